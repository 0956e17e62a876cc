"""Opt-in parity sweep over thousands of seeded random shapes: the checks of
test_gpu_random_shapes.py (layout, bf16 / fp8 / grouped-row dispatch, flat
and grouped combine, all bit for bit against the oracle) on

- 2 x 2000 shapes from that file's generator (seeds 778 and 779), and
- 600 shapes from a wider one: top-k up to 32, up to 1000 experts with
  E + G within the key limit, up to 3000 tokens, hidden up to 4096 (bf16)
  or 128 * 32 (fp8), up to 95% of selections and 30% of tokens masked,
  expert alignment up to 256 rows (seed 31).

About 5 minutes on one MI355X, so it runs only with EP_PARITY_SWEEP=1:
    EP_PARITY_SWEEP=1 python -m pytest tests/test_gpu_parity_sweep.py -m gpu
"""
import os

import numpy as np
import pytest
import torch

import test_gpu_random_shapes as rs

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not os.environ.get("EP_PARITY_SWEEP"), reason="opt-in: set EP_PARITY_SWEEP=1"),
]


def _wide_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([2, 5, 16, 64, 96, 128, 256, 512, 1000]))
        K = int(min(rng.integers(1, 33), E))
        divisors = [g for g in range(1, E + 1) if E % g == 0 and E + g <= 1024]
        G = int(rng.choice(divisors)) if rng.random() < 0.5 else 0
        fp8 = rng.random() < 0.5
        H = int(128 * rng.integers(1, 33)) if fp8 else int(rng.integers(1, 4097))
        T = int(rng.integers(0, 3001))
        routing = "zipf" if rng.random() < 0.3 else "uniform"
        case = dict(
            name=f"w{i}",
            T=T,
            H=H,
            K=K,
            E=E,
            G=max(G, 1),
            routing=routing,
            zipf_s=1.2 if routing == "zipf" else 0.0,
            mask_p=float(rng.choice([0.0, 0.1, 0.5, 0.95])),
            full_mask_frac=float(rng.choice([0.0, 0.05, 0.3])),
            seed=5000 + i,
            groups=G,
            align=int(rng.choice([0, 0, 2, 16, 128, 256])),
        )
        if T > 0:  # T = 0 is covered by the edge-shape tests
            out.append(case)
    return out


@pytest.mark.parametrize("seed,n,wide", [(778, 2000, False), (779, 2000, False), (31, 600, True)])
def test_parity_sweep(seed, n, wide):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cases = _wide_cases(n, seed) if wide else rs._cases(n=n, seed=seed)
    for c in cases:
        rs.test_random_shape_matches_oracle(c)
    print(f"seed {seed}: {len(cases)} shapes match the oracle", flush=True)
