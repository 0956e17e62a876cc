"""Opt-in parity sweep over thousands of seeded random shapes.

The checks of test_gpu_random_shapes.py (layout, bf16 / fp8 / grouped-row
dispatch, flat and grouped combine, all bit for bit against the oracle) on
- 2 x 2000 shapes from that file's generator (seeds 778 and 779), and
- 600 shapes from a wider one: top-k up to 32, up to 1000 experts with
  E + G within the key limit, up to 3000 tokens, hidden up to 4096 (bf16)
  or 128 * 32 (fp8), up to 95% of selections and 30% of tokens masked,
  expert alignment up to 256 rows (seed 31).
The grouped GEMM, exactly, on 150 seeded shapes of small integers (plain
weights, packed weights, and rows gathered from the token matrix).

About 6 minutes on one MI355X, so it runs only with EP_PARITY_SWEEP=1:
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
    for i, c in enumerate(cases):
        rs.test_random_shape_matches_oracle(c)
        if (i + 1) % 200 == 0:
            print(f"seed {seed}: {i + 1} shapes match", flush=True)
    print(f"seed {seed}: {len(cases)} shapes match the oracle", flush=True)


def _gemm_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        E = int(rng.choice([1, 3, 8, 64, 256, 1000]))
        c = dict(
            T=int(rng.integers(1, 3001)),
            K=int(min(rng.integers(1, 9), E)),
            E=E,
            H=int(64 * rng.integers(1, 65)),
            N=int(128 * rng.integers(1, 17)),
            A=int(rng.choice([0, 0, 8, 32, 256])),
            gather=bool(rng.random() < 0.4),
            seed=9000 + len(out),
        )
        rows = c["T"] * c["K"] + c["E"] * max(c["A"] - 1, 0)
        if c["E"] * c["N"] * c["H"] <= 1 << 28 and rows * c["N"] * c["H"] <= 1 << 33:
            out.append(c)
    return out


def test_gemm_exact_sweep():
    """150 seeded GEMM shapes on integers in [-2, 2] (every fp32 partial sum
    exact): plain weights, packed weights and, for 40% of them, rows
    gathered from the token matrix, each equal bit for bit to the bf16
    rounding of the exact sums (a float64 matmul, exact at these sizes)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import combine_ep_layout_03_amd as ep
    import workloads as W
    from oracle import ep_oracle as O

    dev = torch.device("cuda:0")
    for c in _gemm_cases(150, 4242):
        print("exact gemm", c, flush=True)
        w = W.Workload("gx", T=c["T"], H=c["H"], K=c["K"], E=c["E"], mask_p=0.1, seed=c["seed"])
        idx, _ = W.make_routing(w)
        R = O.layout(idx.numpy(), w.E, expert_alignment=c["A"])
        L = ep.ep_layout(idx.to(dev), w.E, expert_alignment=c["A"], expert_row_src=c["gather"])
        wts = W.make_small_ints(w, (w.E, c["N"], w.H), stream=1)
        n = R["n_rows_expert"]
        if c["gather"]:
            x = W.make_small_ints(w, (w.T, w.H), stream=0)
            xin = O.dispatch_bf16(rs.u16(x), R["slot"], n)
        else:
            x = W.make_small_ints(w, (L.max_expert_rows(), w.H), stream=0)
            xin = rs.u16(x)[:n]
        rows = L.max_expert_rows()
        y = torch.zeros(rows, c["N"], dtype=torch.bfloat16, device=dev)
        yp = torch.zeros_like(y)
        ep.ep_expert_gemm(x.to(dev), L, wts.to(dev), out=y, gather=c["gather"])
        ep.ep_expert_gemm(x.to(dev), L, ep.ep_pack_expert_weights(wts.to(dev)), out=yp, gather=c["gather"])
        torch.cuda.synchronize()
        got, gotp = rs.u16(y)[:n], rs.u16(yp)[:n]
        xf = O.bf16_to_f32(xin).astype(np.float64)
        wf = O.bf16_to_f32(rs.u16(wts)).astype(np.float64)
        for e in range(w.E):
            r0, cnt = int(R["offsets"][e]), int(R["counts"][e])
            if cnt == 0:
                continue
            want = O.bf16_rne((xf[r0 : r0 + cnt] @ wf[e].T).astype(np.float32))
            assert np.array_equal(got[r0 : r0 + cnt], want), f"expert {e} of {c}"
            assert np.array_equal(gotp[r0 : r0 + cnt], want), f"expert {e} of {c} (packed)"
    print("150 GEMM shapes exact", flush=True)
