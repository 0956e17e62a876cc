"""The C ABI from plain C: tests/c/ep_c_roundtrip.c (C99, built by gcc
against include/ep_mi355x.h alone) runs layout, bf16 dispatch and combine on
the GPU and checks closed forms: status words, slots forming a permutation,
the unit-weight combine of the dispatched rows equal to K_eff * x, the packed
fp8 rows byte for byte (scale 2^-6 and payload codes of 64 * x), grouped rows,
their row lists and the grouped-order combine, and the grouped GEMM on small
integers (plain and packed weights) equal to the bf16 rounding of the exact
sums; and the allocation-free layout equal to ep_layout's."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "c", "ep_c_roundtrip")

pytestmark = pytest.mark.gpu


def test_c_program_round_trip():
    import torch

    if torch.cuda.device_count() < 1:
        pytest.skip("no GPU")
    assert os.path.exists(BIN), "tests/c/ep_c_roundtrip is not built: run __graft_entry__.build()"
    print("running", BIN, flush=True)
    res = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(res.stdout, res.stderr, flush=True)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("OK")
