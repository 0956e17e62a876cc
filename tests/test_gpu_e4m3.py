"""The gfx950 hardware E4M3FN conversion the fp8 dispatch uses, on
magnitude-clamped inputs, equals the software round-to-nearest-even
saturating encoder on every non-NaN fp32 pattern, and the CPU oracle's
encoder on random and special values."""
import ctypes
import os

import numpy as np
import pytest
import torch

from oracle import ep_oracle as O

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hip", "libep_e4m3_check.so")


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is not built; run __graft_entry__.build()")
    L = ctypes.CDLL(LIB)
    L.e4m3_check_exhaustive.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    L.e4m3_convert_hw.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    return L


def test_hw_equals_software_on_all_fp32(lib):
    dev = torch.device("cuda:0")
    nbad = torch.zeros(1, dtype=torch.int64, device=dev)
    first = torch.zeros(8, dtype=torch.int32, device=dev)
    s = torch.cuda.current_stream(dev).cuda_stream
    assert lib.e4m3_check_exhaustive(nbad.data_ptr(), first.data_ptr(), s) == 0
    torch.cuda.synchronize()
    n = int(nbad.item())
    assert n == 0, f"{n} patterns differ, first {[hex(v & 0xFFFFFFFF) for v in first.tolist()[:min(n, 8)]]}"


def test_hw_equals_oracle(lib):
    rng = np.random.default_rng(9)
    n = 1 << 22
    bits = (
        (rng.integers(0, 2, n, dtype=np.uint32) << 31)
        | (rng.integers(127 - 14, 127 + 12, n, dtype=np.uint32) << 23)
        | rng.integers(0, 1 << 23, n, dtype=np.uint32)
    )
    t = O.e4m3fn_value_table()
    mids = ((t[:-1] + t[1:]) / 2).astype(np.float32).view(np.uint32)
    special = np.concatenate([mids - 1, mids, mids + 1, t.astype(np.float32).view(np.uint32)])
    special = np.concatenate([special, special | np.uint32(0x80000000)])
    extra = np.array([0.0, -0.0, 448.0, 449.0, 464.0, 1e30, -1e30, 1e-45, -1e-45], np.float32).view(np.uint32)
    f = np.concatenate([bits, special, extra]).view(np.float32)
    want = O.e4m3fn_rne_sat(f)
    dev = torch.device("cuda:0")
    fin = torch.from_numpy(f.copy()).to(dev)
    out = torch.empty(len(f), dtype=torch.uint8, device=dev)
    s = torch.cuda.current_stream(dev).cuda_stream
    assert lib.e4m3_convert_hw(fin.data_ptr(), out.data_ptr(), len(f), s) == 0
    got = out.cpu().numpy()
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, [(hex(f.view(np.uint32)[i]), got[i], want[i]) for i in bad[:8]]
