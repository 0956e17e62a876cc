"""Parity at the bench's full size, in the launch configuration bench.py
times: 8192 tokens x 7168, top-8 of 256 experts.  The headline step's ops
are covered in test_gpu_parity.py; these are the extras timed beside it --
grouped combine over 8 groups, grouped fp8 dispatch, fp8 dispatch into
128-row-aligned segments with zeroed padding, and combine seeded by two bias
rows -- each run exactly as the bench runs it (same calls, same 7424-byte
receive pitch) and checked against the oracle on every token or row (the
oracle runs over token chunks, slots renumbered per chunk, so host memory
stays bounded)."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import ep_oracle as O

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def ep():
    import combine_ep_layout_03_amd as m

    return m


def u16(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def pages():
    w = W.by_name("pages")
    idx, wt = W.make_routing(w)
    return {
        "w": w,
        "idx": idx,
        "wt": wt,
        "d_idx": idx.to(DEV),
        "d_wt": wt.to(DEV),
        "x": W.make_x(w, device=DEV),
        "y": W.make_y(w, device=DEV),
        "pitch": ep().fp8_row_pitch(w.H),
    }


CHUNK = 2048


def _sub_slots(slot_rows):
    """A token chunk's slots renumbered over the rows they use."""
    used = np.unique(slot_rows[slot_rows >= 0])
    remap = -np.ones(int(slot_rows.max(initial=-1)) + 2, np.int64)
    remap[used] = np.arange(len(used))
    return used, np.where(slot_rows >= 0, remap[np.maximum(slot_rows, 0)], -1)


def test_combine_grouped_g8_full_size(pages):
    P = pages
    w = P["w"]
    say("bench config: grouped combine, G = 8")
    L = ep().ep_layout(P["d_idx"], w.E, 8, P["d_wt"])
    out = torch.empty(w.T, w.H, dtype=torch.bfloat16, device=DEV)
    ep().ep_combine(P["y"], L, P["d_wt"], P["d_idx"], order=ep().EP_COMBINE_GROUPED, out=out)
    torch.cuda.synchronize()
    R = O.layout(P["idx"].numpy(), w.E, 8, P["wt"].numpy())
    idx, wt = P["idx"].numpy(), P["wt"].numpy()
    for t0 in range(0, w.T, CHUNK):
        used, slot_r = _sub_slots(R["slot"][t0:t0 + CHUNK])
        ysub = u16(P["y"].index_select(0, torch.from_numpy(used).to(DEV)))
        want = O.combine_grouped(ysub, idx[t0:t0 + CHUNK], slot_r, wt[t0:t0 + CHUNK], w.E, 8)
        assert np.array_equal(u16(out[t0:t0 + CHUNK]), want), t0


def test_dispatch_fp8_grouped_rows_full_size(pages):
    """Every grouped fp8 row (payload, scales and zero pad bytes)."""
    P = pages
    w = P["w"]
    say("bench config: grouped fp8 dispatch, G = 8, 7424-byte pitch")
    LG = ep().ep_layout(P["d_idx"], w.E, 8, P["d_wt"])
    R = LG.num_rows(ep().EP_ROWS_GROUP)
    recv = torch.empty(max(R, 1), P["pitch"], dtype=torch.uint8, device=DEV)
    ep().ep_dispatch(P["x"], LG, fp8=True, rows=ep().EP_ROWS_GROUP, out=recv, capacity=R)
    RO = O.layout(P["idx"].numpy(), w.E, 8, P["wt"].numpy())
    assert R == RO["n_rows"]
    rb = O.fp8_row_bytes(w.H)
    want = O.dispatch_fp8(u16(P["x"]), RO["grow"], R)
    got = recv[:R, :rb].cpu().numpy()
    assert np.array_equal(got, want)
    # 7424-byte pitch: each row is zero-filled from its end to its 128-byte line end
    assert bool((recv[:R, rb:] == 0).all())


def test_dispatch_fp8_align128_zero_padding_full_size(pages):
    """Every row of the 128-aligned segments: selections are the packed fp8
    rows, padding rows are zero bytes (the oracle's zero-padding form)."""
    P = pages
    w = P["w"]
    say("bench config: fp8 dispatch into 128-aligned segments, zeroed padding")
    LA = ep().ep_layout(P["d_idx"], w.E, expert_alignment=128)
    n_al = LA.num_rows()
    recv = torch.full((LA.max_expert_rows(), P["pitch"]), 0xA5, dtype=torch.uint8, device=DEV)
    ep().ep_dispatch(P["x"], LA, fp8=True, out=recv, zero_padding=True)
    RO = O.layout(P["idx"].numpy(), w.E, expert_alignment=128)
    assert n_al == len(RO["expert_row_src"])
    rb = O.fp8_row_bytes(w.H)
    want = O.dispatch_fp8(u16(P["x"]), RO["slot"], n_al)
    got = recv[:n_al, :rb].cpu().numpy()
    assert np.array_equal(got, want)
    # selections and padding rows alike are zero-filled to the 7424-byte line end
    assert bool((recv[:n_al, rb:] == 0).all())
    # rows past the layout's rows are never touched
    assert bool((recv[n_al:] == 0xA5).all())


def test_combine_bias2_full_size(pages):
    P = pages
    w = P["w"]
    say("bench config: combine seeded by two bias rows")
    L = ep().ep_layout(P["d_idx"], w.E)
    g = torch.Generator(device=DEV)
    g.manual_seed(77)
    b0 = torch.randn(w.T, w.H, generator=g, device=DEV).to(torch.bfloat16)
    b1 = torch.randn(w.T, w.H, generator=g, device=DEV).to(torch.bfloat16)
    out = torch.empty(w.T, w.H, dtype=torch.bfloat16, device=DEV)
    ep().ep_combine(P["y"], L, P["d_wt"], out=out, bias0=b0, bias1=b1)
    torch.cuda.synchronize()
    R = O.layout(P["idx"].numpy(), w.E)
    wt = P["wt"].numpy()
    for t0 in range(0, w.T, CHUNK):
        t1 = min(t0 + CHUNK, w.T)
        used, slot_r = _sub_slots(R["slot"][t0:t1])
        ysub = u16(P["y"].index_select(0, torch.from_numpy(used).to(DEV)))
        want = O.combine(ysub, slot_r, wt[t0:t1], bias0=u16(b0[t0:t1]), bias1=u16(b1[t0:t1]))
        assert np.array_equal(u16(out[t0:t1]), want), t0
