"""The boundary's data-dependent reports on the GPU, through the C ABI.

- Dispatch overflow: a capacity below the rows the layout needs makes
  ep_dispatch write no row and set EP_STATUS_DISPATCH_OVERFLOW (the PR's
  expand_overflow is known before any payload moves: commit adding DeepEP's
  do_expand); a capacity that fits sets it back to 0 and the rows match the
  oracle.
- Stale layout: an ep_layout_t copied before a later ep_layout on the same
  buffers is a cached handle whose layout is gone (the PR's cached handle=
  dispatch and its _layout_generation check).  Dispatch, combine and the
  grouped GEMM handed it write nothing and set the sticky EP_STATUS_STALE,
  which the next ep_layout clears; a HIP graph captured with the old
  generation is refused the same way on replay.
"""
import ctypes

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


def _stream():
    return torch.cuda.current_stream(DEV).cuda_stream


@pytest.mark.parametrize(
    "fp8,grouped,align",
    [(False, False, 0), (True, False, 0), (False, True, 0), (True, True, 0), (False, False, 16), (True, False, 16)],
)
def test_dispatch_overflow_writes_nothing_and_is_flagged(fp8, grouped, align):
    m = ep()
    w = W.by_name("skewed_masked").replace(T=700, H=256, seed=3)
    print("overflow", fp8, grouped, align, flush=True)
    idx, wt = W.make_routing(w)
    G = 8 if grouped else 0
    L = m.ep_layout(idx.to(DEV), w.E, G, wt.to(DEV), expert_alignment=align)
    rows = m.EP_ROWS_GROUP if grouped else m.EP_ROWS_EXPERT
    need = L.num_rows(rows)
    rb = m.ep_fp8_row_bytes(w.H) if fp8 else 2 * w.H
    x = W.make_x(w).to(DEV)
    poison = torch.full((need, rb), 0xA7, dtype=torch.uint8, device=DEV)
    short = poison[: need - 1]
    dst = short if fp8 else short.view(torch.bfloat16)
    m.ep_dispatch(x, L, fp8=fp8, rows=rows, out=dst, capacity=need - 1, zero_padding=align > 0)
    torch.cuda.synchronize()
    assert L.dispatch_overflowed()
    assert not L.stale_call_seen()
    assert bool((poison == 0xA7).all())
    with pytest.raises(m.EPError):
        m.ep_dispatch(x, L, fp8=fp8, rows=rows, out=dst, capacity=need - 1, check=True)
    # the capacity that fits: flag back to 0, rows as the oracle places them
    full = poison if fp8 else poison.view(torch.bfloat16)
    m.ep_dispatch(x, L, fp8=fp8, rows=rows, out=full, capacity=need, zero_padding=align > 0, check=True)
    torch.cuda.synchronize()
    assert not L.dispatch_overflowed()
    R = O.layout(idx.numpy(), w.E, G, wt.numpy(), expert_alignment=align)
    dest = R["grow"] if grouped else R["slot"]
    xr = u16(x)
    # every row below `need` is a selection's row or zeroed padding
    if fp8:
        want = O.dispatch_fp8(xr, dest, need)
        got = poison.cpu().numpy()
    else:
        want = O.dispatch_bf16(xr, dest, need)
        got = u16(poison.view(torch.bfloat16))
    assert np.array_equal(got, want)


def test_stale_handle_is_refused_on_the_device():
    m = ep()
    lib = m._lib.lib()
    w = W.by_name("mid").replace(T=600, H=256)
    idx, wt = W.make_routing(w)
    idx2, _ = W.make_routing(w.replace(seed=9))
    d_idx, d_wt = idx.to(DEV), wt.to(DEV)
    L = m.ep_layout(d_idx, w.E, expert_row_src=True)
    old = L.struct()  # a cached handle: a copy of the C struct
    assert old.generation != 0
    n = L.num_rows()
    assert L.status_word(m.EP_STATUS_GENERATION) == ctypes.c_int32(old.generation).value
    m.ep_layout(idx2.to(DEV), w.E, out=L)  # the same buffers, another routing
    assert L.generation != old.generation
    x = W.make_x(w).to(DEV)
    y = W.make_y(w, rows=w.T * w.K).to(DEV)
    recv = torch.full((w.T * w.K, w.H), 3.0, dtype=torch.bfloat16, device=DEV)
    out = torch.full((w.T, w.H), 5.0, dtype=torch.bfloat16, device=DEV)
    p = m._lib.Problem(w.T, w.H, w.K, w.E, 0, 0, 0)
    rc = lib.ep_dispatch(ctypes.byref(p), ctypes.byref(old), x.data_ptr(), recv.data_ptr(), w.T * w.K, 0,
                         m.EP_ROWS_EXPERT, m.EP_FORMAT_BF16, _stream())
    assert rc == m._lib.EP_OK
    rc = lib.ep_combine(ctypes.byref(p), ctypes.byref(old), None, d_wt.data_ptr(), y.data_ptr(), y.shape[0],
                        None, None, out.data_ptr(), m.EP_COMBINE_FLAT, _stream())
    assert rc == m._lib.EP_OK
    N = 128
    wts = W.make_expert_weights(w, N, device=DEV)
    yg = torch.full((w.T * w.K, N), 7.0, dtype=torch.bfloat16, device=DEV)
    rc = lib.ep_expert_gemm(ctypes.byref(p), ctypes.byref(old), recv.data_ptr(), 0, wts.data_ptr(), N,
                            yg.data_ptr(), 0, _stream())
    assert rc == m._lib.EP_OK
    torch.cuda.synchronize()
    assert L.stale_call_seen()
    assert bool((recv == 3.0).all()) and bool((out == 5.0).all()) and bool((yg == 7.0).all())
    # the current struct works (the flag stays set until the next layout)
    m.ep_dispatch(x, L, out=recv)
    torch.cuda.synchronize()
    R2 = O.layout(idx2.numpy(), w.E)
    assert np.array_equal(u16(recv)[: R2["n_sel"]], O.dispatch_bf16(u16(x), R2["slot"], R2["n_sel"]))
    assert L.stale_call_seen()
    m.ep_layout(d_idx, w.E, out=L)
    torch.cuda.synchronize()
    assert not L.stale_call_seen()
    assert L.status_word(m.EP_STATUS_GENERATION) == ctypes.c_int32(L.generation).value
    del n


def test_graph_captured_on_an_old_generation_is_refused():
    """A dispatch + combine captured in a graph carries the generation it was
    captured with; after an eager ep_layout rewrites the buffers, replays
    write nothing and flag the layout, and a fresh layout of the original
    routing does not revive them (its generation is new)."""
    m = ep()
    w = W.by_name("mid").replace(T=512, H=512)
    idx, wt = W.make_routing(w)
    d_idx, d_wt = idx.to(DEV), wt.to(DEV)
    x = W.make_x(w, device=DEV)
    y = W.make_y(w, device=DEV)
    L = m.ep_layout(d_idx, w.E)
    recv = torch.zeros(w.T * w.K, w.H, dtype=torch.bfloat16, device=DEV)
    out = torch.zeros(w.T, w.H, dtype=torch.bfloat16, device=DEV)

    def step():
        m.ep_dispatch(x, L, out=recv)
        m.ep_combine(y, L, d_wt, out=out)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    recv.fill_(1.0)
    out.fill_(1.0)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    R = O.layout(idx.numpy(), w.E)
    n = R["n_sel"]
    assert np.array_equal(u16(recv)[:n], O.dispatch_bf16(u16(x), R["slot"], n))
    assert np.array_equal(u16(out), O.combine(u16(y), R["slot"], wt.numpy()))
    assert not L.stale_call_seen()
    for _ in range(2):
        m.ep_layout(d_idx, w.E, out=L)  # same routing, new generation
        recv.fill_(1.0)
        out.fill_(1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert L.stale_call_seen()
        assert bool((recv == 1.0).all()) and bool((out == 1.0).all())
    del g
