"""ep_layout_noalloc, the layout entry point that allocates nothing, against
ep_layout with a caller workspace, through the C ABI.

The allocation-free call keeps its per-block tallies in the library's fixed
per-GPU scratch array instead of a workspace argument; every output must be
the same bytes as ep_layout's on the same routing.  Calls run back to back,
each later one smaller than the one before, so tallies a larger call left in
the shared scratch must not leak into a smaller one.  The largest workspace
any problem needs is checked through the allocation-free call too.
"""
import ctypes

import numpy as np
import pytest
import torch

import workloads as W

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


# layout outputs compared in full (status separately: its generation word differs)
FIELDS = ("counts", "offsets", "slot", "group_counts", "group_offsets", "grow", "row_src",
          "row_topk_idx", "row_topk_weights", "expert_row_src")


def _routing(T, K, E, seed, mask_p=0.0, routing="uniform"):
    w = W.Workload("noalloc", T=T, H=128, K=K, E=E, routing=routing, zipf_s=1.2 if routing == "zipf" else 0.0,
                   mask_p=mask_p, seed=seed)
    idx, wt = W.make_routing(w)
    return idx.to(DEV), wt.to(DEV)


# row lists hold defined values only in the rows the layout produced
ROW_LISTS = {"expert_row_src": "expert", "row_src": "group", "row_topk_idx": "group",
             "row_topk_weights": "group"}


def _compare(ref, got):
    m = ep()
    torch.cuda.synchronize()
    sa, sb = ref.status.cpu().numpy(), got.status.cpu().numpy()
    rows = {"expert": int(sa[m.EP_STATUS_ROWS_EXPERT]), "group": int(sa[m.EP_STATUS_ROWS_GROUP])}
    for f in FIELDS:
        a, b = getattr(ref, f), getattr(got, f)
        if a is None:
            assert b is None, f
            continue
        if f == "row_topk_weights":
            a, b = a.view(torch.int32), b.view(torch.int32)
        if f in ROW_LISTS:
            n = rows[ROW_LISTS[f]]
            a, b = a[:n], b[:n]
        assert torch.equal(a, b), f
    keep = np.arange(m.EP_STATUS_WORDS) != m.EP_STATUS_GENERATION
    assert np.array_equal(sa[keep], sb[keep])
    assert int(sb[m.EP_STATUS_GENERATION]) & 0xFFFFFFFF == got.generation


# (T, K, E, G, alignment, mask_p, routing): each case smaller than the one before
SEQUENCES = {
    "grouped": [(65536, 8, 256, 8, 0, 0.0, "uniform"), (3001, 8, 256, 8, 0, 0.1, "uniform")],
    "flat": [(8192, 8, 256, 0, 0, 0.0, "uniform"), (777, 6, 64, 0, 16, 0.1, "zipf")],
    "wide_keys": [(40000, 4, 448, 64, 0, 0.05, "zipf"), (512, 4, 448, 64, 0, 0.0, "uniform")],
}


@pytest.mark.parametrize("name", sorted(SEQUENCES))
def test_noalloc_layout_equals_workspace_layout(name):
    m = ep()
    for i, (T, K, E, G, A, mask_p, routing) in enumerate(SEQUENCES[name]):
        print(f"noalloc {name} call {i}: T={T} K={K} E={E} G={G} A={A}", flush=True)
        idx, wt = _routing(T, K, E, seed=11 + i, mask_p=mask_p, routing=routing)
        ref = m.ep_layout(idx, E, num_groups=G, topk_weights=wt, expert_alignment=A, expert_row_src=True)
        got = m.alloc_layout(T, K, E, num_groups=G, expert_alignment=A, expert_row_src=True, device=DEV)
        # poison the outputs so an unwritten word cannot match by accident
        for f in FIELDS + ("status",):
            t = getattr(got, f)
            if t is not None:
                t.view(torch.int32).fill_(-7777)
        m.ep_layout_noalloc(idx, E, got, topk_weights=wt)
        _compare(ref, got)
        # the scratch is reused as is by the next call on the same buffers
        m.ep_layout_noalloc(idx, E, got, topk_weights=wt)
        _compare(ref, got)


def test_noalloc_layout_feeds_dispatch_and_combine():
    """A layout from the allocation-free call drives dispatch and combine to
    the same bytes as one from ep_layout."""
    m = ep()
    w = W.by_name("pages").replace(T=2048, H=512, fp8=False)
    idx, wt = (t.to(DEV) for t in W.make_routing(w))
    x = W.make_x(w).to(DEV)
    y = W.make_y(w).to(DEV)
    ref = m.ep_layout(idx, w.E)
    got = m.alloc_layout(w.T, w.K, w.E, device=DEV)
    m.ep_layout_noalloc(idx, w.E, got)
    r1 = m.ep_dispatch(x, ref, fp8=True)
    r2 = m.ep_dispatch(x, got, fp8=True)
    o1 = m.ep_combine(y, ref, wt)
    o2 = m.ep_combine(y, got, wt)
    torch.cuda.synchronize()
    assert torch.equal(r1, r2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_noalloc_at_the_largest_workspace():
    """The shape whose tallies fill the scratch the most (1024 experts, 16,384
    tokens x top-8: 2,230,528 bytes of the 2.25 MiB array) gives the same
    layout as ep_layout with its own workspace."""
    m = ep()
    from combine_ep_layout_03_amd import _lib

    T, K, E = 16384, 8, 1024
    assert m.ep_layout_workspace_bytes(T, K, E) == 2230528 <= _lib.EP_LAYOUT_SCRATCH_BYTES
    idx, _ = _routing(T, K, E, seed=21, mask_p=0.05, routing="zipf")
    ref = m.ep_layout(idx, E)
    got = m.alloc_layout(T, K, E, device=DEV)
    got.status.fill_(-5)
    m.ep_layout_noalloc(idx, E, got)
    _compare(ref, got)


def test_noalloc_through_the_raw_c_call():
    """The export called with a hand-built ep_layout_t (no binding logic)."""
    m = ep()
    from combine_ep_layout_03_amd import _lib

    T, K, E = 1000, 4, 32
    idx, _ = _routing(T, K, E, seed=5, mask_p=0.2)
    ref = m.ep_layout(idx, E)
    got = m.alloc_layout(T, K, E, device=DEV)
    s = got.struct()
    p = _lib.Problem(T, 1, K, E, 0, 0, 0)
    rc = _lib.lib().ep_layout_noalloc(ctypes.byref(p), idx.data_ptr(), None, ctypes.byref(s),
                                      torch.cuda.current_stream(DEV).cuda_stream)
    assert rc == _lib.EP_OK
    got.generation = int(s.generation)
    _compare(ref, got)
