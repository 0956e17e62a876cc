"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Integer layouts, row placement, bf16 rows, fp8 payload/scale bytes and the
bf16 combine output are compared bit for bit: the combine's fp32 order is
fixed, so its tolerance is zero.  Small cases are compared in full; the
workload shapes are compared in full where the oracle finishes in seconds
and on sampled rows / tokens otherwise (the grouped 65536-token case).
"""
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
    import combine_ep_layout_03_amd as ep  # noqa: F401  (fails loudly if not built)

    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def ep():
    import combine_ep_layout_03_amd as m

    return m


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def say(*a):
    print(*a, flush=True)


def check_layout(L, R, E, G=0):
    torch.cuda.synchronize()
    assert np.array_equal(L.counts.cpu().numpy(), R["counts"])
    assert np.array_equal(L.offsets.cpu().numpy(), R["offsets"])
    assert np.array_equal(L.slot.cpu().numpy(), R["slot"])
    st = L.status.cpu().numpy()
    assert st[0] == R["n_invalid"] and st[1] == R["n_sel"]
    if G:
        assert st[2] == R["n_rows"]
        assert np.array_equal(L.group_counts.cpu().numpy(), R["gcounts"])
        assert np.array_equal(L.group_offsets.cpu().numpy(), R["goffsets"])
        assert np.array_equal(L.grow.cpu().numpy(), R["grow"])
        if st[3] == 0:
            n = R["n_rows"]
            assert np.array_equal(L.row_src[:n].cpu().numpy(), R["src"])
            assert np.array_equal(L.row_topk_idx[:n].cpu().numpy(), R["ridx"])
            assert np.array_equal(L.row_topk_weights[:n].cpu().numpy().view(np.uint32), R["rw"].view(np.uint32))
    else:
        assert st[2] == 0


# --------------------------------------------------------------------------- layout
@pytest.mark.parametrize("name", ["tiny", "mid", "pages", "skewed_masked", "grouped"])
def test_layout_workloads(name):
    w = W.by_name(name)
    say("layout", name, w.T, w.K, w.E, w.G)
    idx, wt = W.make_routing(w)
    G = w.G if w.G > 1 else 0
    R = O.layout(idx.numpy(), w.E, G, wt.numpy())
    L = ep().ep_layout(idx.to(DEV), w.E, G, wt.to(DEV) if G else None)
    check_layout(L, R, w.E, G)


@pytest.mark.parametrize(
    "T,K,E,G,mask",
    [
        (0, 8, 256, 0, 0.0),
        (0, 8, 256, 8, 0.0),
        (1, 1, 1, 0, 0.0),
        (5, 3, 7, 0, 0.3),
        (777, 6, 96, 0, 0.2),  # K does not divide a wave; ragged last block
        (1000, 8, 64, 1, 0.1),  # one group: one row per active token
        (1000, 8, 64, 64, 0.1),  # a group per expert
        (513, 5, 40, 8, 0.25),
        (20000, 8, 256, 8, 0.05),  # several rounds per block
        (3000, 32, 512, 16, 0.0),  # K at the limit
        (2000, 4, 1000, 0, 0.0),  # E near the key limit
        (2000, 4, 1024, 0, 0.0),  # E + G at the key limit
        (2000, 4, 992, 32, 0.1),  # E + G at the key limit, grouped
        # count-block geometry: 16-bit tallies (1025 tally columns, more
        # entries than 32-bit tallies admit), K not dividing a wave
        (20000, 7, 992, 32, 0.1),
        # 16-bit tallies with the lane test (K = 8, 8 groups), 512 place blocks
        (16384, 8, 1016, 8, 0.05),
        # 16 rounds per place block, 30 count blocks, 17 tally columns
        (300000, 4, 16, 0, 0.1),
        # K = 16: a token fills a 16-lane row; group bits by row shifts
        (3000, 16, 256, 16, 0.1),
        # up to 2048 entries one block tallies and places everything (1, 2,
        # 4 and 8 rounds); 2056 entries is the first two-launch size
        (32, 8, 64, 8, 0.1),
        (33, 8, 64, 8, 0.1),
        (100, 7, 48, 6, 0.2),
        (256, 8, 1016, 8, 0.05),
        (682, 3, 100, 0, 0.3),
        (64, 32, 512, 16, 0.1),  # fused, K = 32: group tests by LDS permutes
        (100, 13, 96, 8, 0.1),  # fused, K not dividing a wave: per-lane path
        (257, 8, 256, 0, 0.1),
    ],
)
def test_layout_edge_shapes(T, K, E, G, mask):
    say("layout edge", T, K, E, G, mask)
    w = W.Workload("edge", T=T, H=8, K=K, E=E, G=max(G, 1), mask_p=mask, seed=T + K + E)
    if T:
        idx, wt = W.make_routing(w)
    else:
        idx, wt = torch.zeros(0, K, dtype=torch.int64), torch.zeros(0, K)
    R = O.layout(idx.numpy(), E, G, wt.numpy())
    L = ep().ep_layout(idx.to(DEV), E, G, wt.to(DEV) if G else None)
    check_layout(L, R, E, G)


@pytest.mark.parametrize("T", [3000, 200])  # two launches; one fused block
def test_layout_invalid_and_duplicate_ids(T):
    g = torch.Generator().manual_seed(11)
    K, E = 8, 64
    idx = torch.randint(-3, E + 3, (T, K), generator=g)  # -3,-2,E.. invalid; duplicates allowed
    wt = torch.rand(T, K, generator=g)
    for G in (0, 8):
        R = O.layout(idx.numpy(), E, G, wt.numpy())
        L = ep().ep_layout(idx.to(DEV), E, G, wt.to(DEV) if G else None)
        check_layout(L, R, E, G)
        assert R["n_invalid"] > 0


def test_layout_list_overflow_reported():
    w = W.by_name("grouped").replace(T=4000)
    idx, wt = W.make_routing(w)
    R = O.layout(idx.numpy(), w.E, w.G, wt.numpy())
    L = ep().ep_layout(idx.to(DEV), w.E, w.G, wt.to(DEV), row_capacity=R["n_rows"] - 1)
    torch.cuda.synchronize()
    assert L.status[3].item() == 1
    assert np.array_equal(L.grow.cpu().numpy(), R["grow"])


def test_layout_repeat_bit_identical():
    w = W.by_name("skewed_masked")
    idx, wt = W.make_routing(w)
    d_idx, d_wt = idx.to(DEV), wt.to(DEV)
    L0 = ep().ep_layout(d_idx, w.E, 8, d_wt)
    n = L0.num_rows(ep().EP_ROWS_GROUP)

    def outs(L):
        # row lists hold n rows; the rest of their capacity is never written.
        # Every status word but the generation stamp (a new one per call).
        st = L.status.clone()
        st[ep().EP_STATUS_GENERATION] = 0
        return (L.slot, L.grow, L.row_src[:n], L.row_topk_idx[:n], L.row_topk_weights[:n], st)

    ref = [t.clone() for t in outs(L0)]
    for _ in range(200):
        L = ep().ep_layout(d_idx, w.E, 8, d_wt)
        for a, b in zip(ref, outs(L)):
            assert torch.equal(a, b)


# --------------------------------------------------------------------------- dispatch
def _dispatch_case(w, fp8=False, x=None, x_offset=0):
    idx, wt = W.make_routing(w)
    if x is None:
        x = W.make_x(w)
    R = O.layout(idx.numpy(), w.E)
    L = ep().ep_layout(idx.to(DEV), w.E)
    if x_offset:
        buf = torch.empty(w.T * w.H + x_offset, dtype=torch.bfloat16, device=DEV)
        xd = buf[x_offset:].view(w.T, w.H)
        xd.copy_(x)
    else:
        xd = x.to(DEV)
    recv = ep().ep_dispatch(xd, L, fp8=fp8)
    n = R["n_sel"]
    xr = u16(x)
    if fp8:
        want = O.dispatch_fp8(xr, R["slot"], n)
        got = recv[:n].cpu().numpy()
    else:
        want = O.dispatch_bf16(xr, R["slot"], n)
        got = u16(recv[:n])
    assert got.shape == want.shape
    assert np.array_equal(got, want)
    return L, R, recv


@pytest.mark.parametrize("H", [1, 2, 3, 5, 7, 8, 9, 127, 129, 136, 7168])
def test_dispatch_bf16_tails(H):
    say("dispatch bf16 H", H)
    _dispatch_case(W.Workload("tail", T=300, H=H, K=4, E=16, mask_p=0.1, seed=H))


@pytest.mark.parametrize("off", [1, 2, 4])
def test_dispatch_bf16_misaligned_base(off):
    _dispatch_case(W.Workload("mis", T=200, H=64, K=3, E=10, seed=off), x_offset=off)


@pytest.mark.parametrize("name", ["tiny", "mid", "skewed_masked"])
def test_dispatch_bf16_workloads(name):
    say("dispatch bf16", name)
    _dispatch_case(W.by_name(name))


def test_dispatch_bf16_pages_shape():
    say("dispatch bf16 pages shape")
    _dispatch_case(W.by_name("pages").replace(fp8=False))


def test_dispatch_fp8_pages_shape():
    say("dispatch fp8 pages shape")
    _dispatch_case(W.by_name("pages"), fp8=True)


@pytest.mark.parametrize("H", [128, 256, 1152, 2048])
def test_dispatch_fp8_small_hidden(H):
    _dispatch_case(W.Workload("fp8h", T=257, H=H, K=4, E=32, mask_p=0.1, seed=H), fp8=True)


def _special_fp8_rows(H=1024):
    """Rows that exercise every corner of the packed fp8 cast.

    Groups: all zeros; one group per bf16 bit pattern block with a 448
    element (scale exactly 1, so the payload is the E4M3FN code of the bf16
    value itself: together the rows cover every finite bf16 of magnitude
    <= 448); tiny values whose scale is subnormal; -0.0; values exactly on
    E4M3FN midpoints."""
    rows = []
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = O.bf16_to_f32(allb)
    keep = allb[np.isfinite(f) & (np.abs(f) <= 448.0)]
    per = 127
    b448 = O.bf16_rne(np.array([448.0], np.float32))[0]
    groups = []
    for i in range(0, len(keep), per):
        g = np.full(128, b448, np.uint16)
        chunk = keep[i : i + per]
        g[1 : 1 + len(chunk)] = chunk
        groups.append(g)
    groups.append(np.zeros(128, np.uint16))  # scale 0
    groups.append(np.full(128, 0x8000, np.uint16))  # -0.0
    tiny = O.bf16_rne(np.linspace(-1e-38, 1e-38, 128).astype(np.float32))
    groups.append(tiny)  # subnormal scale
    t = O.e4m3fn_value_table()
    mids = O.bf16_rne(((t[:-1] + t[1:]) / 2).astype(np.float32))
    g = np.full(128, b448, np.uint16)
    g[1 : 1 + len(mids)] = mids
    groups.append(g)
    flat = np.concatenate(groups)
    pad = (-len(flat)) % H
    flat = np.concatenate([flat, np.zeros(pad, np.uint16)])
    return flat.reshape(-1, H)


@pytest.mark.parametrize("H", [8320, 16384, 32768])
def test_dispatch_fp8_wide_hidden(H):
    """Rows wider than 8192 elements take the kernel's step-by-step store
    path (8320: nine steps, the last one partly active; 32768: the largest
    supported row, 256 scale groups)."""
    T = 150 if H < 32768 else 60
    _dispatch_case(W.Workload("fp8w", T=T, H=H, K=4, E=16, mask_p=0.1, seed=H), fp8=True)


@pytest.mark.parametrize("H", [1024, 9216])
def test_dispatch_fp8_special_values(H):
    xs = _special_fp8_rows(H)
    T, H = xs.shape
    w = W.Workload("fp8s", T=T, H=H, K=2, E=4)
    x = torch.from_numpy(xs.view(np.int16)).view(torch.bfloat16)
    _dispatch_case(w, fp8=True, x=x)


def test_dispatch_poison_and_capacity():
    w = W.by_name("skewed_masked").replace(T=1500, H=520)
    idx, _ = W.make_routing(w)
    x = W.make_x(w).to(DEV)
    L = ep().ep_layout(idx.to(DEV), w.E)
    n = L.num_rows()
    cap = w.T * w.K
    out = torch.full((cap, w.H), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    ep().ep_dispatch(x, L, out=out)
    torch.cuda.synchronize()
    tail = out[n:].view(torch.int16)
    assert bool((tail == -1).all()), "rows past N_sel were written"
    assert not bool((out[:n].view(torch.int16) == -1).all(dim=1).any()), "a row below N_sel was not written"
    # capacity below the rows needed: nothing is written at all
    out2 = torch.full((n - 1, w.H), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    ep().ep_dispatch(x, L, capacity=n - 1, out=out2)
    rb = ep().ep_fp8_row_bytes(512)
    out3 = torch.full((n - 1, rb), 0xAB, dtype=torch.uint8, device=DEV)
    w2 = w.replace(H=512)
    ep().ep_dispatch(W.make_x(w2).to(DEV), L, fp8=True, capacity=n - 1, out=out3)
    torch.cuda.synchronize()
    assert bool((out2.view(torch.int16) == -1).all())
    assert bool((out3 == 0xAB).all())


def fp8_line_fill_end(rb: int, pitch: int, base_ptr: int) -> int:
    """Where ep_dispatch's fp8 zero fill ends inside a row: the next 128-byte
    boundary when the receive base and the pitch are both multiples of 128
    (never past the pitch), otherwise the packed row's own end."""
    if base_ptr % 128 == 0 and pitch % 128 == 0:
        return min(pitch, (rb + 127) // 128 * 128)
    return rb


@pytest.mark.parametrize("fp8,H,pitch", [(True, 7168, 7424), (True, 128, 256), (True, 128, 384), (True, 384, 416),
                                         (False, 136, 512), (False, 9, 20)])
def test_dispatch_row_pitch(fp8, H, pitch):
    """Rows at a padded pitch: row bytes equal the oracle's; fp8 rows on
    128-byte lines are zero-filled to their line end; every other gap byte
    is untouched."""
    say("dispatch pitch", fp8, H, pitch)
    w = W.Workload("pitch", T=700 if H > 1000 else 1500, H=H, K=8, E=64, mask_p=0.1, seed=H + pitch)
    idx, _ = W.make_routing(w)
    x = W.make_x(w)
    R = O.layout(idx.numpy(), w.E)
    L = ep().ep_layout(idx.to(DEV), w.E)
    n = R["n_sel"]
    cap = w.T * w.K
    if fp8:
        rb = O.fp8_row_bytes(H)
        out = torch.full((cap, pitch), 0xA5, dtype=torch.uint8, device=DEV)
        ep().ep_dispatch(x.to(DEV), L, fp8=True, out=out)
        fe = fp8_line_fill_end(rb, pitch, out.data_ptr())
        assert fe == (rb if pitch % 128 else min(pitch, (rb + 127) // 128 * 128))  # torch bases are 128-aligned
        got = out.cpu().numpy()
        want = O.dispatch_fp8(u16(x), R["slot"], n)
        assert np.array_equal(got[:n, :rb], want)
        assert (got[:n, rb:fe] == 0).all()
        assert (got[:n, fe:] == 0xA5).all() and (got[n:] == 0xA5).all()
    else:
        out = torch.full((cap, pitch // 2), -23131, dtype=torch.int16, device=DEV)  # 0xA5A5
        ep().ep_dispatch(x.to(DEV), L, out=out.view(torch.bfloat16))
        got = out.cpu().numpy().view(np.uint16)
        want = O.dispatch_bf16(u16(x), R["slot"], n)
        assert np.array_equal(got[:n, :H], want)
        assert (got[:n, H:] == 0xA5A5).all() and (got[n:] == 0xA5A5).all()


def test_dispatch_grouped_rows_small():
    w = W.by_name("grouped").replace(T=3000, H=264, mask_p=0.1)
    idx, wt = W.make_routing(w)
    x = W.make_x(w)
    R = O.layout(idx.numpy(), w.E, w.G, wt.numpy())
    L = ep().ep_layout(idx.to(DEV), w.E, w.G, wt.to(DEV))
    recv = ep().ep_dispatch(x.to(DEV), L, rows=ep().EP_ROWS_GROUP)
    n = R["n_rows"]
    assert np.array_equal(u16(recv[:n]), O.dispatch_bf16(u16(x), R["grow"], n))
    w8 = w.replace(H=256)
    x8 = W.make_x(w8)
    recv8 = ep().ep_dispatch(x8.to(DEV), L, fp8=True, rows=ep().EP_ROWS_GROUP)
    assert np.array_equal(recv8[:n].cpu().numpy(), O.dispatch_fp8(u16(x8), R["grow"], n))


def test_dispatch_repeat_bit_identical():
    w = W.by_name("mid")
    idx, _ = W.make_routing(w)
    x = W.make_x(w).to(DEV)
    L = ep().ep_layout(idx.to(DEV), w.E)
    ref = ep().ep_dispatch(x, L).clone()
    out = torch.empty_like(ref)
    for _ in range(100):
        ep().ep_dispatch(x, L, out=out)
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_step_repeat_1000_bit_identical():
    """The whole step (layout, fp8 dispatch, combine) run 1000 times back to
    back on one stream: every run's slots, receive bytes and combine output
    equal the first run's (mismatches are counted on the device and checked
    once at the end)."""
    w = W.by_name("mid").replace(mask_p=0.05)
    idx, wt = W.make_routing(w)
    d_idx, d_wt = idx.to(DEV), wt.to(DEV)
    x = W.make_x(w).to(DEV)
    y = W.make_y(w).to(DEV)
    L = ep().ep_layout(d_idx, w.E)
    recv = ep().ep_dispatch(x, L, fp8=True)
    out = ep().ep_combine(y, L, d_wt)
    torch.cuda.synchronize()
    slot0, recv0, out0 = L.slot.clone(), recv.clone(), out.clone()
    n = L.num_rows()
    bad = torch.zeros((), dtype=torch.int64, device=DEV)
    for _ in range(1000):
        ep().ep_layout(d_idx, w.E, out=L)
        ep().ep_dispatch(x, L, fp8=True, out=recv)
        ep().ep_combine(y, L, d_wt, out=out)
        bad += (L.slot != slot0).sum() + (recv[:n] != recv0[:n]).sum()
        bad += (out.view(torch.int16) != out0.view(torch.int16)).sum()
    torch.cuda.synchronize()
    assert int(bad.item()) == 0


# --------------------------------------------------------------------------- combine
def _combine_case(w, y=None, grouped=False, G=0):
    idx, wt = W.make_routing(w)
    R = O.layout(idx.numpy(), w.E, G, wt.numpy())
    L = ep().ep_layout(idx.to(DEV), w.E, G, wt.to(DEV) if G else None)
    if y is None:
        y = W.make_y(w, rows=max(R["n_sel"], 1))
    order = ep().EP_COMBINE_GROUPED if grouped else ep().EP_COMBINE_FLAT
    out = ep().ep_combine(y.to(DEV), L, wt.to(DEV), idx.to(DEV), order=order)
    yr = u16(y)
    if grouped:
        want = O.combine_grouped(yr, idx.numpy(), R["slot"], wt.numpy(), w.E, G)
    else:
        want = O.combine(yr, R["slot"], wt.numpy())
    got = u16(out)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}"
    return out


def test_combine_tiny_scaled_rows():
    w = W.by_name("tiny")
    idx, wt = W.make_routing(w)
    x = W.make_x(w)
    R = O.layout(idx.numpy(), w.E)
    L = ep().ep_layout(idx.to(DEV), w.E)
    recv = ep().ep_dispatch(x.to(DEV), L)[: R["n_sel"]]
    row_e = np.searchsorted(R["offsets"], np.arange(R["n_sel"]), side="right") - 1
    y = W.tiny_expert_outputs(recv.cpu(), torch.from_numpy(row_e))
    out = ep().ep_combine(y.to(DEV), L, wt.to(DEV))
    assert np.array_equal(u16(out), O.combine(u16(y), R["slot"], wt.numpy()))


@pytest.mark.parametrize("H", [1, 3, 5, 8, 9, 129, 7168])
def test_combine_tails(H):
    say("combine H", H)
    _combine_case(W.Workload("ctail", T=300, H=H, K=4, E=16, mask_p=0.2, seed=H))


@pytest.mark.parametrize("K", [1, 2, 3, 8, 13, 32])
def test_combine_topk_range(K):
    _combine_case(W.Workload("ck", T=200, H=64, K=K, E=64, mask_p=0.1, seed=K))


@pytest.mark.parametrize("name", ["mid", "skewed_masked"])
def test_combine_workloads(name):
    say("combine", name)
    _combine_case(W.by_name(name))


def test_combine_pages_shape():
    say("combine pages shape")
    _combine_case(W.by_name("pages"))


@pytest.mark.parametrize("G", [1, 2, 8, 64])
def test_combine_grouped_small(G):
    _combine_case(W.Workload("cg", T=500, H=136, K=8, E=64, mask_p=0.15, seed=G), grouped=True, G=G)


def test_combine_fully_masked_and_oob():
    w = W.Workload("cm", T=64, H=32, K=4, E=8)
    idx, wt = W.make_routing(w)
    idx[5] = -1
    idx[9] = -1
    L = ep().ep_layout(idx.to(DEV), w.E)
    n = L.num_rows()
    y = W.make_y(w, rows=n).to(DEV)
    out = ep().ep_combine(y, L, wt.to(DEV))
    torch.cuda.synchronize()
    assert bool((out[5].view(torch.int16) == 0).all()) and bool((out[9].view(torch.int16) == 0).all())
    assert L.status[ep().EP_STATUS_COMBINE_OOB].item() == 0
    # y shorter than the rows the layout needs: those rows are skipped and reported
    ep().ep_combine(y[: n // 2], L, wt.to(DEV))
    torch.cuda.synchronize()
    assert L.status[ep().EP_STATUS_COMBINE_OOB].item() == 1


# --------------------------------------------------------------------------- grouped workload
# 65,536 tokens, 8 groups of 32 experts, at its real size: the layout, every
# one of the ~347 K grouped rows and every token's grouped combine against
# the oracle, which runs over token chunks (slots renumbered per chunk) so
# host memory stays bounded.
CHUNK = 4096


def _chunk_slots(dest_rows):
    """A token chunk's destination rows renumbered over the rows it uses."""
    used = np.unique(dest_rows[dest_rows >= 0])
    remap = -np.ones(int(dest_rows.max(initial=-1)) + 2, np.int64)
    remap[used] = np.arange(len(used))
    return used, np.where(dest_rows >= 0, remap[np.maximum(dest_rows, 0)], -1)


@pytest.fixture(scope="module")
def grouped():
    w = W.by_name("grouped")
    say("grouped workload: inputs")
    idx, wt = W.make_routing(w)
    R = O.layout(idx.numpy(), w.E, w.G, wt.numpy())
    d_idx, d_wt = idx.to(DEV), wt.to(DEV)
    L = ep().ep_layout(d_idx, w.E, w.G, d_wt)
    return {"w": w, "idx": idx, "wt": wt, "R": R, "d_idx": d_idx, "d_wt": d_wt, "L": L}


def test_grouped_workload_layout(grouped):
    G = grouped
    check_layout(G["L"], G["R"], G["w"].E, G["w"].G)


def test_grouped_workload_dispatch_every_row(grouped):
    """Every grouped row of the bf16 dispatch against the oracle's dispatch
    of the same tokens, chunk by chunk; the chunks' rows cover all R rows
    exactly once."""
    G = grouped
    w, R = G["w"], G["R"]
    x = W.make_x(w, device=DEV)
    say("grouped workload: dispatch")
    recv = ep().ep_dispatch(x, G["L"], rows=ep().EP_ROWS_GROUP)
    torch.cuda.synchronize()
    grow = R["grow"]
    covered = 0
    for t0 in range(0, w.T, CHUNK):
        t1 = min(t0 + CHUNK, w.T)
        used, dest = _chunk_slots(grow[t0:t1])
        want = O.dispatch_bf16(u16(x[t0:t1]), dest, len(used))
        got = u16(recv.index_select(0, torch.from_numpy(used).to(DEV)))
        assert np.array_equal(got, want), (t0, t1)
        covered += len(used)
    assert covered == R["n_rows"]
    del recv, x


def test_grouped_workload_combine_every_token(grouped):
    """Every token's grouped combine (within-group, then across groups in
    group order) against the oracle, chunk by chunk."""
    G = grouped
    w, R = G["w"], G["R"]
    y = W.make_y(w, device=DEV)
    say("grouped workload: combine")
    out = ep().ep_combine(y, G["L"], G["d_wt"], G["d_idx"], order=ep().EP_COMBINE_GROUPED)
    torch.cuda.synchronize()
    idx, wt = G["idx"].numpy(), G["wt"].numpy()
    for t0 in range(0, w.T, CHUNK):
        t1 = min(t0 + CHUNK, w.T)
        used, slot_r = _chunk_slots(R["slot"][t0:t1])
        ysub = u16(y.index_select(0, torch.from_numpy(used).to(DEV)))
        want = O.combine_grouped(ysub, idx[t0:t1], slot_r, wt[t0:t1], w.E, w.G)
        assert np.array_equal(u16(out[t0:t1]), want), (t0, t1)
    del y, out


@pytest.mark.parametrize("mask_p", [0.0, 0.5])
def test_round_trip_dispatch_then_unit_weight_combine(mask_p):
    """Dispatch bf16 rows, then combine those very rows with unit weights:
    each token comes back as the fp32 sum of K_eff copies of itself, which is
    exactly K_eff * x when K_eff is 1, 2, 4 or 8 (+0 when it is 0), and equal
    to the oracle's dispatch followed by its combine (top-8, then again with
    half the selections masked)."""
    say("round trip", mask_p)
    w = W.Workload("rt", T=600, H=384, K=8, E=32, mask_p=mask_p, seed=41 + int(mask_p * 10))
    idx, _ = W.make_routing(w)
    x = W.make_x(w)
    L = ep().ep_layout(idx.to(DEV), w.E)
    recv = ep().ep_dispatch(x.to(DEV), L)
    ones = torch.ones(w.T, w.K, dtype=torch.float32, device=DEV)
    out = ep().ep_combine(recv, L, ones)
    got = u16(out)
    R = O.layout(idx.numpy(), w.E)
    xs = u16(x)
    rows = O.dispatch_bf16(xs, R["slot"], R["n_sel"])
    want = O.combine(rows, R["slot"], np.ones((w.T, w.K), np.float32))
    assert np.array_equal(got, want)
    k_eff = (idx.numpy() >= 0).sum(axis=1)
    assert (got[k_eff == 0] == 0).all()  # nothing selected: +0, not 0 * x
    exact = np.isin(k_eff, [1, 2, 4, 8])
    assert exact.any()
    scaled = O.bf16_rne((O.bf16_to_f32(xs[exact]) * k_eff[exact, None]).astype(np.float32))
    assert np.array_equal(got[exact], scaled)


@pytest.mark.parametrize("blocks", [1, 3, 64, 5000])
def test_grid_size_sweep_identical_bytes(blocks, monkeypatch):
    """The scatter and combine kernels' cyclic work split gives the same
    bytes at any grid size: one block doing everything, a few blocks (waves
    then take several items, of one token or of several), and more blocks
    than the default one wave per item (the extra waves have nothing to do).
    bf16 and fp8 dispatch (both store paths) and flat and grouped combine
    against the default grid.  5% of the tokens are fully masked, so waves
    that walk several tokens step over tokens they must not read; the
    default grid's fp8 rows are checked against the oracle too."""
    say("grid sweep", blocks)
    w = W.by_name("mid").replace(T=1500, mask_p=0.1, full_mask_frac=0.05, E=64, G=8)
    idx, wt = W.make_routing(w)
    d_idx, d_wt = idx.to(DEV), wt.to(DEV)
    x = W.make_x(w).to(DEV)
    y = W.make_y(w).to(DEV)
    L = ep().ep_layout(d_idx, w.E, w.G, d_wt)
    pitch = ep().fp8_row_pitch(w.H)

    def run():
        outs = [
            ep().ep_dispatch(x, L).view(torch.int16),
            ep().ep_dispatch(x, L, fp8=True),
            ep().ep_dispatch(x, L, fp8=True, row_stride=pitch),
            ep().ep_dispatch(x, L, rows=ep().EP_ROWS_GROUP).view(torch.int16),
            ep().ep_combine(y, L, d_wt).view(torch.int16),
            ep().ep_combine(y, L, d_wt, d_idx, order=ep().EP_COMBINE_GROUPED).view(torch.int16),
        ]
        torch.cuda.synchronize()
        return outs

    ref = run()
    n, R = L.num_rows(), L.num_rows(ep().EP_ROWS_GROUP)
    assert (idx.numpy() < 0).all(axis=1).sum() >= round(0.05 * w.T)
    want = O.dispatch_fp8(u16(x), O.layout(idx.numpy(), w.E)["slot"], n)
    assert np.array_equal(ref[1][:n].cpu().numpy(), want)
    monkeypatch.setenv("EP_MI355X_GRID_BLOCKS", str(blocks))
    got = run()
    monkeypatch.delenv("EP_MI355X_GRID_BLOCKS")
    rows = [n, n, n, R, w.T, w.T]
    for a, b, r in zip(ref, got, rows):
        assert torch.equal(a[:r], b[:r])
