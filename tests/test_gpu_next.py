"""GPU parity of the rows built after the hot path: expert alignment with
zeroed padding rows, cumulative receive stats, combine bias, and the cached
layout handle's stale-layout guard (all through the C ABI, bit-exact against
the CPU oracle)."""
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


@pytest.mark.parametrize("A,T", [(2, 1200), (4, 1200), (64, 1200), (128, 1200), (16, 200)])
@pytest.mark.parametrize("fp8", [False, True])
def test_alignment_zero_padding(A, T, fp8):
    # T = 200: 1600 entries, laid out by one fused block
    w = W.by_name("skewed_masked").replace(T=T, H=256 if fp8 else 200, seed=A)
    print("alignment", A, fp8, flush=True)
    idx, _ = W.make_routing(w)
    x = W.make_x(w)
    R = O.layout(idx.numpy(), w.E, expert_alignment=A)
    L = ep().ep_layout(idx.to(DEV), w.E, expert_alignment=A, expert_row_src=True)
    torch.cuda.synchronize()
    assert np.array_equal(L.counts.cpu().numpy(), R["counts"])
    assert np.array_equal(L.offsets.cpu().numpy(), R["offsets"])
    assert np.array_equal(L.slot.cpu().numpy(), R["slot"])
    n = R["n_rows_expert"]
    assert np.array_equal(L.expert_row_src[:n].cpu().numpy(), R["expert_row_src"])
    st = L.status.cpu().numpy()
    assert st[ep().EP_STATUS_ROWS_EXPERT] == n and st[ep().EP_STATUS_SELECTIONS] == R["n_sel"]
    assert st[ep().EP_STATUS_EXPERT_LIST_OVERFLOW] == 0
    pad = R["expert_row_src"] < 0
    if fp8:
        rb = O.fp8_row_bytes(w.H)
        want = O.dispatch_fp8(u16(x), R["slot"], n)
        # packed rows, then rows on a 128-byte pitch (zero-filled to the line end)
        for pitch in (rb, (rb + 127) // 128 * 128):
            for zp in (True, False):
                out = torch.full((L.max_expert_rows(), pitch), 0xC3, dtype=torch.uint8, device=DEV)
                ep().ep_dispatch(x.to(DEV), L, fp8=True, out=out, zero_padding=zp)
                got = out.cpu().numpy()
                assert np.array_equal(got[:n, :rb][~pad], want[~pad])
                assert not got[:n, rb:][~pad].any()
                if zp:
                    assert np.array_equal(got[:n, :rb][pad], want[pad]) and not got[:n][pad].any()
                else:
                    assert (got[:n][pad] == 0xC3).all()
                assert (got[n:] == 0xC3).all()
    else:
        want = O.dispatch_bf16(u16(x), R["slot"], n)
        for zp in (True, False):
            out = torch.full((L.max_expert_rows(), w.H), -15421, dtype=torch.int16, device=DEV)  # 0xC3C3
            ep().ep_dispatch(x.to(DEV), L, out=out.view(torch.bfloat16), zero_padding=zp)
            got = out.cpu().numpy().view(np.uint16)
            assert np.array_equal(got[:n][~pad], want[~pad])
            if zp:
                assert not got[:n][pad].any()
            else:
                assert (got[:n][pad] == 0xC3C3).all()
            assert (got[n:] == 0xC3C3).all()
    # combine reads the aligned rows through the same slots
    y = W.make_y(w, rows=n)
    wt = W.make_routing(w)[1]
    outc = ep().ep_combine(y.to(DEV), L, wt.to(DEV))
    assert np.array_equal(u16(outc), O.combine(u16(y), R["slot"], wt.numpy()))


def test_expert_row_list_overflow():
    w = W.by_name("mid").replace(T=500)
    idx, _ = W.make_routing(w)
    L = ep().ep_layout(idx.to(DEV), w.E, expert_alignment=16, expert_row_src=True)
    n = L.num_rows()
    L2 = ep().Layout(**{**L.__dict__, "expert_row_capacity": n - 1, "generation": 0})
    ep().ep_layout(idx.to(DEV), w.E, expert_alignment=16, out=L2)
    torch.cuda.synchronize()
    assert L2.status[ep().EP_STATUS_EXPERT_LIST_OVERFLOW].item() == 1


@pytest.mark.parametrize("T", [3000, 150])  # two launches; one fused block
def test_cumulative_recv_stats(T):
    """Three accumulating layouts; 25% of the selections are masked."""
    w = W.by_name("pages").replace(T=T, mask_p=0.25)
    stats = torch.zeros(w.E, dtype=torch.int32, device=DEV)
    want = np.zeros(w.E, np.int64)
    for s in range(3):
        idx, _ = W.make_routing(w.replace(seed=s))
        ep().ep_layout(idx.to(DEV), w.E, recv_stats=stats)
        want += O.layout(idx.numpy(), w.E)["counts"]
    torch.cuda.synchronize()
    assert np.array_equal(stats.cpu().numpy().astype(np.int64), want)


@pytest.mark.parametrize("nb", [1, 2])
@pytest.mark.parametrize("grouped", [False, True])
def test_combine_bias(nb, grouped):
    w = W.Workload("bias", T=600, H=264, K=8, E=64, G=8, mask_p=0.15, full_mask_frac=0.05, seed=nb)
    idx, wt = W.make_routing(w)
    G = w.G if grouped else 0
    R = O.layout(idx.numpy(), w.E, G, wt.numpy())
    L = ep().ep_layout(idx.to(DEV), w.E, G, wt.to(DEV) if G else None)
    y = W.make_y(w, rows=R["n_sel"])
    g = torch.Generator().manual_seed(40 + nb)
    b0 = torch.randn(w.T, w.H, generator=g).to(torch.bfloat16)
    b1 = torch.randn(w.T, w.H, generator=g).to(torch.bfloat16) if nb == 2 else None
    order = ep().EP_COMBINE_GROUPED if grouped else ep().EP_COMBINE_FLAT
    out = ep().ep_combine(
        y.to(DEV), L, wt.to(DEV), idx.to(DEV), order=order, bias0=b0.to(DEV), bias1=None if b1 is None else b1.to(DEV)
    )
    args = dict(bias0=u16(b0), bias1=None if b1 is None else u16(b1))
    if grouped:
        want = O.combine_grouped(u16(y), idx.numpy(), R["slot"], wt.numpy(), w.E, w.G, **args)
    else:
        want = O.combine(u16(y), R["slot"], wt.numpy(), **args)
    got = u16(out)
    assert np.array_equal(got, want)
    masked = (idx.numpy() < 0).all(axis=1)
    assert masked.any()
    if nb == 1:
        assert np.array_equal(got[masked], u16(b0)[masked])


def test_cached_handle_and_stale_guard():
    """Fresh, cached and cached-twice dispatches agree; a handle whose layout
    buffers were recomputed for another routing is rejected."""
    w = W.by_name("mid").replace(T=1000)
    idx, _ = W.make_routing(w)
    x = W.make_x(w).to(DEV)
    L = ep().ep_layout(idx.to(DEV), w.E)
    h = L.handle()
    fresh = ep().ep_dispatch(x, L).clone()
    cached = ep().ep_dispatch(x, h).clone()
    twice = ep().ep_dispatch(x, h).clone()
    n = L.num_rows()
    assert torch.equal(fresh[:n].view(torch.int16), cached[:n].view(torch.int16))
    assert torch.equal(fresh[:n].view(torch.int16), twice[:n].view(torch.int16))
    idx2, _ = W.make_routing(w.replace(seed=5))
    ep().ep_layout(idx2.to(DEV), w.E, out=L)  # same buffers, another routing
    with pytest.raises(ep().StaleLayoutError):
        ep().ep_dispatch(x, h)
    ep().ep_dispatch(x, L.handle())  # a fresh handle is fine
