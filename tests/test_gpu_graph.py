"""The dispatch/combine step, and the grouped path with the GEMM, captured
in a HIP graph (torch.cuda.graph).

The library only enqueues kernels on the caller's stream: it allocates,
clears and synchronises nothing, so a step with preallocated outputs can be
captured once and replayed.  Inputs are rewritten in place between replays
(new routing, weights and token rows each time), with eager work and
synchronisations in between, and every replay must equal an eager run of the
same step on separate buffers bit for bit; the first replay is also checked
against the oracle."""
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


def u16(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def test_step_graph_replays_match_eager_and_oracle():
    import combine_ep_layout_03_amd as ep

    base = W.by_name("mid").replace(mask_p=0.05)
    T, H, K, E = base.T, base.H, base.K, base.E
    pitch = ep.fp8_row_pitch(H)
    idx0, wt0 = W.make_routing(base)
    d_idx, d_wt = idx0.to(DEV), wt0.to(DEV)
    x = W.make_x(base, device=DEV)
    y = W.make_y(base, device=DEV)

    # graph-side buffers
    L = ep.ep_layout(d_idx, E)
    recv = torch.full((T * K, pitch), 0x5A, dtype=torch.uint8, device=DEV)
    out = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)
    # eager-side buffers
    Le = ep.ep_layout(d_idx, E)
    recv_e = torch.full((T * K, pitch), 0x5A, dtype=torch.uint8, device=DEV)
    out_e = torch.empty(T, H, dtype=torch.bfloat16, device=DEV)

    def step(Lx, rx, ox):
        ep.ep_layout(d_idx, E, out=Lx)
        ep.ep_dispatch(x, Lx, fp8=True, out=rx)
        ep.ep_combine(y, Lx, d_wt, out=ox)

    # warm up on a side stream, as torch's capture requires, then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(L, recv, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(L, recv, out)
    torch.cuda.synchronize()

    rb = ep.ep_fp8_row_bytes(H)
    for rep in range(4):
        w = base.replace(seed=100 + rep)
        idx, wt = W.make_routing(w)
        d_idx.copy_(idx.to(DEV))
        d_wt.copy_(wt.to(DEV))
        x.copy_(W.make_x(w, device=DEV))
        torch.cuda.synchronize()
        step(Le, recv_e, out_e)  # eager reference on its own buffers
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        n = Le.num_rows()
        assert L.num_rows() == n
        for name in ("counts", "offsets", "slot"):
            assert torch.equal(getattr(L, name), getattr(Le, name)), f"replay {rep}: {name}"
        assert torch.equal(recv[:n, :rb], recv_e[:n, :rb]), f"replay {rep}: dispatch rows"
        assert torch.equal(out.view(torch.int16), out_e.view(torch.int16)), f"replay {rep}: combine"
        if rep == 0:
            R = O.layout(idx.numpy(), E)
            assert np.array_equal(L.slot.cpu().numpy(), R["slot"])
            want = O.combine(u16(y), R["slot"], wt.numpy())
            assert np.array_equal(u16(out), want)
            xs = u16(x)
            got = recv[:n, :rb].cpu().numpy()
            want_rows = O.dispatch_fp8(xs, R["slot"], n)
            assert np.array_equal(got, want_rows)


def test_grouped_step_graph_replays_match_eager_and_oracle():
    """The grouped path captured once and replayed: grouped layout with row
    lists and expert-row map (96,000 entries, past 65,536, so the wide column
    scan runs), one bf16 row per (token, group hit), the grouped-order
    combine, and the grouped GEMM gathering its rows from the token matrix
    through packed weights.  Every replay, on new routing, weights and token
    rows, equals an eager run on separate buffers bit for bit; the first is
    also checked against the oracle (layout, group rows, grouped combine)."""
    import combine_ep_layout_03_amd as ep

    base = W.Workload("graph_grouped", T=12000, H=256, K=8, E=64, G=8, mask_p=0.05, seed=3)
    T, H, K, E, G = base.T, base.H, base.K, base.E, base.G
    N = 256
    idx0, wt0 = W.make_routing(base)
    d_idx, d_wt = idx0.to(DEV), wt0.to(DEV)
    x = W.make_x(base, device=DEV)
    y = W.make_y(base, device=DEV)
    packed = ep.ep_pack_expert_weights(W.make_expert_weights(base, N).to(DEV))

    def buffers():
        Lx = ep.ep_layout(d_idx, E, G, d_wt, expert_row_src=True)
        return (
            Lx,
            torch.full((Lx.max_group_rows(), H), 7.0, dtype=torch.bfloat16, device=DEV),
            torch.empty(T, H, dtype=torch.bfloat16, device=DEV),
            torch.zeros(Lx.max_expert_rows(), N, dtype=torch.bfloat16, device=DEV),
        )

    def step(Lx, rx, ox, gx):
        ep.ep_layout(d_idx, E, G, d_wt, out=Lx)
        ep.ep_dispatch(x, Lx, rows=ep.EP_ROWS_GROUP, out=rx)
        ep.ep_combine(y, Lx, d_wt, d_idx, order=ep.EP_COMBINE_GROUPED, out=ox)
        ep.ep_expert_gemm(x, Lx, packed, out=gx, gather=True)

    L, recv, out, yg = buffers()
    Le, recv_e, out_e, yg_e = buffers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(L, recv, out, yg)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(L, recv, out, yg)
    torch.cuda.synchronize()

    for rep in range(4):
        w = base.replace(seed=200 + rep)
        idx, wt = W.make_routing(w)
        d_idx.copy_(idx.to(DEV))
        d_wt.copy_(wt.to(DEV))
        x.copy_(W.make_x(w, device=DEV))
        torch.cuda.synchronize()
        step(Le, recv_e, out_e, yg_e)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name in ("counts", "offsets", "slot", "grow", "group_counts", "group_offsets"):
            assert torch.equal(getattr(L, name), getattr(Le, name)), f"replay {rep}: {name}"
        ng = int(L.status[2].item())
        ne = int(L.status[1].item())
        assert ng == int(Le.status[2].item()) and ne == int(Le.status[1].item())
        # the expert-row map holds ne rows; the rest of its capacity is never written
        assert torch.equal(L.expert_row_src[:ne], Le.expert_row_src[:ne]), f"replay {rep}: expert_row_src"
        for name in ("row_src", "row_topk_idx"):
            assert torch.equal(getattr(L, name)[:ng], getattr(Le, name)[:ng]), f"replay {rep}: {name}"
        assert torch.equal(L.row_topk_weights[:ng].view(torch.int32), Le.row_topk_weights[:ng].view(torch.int32))
        assert torch.equal(recv[:ng].view(torch.int16), recv_e[:ng].view(torch.int16)), f"replay {rep}: group rows"
        assert torch.equal(out.view(torch.int16), out_e.view(torch.int16)), f"replay {rep}: grouped combine"
        assert torch.equal(yg[:ne].view(torch.int16), yg_e[:ne].view(torch.int16)), f"replay {rep}: gemm"
        if rep == 0:
            R = O.layout(idx.numpy(), E, G, wt.numpy())
            assert np.array_equal(L.grow.cpu().numpy(), R["grow"])
            assert np.array_equal(L.slot.cpu().numpy(), R["slot"])
            assert np.array_equal(u16(recv[:ng]), O.dispatch_bf16(u16(x), R["grow"], R["n_rows"]))
            want = O.combine_grouped(u16(y), idx.numpy(), R["slot"], wt.numpy(), E, G)
            assert np.array_equal(u16(out), want)
