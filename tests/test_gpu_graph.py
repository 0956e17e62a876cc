"""The dispatch/combine step captured in a HIP graph (torch.cuda.graph).

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
