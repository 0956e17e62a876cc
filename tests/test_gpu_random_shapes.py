"""Seeded random shapes within the documented limits, each checked against
the oracle bit for bit: the layout (counts, offsets, slots, grouped rows),
bf16 dispatch of expert rows (and, with groups, of grouped rows), fp8
dispatch where H % 128 == 0 (with zeroed alignment padding), and flat and
grouped combine.  Tokens, top-k, experts, groups, hidden size (ragged
vector tails included), routing, masking and expert alignment are drawn
from a fixed generator, so every run tests the same 24 cases."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import ep_oracle as O

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _cases(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([1, 3, 8, 16, 40, 64, 100, 256]))
        K = int(min(rng.integers(1, 17), E))
        divisors = [g for g in range(1, E + 1) if E % g == 0]
        G = int(rng.choice([0] + divisors)) if rng.random() < 0.6 else 0
        fp8 = rng.random() < 0.5
        H = int(128 * rng.integers(1, 9)) if fp8 else int(rng.integers(1, 600))
        T = int(rng.integers(1, 1500))
        routing = "zipf" if rng.random() < 0.3 else "uniform"
        out.append(
            dict(
                name=f"r{i}",
                T=T,
                H=H,
                K=K,
                E=E,
                G=max(G, 1),
                routing=routing,
                zipf_s=1.2 if routing == "zipf" else 0.0,
                mask_p=float(rng.choice([0.0, 0.1, 0.5])),
                full_mask_frac=float(rng.choice([0.0, 0.05])),
                seed=1000 + i,
                groups=G,
                align=int(rng.choice([0, 0, 2, 8, 64])),
            )
        )
    return out


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


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_random_shape_matches_oracle(case):
    c = dict(case)
    G, A = c.pop("groups"), c.pop("align")
    print("random shape", case, flush=True)
    w = W.Workload(**c)
    idx, wt = W.make_routing(w)
    x = W.make_x(w)
    R = O.layout(idx.numpy(), w.E, G, wt.numpy(), expert_alignment=A)
    L = ep().ep_layout(idx.to(DEV), w.E, G, wt.to(DEV) if G else None, expert_alignment=A,
                       expert_row_src=A > 1)
    torch.cuda.synchronize()
    assert np.array_equal(L.counts.cpu().numpy(), R["counts"])
    assert np.array_equal(L.offsets.cpu().numpy(), R["offsets"])
    assert np.array_equal(L.slot.cpu().numpy(), R["slot"])
    n = R["n_rows_expert"]
    sel = np.ones(n, bool) if A <= 1 else R["expert_row_src"] >= 0
    xr = u16(x)
    # bf16 dispatch of expert rows (padding rows are not written)
    recv = ep().ep_dispatch(x.to(DEV), L)
    if n:
        assert np.array_equal(u16(recv[:n])[sel], O.dispatch_bf16(xr, R["slot"], n)[sel])
    # fp8 dispatch, alignment padding zeroed
    if w.H % 128 == 0:
        recv8 = ep().ep_dispatch(x.to(DEV), L, fp8=True, zero_padding=A > 1)
        if n:
            want8 = O.dispatch_fp8(xr, R["slot"], n)
            got8 = recv8[:n].cpu().numpy()
            assert np.array_equal(got8 if A > 1 else got8[sel], want8 if A > 1 else want8[sel])
    # grouped rows
    if G:
        assert np.array_equal(L.grow.cpu().numpy(), R["grow"])
        ng = R["n_rows"]
        recvg = ep().ep_dispatch(x.to(DEV), L, rows=ep().EP_ROWS_GROUP)
        if ng:
            assert np.array_equal(u16(recvg[:ng]), O.dispatch_bf16(xr, R["grow"], ng))
    # combine, flat and (with groups) grouped, over one row per expert row
    y = W.make_y(w, rows=max(n, 1))
    out = ep().ep_combine(y.to(DEV), L, wt.to(DEV))
    assert np.array_equal(u16(out), O.combine(u16(y), R["slot"], wt.numpy()))
    if G:
        outg = ep().ep_combine(y.to(DEV), L, wt.to(DEV), idx.to(DEV), order=ep().EP_COMBINE_GROUPED)
        assert np.array_equal(u16(outg), O.combine_grouped(u16(y), idx.numpy(), R["slot"], wt.numpy(), w.E, G))
