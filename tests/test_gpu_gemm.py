"""GPU parity of the grouped GEMM over expert segments (MFMA, bf16 in, fp32
accumulate, bf16 out) against the float64 oracle, within the bound derived
from the arithmetic: |y - y64| <= 2^-8 |y64| + H 2^-24 sum |x w| per element,
and rel_l2 <= 1e-2 overall."""
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


def _check(got_u16, x_u16, counts, offsets, w_u16, rows=None):
    y64 = O.expert_gemm(x_u16, counts, offsets, w_u16, rows=rows)
    bound = O.expert_gemm_bound(x_u16, counts, offsets, w_u16, y64)
    ok = ~np.isnan(y64)
    got = O.bf16_to_f32(got_u16).astype(np.float64)
    err = np.abs(got - y64)
    bad = ok & ~(err <= bound)
    assert not bad.any(), f"{bad.sum()} elements out of bound, worst {np.nanmax(err - bound)}"
    rel = np.linalg.norm((got - y64)[ok]) / np.linalg.norm(y64[ok])
    assert rel <= 1e-2, rel
    return rel


@pytest.mark.parametrize(
    "T,K,E,H,N,A",
    [
        (300, 2, 8, 256, 256, 0),
        (257, 4, 16, 128, 128, 0),
        (700, 3, 12, 192, 384, 64),
        (90, 2, 4, 64, 128, 0),  # two reduction steps: fewer than the ring's depth
        (1500, 2, 4, 320, 256, 0),  # ~750 rows per expert: three row tiles each
        (600, 2, 1024, 64, 128, 0),  # the largest expert count, most experts empty
    ],
)
def test_expert_gemm_small(T, K, E, H, N, A):
    w = W.Workload("g", T=T, H=H, K=K, E=E, mask_p=0.1, seed=T)
    idx, _ = W.make_routing(w)
    R = O.layout(idx.numpy(), E, expert_alignment=A)
    L = ep().ep_layout(idx.to(DEV), E, expert_alignment=A)
    rows = L.max_expert_rows()
    x = W.make_rows(w, rows)
    wts = W.make_expert_weights(w, N)
    y = torch.full((rows, N), -1, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    ep().ep_expert_gemm(x.to(DEV), L, wts.to(DEV), out=y)
    got = u16(y)
    _check(got, u16(x), R["counts"], R["offsets"], u16(wts))
    # rows outside every expert's selections stay untouched
    occupied = np.zeros(rows, bool)
    for e in range(E):
        occupied[R["offsets"][e] : R["offsets"][e] + R["counts"][e]] = True
    assert (got[~occupied] == 0xFFFF).all()


def test_expert_gemm_exact_on_small_integers():
    """Integer inputs in [-2, 2] make every fp32 partial sum exact, so the
    kernel's output must equal the bf16 rounding of the exact sum bit for bit:
    any row, column or k misplacement shows as a mismatch."""
    w = W.Workload("gi", T=1200, H=448, K=3, E=6, mask_p=0.05, seed=11)
    N = 384
    idx, _ = W.make_routing(w)
    R = O.layout(idx.numpy(), w.E, expert_alignment=32)
    L = ep().ep_layout(idx.to(DEV), w.E, expert_alignment=32)
    rows = L.max_expert_rows()
    x = W.make_small_ints(w, (rows, w.H), stream=0)
    wts = W.make_small_ints(w, (w.E, N, w.H), stream=1)
    y = ep().ep_expert_gemm(x.to(DEV), L, wts.to(DEV))
    y64 = O.expert_gemm(u16(x), R["counts"], R["offsets"], u16(wts))
    ok = ~np.isnan(y64)
    want = O.bf16_rne(y64[ok].astype(np.float32))
    assert np.array_equal(u16(y)[ok], want)


def test_expert_gemm_skewed_with_empty_experts():
    w = W.by_name("skewed_masked").replace(T=2000, H=256, E=64)
    idx, _ = W.make_routing(w)
    R = O.layout(idx.numpy(), w.E, expert_alignment=16)
    assert (R["counts"] == 0).any() or R["counts"].max() > 3 * 128
    L = ep().ep_layout(idx.to(DEV), w.E, expert_alignment=16)
    x = W.make_rows(w, L.max_expert_rows())
    wts = W.make_expert_weights(w, 256)
    y = ep().ep_expert_gemm(x.to(DEV), L, wts.to(DEV))
    _check(u16(y), u16(x), R["counts"], R["offsets"], u16(wts))


def test_expert_gemm_pages_shape_sampled():
    """8192 tokens x top-8 of 256 experts, H = 7168 -> N = 2048, on 64 sampled
    rows from 8 experts (their first, last and random rows)."""
    w = W.by_name("pages")
    N = 2048
    print("gemm pages shape: inputs", flush=True)
    idx, _ = W.make_routing(w)
    R = O.layout(idx.numpy(), w.E)
    L = ep().ep_layout(idx.to(DEV), w.E)
    x = W.make_rows(w, L.max_expert_rows(), device=DEV)
    wts = W.make_expert_weights(w, N, device=DEV)
    print("gemm pages shape: run", flush=True)
    y = ep().ep_expert_gemm(x, L, wts)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    experts = rng.choice(w.E, 8, replace=False)
    rows = []
    for e in experts:
        r0, c = int(R["offsets"][e]), int(R["counts"][e])
        rows += [r0, r0 + c - 1] + list(rng.choice(np.arange(r0, r0 + c), 6, replace=False))
    rows = np.array(sorted(set(rows)))
    # the oracle sees only the sampled rows and their experts' weights
    sub_counts = np.zeros(len(experts), np.int64)
    sub_offsets = np.zeros(len(experts) + 1, np.int64)
    order = []
    for i, e in enumerate(sorted(experts)):
        r0, c = int(R["offsets"][e]), int(R["counts"][e])
        mine = [r for r in rows if r0 <= r < r0 + c]
        order += mine
        sub_counts[i] = len(mine)
        sub_offsets[i + 1] = sub_offsets[i] + len(mine)
    sel = torch.from_numpy(np.array(order)).to(DEV)
    xs = u16(x.index_select(0, sel))
    ws = u16(wts.index_select(0, torch.from_numpy(np.sort(experts)).to(DEV)))
    ys = u16(y.index_select(0, sel))
    rel = _check(ys, xs, sub_counts, sub_offsets, ws)
    print("rel_l2", rel, flush=True)


@pytest.mark.parametrize(
    "name,T,K,E,H,N,A",
    [
        ("gf1", 300, 2, 8, 256, 256, 0),
        ("gf2", 700, 3, 12, 192, 384, 64),  # aligned segments with padding rows
        ("gf3", 1500, 2, 4, 320, 256, 0),   # several row tiles per expert
    ],
)
def test_gathered_gemm_equals_dispatch_then_gemm(name, T, K, E, H, N, A):
    """Rows gathered through expert_row_src inside the GEMM (dispatch fused
    into the GEMM's loads) give exactly the dispatch-then-GEMM result: same
    operands, same accumulation order.  The first case is also checked
    against the oracle's bound."""
    w = W.Workload(name, T=T, H=H, K=K, E=E, mask_p=0.1, seed=T + H)
    idx, _ = W.make_routing(w)
    L = ep().ep_layout(idx.to(DEV), E, expert_alignment=A, expert_row_src=True)
    x = W.make_x(w).to(DEV)
    wts = W.make_expert_weights(w, N).to(DEV)
    recv = ep().ep_dispatch(x, L)
    y_unfused = ep().ep_expert_gemm(recv, L, wts)
    y_fused = ep().ep_expert_gemm(x, L, wts, gather=True)
    torch.cuda.synchronize()
    R = O.layout(idx.numpy(), E, expert_alignment=A)
    n = len(R["expert_row_src"])
    valid = R["expert_row_src"] >= 0
    assert np.array_equal(u16(y_fused)[:n][valid], u16(y_unfused)[:n][valid])
    if name == "gf1":
        rows = O.dispatch_bf16(u16(x), R["slot"], R["n_rows_expert"])
        _check(u16(y_fused)[:n], rows, R["counts"], R["offsets"], u16(wts))


def test_gathered_gemm_pages_shape_equals_unfused():
    """8192 tokens x top-8 of 256, H = 7168 -> N = 2048: the fused gather
    equals dispatch then GEMM on every one of the 65536 expert rows."""
    w = W.by_name("pages")
    idx, _ = W.make_routing(w)
    L = ep().ep_layout(idx.to(DEV), w.E, expert_row_src=True)
    x = W.make_x(w, device=DEV)
    wts = W.make_expert_weights(w, 2048, device=DEV)
    print("gathered gemm pages shape: run", flush=True)
    y_unfused = ep().ep_expert_gemm(ep().ep_dispatch(x, L), L, wts)
    y_fused = ep().ep_expert_gemm(x, L, wts, gather=True)
    torch.cuda.synchronize()
    n = L.num_rows()
    assert torch.equal(y_fused[:n].view(torch.int16), y_unfused[:n].view(torch.int16))


def test_pack_expert_weights_layout():
    """The packed order is the documented permutation: block (e, j, k) holds
    rows 256 j .. 256 j + 255 of expert e, elements 32 k .. 32 k + 31, rows
    past N zero.  N = 384 leaves the second column tile half padding."""
    E, N, H = 3, 384, 128
    w = W.make_expert_weights(W.Workload("pk", T=8, H=H, K=1, E=E), N)
    packed = ep().ep_pack_expert_weights(w.to(DEV))
    torch.cuda.synchronize()
    wn = u16(w).reshape(E, N, H)
    ntn = (N + 255) // 256
    full = np.zeros((E, ntn * 256, H), np.uint16)
    full[:, :N] = wn
    want = full.reshape(E, ntn, 256, H // 32, 32).transpose(0, 1, 3, 2, 4).reshape(-1)
    assert np.array_equal(u16(packed.data), want)


@pytest.mark.parametrize(
    "T,K,E,H,N,A,gather",
    [
        (300, 2, 8, 256, 256, 0, False),
        (700, 3, 12, 192, 384, 64, False),  # half-padded last column tile
        (90, 2, 4, 64, 128, 0, False),
        (1500, 2, 4, 320, 256, 0, False),
        (600, 2, 1024, 64, 128, 0, False),
        (700, 3, 12, 192, 384, 64, True),   # packed weights with gathered rows
    ],
)
def test_packed_weights_gemm_equals_plain(T, K, E, H, N, A, gather):
    """Packed weights change where the weight stages come from, not the
    operands or the order: the result equals the plain GEMM bit for bit on
    every expert row."""
    w = W.Workload("gp", T=T, H=H, K=K, E=E, mask_p=0.1, seed=T + N)
    idx, _ = W.make_routing(w)
    L = ep().ep_layout(idx.to(DEV), E, expert_alignment=A, expert_row_src=gather)
    wts = W.make_expert_weights(w, N).to(DEV)
    packed = ep().ep_pack_expert_weights(wts)
    if gather:
        x = W.make_x(w).to(DEV)
    else:
        x = W.make_rows(w, L.max_expert_rows()).to(DEV)
    y_plain = ep().ep_expert_gemm(x, L, wts, gather=gather)
    y_packed = ep().ep_expert_gemm(x, L, packed, gather=gather)
    torch.cuda.synchronize()
    R = O.layout(idx.numpy(), E, expert_alignment=A)
    occupied = np.zeros(y_plain.shape[0], bool)
    for e in range(E):
        occupied[R["offsets"][e] : R["offsets"][e] + R["counts"][e]] = True
    assert np.array_equal(u16(y_packed)[occupied], u16(y_plain)[occupied])


def test_packed_weights_gemm_pages_shape_equals_plain():
    """65,536 rows x 7168 -> 2048 over 256 experts: packed and plain weights
    give the same bytes on every expert row."""
    w = W.by_name("pages")
    idx, _ = W.make_routing(w)
    L = ep().ep_layout(idx.to(DEV), w.E)
    x = W.make_rows(w, L.max_expert_rows(), device=DEV)
    wts = W.make_expert_weights(w, 2048, device=DEV)
    print("packed gemm pages shape: run", flush=True)
    packed = ep().ep_pack_expert_weights(wts)
    y_plain = ep().ep_expert_gemm(x, L, wts)
    y_packed = ep().ep_expert_gemm(x, L, packed)
    torch.cuda.synchronize()
    n = L.num_rows()
    assert torch.equal(y_packed[:n].view(torch.int16), y_plain[:n].view(torch.int16))


def _gemm_cases(n=8, seed=77):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([1, 5, 16, 64, 300]))
        out.append(
            dict(
                T=int(rng.integers(20, 1200)),
                K=int(min(rng.integers(1, 9), E)),
                E=E,
                H=int(64 * rng.integers(1, 7)),
                N=int(128 * rng.integers(1, 5)),
                A=int(rng.choice([0, 0, 8, 64])),
                gather=bool(rng.random() < 0.4),
                seed=500 + i,
            )
        )
    return out


@pytest.mark.parametrize("c", _gemm_cases(), ids=lambda c: f"E{c['E']}-H{c['H']}-N{c['N']}-A{c['A']}-g{int(c['gather'])}")
def test_expert_gemm_random_shapes(c):
    """Seeded random shapes: within the oracle's bound, and packed weights
    bit-identical to plain ones."""
    print("random gemm", c, flush=True)
    w = W.Workload("gr", T=c["T"], H=c["H"], K=c["K"], E=c["E"], mask_p=0.1, seed=c["seed"])
    idx, _ = W.make_routing(w)
    A = c["A"]
    R = O.layout(idx.numpy(), w.E, expert_alignment=A)
    L = ep().ep_layout(idx.to(DEV), w.E, expert_alignment=A, expert_row_src=c["gather"])
    wts = W.make_expert_weights(w, c["N"])
    if c["gather"]:
        x = W.make_x(w)
        rows = O.dispatch_bf16(u16(x), R["slot"], R["n_rows_expert"])
    else:
        x = W.make_rows(w, L.max_expert_rows())
        rows = None
    # padding rows are never written: start from zeros so they hold no NaN patterns
    y = torch.zeros(L.max_expert_rows(), c["N"], dtype=torch.bfloat16, device=DEV)
    yp = torch.zeros_like(y)
    ep().ep_expert_gemm(x.to(DEV), L, wts.to(DEV), out=y, gather=c["gather"])
    ep().ep_expert_gemm(x.to(DEV), L, ep().ep_pack_expert_weights(wts.to(DEV)), out=yp, gather=c["gather"])
    torch.cuda.synchronize()
    n = R["n_rows_expert"]
    occupied = np.zeros(n, bool)
    for e in range(w.E):
        occupied[R["offsets"][e] : R["offsets"][e] + R["counts"][e]] = True
    got = u16(y)[:n]
    assert np.array_equal(u16(yp)[:n][occupied], got[occupied])
    xin = rows if rows is not None else u16(x)[:n]
    if occupied.any():
        _check(got, xin, R["counts"], R["offsets"], u16(wts))
