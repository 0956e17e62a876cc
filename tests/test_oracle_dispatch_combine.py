"""Pins for the oracle's dispatch and combine (CPU only).

Dispatch rows carry their token's identity, so a misplaced row cannot look
plausible.  Combine is pinned by the invariants the method fixes (a fully
masked token gives +0; unit weights over rows equal to the token give K*x;
K = 1 with unit weight is the identity), by a float64 reference within the
bf16 bound, by the tiny workload's closed form, and by a scalar per-token
brute force in a different evaluation order where the grouped sum reduces to
a plain one.
"""
import numpy as np
import pytest
import torch

from oracle import ep_oracle as O
import workloads as W


def _u16(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _identity_x(T, H):
    """bf16 rows whose every element encodes (token, column) exactly."""
    t = np.arange(T)[:, None]
    h = np.arange(H)[None, :]
    v = ((t % 251) + 1) * 2.0 ** -(h % 5)  # exact in bf16 (8 significant bits)
    sign = np.where((t * 7 + h) % 3 == 0, -1.0, 1.0)
    return O.bf16_rne((sign * v).astype(np.float32))


def test_dispatch_bf16_rows_carry_token_identity():
    w = W.by_name("skewed_masked").replace(T=600, H=136)
    idx, _ = W.make_routing(w)
    idx = idx.numpy()
    L = O.layout(idx, w.E)
    x = _identity_x(w.T, w.H)
    recv = O.dispatch_bf16(x, L["slot"], L["n_sel"])
    for t in range(w.T):
        for k in range(w.K):
            if idx[t, k] >= 0:
                assert np.array_equal(recv[L["slot"][t, k]], x[t])
    # each expert segment holds exactly the tokens that picked it
    for e in range(w.E):
        seg = recv[L["offsets"][e] : L["offsets"][e + 1]]
        toks = sorted(np.nonzero((idx == e).any(axis=1))[0].tolist())
        got = sorted(int(np.flatnonzero((x == r).all(axis=1))[0]) for r in seg)
        assert got == toks


def test_dispatch_grouped_rows():
    w = W.by_name("grouped").replace(T=300, H=64)
    idx, wt = W.make_routing(w)
    L = O.layout(idx.numpy(), w.E, w.G, wt.numpy())
    x = _identity_x(w.T, w.H)
    recv = O.dispatch_bf16(x, L["grow"], L["n_rows"])
    assert np.array_equal(recv, x[L["src"]])
    # no duplicate (group, token) pairs
    g_of_row = np.searchsorted(L["goffsets"], np.arange(L["n_rows"]), side="right") - 1
    pairs = set(zip(g_of_row.tolist(), L["src"].tolist()))
    assert len(pairs) == L["n_rows"]


def test_dispatch_fp8_rows_equal_quantized_token():
    w = W.by_name("pages").replace(T=40, H=512)
    idx, _ = W.make_routing(w)
    L = O.layout(idx.numpy(), w.E)
    x = _u16(W.make_x(w))
    recv = O.dispatch_fp8(x, L["slot"], L["n_sel"])
    assert recv.shape == (L["n_sel"], O.fp8_row_bytes(w.H))
    for t in range(w.T):
        row = O.quantize_row_fp8(x[t])
        for k in range(w.K):
            assert np.array_equal(recv[L["slot"][t, k]], row)


# ---------------------------------------------------------------- combine
def test_fully_masked_token_combines_to_positive_zero():
    rng = np.random.default_rng(1)
    y = O.bf16_rne(rng.standard_normal((6, 32)).astype(np.float32))
    slot = np.array([[0, 1], [-1, -1], [2, -1], [-1, -1], [4, 5]])
    w = rng.random((5, 2)).astype(np.float32)
    out = O.combine(y, slot, w)
    assert np.all(out[1] == 0x0000) and np.all(out[3] == 0x0000)
    out_g = O.combine_grouped(y, np.array([[0, 1], [-1, -1], [1, -1], [-1, -1], [0, 1]]), slot, w, 2, 2)
    assert np.all(out_g[1] == 0x0000)


@pytest.mark.parametrize("K", [1, 2, 4, 8])
def test_unit_weights_over_dispatched_rows_give_K_x(K):
    w = W.Workload("kx", T=200, H=96, K=K, E=32)
    idx, _ = W.make_routing(w)
    idx = idx.numpy()
    L = O.layout(idx, w.E)
    x = _u16(W.make_x(w))
    y = O.dispatch_bf16(x, L["slot"], L["n_sel"])
    ones = np.ones((w.T, K), np.float32)
    out = O.combine(y, L["slot"], ones)
    # K * x is exact in fp32 and in bf16 for K a power of two
    expect = O.bf16_rne((O.bf16_to_f32(x) * np.float32(K)).astype(np.float32))
    assert np.array_equal(out, expect)
    if K == 1:
        assert np.array_equal(out, x)


def test_masked_unit_weights_give_keff_x():
    w = W.Workload("keff", T=300, H=64, K=8, E=64, mask_p=0.5)
    idx, _ = W.make_routing(w)
    idx = idx.numpy()
    L = O.layout(idx, w.E)
    x = _u16(W.make_x(w))
    y = O.dispatch_bf16(x, L["slot"], L["n_sel"])
    out = O.combine(y, L["slot"], np.ones((w.T, w.K), np.float32))
    keff = (idx >= 0).sum(axis=1).astype(np.float64)
    exact = O.bf16_to_f32(x).astype(np.float64) * keff[:, None]
    # sums of up to 8 bf16 copies are exact in fp32; output is one bf16 rounding
    assert np.array_equal(out, O.bf16_rne(exact.astype(np.float32)))


def test_combine_within_bf16_bound_of_float64():
    w = W.by_name("mid").replace(T=256, H=512)
    idx, wt = W.make_routing(w)
    idx, wt = idx.numpy(), wt.numpy()
    L = O.layout(idx, w.E)
    y = _u16(W.make_y(w, rows=L["n_sel"]))
    out = O.bf16_to_f32(O.combine(y, L["slot"], wt)).astype(np.float64)
    yf = O.bf16_to_f32(y).astype(np.float64)
    ref = np.zeros((w.T, w.H))
    for k in range(w.K):
        ref += wt[:, k : k + 1].astype(np.float64) * yf[L["slot"][:, k]]
    absw = np.zeros_like(ref)
    for k in range(w.K):
        absw += np.abs(wt[:, k : k + 1].astype(np.float64) * yf[L["slot"][:, k]])
    # bf16 output rounding (2^-9 relative) plus K fp32 roundings on |terms|
    assert np.all(np.abs(out - ref) <= np.abs(ref) * 2.0**-8 + absw * 2.0**-20 + 1e-30)
    rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert rel < 1e-2


def test_tiny_closed_form():
    w = W.by_name("tiny")
    idx, wt = W.make_routing(w)
    idx, wt = idx.numpy(), wt.numpy()
    L = O.layout(idx, w.E)
    xt = W.make_x(w)
    x = _u16(xt)
    recv = O.dispatch_bf16(x, L["slot"], L["n_sel"])
    row_e = np.searchsorted(L["offsets"], np.arange(L["n_sel"]), side="right") - 1
    y = _u16(W.tiny_expert_outputs(torch.from_numpy(recv.view(np.int16)).view(torch.bfloat16), torch.from_numpy(row_e)))
    out = O.bf16_to_f32(O.combine(y, L["slot"], wt)).astype(np.float64)
    xf = O.bf16_to_f32(x).astype(np.float64)
    f = (wt.astype(np.float64) * (1.0 + idx / 16.0)).sum(axis=1)
    ref = f[:, None] * xf
    # y carries one bf16 rounding per term, plus the output rounding
    assert np.all(np.abs(out - ref) <= (np.abs(ref) + np.abs(xf) * 2) * 2.0**-7 + 1e-30)


def _scalar_grouped(y, idx, slot, w, E, G, t, h):
    """Per-element scalar evaluation: sort the token's entries by (group, k)."""
    epg = E // G
    ents = sorted((int(idx[t, k]) // epg, k) for k in range(idx.shape[1]) if slot[t, k] >= 0)
    tot = np.float32(0.0)
    cur_g, P = None, np.float32(0.0)
    for g, k in ents:
        if g != cur_g:
            if cur_g is not None:
                tot = np.float32(tot + P)
            cur_g, P = g, np.float32(0.0)
        yv = O.bf16_to_f32(np.array([y[slot[t, k], h]], np.uint16))[0]
        P = np.float32(P + np.float32(w[t, k] * yv))
    if cur_g is not None:
        tot = np.float32(tot + P)
    return tot


def test_grouped_combine_scalar_bruteforce_and_reductions():
    w = W.by_name("grouped").replace(T=48, H=16, mask_p=0.2)
    idx, wt = W.make_routing(w)
    idx, wt = idx.numpy(), wt.numpy()
    L = O.layout(idx, w.E, w.G, wt)
    y = _u16(W.make_y(w, rows=max(L["n_sel"], 1)))
    out = O.combine_grouped(y, idx, L["slot"], wt, w.E, w.G)
    for t in range(w.T):
        for h in range(w.H):
            ref = _scalar_grouped(y, idx, L["slot"], wt, w.E, w.G, t, h)
            assert out[t, h] == O.bf16_rne(np.array([ref], np.float32))[0]
    # G = 1 is the flat combine
    assert np.array_equal(O.combine_grouped(y, idx, L["slot"], wt, w.E, 1), O.combine(y, L["slot"], wt))
    # G = E sums in ascending expert order
    outE = O.combine_grouped(y, idx, L["slot"], wt, w.E, w.E)
    for t in range(0, w.T, 7):
        ks = sorted((int(idx[t, k]), k) for k in range(w.K) if idx[t, k] >= 0)
        for h in range(w.H):
            acc = np.float32(0.0)
            for _, k in ks:
                yv = O.bf16_to_f32(np.array([y[L["slot"][t, k], h]], np.uint16))[0]
                acc = np.float32(acc + np.float32(wt[t, k] * yv))
            assert outE[t, h] == O.bf16_rne(np.array([acc], np.float32))[0]


def test_flat_combine_scalar_bruteforce():
    w = W.by_name("skewed_masked").replace(T=40, H=24)
    idx, wt = W.make_routing(w)
    idx, wt = idx.numpy(), wt.numpy()
    L = O.layout(idx, w.E)
    y = _u16(W.make_y(w, rows=max(L["n_sel"], 1)))
    out = O.combine(y, L["slot"], wt)
    for t in range(w.T):
        for h in range(w.H):
            acc = np.float32(0.0)
            for k in range(w.K):
                if L["slot"][t, k] >= 0:
                    yv = O.bf16_to_f32(np.array([y[L["slot"][t, k], h]], np.uint16))[0]
                    acc = np.float32(acc + np.float32(wt[t, k] * yv))
            assert out[t, h] == O.bf16_rne(np.array([acc], np.float32))[0]


def test_summation_order_is_visible_and_fixed():
    """Values chosen so that each summation order gives a different bf16.

    Token 0: k0 -> expert 2 (group 1) value 2^25, k1 -> expert 0 (group 0)
    value 1, k2 -> expert 3 (group 1) value -2^25, unit weights.
      flat ascending k:  (2^25 + 1) - 2^25 = 0   (the 1 is absorbed)
      grouped (2 groups): P0 = 1, P1 = 2^25 - 2^25 = 0, total = 1
    """
    vals = np.array([2.0**25, 1.0, -(2.0**25)], np.float32)
    y = O.bf16_rne(np.repeat(vals[:, None], 4, axis=1))
    idx = np.array([[2, 0, 3]])
    L = O.layout(idx, 4)
    # rows in expert-major order: expert 0 -> row 0, expert 2 -> 1, expert 3 -> 2
    assert L["slot"].tolist() == [[1, 0, 2]]
    yr = y[[1, 0, 2]]
    w = np.ones((1, 3), np.float32)
    flat = O.bf16_to_f32(O.combine(yr, L["slot"], w))
    grouped = O.bf16_to_f32(O.combine_grouped(yr, idx, L["slot"], w, 4, 2))
    assert np.all(flat == 0.0)
    assert np.all(grouped == 1.0)


def test_group_order_is_ascending():
    """Three groups of two experts; one selection per group, unit weights.

    k0 -> expert 4 (group 2) value 1, k1 -> expert 0 (group 0) value 2^25,
    k2 -> expert 2 (group 1) value -2^25.
      ascending groups: (2^25 - 2^25) + 1 = 1
      descending groups: (1 - 2^25) + 2^25 = 0   (the 1 is absorbed)
      flat ascending k: (1 + 2^25) - 2^25 = 0
    """
    idx = np.array([[4, 0, 2]])
    L = O.layout(idx, 6)
    vals_by_k = np.array([1.0, 2.0**25, -(2.0**25)], np.float32)
    y = np.zeros((3, 4), np.uint16)
    for k in range(3):
        y[L["slot"][0, k]] = O.bf16_rne(np.full(4, vals_by_k[k], np.float32))
    w = np.ones((1, 3), np.float32)
    assert np.all(O.bf16_to_f32(O.combine_grouped(y, idx, L["slot"], w, 6, 3)) == 1.0)
    assert np.all(O.bf16_to_f32(O.combine(y, L["slot"], w)) == 0.0)


def test_fp8_quotient_is_a_true_division():
    """The fp8 quotient is the IEEE fp32 division x / s (reading of the
    spec formula), not x * (1 / s): for this bf16 group the exact
    quotient rounds to fp32 84.0, the midpoint between the E4M3 values 80
    and 88, so ties-to-even gives 80 (code 0x6A).  The product with the
    rounded reciprocal is 84.0000076, which would encode as 88 (0x6B)."""
    from fractions import Fraction

    a = O.bf16_to_f32(np.array([0x3D98], np.uint16))[0]  # the group's amax
    xv = O.bf16_to_f32(np.array([0x3C64], np.uint16))[0]
    s = np.float32(Fraction(float(a)) / 448)  # exact a/448 rounded once to fp32
    # the exact quotient, rounded to the nearest fp32 by comparing neighbours
    q = Fraction(float(xv)) / Fraction(float(s))
    c = np.float32(float(q))
    cands = [np.nextafter(c, np.float32(0)), c, np.nextafter(c, np.float32(np.inf))]
    nearest = min(cands, key=lambda f: abs(Fraction(float(f)) - q))
    assert nearest == np.float32(84.0)
    g = np.zeros(128, np.uint16)
    g[0], g[1] = 0x3D98, 0x3C64
    row = O.quantize_row_fp8(g)
    assert row[0] == 0x7E  # the amax element encodes to 448
    assert row[1] == 0x6A  # 80: the tie at 84 goes to the even code
    assert np.frombuffer(row[128:132].tobytes(), "<f4")[0] == s
