"""Pins for the oracle's expert alignment / padding rows and combine bias.

Alignment is checked by an exhaustive brute force over small routings
(segment bases from a sort of (e, t, k) tuples plus a closed-form rounding),
by its reduction to the unaligned layout, and by invariants.  The bias is
checked by the cases the pages state (a fully masked token returns its
bias), a zero bias reducing to no bias, and a float64 bound.
"""
import itertools

import numpy as np
import pytest
import torch

from oracle import ep_oracle as O
import workloads as W


def _u16(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _aligned_by_sort(idx, E, A):
    T, K = idx.shape
    ents = sorted((int(idx[t, k]), t, k) for t in range(T) for k in range(K) if 0 <= idx[t, k] < E)
    cnt = np.bincount([e for e, _, _ in ents], minlength=E)
    seg = [(-(-c // A)) * A for c in cnt]  # ceil(c / A) * A
    base = np.concatenate([[0], np.cumsum(seg)])
    slot = np.full((T, K), -1, np.int64)
    seen = np.zeros(E, np.int64)
    for e, t, k in ents:
        slot[t, k] = base[e] + seen[e]
        seen[e] += 1
    src = -np.ones(base[-1], np.int64)
    for e, t, k in ents:
        src[slot[t, k]] = t
    return slot, base, src


@pytest.mark.parametrize("T,K,E,A", [(2, 2, 3, 2), (3, 2, 2, 4), (2, 3, 3, 3)])
def test_alignment_bruteforce(T, K, E, A):
    vals = list(range(-1, E))
    for combo in itertools.product(vals, repeat=T * K):
        idx = np.array(combo, np.int64).reshape(T, K)
        L = O.layout(idx, E, expert_alignment=A)
        slot, base, src = _aligned_by_sort(idx, E, A)
        assert np.array_equal(L["slot"], slot)
        assert np.array_equal(L["offsets"], base)
        assert np.array_equal(L["expert_row_src"], src)
        assert L["n_sel"] == int((idx >= 0).sum())
        assert L["n_rows_expert"] == base[-1]


def test_alignment_one_is_unaligned_and_invariants():
    w = W.by_name("skewed_masked").replace(T=700)
    idx, _ = W.make_routing(w)
    idx = idx.numpy()
    L0 = O.layout(idx, w.E)
    L1 = O.layout(idx, w.E, expert_alignment=1)
    for k in ("counts", "offsets", "slot", "expert_row_src"):
        assert np.array_equal(L0[k], L1[k])
    assert L0["n_rows_expert"] == L0["n_sel"]
    for A in (8, 128):
        L = O.layout(idx, w.E, expert_alignment=A)
        off, cnt = L["offsets"], L["counts"]
        assert np.all(off % A == 0)
        assert np.all(np.diff(off) == -(-cnt // A) * A)
        # relative placement inside each segment is the unaligned one
        for e in range(w.E):
            sel = idx == e
            assert np.array_equal(L["slot"][sel] - off[e], L0["slot"][sel] - L0["offsets"][e])
        # padding rows are exactly the rows past each expert's selections
        pad = np.ones(L["n_rows_expert"], bool)
        for e in range(w.E):
            pad[off[e] : off[e] + cnt[e]] = False
        assert np.array_equal(L["expert_row_src"] < 0, pad)
        x = O.bf16_rne(np.random.default_rng(A).standard_normal((w.T, 16)).astype(np.float32))
        recv = O.dispatch_bf16(x, L["slot"], L["n_rows_expert"])
        assert not recv[pad].any()
        assert np.array_equal(recv[~pad], x[L["expert_row_src"][~pad]])


def test_bias_masked_token_returns_bias_and_zero_bias_is_no_bias():
    rng = np.random.default_rng(2)
    T, H, K = 6, 32, 3
    y = O.bf16_rne(rng.standard_normal((T * K, H)).astype(np.float32))
    slot = np.arange(T * K).reshape(T, K)
    slot[2] = -1
    slot[4, 1] = -1
    w = rng.random((T, K)).astype(np.float32)
    b0 = O.bf16_rne(rng.standard_normal((T, H)).astype(np.float32))
    b1 = O.bf16_rne(rng.standard_normal((T, H)).astype(np.float32))
    out1 = O.combine(y, slot, w, bias0=b0)
    assert np.array_equal(out1[2], b0[2])  # fully masked: its bias, exactly
    out2 = O.combine(y, slot, w, bias0=b0, bias1=b1)
    two = (O.bf16_to_f32(b0[2]) + O.bf16_to_f32(b1[2])).astype(np.float32)
    assert np.array_equal(out2[2], O.bf16_rne(two))
    zero = np.zeros((T, H), np.uint16)
    assert np.array_equal(O.combine(y, slot, w, bias0=zero), O.combine(y, slot, w))
    # float64 reference: bias plus the weighted rows, within bf16 rounding
    ref = O.bf16_to_f32(b0).astype(np.float64) + O.bf16_to_f32(b1).astype(np.float64)
    for k in range(K):
        m = slot[:, k] >= 0
        ref[m] += w[m, k][:, None].astype(np.float64) * O.bf16_to_f32(y[slot[m, k]]).astype(np.float64)
    got = O.bf16_to_f32(out2).astype(np.float64)
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2.0**-8 + 1e-6)
    # grouped order: the bias seeds the cross-group total
    idx = np.where(slot >= 0, (np.arange(T * K).reshape(T, K) * 7) % 12, -1)
    g1 = O.combine_grouped(y, idx, slot, w, 12, 3, bias0=b0)
    assert np.array_equal(g1[2], b0[2])
    assert np.array_equal(O.combine_grouped(y, idx, slot, w, 12, 1, bias0=b0, bias1=b1), out2)


def test_expert_gemm_bruteforce_and_segments():
    rng = np.random.default_rng(12)
    E, N, H = 3, 5, 7
    counts = np.array([2, 0, 3])
    offsets = np.array([0, 4, 4, 8])  # aligned to 4: rows 2,3 and 7 are padding
    x = O.bf16_rne(rng.standard_normal((8, H)).astype(np.float32))
    w = O.bf16_rne(rng.standard_normal((E, N, H)).astype(np.float32))
    y = O.expert_gemm(x, counts, offsets, w)
    xf, wf = O.bf16_to_f32(x).astype(np.float64), O.bf16_to_f32(w).astype(np.float64)
    for r in range(8):
        e = 0 if r < 2 else (2 if 4 <= r < 7 else None)
        for n in range(N):
            if e is None:
                assert np.isnan(y[r, n])
            else:
                ref = sum(xf[r, h] * wf[e, n, h] for h in range(H))
                assert abs(y[r, n] - ref) <= 1e-12 * max(1.0, abs(ref))
    sub = O.expert_gemm(x, counts, offsets, w, rows=[1, 5])
    assert np.array_equal(sub[[1, 5]], y[[1, 5]]) and np.isnan(sub[[0, 4, 6]]).all()
    b = O.expert_gemm_bound(x, counts, offsets, w, y)
    assert np.all(b[[0, 1, 4, 5, 6]] > 0)
    # an fp32 sum in k order, rounded to bf16, sits inside the bound
    got = np.full(8, np.nan)
    for e in range(E):
        for r in range(offsets[e], offsets[e] + counts[e]):
            acc = np.float32(0.0)
            for h in range(H):
                acc = np.float32(acc + np.float32(xf[r, h] * wf[e, 0, h]))
            got[r] = O.bf16_to_f32(O.bf16_rne(np.array([acc], np.float32)))[0]
    ok = ~np.isnan(y[:, 0])
    assert np.all(np.abs(got[ok] - y[ok, 0]) <= b[ok, 0])


def test_bias_seeds_the_accumulator_not_added_after():
    """The bias starts the fp32 sum (the reading of "seeds the reduce
    accumulator"): with bias -1 and terms 1 and 2^-30 the seeded flat sum is
    (-1 + 1) + 2^-30 = 2^-30, while adding the bias after the terms would
    give (1 + 2^-30) - 1 = 0 in fp32."""
    one = O.bf16_rne(np.array([1.0], np.float32))[0]
    tiny = O.bf16_rne(np.array([2.0**-30], np.float32))[0]
    minus_one = O.bf16_rne(np.array([-1.0], np.float32))[0]
    y = np.array([[one], [tiny]], np.uint16)
    slot = np.array([[0, 1]])
    w = np.ones((1, 2), np.float32)
    out = O.combine(y, slot, w, bias0=np.array([[minus_one]], np.uint16))
    assert out[0, 0] == tiny
    # grouped order: the bias seeds the cross-group total, each group's
    # partial starts from +0.  Two groups: (-1 + 1) + 2^-30 = 2^-30; one
    # group: -1 + (1 + 2^-30 -> 1) = +0.
    b = np.array([[minus_one]], np.uint16)
    assert O.combine_grouped(y, np.array([[0, 1]]), slot, w, 2, 2, bias0=b)[0, 0] == tiny
    assert O.combine_grouped(y, np.array([[0, 1]]), slot, w, 2, 1, bias0=b)[0, 0] == 0x0000


def test_gemm_bound_covers_fp32_cancellation():
    """The bound's accumulation term matters: the fp32 sum in k order of
    2^20 + 2^-5 - 2^20 is 0 (2^-5 is lost against 2^20), the exact value
    2^-5; the bf16 rounding term alone (2^-8 |y|) would not cover that."""
    vals = [2.0**20, 2.0**-5, -(2.0**20)]
    x = O.bf16_rne(np.ones((1, 3), np.float32))
    w = O.bf16_rne(np.array([[vals]], np.float32))  # [E=1, N=1, H=3]
    y64 = O.expert_gemm(x, np.array([1]), np.array([0, 1]), w)
    assert y64[0, 0] == 2.0**-5
    acc = np.float32(0.0)
    for v in vals:
        acc = np.float32(acc + np.float32(v))
    assert acc == 0.0
    b = O.expert_gemm_bound(x, np.array([1]), np.array([0, 1]), w, y64)
    assert abs(float(acc) - y64[0, 0]) <= b[0, 0]
    assert abs(float(acc) - y64[0, 0]) > abs(y64[0, 0]) * 2.0**-8
