"""Property tests (hypothesis) of the oracle on random tiny shapes.

Each property compares the oracle with something other than itself: the
placement by sorting (expert, token, k) tuples, the set of (group, token)
pairs, segment invariants the pages state, and the E4M3FN value table for the
quantised payload.  Sizes stay tiny so the whole file runs in seconds.
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import ep_oracle as O

SETTINGS = dict(max_examples=60, deadline=None)


@st.composite
def routing(draw, max_T=6, max_K=4, max_E=6, with_groups=False):
    E = draw(st.integers(1, max_E))
    G = 0
    if with_groups:
        G = draw(st.sampled_from([g for g in range(1, E + 1) if E % g == 0]))
    T = draw(st.integers(0, max_T))
    K = draw(st.integers(1, max_K))
    ids = draw(st.lists(st.integers(-2, E), min_size=T * K, max_size=T * K))
    return np.array(ids, np.int64).reshape(T, K), E, G


def _by_sort(idx, E):
    T, K = idx.shape
    ents = sorted((int(idx[t, k]), t, k) for t in range(T) for k in range(K) if 0 <= idx[t, k] < E)
    slot = np.full((T, K), -1, np.int64)
    for pos, (_, t, k) in enumerate(ents):
        slot[t, k] = pos
    return slot


@settings(**SETTINGS)
@given(routing())
def test_slot_equals_sorted_placement(case):
    idx, E, _ = case
    L = O.layout(idx, E)
    assert np.array_equal(L["slot"], _by_sort(idx, E))
    valid = (idx >= 0) & (idx < E)
    assert L["n_sel"] == int(valid.sum())
    assert L["n_invalid"] == int(((idx != -1) & ~valid).sum())
    # every selection placed exactly once, onto [0, n_sel)
    placed = np.sort(L["slot"][valid])
    assert np.array_equal(placed, np.arange(L["n_sel"]))


@settings(**SETTINGS)
@given(routing(), st.sampled_from([1, 2, 3, 4, 8]))
def test_aligned_segments(case, A):
    idx, E, _ = case
    L = O.layout(idx, E, expert_alignment=A)
    U = O.layout(idx, E)
    off, cnt = L["offsets"], L["counts"]
    assert np.array_equal(cnt, U["counts"])
    seg = np.diff(off)
    assert np.all(seg % A == 0) and np.all(seg >= cnt) and np.all(seg - cnt < A)
    # rank inside the segment is unchanged by alignment
    valid = L["slot"] >= 0
    e = idx[valid]
    assert np.array_equal(L["slot"][valid] - off[e], U["slot"][valid] - U["offsets"][e])
    src = L["expert_row_src"]
    assert len(src) == off[-1]
    assert int((src >= 0).sum()) == L["n_sel"]
    for ee in range(E):
        rows = src[off[ee] : off[ee + 1]]
        assert np.all(rows[: cnt[ee]] >= 0) and np.all(rows[cnt[ee] :] == -1)
        assert np.all(np.diff(rows[: cnt[ee]]) >= 0)  # stable by token


@settings(**SETTINGS)
@given(routing(with_groups=True))
def test_grouped_rows_are_the_sorted_group_token_pairs(case):
    idx, E, G = case
    T, K = idx.shape
    w = np.arange(T * K, dtype=np.float32).reshape(T, K) + 0.5
    L = O.layout(idx, E, G, w)
    epg = E // G
    pairs = sorted({(int(idx[t, k]) // epg, t) for t in range(T) for k in range(K) if 0 <= idx[t, k] < E})
    assert L["n_rows"] == len(pairs)
    assert [(int(L["src"][r]), r) for r in range(len(pairs))] == [(t, r) for r, (_, t) in enumerate(pairs)]
    row = {p: r for r, p in enumerate(pairs)}
    for t in range(T):
        for k in range(K):
            e = int(idx[t, k])
            if 0 <= e < E:
                r = row[(e // epg, t)]
                assert L["grow"][t, k] == r
                assert L["ridx"][r, k] == e - (e // epg) * epg
                assert L["rw"][r, k] == w[t, k]
            else:
                assert L["grow"][t, k] == -1
    # list entries outside a row's group are empty
    for r, (g, t) in enumerate(pairs):
        for k in range(K):
            e = int(idx[t, k])
            if not (0 <= e < E and e // epg == g):
                assert L["ridx"][r, k] == -1 and L["rw"][r, k] == 0.0


@settings(**SETTINGS)
@given(st.integers(0, 2**32 - 1), st.floats(1e-3, 1e3))
def test_fp8_payload_codes_lie_on_the_grid_around_each_value(seed, scale):
    """Every quantised element decodes to one of the two E4M3FN grid values
    around x/s (or to +-448 at the top), and the group maximum to +-448."""
    rng = np.random.default_rng(seed)
    x = O.bf16_rne((rng.standard_normal(256) * scale).astype(np.float32))
    row = O.quantize_row_fp8(x)
    q = row[:256]
    s = row[256 : 256 + 8].view("<f4")
    table = O.e4m3fn_value_table()
    xf = O.bf16_to_f32(x)
    for g in range(2):
        xs = xf[g * 128 : (g + 1) * 128]
        sg = np.float32(s[g])
        assert sg == np.float32(np.abs(xs).max() / np.float32(448.0))
        v = (xs / sg).astype(np.float32)
        mag = np.minimum(np.abs(v), 448.0)
        dec = table[q[g * 128 : (g + 1) * 128] & 0x7F]
        lo = np.array([table[table <= m].max() for m in mag])
        hi = np.array([table[table >= m].min() for m in mag])
        assert np.all((dec == lo) | (dec == hi))
        top = np.argmax(np.abs(xs))
        assert dec[top] == 448.0
