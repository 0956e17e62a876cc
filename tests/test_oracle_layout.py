"""Pins for the oracle's layout (count, exclusive scan, slot; grouped rows).

Checked against things other than the oracle itself: an exhaustive brute
force over every routing of tiny problems (placement by sorting (expert,
token, k) tuples), numpy's stable argsort, the invariants the pages state
(every selection placed exactly once, counts summing to the selections, no
duplicate (source, token) pairs) and a closed-form expectation of the number
of grouped rows.
"""
import itertools
import math

import numpy as np
import pytest
import torch

from oracle import ep_oracle as O
import workloads as W


def _placement_by_sort(idx, E):
    """slot by sorting valid (e, t, k) tuples: position in sorted order."""
    T, K = idx.shape
    ents = sorted((int(idx[t, k]), t, k) for t in range(T) for k in range(K) if 0 <= idx[t, k] < E)
    slot = np.full((T, K), -1, np.int64)
    for pos, (_, t, k) in enumerate(ents):
        slot[t, k] = pos
    return slot


def _grouped_by_sort(idx, E, G):
    T, K = idx.shape
    epg = E // G
    pairs = sorted({(int(idx[t, k]) // epg, t) for t in range(T) for k in range(K) if 0 <= idx[t, k] < E})
    row = {p: r for r, p in enumerate(pairs)}
    grow = np.full((T, K), -1, np.int64)
    for t in range(T):
        for k in range(K):
            if 0 <= idx[t, k] < E:
                grow[t, k] = row[(int(idx[t, k]) // epg, t)]
    return grow, len(pairs)


@pytest.mark.parametrize("T,K,E", [(2, 2, 3), (3, 2, 2), (1, 3, 4), (4, 1, 3)])
def test_layout_bruteforce_all_routings(T, K, E):
    vals = list(range(-2, E + 1))  # -2 and E are invalid ids, -1 "no selection"
    n = 0
    for combo in itertools.product(vals, repeat=T * K):
        idx = np.array(combo, np.int64).reshape(T, K)
        L = O.layout(idx, E)
        assert np.array_equal(L["slot"], _placement_by_sort(idx, E))
        valid = (idx >= 0) & (idx < E)
        assert L["n_invalid"] == int(((idx == -2) | (idx == E)).sum())
        assert L["n_sel"] == int(valid.sum())
        assert np.array_equal(L["counts"], np.bincount(idx[valid], minlength=E))
        n += 1
    assert n == len(vals) ** (T * K)


@pytest.mark.parametrize("T,K,E,G", [(3, 2, 4, 2), (2, 3, 4, 4), (4, 2, 4, 1), (2, 2, 6, 3)])
def test_grouped_layout_bruteforce(T, K, E, G):
    vals = list(range(-1, E))
    rng = np.random.default_rng(T * 100 + K * 10 + E + G)
    combos = list(itertools.product(vals, repeat=T * K))
    if len(combos) > 4000:
        combos = [combos[i] for i in rng.choice(len(combos), 4000, replace=False)]
    w = rng.random((T, K)).astype(np.float32)
    epg = E // G
    for combo in combos:
        idx = np.array(combo, np.int64).reshape(T, K)
        L = O.layout(idx, E, G, w)
        grow, R = _grouped_by_sort(idx, E, G)
        assert L["n_rows"] == R
        assert np.array_equal(L["grow"], grow)
        # row lists: K-wide, local ids and weights of the row's group only
        for r in range(R):
            t = L["src"][r]
            ks = [k for k in range(K) if grow[t, k] == r]
            assert ks
            for k in range(K):
                if k in ks:
                    assert L["ridx"][r, k] == idx[t, k] - (idx[t, k] // epg) * epg
                    assert L["rw"][r, k] == w[t, k]
                else:
                    assert L["ridx"][r, k] == -1 and L["rw"][r, k] == 0.0


def test_slot_is_inverse_of_stable_argsort():
    rng = np.random.default_rng(7)
    T, K, E = 700, 6, 37
    idx = rng.integers(-1, E, (T, K))
    L = O.layout(idx, E)
    flat = idx.reshape(-1)
    valid = flat >= 0
    order = np.flatnonzero(valid)[np.argsort(flat[valid], kind="stable")]
    slot = L["slot"].reshape(-1)
    assert np.array_equal(slot[order], np.arange(valid.sum()))
    assert np.all(slot[~valid] == -1)


def test_layout_invariants_on_workloads():
    for name in ("tiny", "mid", "skewed_masked"):
        w = W.by_name(name)
        if w.T > 2048:
            w = w.replace(T=2048)
        idx, _ = W.make_routing(w)
        idx = idx.numpy()
        L = O.layout(idx, w.E)
        valid = idx >= 0
        s = L["slot"][valid]
        # every valid selection appears exactly once
        assert np.array_equal(np.sort(s), np.arange(valid.sum()))
        assert L["counts"].sum() == valid.sum() == L["n_sel"]
        assert L["offsets"][0] == 0 and np.all(np.diff(L["offsets"]) == L["counts"])
        # inside a segment the source tokens strictly increase (distinct experts per token)
        for e in range(w.E):
            t, k = np.nonzero((idx == e))
            order = np.argsort(L["slot"][t, k])
            assert np.all(np.diff(t[order]) > 0)
            assert np.all((L["slot"][t, k] >= L["offsets"][e]) & (L["slot"][t, k] < L["offsets"][e + 1]))


def test_duplicate_expert_in_token_gets_two_rows():
    idx = np.array([[3, 3, -1], [3, 0, 3]])
    L = O.layout(idx, 4)
    assert L["slot"].tolist() == [[1, 2, -1], [3, 0, 4]]
    Lg = O.layout(idx, 4, 2)  # group of expert 3 is 1; hit once per token
    assert Lg["n_rows"] == 3
    assert Lg["grow"].tolist() == [[1, 1, -1], [2, 0, 2]]


def test_group1_one_row_per_token_and_groupE_equals_expert_rows():
    w = W.by_name("skewed_masked").replace(T=1024)
    idx, wt = W.make_routing(w)
    idx, wt = idx.numpy(), wt.numpy()
    L1 = O.layout(idx, w.E, 1, wt)
    active = (idx >= 0).any(axis=1)
    assert L1["n_rows"] == active.sum()
    assert np.array_equal(L1["src"], np.flatnonzero(active))
    LE = O.layout(idx, w.E, w.E, wt)
    # one expert per group and distinct experts per token: rows == selections
    assert np.array_equal(LE["grow"], LE["slot"])
    assert np.array_equal(LE["gcounts"], LE["counts"])


def test_grouped_rows_per_token_closed_form():
    """Uniform top-8 of 256 in 8 groups: E[#groups hit] = G(1 - C(E-E/G,K)/C(E,K))."""
    w = W.by_name("grouped").replace(T=8192)
    idx, wt = W.make_routing(w)
    L = O.layout(idx.numpy(), w.E, w.G, wt.numpy())
    epg = w.E // w.G
    expect = w.G * (1 - math.comb(w.E - epg, w.K) / math.comb(w.E, w.K))
    assert abs(expect - 5.2947) < 1e-4
    got = L["n_rows"] / w.T
    # per-token count has variance < 2; 5 sigma over 8192 tokens ~ 0.08
    assert abs(got - expect) < 0.08, got
    assert L["gcounts"].sum() == L["n_rows"]
