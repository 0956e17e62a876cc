"""Layout, bf16 dispatch and combine at the largest selection count the
library accepts: T * K = 2,147,483,640 (268,435,455 tokens, top-8 of 256
experts), just below the int32 limit on slots and rows.  Hidden is 8
(16-byte rows) so the receive rows fit in HBM (34 GB).

Routing: expert (7 t + 37 k) mod 256, distinct within a token; every 97th
selection masked (-1), every 1009th an invalid id (259), every 1000th token
fully masked.

Checks, at full size on the GPU with torch:
- counts against a bincount, status[0] against the invalid-id count;
- slot against its definition (the PR's layout: expert-major segments, rows
  of a segment in (t, k) order), as the inverse of a stable sort of the
  flattened expert ids: the j-th entry in (expert, t, k) order holds row j;
- every valid receive row equals its token's row, byte for byte;
- combine with unit weights equals bf16(K_eff * x) bit for bit (K_eff <= 8
  equal terms sum exactly in fp32, and torch's bf16 conversion rounds to
  nearest even), fully masked tokens +0;
and combine with random weights against the oracle on 2,112 sampled tokens,
the last 64 among them."""
import numpy as np
import pytest
import torch

from oracle import ep_oracle as O

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
K, E, H = 8, 256, 8
T = (2**31 - 1) // K
N = T * K
NEED_BYTES = 150 * 10**9


def say(*a):
    print(*a, flush=True)


def u16(t):
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def test_max_selection_count():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    free, _ = torch.cuda.mem_get_info(DEV)
    if free < NEED_BYTES:
        pytest.skip(f"needs {NEED_BYTES / 1e9:.0f} GB of free device memory, {free / 1e9:.0f} GB free")
    import combine_ep_layout_03_amd as ep

    assert N < 2**31
    say(f"max size: T={T} K={K} E={E} H={H}, {N} selections")
    # routing
    kk = torch.arange(K, dtype=torch.int64, device=DEV).view(1, K)
    idx = torch.arange(T, dtype=torch.int64, device=DEV).view(T, 1) * 7 + kk * 37
    idx.remainder_(E)
    flat = idx.view(-1)
    pos = torch.arange(N, dtype=torch.int32, device=DEV)
    flat.masked_fill_(pos.remainder(97) == 0, -1)
    flat.masked_fill_(pos.remainder(1009) == 5, E + 3)
    del pos
    tok_masked = torch.arange(T, dtype=torch.int32, device=DEV).remainder(1000) == 999
    idx.masked_fill_(tok_masked.view(T, 1), -1)
    del tok_masked
    valid = (flat >= 0) & (flat < E)
    n_invalid = int(((flat != -1) & ~valid).sum())
    keys = torch.where(valid, flat, E).to(torch.int32)
    del valid
    torch.cuda.synchronize()
    say("routing built")

    L = ep.ep_layout(idx, E)
    torch.cuda.synchronize()
    say("layout done")
    counts_ref = torch.bincount(keys, minlength=E + 1)[:E].to(torch.int32)
    assert torch.equal(L.counts, counts_ref)
    n_sel = int(counts_ref.sum())
    offs_ref = torch.zeros(E + 1, dtype=torch.int64, device=DEV)
    offs_ref[1:] = torch.cumsum(counts_ref.to(torch.int64), 0)
    assert torch.equal(L.offsets.to(torch.int64), offs_ref)
    st = L.status.cpu().numpy()
    assert st[0] == n_invalid and st[1] == n_sel
    say(f"counts ok: {n_sel} valid selections, {n_invalid} invalid ids")

    # slot is the inverse of the stable sort of the expert ids
    _, order = torch.sort(keys, stable=True)
    del keys
    sflat = L.slot.view(-1)
    got = sflat[order[:n_sel]]
    assert torch.equal(got, torch.arange(n_sel, dtype=torch.int32, device=DEV))
    del got
    assert bool((sflat[order[n_sel:]] == -1).all())
    # token of receive row j (the j-th valid selection in (expert, t, k) order)
    row_tok = (order[:n_sel] // K).to(torch.int32)
    del order
    torch.cuda.synchronize()
    say("slot ok")

    g = torch.Generator(device=DEV)
    g.manual_seed(0)
    x = torch.randn(T, H, generator=g, device=DEV).to(torch.bfloat16)
    recv = ep.ep_dispatch(x, L)
    torch.cuda.synchronize()
    say("dispatch done")
    # recv[slot[t,k]] == x[t], read as: receive row j holds the row of token
    # row_tok[j] (slot was shown to be the inverse of that order above).  The
    # receive rows are read in contiguous slices: torch's advanced indexing
    # returned wrong rows from this 1.7e10-element tensor, and its
    # index_select over 2^26 indices failed to launch, so nothing here indexes
    # a tensor of 2^31 elements or more, and each torch call takes 2^24 rows.
    xi = x.view(torch.int16)
    ri = recv.view(torch.int16)
    step = 1 << 24
    for j0 in range(0, n_sel, step):
        j1 = min(n_sel, j0 + step)
        want = torch.index_select(xi, 0, row_tok[j0:j1].to(torch.int64))
        assert torch.equal(ri[j0:j1], want), f"receive rows {j0}..{j1}"
    del row_tok
    torch.cuda.synchronize()
    say("dispatch ok")

    # combine, unit weights: exact
    wt = torch.ones(T, K, dtype=torch.float32, device=DEV)
    out = ep.ep_combine(recv, L, wt)
    torch.cuda.synchronize()
    say("combine (unit weights) done")
    keff = (L.slot >= 0).sum(1, dtype=torch.int32)
    tstep = 1 << 24
    for t0 in range(0, T, tstep):
        t1 = min(T, t0 + tstep)
        want = (x[t0:t1].float() * keff[t0:t1, None].float() + 0.0).to(torch.bfloat16)
        assert torch.equal(out[t0:t1].view(torch.int16), want.view(torch.int16)), f"combine tokens {t0}..{t1}"
    assert int((keff == 0).sum()) >= T // 1000
    say("combine (unit weights) ok")

    # combine, random weights: sampled tokens against the oracle
    wt.uniform_(generator=g)
    out = ep.ep_combine(recv, L, wt, out=out)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    toks = np.concatenate([np.arange(T - 64, T), rng.choice(T - 64, 2048, replace=False)])
    ti = torch.from_numpy(toks).to(DEV)
    slot_s = L.slot[ti].cpu().numpy()
    used = np.unique(slot_s[slot_s >= 0])  # sorted receive rows of the sample
    y_s = np.concatenate([  # gathered slice by slice, each below 2^31 elements
        u16(recv[r0 : r0 + step][torch.from_numpy(used[(used >= r0) & (used < r0 + step)] - r0).to(DEV)])
        for r0 in range(0, n_sel, step)
    ])
    slot_r = np.where(slot_s >= 0, np.searchsorted(used, slot_s), -1)
    want = O.combine(y_s, slot_r, wt[ti].cpu().numpy())
    assert np.array_equal(u16(out[ti]), want)
    say("combine (random weights) ok on sampled tokens")
    del idx, L, x, recv, wt, out, keff
    torch.cuda.empty_cache()


def test_large_hidden_bf16():
    """Hidden 2^20 + 8 (2 MiB rows, a ragged last chunk): bf16 dispatch and
    flat and grouped combine against the oracle element by element; offsets
    inside a row stay 32-bit there (row bytes < 2^32)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import combine_ep_layout_03_amd as ep
    import workloads as W

    w = W.Workload("wide", T=48, H=(1 << 20) + 8, K=4, E=8, G=2, mask_p=0.2, full_mask_frac=0.05, seed=5)
    say(f"large hidden: T={w.T} H={w.H} K={w.K} E={w.E}")
    idx, wt = W.make_routing(w)
    x = W.make_x(w)
    R = O.layout(idx.numpy(), w.E)
    L = ep.ep_layout(idx.to(DEV), w.E)
    recv = ep.ep_dispatch(x.to(DEV), L)
    torch.cuda.synchronize()
    n = R["n_sel"]
    assert np.array_equal(u16(recv[:n]), O.dispatch_bf16(u16(x), R["slot"], n))
    say("dispatch ok")
    y = W.make_y(w, rows=n)
    out = ep.ep_combine(y.to(DEV), L, wt.to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(u16(out), O.combine(u16(y), R["slot"], wt.numpy()))
    d_idx = idx.to(DEV)
    Lg = ep.ep_layout(d_idx, w.E, w.G, wt.to(DEV))  # the grouped order needs the groups
    outg = ep.ep_combine(y.to(DEV), Lg, wt.to(DEV), topk_idx=d_idx, order=ep.EP_COMBINE_GROUPED)
    torch.cuda.synchronize()
    assert np.array_equal(u16(outg), O.combine_grouped(u16(y), idx.numpy(), R["slot"], wt.numpy(), w.E, w.G))
    say("combine (flat and grouped) ok")
