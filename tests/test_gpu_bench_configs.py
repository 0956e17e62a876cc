"""Parity at the bench's full size, in the launch configuration bench.py
times: 8192 tokens x 7168, top-8 of 256 experts.  The headline step's ops
are covered in test_gpu_parity.py; these are the extras timed beside it --
grouped combine over 8 groups, grouped fp8 dispatch, fp8 dispatch into
128-row-aligned segments with zeroed padding, and combine seeded by two bias
rows -- each run exactly as the bench runs it (same calls, same 7424-byte
receive pitch) and checked on sampled tokens or rows against the oracle."""
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


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def pages():
    w = W.by_name("pages")
    idx, wt = W.make_routing(w)
    return {
        "w": w,
        "idx": idx,
        "wt": wt,
        "d_idx": idx.to(DEV),
        "d_wt": wt.to(DEV),
        "x": W.make_x(w, device=DEV),
        "y": W.make_y(w, device=DEV),
        "pitch": ep().fp8_row_pitch(w.H),
        "gen": np.random.default_rng(1),
    }


def _sampled_tokens(gen, T, n=600):
    return np.concatenate([[0, T - 1], gen.choice(T, n, replace=False)])


def _sub_slots(slot_rows, n_sel):
    """The sampled tokens' slots renumbered over the rows they use."""
    used = np.unique(slot_rows[slot_rows >= 0])
    remap = -np.ones(n_sel + 1, np.int64)
    remap[used] = np.arange(len(used))
    return used, np.where(slot_rows >= 0, remap[np.maximum(slot_rows, 0)], -1)


def test_combine_grouped_g8_full_size(pages):
    P = pages
    w = P["w"]
    say("bench config: grouped combine, G = 8")
    L = ep().ep_layout(P["d_idx"], w.E, 8, P["d_wt"])
    out = torch.empty(w.T, w.H, dtype=torch.bfloat16, device=DEV)
    ep().ep_combine(P["y"], L, P["d_wt"], P["d_idx"], order=ep().EP_COMBINE_GROUPED, out=out)
    R = O.layout(P["idx"].numpy(), w.E, 8, P["wt"].numpy())
    toks = _sampled_tokens(P["gen"], w.T)
    used, slot_r = _sub_slots(R["slot"][toks], R["n_sel"])
    ysub = u16(P["y"].index_select(0, torch.from_numpy(used).to(DEV)))
    want = O.combine_grouped(ysub, P["idx"].numpy()[toks], slot_r, P["wt"].numpy()[toks], w.E, 8)
    got = u16(out.index_select(0, torch.from_numpy(toks).to(DEV)))
    assert np.array_equal(got, want)


def test_dispatch_fp8_grouped_rows_full_size(pages):
    P = pages
    w = P["w"]
    say("bench config: grouped fp8 dispatch, G = 8, 7424-byte pitch")
    LG = ep().ep_layout(P["d_idx"], w.E, 8, P["d_wt"])
    R = LG.num_rows(ep().EP_ROWS_GROUP)
    recv = torch.empty(max(R, 1), P["pitch"], dtype=torch.uint8, device=DEV)
    ep().ep_dispatch(P["x"], LG, fp8=True, rows=ep().EP_ROWS_GROUP, out=recv, capacity=R)
    RO = O.layout(P["idx"].numpy(), w.E, 8, P["wt"].numpy())
    assert R == RO["n_rows"]
    rb = O.fp8_row_bytes(w.H)
    rows = np.concatenate([[0, R - 1], P["gen"].choice(R, 400, replace=False)])
    got = recv.index_select(0, torch.from_numpy(rows).to(DEV))[:, :rb].cpu().numpy()
    src = u16(P["x"].index_select(0, torch.from_numpy(RO["src"][rows]).to(DEV)))
    want = np.stack([O.quantize_row_fp8(r) for r in src])
    assert np.array_equal(got, want)


def test_dispatch_fp8_align128_zero_padding_full_size(pages):
    P = pages
    w = P["w"]
    say("bench config: fp8 dispatch into 128-aligned segments, zeroed padding")
    LA = ep().ep_layout(P["d_idx"], w.E, expert_alignment=128)
    n_al = LA.num_rows()
    recv = torch.full((LA.max_expert_rows(), P["pitch"]), 0xA5, dtype=torch.uint8, device=DEV)
    ep().ep_dispatch(P["x"], LA, fp8=True, out=recv, zero_padding=True)
    RO = O.layout(P["idx"].numpy(), w.E, expert_alignment=128)
    src_of = RO["expert_row_src"]
    assert n_al == len(src_of)
    rb = O.fp8_row_bytes(w.H)
    pad_rows = np.flatnonzero(src_of < 0)
    sel_rows = np.flatnonzero(src_of >= 0)
    rows = np.concatenate([P["gen"].choice(sel_rows, 300, replace=False), P["gen"].choice(pad_rows, 100, replace=False)])
    got = recv.index_select(0, torch.from_numpy(rows).to(DEV))[:, :rb].cpu().numpy()
    toks = np.maximum(src_of[rows], 0)
    srcx = u16(P["x"].index_select(0, torch.from_numpy(toks).to(DEV)))
    want = np.stack([O.quantize_row_fp8(r) if s >= 0 else np.zeros(rb, np.uint8) for r, s in zip(srcx, src_of[rows])])
    assert np.array_equal(got, want)


def test_combine_bias2_full_size(pages):
    P = pages
    w = P["w"]
    say("bench config: combine seeded by two bias rows")
    L = ep().ep_layout(P["d_idx"], w.E)
    g = torch.Generator(device=DEV)
    g.manual_seed(77)
    b0 = torch.randn(w.T, w.H, generator=g, device=DEV).to(torch.bfloat16)
    b1 = torch.randn(w.T, w.H, generator=g, device=DEV).to(torch.bfloat16)
    out = torch.empty(w.T, w.H, dtype=torch.bfloat16, device=DEV)
    ep().ep_combine(P["y"], L, P["d_wt"], out=out, bias0=b0, bias1=b1)
    R = O.layout(P["idx"].numpy(), w.E)
    toks = _sampled_tokens(P["gen"], w.T)
    used, slot_r = _sub_slots(R["slot"][toks], R["n_sel"])
    ysub = u16(P["y"].index_select(0, torch.from_numpy(used).to(DEV)))
    tsel = torch.from_numpy(toks).to(DEV)
    want = O.combine(ysub, slot_r, P["wt"].numpy()[toks], bias0=u16(b0.index_select(0, tsel)), bias1=u16(b1.index_select(0, tsel)))
    got = u16(out.index_select(0, tsel))
    assert np.array_equal(got, want)
