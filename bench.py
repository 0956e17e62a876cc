"""Benchmark of the MoE dispatch / combine hot path on one MI355X.

One step = layout (count, scan, place) + fp8 packed dispatch + bf16 combine
over the 8192-token, hidden-7168, top-8-of-256-experts workload, with every
input already resident in HBM.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Per-op times come from HIP events recorded on the stream the kernels run on
(torch's current stream, which the binding passes to every entry point).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E
METRIC = "dispatch / combine µs and achieved HBM GB/s (% of peak), 8192×7168 top-8 E=256"


def algorithmic_bytes(T, H, K, E, n_sel, fp8_row_bytes):
    """Bytes each op must move at minimum (reads + writes), per launch."""
    layout = T * K * 8 + T * K * 4 + (2 * E + 1) * 4  # idx in, slot out, counts/offsets
    disp_fp8 = T * H * 2 + T * K * 4 + n_sel * fp8_row_bytes  # x in, slot in, rows out
    disp_bf16 = T * H * 2 + T * K * 4 + n_sel * H * 2
    combine = n_sel * H * 2 + T * K * (4 + 4) + T * H * 2  # y rows in, slot+w in, out
    return {"layout": layout, "dispatch_fp8": disp_fp8, "dispatch_bf16": disp_bf16, "combine": combine}


def _code_only(text):
    """C/C++/HIP source with its comments and all whitespace removed (string
    and character literals kept as written), so that a comment edit does not
    count as a change of the code."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            if not c.isspace():
                out.append(c)
            i += 1
    return "".join(out)


def source_hash(files):
    """First 16 hex digits of the sha256 of the listed sources' code (comments
    and whitespace excluded, see _code_only), in the order given."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode("utf-8"))
    return h.hexdigest()[:16]


def counted_traffic(op, workload):
    """HBM bytes per launch of `op` from the committed FETCH_SIZE/WRITE_SIZE
    passes (profiles/traffic_<op>_<workload>.json), or None when there is no
    such record or the kernel code changed since the counters were taken (the
    record keeps source_hash() of the sources it was measured on)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{op}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if source_hash(rec.get("sources", [])) != rec.get("source_sha256_16"):
        return None
    return rec.get("bytes_per_launch")


def time_extras(ep, W, w, d_idx, d_wt, x, y, L, n_sel, rb, pitch, reps, only=None, flush=None):
    """Each op beside the headline step, timed alone (back to back, HIP
    events on the current stream) at the same 8192 x 7168 workload: the
    plain bf16 dispatch, grouped-order combine over 8 groups of 32 experts,
    the grouped (deduped)
    fp8 dispatch, dispatch into 128-row-aligned expert segments with zeroed
    padding, combine seeded by two bias rows, and the layout with
    receive-stats accumulation, the grouped GEMM consumer (plain weights,
    packed weights, and fused with the dispatch), the skewed and
    masked routing, and one GPU's grouped receive share at 65,536 tokens;
    also the fp8 dispatch at the packed 7392-byte pitch and the tiny and mid
    configurations, warm and with cold caches (``flush`` runs before each
    cold call).  ``only``, if given, names the cases to run."""
    import torch

    dev = x.device
    if flush is None:
        flush = CacheFlush(dev)
    T, H, K, E = w.T, w.H, w.K, w.E
    stream = torch.cuda.current_stream(dev)
    G = 8
    LG = ep.ep_layout(d_idx, E, G, d_wt)
    R = LG.num_rows(ep.EP_ROWS_GROUP)
    LA = ep.ep_layout(d_idx, E, expert_alignment=128)
    n_al = LA.num_rows()
    out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    recv_g = torch.empty(max(R, 1), pitch, dtype=torch.uint8, device=dev)
    recv_a = torch.empty(LA.max_expert_rows(), pitch, dtype=torch.uint8, device=dev)
    recv_b = torch.empty(max(n_sel, 1), H, dtype=torch.bfloat16, device=dev)
    g = torch.Generator(device=dev)
    g.manual_seed(77)
    b0 = torch.randn(T, H, generator=g, device=dev).to(torch.bfloat16)
    b1 = torch.randn(T, H, generator=g, device=dev).to(torch.bfloat16)
    stats = torch.zeros(E, dtype=torch.int32, device=dev)
    comb_b = n_sel * H * 2 + T * K * 8 + T * H * 2
    cases = {
        # the plain bf16 row scatter (no quantisation) of the same step
        "dispatch_bf16": (
            lambda: ep.ep_dispatch(x, L, out=recv_b, capacity=n_sel),
            T * H * 2 + T * K * 4 + n_sel * H * 2,
        ),
        "combine_grouped_g8": (
            lambda: ep.ep_combine(y, LG, d_wt, d_idx, order=ep.EP_COMBINE_GROUPED, out=out),
            comb_b + T * K * 8,
        ),
        "dispatch_fp8_grouped_rows_g8": (
            lambda: ep.ep_dispatch(x, LG, fp8=True, rows=ep.EP_ROWS_GROUP, out=recv_g, capacity=R),
            T * H * 2 + T * K * 4 + R * rb,
        ),
        "dispatch_fp8_align128_zero_padding": (
            lambda: ep.ep_dispatch(x, LA, fp8=True, out=recv_a, zero_padding=True),
            T * H * 2 + T * K * 4 + n_al * rb,
        ),
        "combine_bias2": (
            lambda: ep.ep_combine(y, L, d_wt, out=out, bias0=b0, bias1=b1),
            comb_b + 2 * T * H * 2,
        ),
        "layout_recv_stats": (
            lambda: ep.ep_layout(d_idx, E, out=L, recv_stats=stats),
            T * K * 12 + (2 * E + 1) * 4 + 2 * E * 4,
        ),
    }
    res = {}
    for name, (fn, nbytes) in cases.items():
        if only is not None and name not in only:
            continue
        fn()
        a0 = torch.cuda.Event(enable_timing=True)
        a1 = torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        for _ in range(reps):
            fn()
        a1.record(stream)
        torch.cuda.synchronize()
        us = a0.elapsed_time(a1) * 1e3 / reps
        res[name] = {
            "us": round(us, 2),
            "bytes": int(nbytes),
            "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "pct_of_peak": round(100.0 * nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 1),
        }
    def want(name):
        return only is None or name in only

    # grouped GEMM consumer: receive rows @ per-expert weights, H -> 2048
    N = 2048
    gemm_reps = max(3, reps // 5)
    flops = 2.0 * n_sel * H * N

    def timed(fn, n):
        fn()
        b0 = torch.cuda.Event(enable_timing=True)
        b1 = torch.cuda.Event(enable_timing=True)
        b0.record(stream)
        for _ in range(n):
            fn()
        b1.record(stream)
        torch.cuda.synchronize()
        return b0.elapsed_time(b1) * 1e3 / n

    gemm_cases = ("expert_gemm_bf16_n2048", "expert_gemm_fused_dispatch_n2048", "expert_gemm_packed_weights_n2048")
    if any(want(c) for c in gemm_cases):
        wts = W.make_expert_weights(w, N, device=dev)
        yg = torch.empty(L.max_expert_rows(), N, dtype=torch.bfloat16, device=dev)
        if want("expert_gemm_bf16_n2048"):
            xr = W.make_rows(w, L.max_expert_rows(), device=dev)
            us = timed(lambda: ep.ep_expert_gemm(xr, L, wts, out=yg), gemm_reps)
            nbytes = E * N * H * 2 + n_sel * H * 2 + n_sel * N * 2
            res["expert_gemm_bf16_n2048"] = {
                "us": round(us, 1),
                "TFLOPs": round(flops / (us * 1e-6) / 1e12, 1),
                "pct_of_mfma_peak": round(100.0 * flops / (us * 1e-6) / 2.5e15, 1),
                "bytes": int(nbytes),
                "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                "pct_of_hbm_peak": round(100.0 * nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 1),
                "bound_us": {"mfma": round(flops / 2.5e15 * 1e6, 1), "hbm": round(nbytes / 8e12 * 1e6, 1)},
                "traffic": counted_traffic("expert_gemm_n2048", w.name),
            }
            del xr
        if want("expert_gemm_packed_weights_n2048"):
            # weights packed once into the kernel's tile order (outside the
            # timed region, as static weights are), then the same GEMM
            xr = W.make_rows(w, L.max_expert_rows(), device=dev)
            packed = ep.ep_pack_expert_weights(wts)
            us_p = timed(lambda: ep.ep_expert_gemm(xr, L, packed, out=yg), gemm_reps)
            us_plain = timed(lambda: ep.ep_expert_gemm(xr, L, wts, out=yg), gemm_reps)
            nbytes = E * N * H * 2 + n_sel * H * 2 + n_sel * N * 2
            res["expert_gemm_packed_weights_n2048"] = {
                "us": round(us_p, 1),
                "us_plain_weights": round(us_plain, 1),
                "TFLOPs": round(flops / (us_p * 1e-6) / 1e12, 1),
                "pct_of_mfma_peak": round(100.0 * flops / (us_p * 1e-6) / 2.5e15, 1),
                "GBps": round(nbytes / (us_p * 1e-6) / 1e9, 1),
                "pct_of_hbm_peak": round(100.0 * nbytes / (us_p * 1e-6) / 1e9 / HBM_PEAK_GBS, 1),
            }
            del xr, packed
        if want("expert_gemm_fused_dispatch_n2048"):
            # the same GEMM with the dispatch folded into its loads (rows
            # gathered from the token matrix through expert_row_src), against
            # bf16 dispatch followed by the GEMM on the receive rows
            Lf = ep.ep_layout(d_idx, E, expert_row_src=True)
            recv16 = torch.empty(Lf.max_expert_rows(), H, dtype=torch.bfloat16, device=dev)

            def unfused():
                ep.ep_dispatch(x, Lf, out=recv16)
                ep.ep_expert_gemm(recv16, Lf, wts, out=yg)

            us_f = timed(lambda: ep.ep_expert_gemm(x, Lf, wts, out=yg, gather=True), gemm_reps)
            us_u = timed(unfused, gemm_reps)
            packed = ep.ep_pack_expert_weights(wts)
            us_fp = timed(lambda: ep.ep_expert_gemm(x, Lf, packed, out=yg, gather=True), gemm_reps)
            del packed
            fbytes = E * N * H * 2 + T * H * 2 + n_sel * N * 2
            res["expert_gemm_fused_dispatch_n2048"] = {
                "us": round(us_f, 1),
                "us_dispatch_then_gemm": round(us_u, 1),
                "us_packed_weights": round(us_fp, 1),
                "TFLOPs": round(flops / (us_f * 1e-6) / 1e12, 1),
                "bytes": int(fbytes),
                "GBps": round(fbytes / (us_f * 1e-6) / 1e9, 1),
                "pct_of_hbm_peak": round(100.0 * fbytes / (us_f * 1e-6) / 1e9 / HBM_PEAK_GBS, 1),
            }
            del recv16, Lf
        del wts, yg
    if want("dispatch_fp8_packed_pitch"):
        # the packed fp8 rows back to back (7392-byte pitch at hidden 7168),
        # the PR's own row, against the 128-byte aligned pitch of the step
        recv_p = torch.empty(T * K, rb, dtype=torch.uint8, device=dev)
        fn = lambda: ep.ep_dispatch(x, L, fp8=True, out=recv_p)  # noqa: E731
        nbytes = T * H * 2 + T * K * 4 + n_sel * rb
        res["dispatch_fp8_packed_pitch"] = {
            "row_bytes": int(rb),
            "warm": us_stats(per_call_us(fn, reps, stream), nbytes),
            "cold": us_stats(per_call_us(fn, reps, stream, before=flush), nbytes),
        }
        del recv_p
    if want("tiny"):
        res["tiny"] = time_tiny(ep, W, dev, stream, reps)
    if want("mid"):
        res["mid"] = time_mid(ep, W, dev, stream, reps, flush)
    if want("grouped_t65536_g8"):
        res["grouped_t65536_g8"] = time_grouped_receive_share(ep, W, dev, stream, gemm_reps)
    if want("skewed_masked"):
        res["skewed_masked"] = time_skewed_masked(ep, W, x, y, dev, stream, reps)
    res["_note"] = (
        f"grouped rows R={R} ({R / T:.3f} per token); aligned expert rows {n_al} "
        f"(of which {n_al - n_sel} padding, counted as written bytes)"
    )
    ep.ep_layout(d_idx, E, out=L)  # restore the headline layout
    return res


class CacheFlush:
    """Reads a 1 GiB buffer, which evicts whatever the next op reads from L2
    and from the 256 MB memory-side cache without leaving dirty lines to be
    written back during that op (a write flush was measured to time its own
    write-back instead)."""

    def __init__(self, dev):
        import torch

        self.buf = torch.ones(1 << 28, dtype=torch.int32, device=dev)
        self.sink = torch.zeros((), dtype=torch.int64, device=dev)

    def __call__(self):
        self.sink += self.buf.sum()


def per_call_us(fn, reps, stream, before=None):
    """Each of `reps` calls of `fn` bracketed by its own HIP events on
    `stream` (the stream the kernels run on); `before`, if given, runs
    untimed ahead of every call.  Returns the sorted durations in us."""
    import torch

    fn()
    torch.cuda.synchronize()
    marks = []
    for _ in range(reps):
        if before is not None:
            before()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        marks.append((a, b))
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) * 1e3 for a, b in marks)


def us_stats(v, nbytes=None):
    med = statistics.median(v)
    out = {"us_median": round(med, 2), "us_min": round(min(v), 2), "us_max": round(max(v), 2)}
    if nbytes is not None:
        out.update({
            "bytes": int(nbytes),
            "GBps": round(nbytes / (med * 1e-6) / 1e9, 1),
            "pct_of_peak": round(100.0 * nbytes / (med * 1e-6) / 1e9 / HBM_PEAK_GBS, 1),
        })
    return out


def time_tiny(ep, W, dev, stream, reps):
    """The tiny configuration (128 tokens x 256, top-2 of 16 experts, expert
    outputs = dispatched rows x (1 + e/16)): layout, bf16 dispatch and
    combine, each call timed on its own.  Latency-bound (0.2 MB per op), so
    only microseconds are reported."""
    import torch

    w = W.by_name("tiny")
    idx, wt = W.make_routing(w)
    d_idx, d_wt = idx.to(dev), wt.to(dev)
    x = W.make_x(w, device=dev)
    L = ep.ep_layout(d_idx, w.E)
    n_sel = L.num_rows()
    recv = ep.ep_dispatch(x, L)
    row_expert = torch.repeat_interleave(torch.arange(w.E, device=dev), L.counts.long())
    y = W.tiny_expert_outputs(recv[:n_sel], row_expert)
    out = torch.empty(w.T, w.H, dtype=torch.bfloat16, device=dev)
    res = {"selections": int(n_sel),
           "_note": "per call: one host launch per timed call, so mostly the host's launch path; "
                    "graph_us: 32 calls captured in one HIP graph and replayed, the GPU time per call"}
    for name, fn in (
        ("layout", lambda: ep.ep_layout(d_idx, w.E, out=L)),
        ("dispatch_bf16", lambda: ep.ep_dispatch(x, L, out=recv)),
        ("combine", lambda: ep.ep_combine(y, L, d_wt, out=out)),
    ):
        res[name] = us_stats(per_call_us(fn, reps, stream))
        res[name]["graph_us"] = round(graph_per_call_us(fn, 32, max(5, reps // 20), dev), 2)
    return res


def graph_per_call_us(fn, calls, replays, dev):
    """GPU time per call of `fn`: `calls` calls captured back to back in one
    HIP graph, the graph replayed `replays` times between two events, so no
    host work sits between the kernels."""
    import torch

    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        fn()  # warm the allocator and the library on the capture stream
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(replays):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / (replays * calls)
    del g
    return us


def time_mid(ep, W, dev, stream, reps, flush):
    """The mid configuration (4096 tokens x 4096, top-4 of 64 experts,
    uniform): bf16 dispatch and combine, each call timed on its own, warm and
    with cold caches.  Both ops' working sets (about 168 MB) fit the 256 MB
    memory-side cache, so only the cold figure measures HBM."""
    import torch

    w = W.by_name("mid")
    T, H, K, E = w.T, w.H, w.K, w.E
    idx, wt = W.make_routing(w)
    d_idx, d_wt = idx.to(dev), wt.to(dev)
    x = W.make_x(w, device=dev)
    y = W.make_y(w, device=dev)
    L = ep.ep_layout(d_idx, E)
    n_sel = L.num_rows()
    recv = torch.empty(n_sel, H, dtype=torch.bfloat16, device=dev)
    out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    nb = algorithmic_bytes(T, H, K, E, n_sel, 0)
    res = {"selections": int(n_sel)}
    for name, fn, nbytes in (
        ("dispatch_bf16", lambda: ep.ep_dispatch(x, L, out=recv, capacity=n_sel), nb["dispatch_bf16"]),
        ("combine", lambda: ep.ep_combine(y, L, d_wt, out=out), nb["combine"]),
    ):
        res[name] = {
            "warm": us_stats(per_call_us(fn, reps, stream), nbytes),
            "cold": us_stats(per_call_us(fn, reps, stream, before=flush), nbytes),
        }
    del x, y, recv, out
    return res


def time_skewed_masked(ep, W, x, y, dev, stream, reps):
    """The skewed, masked routing at the bench shape (8192 x 7168, top-8 of
    256): expert popularity Zipf(1.2) over a seeded permutation, each
    selection masked with probability 0.1 and 1% of the tokens fully masked.
    Times its layout, bf16 dispatch and combine on the bench's x and y rows;
    a fully masked token's row is not read, so dispatch counts the active
    tokens' rows."""
    import torch

    w = W.by_name("skewed_masked")
    T, H, K, E = w.T, w.H, w.K, w.E
    si, sw = W.make_routing(w)
    active = int((si >= 0).any(dim=1).sum())
    si, sw = si.to(dev), sw.to(dev)
    Ls = ep.ep_layout(si, E)
    n_sel = Ls.num_rows()
    counts = Ls.counts.cpu()
    recv = torch.empty(n_sel, H, dtype=torch.bfloat16, device=dev)
    out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    nb = algorithmic_bytes(T, H, K, E, n_sel, 0)
    cases = {
        "layout": (lambda: ep.ep_layout(si, E, out=Ls), nb["layout"]),
        "dispatch_bf16": (
            lambda: ep.ep_dispatch(x, Ls, out=recv, capacity=n_sel),
            active * H * 2 + T * K * 4 + n_sel * H * 2,
        ),
        "combine": (lambda: ep.ep_combine(y, Ls, sw, out=out), nb["combine"]),
    }
    res = {
        "selections": int(n_sel),
        "active_tokens": active,
        "rows_per_expert": {"max": int(counts.max()), "median": int(counts.median()), "min": int(counts.min())},
    }
    for name, (fn, nbytes) in cases.items():
        fn()
        a0 = torch.cuda.Event(enable_timing=True)
        a1 = torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        for _ in range(reps):
            fn()
        a1.record(stream)
        torch.cuda.synchronize()
        us = a0.elapsed_time(a1) * 1e3 / reps
        res[name] = {
            "us": round(us, 2),
            "bytes": int(nbytes),
            "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "pct_of_peak": round(100.0 * nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 1),
        }
    del recv, out, Ls
    return res


def time_grouped_receive_share(ep, W, dev, stream, reps):
    """One GPU's receive share with grouped dedup at its real size: 65536
    source tokens x 7168, top-8 of 256 experts in 8 groups of 32.  Times the
    grouped layout, the bf16 dispatch of one row per (token, group hit) and
    the grouped-order combine over one expert-output row per selection."""
    import torch

    w = W.by_name("grouped")
    T, H, K, E, G = w.T, w.H, w.K, w.E, w.G
    gi, gw = W.make_routing(w, device=dev)
    gx = W.make_x(w, device=dev)
    gy = W.make_y(w, device=dev)
    LG = ep.ep_layout(gi, E, G, gw)
    R = LG.num_rows(ep.EP_ROWS_GROUP)
    n_sel = LG.num_rows()
    recv = torch.empty(R, H, dtype=torch.bfloat16, device=dev)
    out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    cases = {
        # ids and weights read; slot and group row written per selection;
        # source token and K-wide id / weight lists written per row
        "layout": (lambda: ep.ep_layout(gi, E, G, gw, out=LG), T * K * (8 + 4 + 4 + 4) + R * (4 + K * 8)),
        "dispatch_bf16_group_rows": (
            lambda: ep.ep_dispatch(gx, LG, rows=ep.EP_ROWS_GROUP, out=recv, capacity=R),
            T * H * 2 + T * K * 4 + R * H * 2,
        ),
        "combine_grouped": (
            lambda: ep.ep_combine(gy, LG, gw, gi, order=ep.EP_COMBINE_GROUPED, out=out),
            n_sel * H * 2 + T * K * (4 + 4 + 8) + T * H * 2,
        ),
    }
    res = {"rows_R": int(R), "selections": int(n_sel)}
    for name, (fn, nbytes) in cases.items():
        fn()
        a0 = torch.cuda.Event(enable_timing=True)
        a1 = torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        for _ in range(reps):
            fn()
        a1.record(stream)
        torch.cuda.synchronize()
        us = a0.elapsed_time(a1) * 1e3 / reps
        res[name] = {
            "us": round(us, 1),
            "bytes": int(nbytes),
            "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
            "pct_of_peak": round(100.0 * nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 1),
        }
    del gx, gy, recv, out, LG
    torch.cuda.empty_cache()
    return res


def cpu_baseline(w, idx, wt, x_host, y_host, sample_tokens, passes=3):
    """The CPU oracle, as it stands, timed on a bounded sample of the workload:
    the full layout, then fp8 dispatch and combine of the first
    ``sample_tokens`` tokens, ``passes`` times; each phase reports its median
    pass.  Reported in the metric's unit (GB/s of the same algorithmic
    bytes)."""
    import numpy as np

    from oracle import ep_oracle as O

    threads = 1  # numpy's elementwise, indexing and searchsorted kernels run on one thread
    S = sample_tokens
    rb = O.fp8_row_bytes(w.H)
    t_lay, t_disp, t_comb = [], [], []
    for _ in range(passes):
        t0 = time.perf_counter()
        R = O.layout(idx, w.E)
        t1 = time.perf_counter()
        slot_s = R["slot"][:S]
        used = np.unique(slot_s[slot_s >= 0])
        remap = -np.ones(R["n_sel"] + 1, np.int64)
        remap[used] = np.arange(len(used))
        slot_r = np.where(slot_s >= 0, remap[np.maximum(slot_s, 0)], -1)
        t2 = time.perf_counter()
        O.dispatch_fp8(x_host[:S], slot_r, len(used))
        t3 = time.perf_counter()
        ysub = y_host[used]
        t4 = time.perf_counter()
        O.combine(ysub, slot_r, wt[:S])
        t5 = time.perf_counter()
        t_lay.append(t1 - t0)
        t_disp.append(t3 - t2)
        t_comb.append(t5 - t4)
    b_layout = w.T * w.K * 12
    b_disp = S * w.H * 2 + S * w.K * 4 + len(used) * rb
    b_comb = len(used) * w.H * 2 + S * w.K * 8 + S * w.H * 2
    med = statistics.median
    secs = med(t_lay) + med(t_disp) + med(t_comb)
    total = sum(t_lay) + sum(t_disp) + sum(t_comb)
    return {
        "value": round((b_layout + b_disp + b_comb) / secs / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"full layout of {w.T}x{w.K} ids; fp8 dispatch + combine of the first {S} tokens "
        f"({len(used)} rows); median of {passes} passes, {secs:.1f} s per pass, {total:.1f} s of CPU "
        "time in all; numpy single-threaded elementwise",
        "seconds": {"layout": round(med(t_lay), 3), "dispatch_fp8": round(med(t_disp), 3),
                    "combine": round(med(t_comb), 3)},
        "cpu_model": host_cpu_model(),
        "host_cpu_count": os.cpu_count(),
        "affinity_cpus": len(os.sched_getaffinity(0)),
    }


def host_cpu_model():
    """The host CPU's model name from /proc/cpuinfo, else what platform gives."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def smi_snapshot():
    """GPU busy percentage of every amdgpu device and the processes holding a
    GPU context, read from sysfs (the driver's gpu_busy_percent and the KFD
    process list): the idle check, without starting any other program."""
    import glob

    out = {"busy_percent": {}, "kfd_processes": None}
    for f in sorted(glob.glob("/sys/class/drm/card[0-9]*/device/gpu_busy_percent")):
        try:
            with open(f) as fh:
                out["busy_percent"][f.split("/")[4]] = int(fh.read().strip())
        except (OSError, ValueError):
            pass
    try:
        pids = sorted(int(p) for p in os.listdir("/sys/class/kfd/kfd/proc") if p.isdigit())
        out["kfd_processes"] = {"count": len(pids), "self_listed": os.getpid() in pids}
    except OSError:
        pass
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="pages")
    ap.add_argument("--seed", type=int, default=None, help="override the workload's seed")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=8192)
    ap.add_argument("--bf16-dispatch", action="store_true", help="also time the bf16 dispatch variant")
    ap.add_argument(
        "--no-extras",
        action="store_true",
        help="skip the extra per-op timings (grouped combine, aligned dispatch, bias, stats)",
    )
    ap.add_argument(
        "--isolated",
        action="store_true",
        help="also time each op alone, back to back, outside the step (diagnostic)",
    )
    ap.add_argument(
        "--extras",
        default=None,
        metavar="NAMES",
        help="comma-separated names of the extra timings to run (default: all)",
    )
    ap.add_argument(
        "--no-graph",
        action="store_true",
        help="skip timing the step as a captured HIP graph",
    )
    ap.add_argument(
        "--no-cold",
        action="store_true",
        help="skip the cold-cache pass (a 1 GiB buffer is read before each step, so the "
        "256 MB memory-side cache cannot serve the step's inputs)",
    )
    ap.add_argument(
        "--calibrate-copy",
        type=int,
        default=0,
        metavar="MIB",
        help="after the run, copy a MIB-mebibyte buffer 5 times with torch (a plain copy "
        "kernel of known size, the reference for HBM byte counters)",
    )
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(
            f"bench.py measures one GPU's share of dispatch/combine; --gpus {args.gpus} is not "
            "supported (the library has no collectives)",
            file=sys.stderr,
        )
        return 2

    import numpy as np
    import torch

    import combine_ep_layout_03_amd as ep
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    w = W.by_name(args.workload)
    if args.seed is not None:
        w = w.replace(seed=args.seed)
    T, H, K, E = w.T, w.H, w.K, w.E
    print(f"# workload {w.name}: T={T} H={H} K={K} E={E}; generating inputs", file=sys.stderr, flush=True)
    idx, wt = W.make_routing(w)
    d_idx, d_wt = idx.to(dev), wt.to(dev)
    x = W.make_x(w, device=dev)
    y = W.make_y(w, device=dev)  # T*K expert-output rows
    rb = ep.ep_fp8_row_bytes(H)
    pitch = ep.fp8_row_pitch(H)  # 128-byte aligned receive-row pitch (7424 at H=7168)

    inputs_sha256 = {
        name: hashlib.sha256(t.contiguous().cpu().view(torch.uint8).numpy().tobytes()).hexdigest()[:16]
        for name, t in (("topk_idx", idx), ("topk_weights", wt), ("x", x), ("y", y))
    }
    L = ep.ep_layout(d_idx, E)
    n_sel = L.num_rows()
    recv8 = torch.empty(T * K, pitch, dtype=torch.uint8, device=dev)
    recv8_packed = torch.empty(T * K, rb, dtype=torch.uint8, device=dev) if args.isolated else None
    out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    recv16 = torch.empty(T * K, H, dtype=torch.bfloat16, device=dev) if args.bf16_dispatch else None
    nb = algorithmic_bytes(T, H, K, E, n_sel, rb)

    stream = torch.cuda.current_stream(dev)
    ev = {k: [] for k in ("start", "layout", "dispatch", "combine", "bf16")}
    gpu_state = {"before": smi_snapshot()}

    def step(record, ev=ev):
        if record:
            e0 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        ep.ep_layout(d_idx, E, out=L)
        if record:
            e1 = torch.cuda.Event(enable_timing=True)
            e1.record(stream)
        ep.ep_dispatch(x, L, fp8=True, out=recv8)
        if record:
            e2 = torch.cuda.Event(enable_timing=True)
            e2.record(stream)
        ep.ep_combine(y, L, d_wt, out=out)
        if record:
            e3 = torch.cuda.Event(enable_timing=True)
            e3.record(stream)
            ev["start"].append(e0)
            ev["layout"].append(e1)
            ev["dispatch"].append(e2)
            ev["combine"].append(e3)
        if recv16 is not None:
            ep.ep_dispatch(x, L, fp8=False, out=recv16)
            if record:
                e4 = torch.cuda.Event(enable_timing=True)
                e4.record(stream)
                ev["bf16"].append(e4)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    print(f"# warmup done; timing {args.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_state["after"] = smi_snapshot()

    # the same step (layout, fp8 dispatch, combine) captured once in a HIP
    # graph and replayed: every launch is recorded, only the host's per-launch
    # work goes away
    t_graph = []
    if not args.no_graph:
        def core_step():
            ep.ep_layout(d_idx, E, out=L)
            ep.ep_dispatch(x, L, fp8=True, out=recv8)
            ep.ep_combine(y, L, d_wt, out=out)

        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            core_step()
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            core_step()
        torch.cuda.synchronize()
        for _ in range(3):
            graph.replay()
        marks = []
        for _ in range(args.steps):
            g0 = torch.cuda.Event(enable_timing=True)
            g1 = torch.cuda.Event(enable_timing=True)
            g0.record(stream)
            graph.replay()
            g1.record(stream)
            marks.append((g0, g1))
        torch.cuda.synchronize()
        t_graph = [a.elapsed_time(b) for a, b in marks]
        del graph

    ev_cold = {k: [] for k in ev}
    flush = CacheFlush(dev)
    if not args.no_cold:
        # cold caches: read 1 GiB before every step (outside the timed
        # events), which evicts the step's inputs from L2 and the 256 MB
        # memory-side cache without leaving dirty lines to write back during
        # the step
        for _ in range(args.steps):
            flush()
            step(True, ev_cold)
        torch.cuda.synchronize()
        print("# cold-cache pass done", file=sys.stderr, flush=True)

    def ms(a, b, evd=ev):
        return [x.elapsed_time(y) for x, y in zip(evd[a], evd[b])]

    t_layout = ms("start", "layout")
    t_disp = ms("layout", "dispatch")
    t_comb = ms("dispatch", "combine")
    t_step = [a + b + c for a, b, c in zip(t_layout, t_disp, t_comb)]
    t_bf16 = ms("combine", "bf16") if recv16 is not None else []

    def stats(v, nbytes):
        med = statistics.median(v)
        return {
            "us_median": round(med * 1e3, 2),
            "us_min": round(min(v) * 1e3, 2),
            "us_max": round(max(v) * 1e3, 2),
            "bytes": nbytes,
            "GBps": round(nbytes / (med * 1e-3) / 1e9, 1),
            "pct_of_peak": round(100.0 * nbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 1),
        }

    ops = {
        "layout": stats(t_layout, nb["layout"]),
        "dispatch_fp8": stats(t_disp, nb["dispatch_fp8"]),
        "combine": stats(t_comb, nb["combine"]),
        # dispatch as the pages time a collective: layout and scatter together
        "dispatch_e2e": stats([a + b for a, b in zip(t_layout, t_disp)], nb["layout"] + nb["dispatch_fp8"]),
    }
    if t_bf16:
        ops["dispatch_bf16"] = stats(t_bf16, nb["dispatch_bf16"])
    if t_graph:
        ops["step_graph"] = stats(t_graph, nb["layout"] + nb["dispatch_fp8"] + nb["combine"])
    ops_cold = None
    if ev_cold["start"]:
        c_layout = ms("start", "layout", ev_cold)
        c_disp = ms("layout", "dispatch", ev_cold)
        c_comb = ms("dispatch", "combine", ev_cold)
        ops_cold = {
            "layout": stats(c_layout, nb["layout"]),
            "dispatch_fp8": stats(c_disp, nb["dispatch_fp8"]),
            "combine": stats(c_comb, nb["combine"]),
            "dispatch_e2e": stats([a + b for a, b in zip(c_layout, c_disp)], nb["layout"] + nb["dispatch_fp8"]),
            "step": stats([a + b + c for a, b, c in zip(c_layout, c_disp, c_comb)],
                          nb["layout"] + nb["dispatch_fp8"] + nb["combine"]),
        }
        if recv16 is not None:
            ops_cold["dispatch_bf16"] = stats(ms("combine", "bf16", ev_cold), nb["dispatch_bf16"])
    if args.isolated:
        iso = {
            "layout": lambda: ep.ep_layout(d_idx, E, out=L),
            "dispatch_fp8": lambda: ep.ep_dispatch(x, L, fp8=True, out=recv8),
            "dispatch_fp8_packed_pitch": lambda: ep.ep_dispatch(x, L, fp8=True, out=recv8_packed),
            "combine": lambda: ep.ep_combine(y, L, d_wt, out=out),
        }
        if recv16 is not None:
            iso["dispatch_bf16"] = lambda: ep.ep_dispatch(x, L, fp8=False, out=recv16)
        for name, fn in iso.items():
            if name not in ops:
                ops[name] = {"bytes": nb["dispatch_fp8"]}
            fn()
            a0 = torch.cuda.Event(enable_timing=True)
            a1 = torch.cuda.Event(enable_timing=True)
            a0.record(stream)
            for _ in range(args.steps):
                fn()
            a1.record(stream)
            torch.cuda.synchronize()
            us = a0.elapsed_time(a1) * 1e3 / args.steps
            ops[name]["isolated_us"] = round(us, 2)
            ops[name]["isolated_GBps"] = round(ops[name]["bytes"] / (us * 1e-6) / 1e9, 1)
    only = None if args.extras is None else set(s for s in args.extras.split(",") if s)
    extras = {} if args.no_extras else time_extras(ep, W, w, d_idx, d_wt, x, y, L, n_sel, rb, pitch, args.steps,
                                                   only, flush)
    del flush
    step_bytes = nb["layout"] + nb["dispatch_fp8"] + nb["combine"]
    step_ms = statistics.median(t_step)
    value = step_bytes / (step_ms * 1e-3) / 1e9

    # roofline of the dominant kernel (largest median time of the step's ops)
    dom = max(("dispatch_fp8", "combine"), key=lambda k: ops[k]["us_median"])
    avg_us = statistics.mean(t_disp if dom == "dispatch_fp8" else t_comb) * 1e3
    achieved = nb[dom] / (avg_us * 1e-6) / 1e9
    traffic = counted_traffic(dom, w.name)

    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3+bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: T={T} tokens, H={H}, top-{K} of E={E} experts, uniform routing; "
            f"fp8 packed dispatch ({rb}-byte rows at a {pitch}-byte receive pitch) + bf16 combine",
            "global_batch": T,
            "seq_len": 1,
            "parallelism": "single-GPU",
        },
        "inputs": {"seed": w.seed, "sha256_16": inputs_sha256},
        "ops": ops,
        "ops_cold_cache": ops_cold,
        "extras": extras,
        "gpu_state": gpu_state,
        "wall_ms_per_step": round(wall / args.steps * 1e3, 4),
        "roofline": {
            "bound": "hbm",
            "kernel": dom,
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "avg_launch_us": round(avg_us, 2),
        },
    }
    if ops_cold is not None:
        # The >= 60%-of-HBM target is judged on the cold-cache figures: with
        # warm caches the fp8 dispatch reads its 117 MB of token rows from the
        # memory-side cache (a rate that in a model's forward pass, where the
        # previous layer just wrote those rows, is the realistic one, but not
        # an HBM rate).  The combine reads 940 MB, far more than that cache,
        # so its warm and cold figures agree.
        res["hbm_target_60pct"] = {
            "basis": "cold caches: a 1 GiB read before each step evicts L2 and the 256 MB memory-side cache",
            "pct_of_peak": {k: ops_cold[k]["pct_of_peak"] for k in ("dispatch_fp8", "dispatch_e2e", "combine")},
            "warm_is_cache_assisted": {k: ops[k]["pct_of_peak"] for k in ("dispatch_fp8", "dispatch_e2e")},
            "met": all(ops_cold[k]["pct_of_peak"] >= 60.0 for k in ("dispatch_fp8", "dispatch_e2e", "combine")),
        }
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        x_host = x.cpu().view(torch.int16).numpy().view(np.uint16)
        S = args.cpu_sample_tokens
        y_host = y[: int(n_sel)].cpu().view(torch.int16).numpy().view(np.uint16)
        res["cpu_baseline"] = cpu_baseline(w, idx.numpy(), wt.numpy(), x_host, y_host, S)
    if args.calibrate_copy:
        nbytes = args.calibrate_copy << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        res["calibrate_copy_bytes"] = nbytes
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
