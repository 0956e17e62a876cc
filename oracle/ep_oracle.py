"""CPU oracle for MoE token dispatch and combine.

TEST INFRASTRUCTURE ONLY.  This is a plain, slow, obviously correct numpy
implementation of what the dispatch/combine hot path computes.  Only the test
suite, the package's smoke entry and the benchmark's cpu_baseline leg may
import it; the product path (the C-ABI library and its Python binding) never
does, and this module imports nothing from the product.

Floating point: every fp32 operation below is a single numpy float32 array
operation (IEEE binary32, round to nearest even, no fused multiply-add),
which is the precision the method fixes for the fp8 scale and the combine
accumulator.  bf16 values travel as their uint16 bit patterns.

Sources (TileScale pull request #68, "[Example] EP v2 intranode
dispatch/combine", unless stated otherwise):
* three-phase layout (count per destination, base from the counts, locally
  claimed slot) and the expert-major layout whose segment base is an
  exclusive prefix sum of per-expert counts: the commit adding DeepEP's
  ``do_expand``, and the Design section of the PR description;
* ``-1`` as the no-selection marker, skipped, so a fully masked token combines
  to zero: the commit on masked ``topk_idx``;
* the packed fp8 row (payload, then the per-128-element fp32 scales, padded
  to 16 bytes) written in one store: the commit packing payload and scales;
* one scale per token and per run of 128 elements (the layout of DeepEP's
  per_token_cast_to_fp8): the PR description's opening paragraph;
* rows deduplicated per (token, destination), each carrying the token's
  local experts as a K-wide list: the Design section and the commit adding
  receive stats and combine bias;
* the rows of one token that share a destination added together first, then
  the destinations' partial sums: the commit adding the expanded combine
  (``kDoExpandedSend``).

Readings where the pages are silent (each repeated at its function):
* rows inside one destination segment are ordered by ascending (token, k);
* an id outside ``{-1} U [0, E)`` is counted as invalid and treated as -1;
* scale ``s = fl(amax / 448)`` and payload ``q = e4m3(fl(x / s))``: two IEEE
  fp32 divisions, then OCP E4M3FN round-to-nearest-even with saturation to
  448; ``s == 0`` gives an all-zero payload;
* combine multiplies and adds as two separately rounded fp32 operations in
  ascending k order starting from +0; grouped combine sums within a group in
  ascending k, then across groups in ascending group order, all in fp32.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_to_f32",
    "bf16_rne",
    "e4m3fn_value_table",
    "e4m3fn_rne_sat",
    "fp8_row_bytes",
    "layout",
    "dispatch_bf16",
    "quantize_row_fp8",
    "dispatch_fp8",
    "combine",
    "combine_grouped",
    "expert_gemm",
    "expert_gemm_bound",
]

FP8_GROUP = 128  # elements per fp32 scale
FP8_MAX = 448.0  # largest finite E4M3FN magnitude


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------
def bf16_to_f32(u16) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact: bf16 is the top half of fp32)."""
    u = np.asarray(u16, dtype=np.uint16)
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_rne(f32) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even.

    Keep the top 16 bits; the dropped 16 bits decide: above one half of the
    kept unit rounds up, exactly one half rounds up only when the kept
    pattern is odd.  Incrementing the kept pattern steps to the next bf16
    magnitude (carrying into the exponent, up to infinity).  Inputs must not
    be NaN.
    """
    f = np.asarray(f32, dtype=np.float32)
    if np.isnan(f).any():
        raise ValueError("bf16_rne: NaN input is outside the oracle's domain")
    b = f.view(np.uint32)
    hi = b >> np.uint32(16)
    lo = b & np.uint32(0xFFFF)
    up = (lo > 0x8000) | ((lo == 0x8000) & ((hi & np.uint32(1)) == 1))
    return (hi + up.astype(np.uint32)).astype(np.uint16)


def e4m3fn_value_table() -> np.ndarray:
    """Magnitudes of the 127 finite non-negative OCP E4M3FN codes 0x00..0x7E.

    Code bits are S.EEEE.MMM with exponent bias 7.  Exponent field 0 encodes
    subnormals m * 2^-9; fields 1..15 encode (1 + m/8) * 2^(e-7).  The
    pattern S.1111.111 is NaN and there is no infinity, so the largest
    finite magnitude is code 0x7E = 1.75 * 2^8 = 448.  The table is
    increasing in the code.
    """
    vals = []
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        if e == 0:
            vals.append(m * 2.0**-9)
        else:
            vals.append((1.0 + m / 8.0) * 2.0 ** (e - 7))
    return np.array(vals, dtype=np.float64)


_E4M3_TABLE = e4m3fn_value_table()


def e4m3fn_rne_sat(v) -> np.ndarray:
    """float32 -> E4M3FN codes (uint8), nearest with ties to the even code,
    magnitudes above 448 saturated to 448.

    The magnitude is clamped to 448 and compared against the midpoint of its
    two neighbouring table values (midpoints of dyadic values with a few
    bits are exact in float64, and so is every float32).  The sign bit is
    copied from the input, so negative values that round to zero encode as
    0x80.  NaN is outside the domain.
    """
    f = np.asarray(v, dtype=np.float32)
    if np.isnan(f).any():
        raise ValueError("e4m3fn_rne_sat: NaN input is outside the oracle's domain")
    sign = (f.view(np.uint32) >> np.uint32(31)).astype(np.uint8)
    m = np.minimum(np.abs(f.astype(np.float64)), FP8_MAX)
    t = _E4M3_TABLE
    hi = np.searchsorted(t, m, side="left")  # first table value >= m
    hi = np.minimum(hi, len(t) - 1)
    lo = np.maximum(hi - 1, 0)
    exact = t[hi] == m
    mid = (t[lo] + t[hi]) / 2.0
    pick_hi = exact | (m > mid) | ((m == mid) & ((hi & 1) == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return code | (sign << np.uint8(7))


def fp8_row_bytes(hidden: int) -> int:
    """Bytes of one packed fp8 row: H payload bytes, then H/128 fp32 scales,
    zero-padded up to a multiple of 16 bytes.  -1 if H is not a multiple of
    128 (the scale groups would not tile the row)."""
    if hidden <= 0 or hidden % FP8_GROUP:
        return -1
    raw = hidden + 4 * (hidden // FP8_GROUP)
    return (raw + 15) // 16 * 16


# --------------------------------------------------------------------------
# layout: count, exclusive scan, slot
# --------------------------------------------------------------------------
def layout(
    topk_idx, num_experts: int, num_groups: int = 0, topk_weights=None, expert_alignment: int = 0
) -> dict:
    """Placement of every selection, as the three dispatch phases define it.

    Expert-major layout (always computed):
      valid(t,k)  <=> 0 <= idx[t,k] < E; -1 is "no selection"; any other id is
                      counted in ``n_invalid`` and treated as -1;
      counts[e]   = #valid (t,k) with idx[t,k] = e;
      offsets     = exclusive prefix sum of the segment sizes, where a
                    segment is counts[e] rounded up to a multiple of the
                    expert alignment A (A <= 1: no rounding; the commit
                    adding do_expand rounds each segment up and marks the
                    gap unoccupied); offsets[E] = n_rows_expert;
      slot[t,k]   = offsets[e] + #valid (t',k') before (t,k) in (t,k) order
                    with the same expert, or -1;
      expert_row_src[r] = the token of expert row r, or -1 for a padding row.
    The pages leave the order of rows inside a segment to whichever lane
    claims a slot first; this oracle fixes ascending (t,k).

    Grouped layout (``num_groups = G >= 1``): the E experts form G contiguous
    groups of E/G; a token sends one row per group it hits:
      hit(t,g)    <=> some valid k of t has idx[t,k] // (E/G) = g;
      gcounts[g]  = #tokens hitting g; goffsets = its exclusive prefix sum;
      row of (t,g) = goffsets[g] + #tokens t' < t hitting g;
      grow[t,k]   = row of (t, group of idx[t,k]) for valid (t,k), else -1;
      src[r]      = token of row r;
      ridx[r,k]   = idx[t,k] - g*(E/G) if (t,k) is valid and in g, else -1;
      rw[r,k]     = topk_weights[t,k] under the same condition, else 0.
    ``num_groups = 0`` means expert mode only.
    """
    idx = np.asarray(topk_idx, dtype=np.int64)
    if idx.ndim != 2:
        raise ValueError("topk_idx must be [T, K]")
    T, K = idx.shape
    E = int(num_experts)
    G = int(num_groups)
    if E < 1 or G < 0 or (G > 0 and E % G):
        raise ValueError("need E >= 1 and G dividing E")
    valid = (idx >= 0) & (idx < E)
    n_invalid = int(np.count_nonzero((idx != -1) & ~valid))
    idl = idx.tolist()
    vl = valid.tolist()

    # phase 1: count per destination
    counts = [0] * E
    for t in range(T):
        for k in range(K):
            if vl[t][k]:
                counts[idl[t][k]] += 1
    # phase 2: exclusive prefix sum -> segment bases
    A = max(1, int(expert_alignment))
    offsets = [0] * (E + 1)
    for e in range(E):
        seg = (counts[e] + A - 1) // A * A
        offsets[e + 1] = offsets[e] + seg
    # phase 3: base + locally claimed slot, claims taken in (t,k) order
    claimed = [0] * E
    slot = [[-1] * K for _ in range(T)]
    for t in range(T):
        for k in range(K):
            if vl[t][k]:
                e = idl[t][k]
                slot[t][k] = offsets[e] + claimed[e]
                claimed[e] += 1
    expert_row_src = [-1] * offsets[E]
    for t in range(T):
        for k in range(K):
            if slot[t][k] >= 0:
                expert_row_src[slot[t][k]] = t
    out = {
        "counts": np.array(counts, dtype=np.int64),
        "offsets": np.array(offsets, dtype=np.int64),
        "slot": np.array(slot, dtype=np.int64).reshape(T, K),
        "expert_row_src": np.array(expert_row_src, dtype=np.int64),
        "n_invalid": n_invalid,
        "n_sel": sum(counts),
        "n_rows_expert": offsets[E],
    }
    if G == 0:
        return out

    epg = E // G
    w = None if topk_weights is None else np.asarray(topk_weights, dtype=np.float32)
    hit = [[False] * G for _ in range(T)]
    for t in range(T):
        for k in range(K):
            if vl[t][k]:
                hit[t][idl[t][k] // epg] = True
    gcounts = [0] * G
    for t in range(T):
        for g in range(G):
            if hit[t][g]:
                gcounts[g] += 1
    goffsets = [0] * (G + 1)
    for g in range(G):
        goffsets[g + 1] = goffsets[g] + gcounts[g]
    R = goffsets[G]
    claimed_g = [0] * G
    grow = np.full((T, K), -1, dtype=np.int64)
    src = np.zeros(R, dtype=np.int64)
    ridx = np.full((R, K), -1, dtype=np.int64)
    rw = np.zeros((R, K), dtype=np.float32)
    for t in range(T):
        for g in range(G):
            if not hit[t][g]:
                continue
            r = goffsets[g] + claimed_g[g]
            claimed_g[g] += 1
            src[r] = t
            for k in range(K):
                if vl[t][k] and idl[t][k] // epg == g:
                    grow[t, k] = r
                    ridx[r, k] = idl[t][k] - g * epg
                    if w is not None:
                        rw[r, k] = w[t, k]
    out.update(
        {
            "gcounts": np.array(gcounts, dtype=np.int64),
            "goffsets": np.array(goffsets, dtype=np.int64),
            "grow": grow,
            "src": src,
            "ridx": ridx,
            "rw": rw,
            "n_rows": R,
        }
    )
    return out


# --------------------------------------------------------------------------
# dispatch
# --------------------------------------------------------------------------
def dispatch_bf16(x_u16, dest, n_rows: int) -> np.ndarray:
    """recv[dest[t,k]] = x[t] for every dest >= 0 (bytes copied unchanged).

    ``dest`` is ``slot`` for the expert-major layout or ``grow`` for the
    grouped one (several k of a token then name the same row, which receives
    the same bytes).  Rows no selection names are alignment padding and are
    zero (the zero_padding form)."""
    x = np.asarray(x_u16, dtype=np.uint16)
    dest = np.asarray(dest, dtype=np.int64)
    T, K = dest.shape
    recv = np.zeros((n_rows, x.shape[1]), dtype=np.uint16)
    for k in range(K):
        sel = dest[:, k] >= 0
        recv[dest[sel, k]] = x[sel]
    return recv


def quantize_row_fp8(x_row_u16) -> np.ndarray:
    """One token's packed fp8 row (uint8, ``fp8_row_bytes(H)`` long).

    For each 128-element group j: a = max |x| (exact in fp32),
    s = fl32(a / 448), q_i = e4m3fn_rne_sat(fl32(x_i / s)) or 0x00 for every
    element when s == 0.  Bytes: q[0..H), then s_0..s_{H/128-1} as
    little-endian fp32, then zeros to the 16-byte boundary.
    """
    xr = np.asarray(x_row_u16, dtype=np.uint16)
    H = xr.shape[0]
    rb = fp8_row_bytes(H)
    if rb < 0:
        raise ValueError("fp8 rows need H % 128 == 0")
    xf = bf16_to_f32(xr).reshape(H // FP8_GROUP, FP8_GROUP)
    a = np.max(np.abs(xf), axis=1).astype(np.float32)
    s = (a / np.float32(FP8_MAX)).astype(np.float32)
    q = np.zeros((H // FP8_GROUP, FP8_GROUP), dtype=np.uint8)
    nz = s != 0
    if nz.any():
        v = (xf[nz] / s[nz][:, None]).astype(np.float32)
        q[nz] = e4m3fn_rne_sat(v)
    row = np.zeros(rb, dtype=np.uint8)
    row[:H] = q.reshape(-1)
    row[H : H + 4 * (H // FP8_GROUP)] = s.astype("<f4").view(np.uint8)
    return row


def dispatch_fp8(x_u16, dest, n_rows: int) -> np.ndarray:
    """recv[dest[t,k]] = packed fp8 row of token t (see ``quantize_row_fp8``);
    rows no selection names (alignment padding) are all zero bytes."""
    x = np.asarray(x_u16, dtype=np.uint16)
    dest = np.asarray(dest, dtype=np.int64)
    T, K = dest.shape
    rb = fp8_row_bytes(x.shape[1])
    if rb < 0:
        raise ValueError("fp8 rows need H % 128 == 0")
    recv = np.zeros((n_rows, rb), dtype=np.uint8)
    for t in range(T):
        ds = [int(d) for d in dest[t] if d >= 0]
        if not ds:
            continue
        row = quantize_row_fp8(x[t])
        for d in ds:
            recv[d] = row
    return recv


# --------------------------------------------------------------------------
# combine
# --------------------------------------------------------------------------
def _bias_seed(bias0, bias1, shape) -> np.ndarray:
    """The combine accumulator's starting value: +0 without a bias,
    f32(bias) with one, fl32(f32(bias0) + f32(bias1)) with two.  The bias
    seeds the reduction instead of being added after it (commit adding
    receive stats and combine bias)."""
    given = [b for b in (bias0, bias1) if b is not None]
    if not given:
        return np.zeros(shape, dtype=np.float32)
    acc = bf16_to_f32(np.asarray(given[0], dtype=np.uint16)).reshape(shape).astype(np.float32)
    if len(given) == 2:
        acc = (acc + bf16_to_f32(np.asarray(given[1], dtype=np.uint16)).reshape(shape)).astype(np.float32)
    return acc


def combine(y_u16, slot, topk_weights, bias0=None, bias1=None) -> np.ndarray:
    """out[t] = bf16_rne(sum over k = 0..K-1 with slot[t,k] >= 0 of
    w[t,k] * y[slot[t,k]]), accumulated in fp32 with the product and the sum
    rounded separately, in ascending k, starting from +0 or from the bias
    (``_bias_seed``).  A token with no selection gives +0, or its bias."""
    y = np.asarray(y_u16, dtype=np.uint16)
    slot = np.asarray(slot, dtype=np.int64)
    w = np.asarray(topk_weights, dtype=np.float32)
    T, K = slot.shape
    acc = _bias_seed(bias0, bias1, (T, y.shape[1]))
    for k in range(K):
        sel = slot[:, k] >= 0
        rows = bf16_to_f32(y[slot[sel, k]])
        p = (w[sel, k][:, None] * rows).astype(np.float32)
        acc[sel] = (acc[sel] + p).astype(np.float32)
    return bf16_rne(acc)


def combine_grouped(
    y_u16, topk_idx, slot, topk_weights, num_experts: int, num_groups: int, bias0=None, bias1=None
):
    """out[t] = bf16_rne(sum over g ascending of P_g) where
    P_g = sum over k ascending with (t,k) valid and in group g of
    w[t,k] * y[slot[t,k]]; every product and sum is one fp32 rounding; each
    P_g starts from +0 and the cross-group total from +0 or the bias.  A token's rows inside one group are summed
    before the cross-group sum, the order of the expanded combine, which adds
    up a token's rows on one destination before that destination's single
    row goes out."""
    y = np.asarray(y_u16, dtype=np.uint16)
    idx = np.asarray(topk_idx, dtype=np.int64)
    slot = np.asarray(slot, dtype=np.int64)
    w = np.asarray(topk_weights, dtype=np.float32)
    T, K = slot.shape
    epg = num_experts // num_groups
    tot = _bias_seed(bias0, bias1, (T, y.shape[1]))
    for g in range(num_groups):
        P = np.zeros_like(tot)
        for k in range(K):
            sel = (slot[:, k] >= 0) & (idx[:, k] // epg == g)
            if not sel.any():
                continue
            rows = bf16_to_f32(y[slot[sel, k]])
            p = (w[sel, k][:, None] * rows).astype(np.float32)
            P[sel] = (P[sel] + p).astype(np.float32)
        tot = (tot + P).astype(np.float32)
    return bf16_rne(tot)


# --------------------------------------------------------------------------
# grouped GEMM over the expert-major segments (the dispatch's consumer)
# --------------------------------------------------------------------------
def expert_gemm(x_u16, counts, offsets, w_u16, rows=None) -> np.ndarray:
    """float64 y[r] = x[r] @ w[e]^T for every row r of expert e's segment
    [offsets[e], offsets[e] + counts[e]); other rows are NaN (not defined).

    ``w`` is bf16 [E, N, H] (expert e's N output rows, each H long).  The
    products of bf16 values are exact in float64 and the sum is float64, so
    this is the exact value to about 2^-50 relative; the GPU's fp32 sum and
    bf16 output are compared against it within ``expert_gemm_bound``.  With
    ``rows`` only those receive rows are computed (others NaN).  Used as the
    grouped GEMM that consumes each expert's contiguous block of rows
    (the mKernel article's MoE dispatch + grouped GEMM, consumer half).
    """
    x = bf16_to_f32(np.asarray(x_u16, dtype=np.uint16)).astype(np.float64)
    w = bf16_to_f32(np.asarray(w_u16, dtype=np.uint16)).astype(np.float64)
    E, N, H = w.shape
    y = np.full((x.shape[0], N), np.nan)
    want = None if rows is None else set(int(r) for r in rows)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e]) + int(counts[e])
        rs = [r for r in range(r0, r1) if want is None or r in want]
        if rs:
            y[rs] = x[rs] @ w[e].T
    return y


def expert_gemm_bound(x_u16, counts, offsets, w_u16, y64) -> np.ndarray:
    """Per-element error bound for a bf16 result of an fp32-accumulated
    expert GEMM: 2^-8 |y| (bf16 output rounding, with slack) plus
    H * 2^-24 * sum_h |x w| (any order of H fp32 additions of exact
    products).  NaN where y64 is NaN."""
    x = np.abs(bf16_to_f32(np.asarray(x_u16, dtype=np.uint16)).astype(np.float64))
    w = np.abs(bf16_to_f32(np.asarray(w_u16, dtype=np.uint16)).astype(np.float64))
    E, N, H = w.shape
    absdot = np.full_like(y64, np.nan)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e]) + int(counts[e])
        rs = [r for r in range(r0, r1) if not np.isnan(y64[r]).all()]
        if rs:
            absdot[rs] = x[rs] @ w[e].T
    return np.abs(y64) * 2.0**-8 + absdot * H * 2.0**-24
