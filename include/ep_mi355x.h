/*
 * ep_mi355x.h — C ABI of the MoE token dispatch / combine hot path for one
 * MI355X (gfx950) GPU.
 *
 * The operations follow TileScale pull request #68, "[Example] EP v2
 * intranode dispatch/combine":
 *   - dispatch counts each token's selections per destination, turns the
 *     counts into a base per destination, and writes every row straight to
 *     base + a claimed slot, already its place in the dense receive buffer,
 *     so no later pass moves rows (PR summary; PR description, Design
 *     section; commit adding DeepEP's do_expand, where the destination
 *     becomes the expert and the base is an exclusive prefix sum of
 *     per-expert counts);
 *   - the fp8 payload is DeepEP's per-token, per-128-element cast, packed
 *     with its fp32 scales into one row moved by one store (commit packing
 *     the fp8 payload and scales into one row);
 *   - topk_idx == -1 means "no selection" and is skipped (commit on masked
 *     topk_idx);
 *   - combine gathers each token's expert-output rows and reduces them per
 *     source token (PR summary; Design section), summing a token's rows
 *     inside one expert group before the sum across groups (commit adding
 *     the expanded combine, kDoExpandedSend).
 *
 * Conventions for every entry point
 *   - All device pointers are caller-owned allocations on the current HIP
 *     device.  The library never allocates, frees or synchronises; every
 *     call only enqueues kernels on `stream`, and pointers must stay valid
 *     until the stream reaches that work.
 *   - Inputs are read-only.  Outputs are fully overwritten as documented.
 *   - Host-checkable errors return a nonzero code before anything is
 *     enqueued.  Data-dependent conditions are reported in the device
 *     status words (EP_STATUS_*), never by corrupting memory.
 *   - bf16 values are 16-bit IEEE-style bfloat16 bit patterns; fp32 is IEEE
 *     binary32; all integers are little-endian.
 *   - The environment variable EP_MI355X_GRID_BLOCKS=<n> (1 <= n <= 2^20),
 *     read at every launch, replaces the grid size of the dispatch and
 *     combine kernels, for launch sweeps; results are the same at any grid.
 */
#ifndef EP_MI355X_H
#define EP_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes ---------------------------------------------------- */
#define EP_OK 0
#define EP_EINVAL 1     /* null pointer, bad size, misaligned base pointer */
#define EP_ENOTSUP 2    /* valid but unsupported (fp8 with hidden % 128 != 0, limits) */
#define EP_EHIP 3       /* a HIP launch failed (hipGetLastError) */
#define EP_EWORKSPACE 4 /* workspace smaller than ep_layout_workspace_bytes() */
#define EP_ESCRATCH 5   /* ep_layout_noalloc: the problem needs more than the
                         * library's fixed EP_LAYOUT_SCRATCH_BYTES of scratch */

/* ---- limits ---------------------------------------------------------- */
#define EP_MAX_TOPK 32     /* K */
#define EP_MAX_KEYS 1024   /* E + G (destinations counted by the layout) */
#define EP_LAYOUT_SCRATCH_BYTES (9u << 18) /* ep_layout_noalloc's fixed scratch per GPU, 2.25 MiB */

/* ---- device status words ---------------------------------------------
 * ep_layout writes every word (words 4, 7 and 9 as 0); the other calls
 * write only the words named here.  Data-dependent conditions are reported
 * here rather than by corrupting memory, as the PR's expanded dispatch
 * reports expand_overflow before any payload moves (commit adding DeepEP's
 * do_expand). */
#define EP_STATUS_INVALID_IDS 0 /* ids outside {-1} U [0,E): counted, treated as -1 */
#define EP_STATUS_ROWS_EXPERT 1 /* rows of the expert-major layout (selections + padding) */
#define EP_STATUS_ROWS_GROUP 2  /* R: rows of the grouped layout (0 without groups) */
#define EP_STATUS_LIST_OVERFLOW 3 /* 1 if R > row_capacity: row lists not written */
#define EP_STATUS_COMBINE_OOB 4 /* set to 1 by ep_combine if a slot >= y_rows was met */
#define EP_STATUS_EXPERT_LIST_OVERFLOW 5 /* 1 if expert rows > expert_row_capacity */
#define EP_STATUS_SELECTIONS 6  /* valid selections (EP_STATUS_ROWS_EXPERT minus padding) */
#define EP_STATUS_DISPATCH_OVERFLOW 7 /* written by every ep_dispatch: 1 if the rows it
                                       * needed exceeded capacity_rows (it then wrote no
                                       * row), else 0 */
#define EP_STATUS_GENERATION 8  /* the generation ep_layout stamped on these buffers */
#define EP_STATUS_STALE 9       /* set to 1 (sticky until the next ep_layout) by a
                                 * dispatch, combine or GEMM handed an ep_layout_t whose
                                 * generation is not EP_STATUS_GENERATION; that call
                                 * wrote nothing else */
#define EP_STATUS_WORDS 16

/* ---- problem flags ---------------------------------------------------- */
#define EP_FLAG_ZERO_PADDING 1 /* dispatch zeroes the alignment padding rows */
#define EP_FLAG_GATHER_ROWS 2  /* ep_expert_gemm reads token rows through expert_row_src */
#define EP_FLAG_PACKED_WEIGHTS 4 /* ep_expert_gemm's w is in ep_pack_expert_weights' order */

/* ---- formats, row kinds, combine orders ------------------------------ */
#define EP_FORMAT_BF16 0       /* receive row = the token's H bf16 values */
#define EP_FORMAT_FP8_PACKED 1 /* receive row = ep_fp8_row_bytes(H) bytes */

#define EP_ROWS_EXPERT 0 /* one row per valid (token, k), expert-major */
#define EP_ROWS_GROUP 1  /* one row per (token, group hit), group-major */

#define EP_COMBINE_FLAT 0    /* ascending k */
#define EP_COMBINE_GROUPED 1 /* within each group ascending k, then groups ascending */

/* Problem shape.
 *   num_tokens  T >= 0 source tokens
 *   hidden      H >= 1 elements per token row
 *   topk        K in [1, EP_MAX_TOPK]
 *   num_experts E >= 1
 *   num_groups  G: 0 = expert-major layout only; G >= 1 dividing E = the E
 *               experts also form G contiguous groups of E/G (a group plays
 *               the role of a destination rank) and the layout adds one
 *               deduplicated row per (token, group hit).  E + G must not
 *               exceed EP_MAX_KEYS.
 *   expert_alignment  0 or 1 = none; A >= 2 rounds every expert segment of
 *               the expert-major layout up to a multiple of A rows, so each
 *               expert's rows form an A-aligned block a grouped GEMM can
 *               consume (PR commit adding do_expand: expert_alignment).  The
 *               rows past an expert's selections are padding.
 *   flags       EP_FLAG_ZERO_PADDING: ep_dispatch also zeroes every byte of
 *               the padding rows' row size (the PR's zero_padding), and for
 *               fp8 rows the line fill ep_dispatch describes.
 *               EP_FLAG_GATHER_ROWS: ep_expert_gemm takes the token rows
 *               themselves and gathers each expert row's operand through
 *               the layout's expert_row_src (dispatch fused into the GEMM).
 *               EP_FLAG_PACKED_WEIGHTS: ep_expert_gemm's weights are in the
 *               packed tile order ep_pack_expert_weights writes.
 *               Other entry points ignore these two. */
typedef struct ep_problem {
  int64_t num_tokens;
  int32_t hidden;
  int32_t topk;
  int32_t num_experts;
  int32_t num_groups;
  int32_t expert_alignment;
  int32_t flags;
} ep_problem_t;

/* Layout outputs: device pointers, caller-owned, all int32 unless noted.
 *   counts[E]          selections per expert
 *   offsets[E+1]       exclusive prefix sum of the (aligned) counts;
 *                      offsets[E] = rows of the expert-major layout
 *   slot[T*K]          expert-major row of (t,k): offsets[e] + number of
 *                      earlier (t',k') in (t,k) order with the same expert;
 *                      -1 for masked or invalid entries
 *   status[EP_STATUS_WORDS]
 *   expert_row_src[expert_row_capacity]   optional (NULL = not written):
 *                      source token of each expert-major row, -1 for an
 *                      alignment padding row (marked unoccupied); not
 *                      written if the rows exceed the capacity
 *                      (EP_STATUS_EXPERT_LIST_OVERFLOW)
 *   recv_stats[E]      optional uint32 (NULL = not touched): counts[e] is
 *                      ADDED to recv_stats[e], so the caller chooses the
 *                      accumulation window by when it clears it (the PR's
 *                      cumulative_local_expert_recv_stats, commit adding
 *                      receive stats and combine bias)
 * Grouped layout (only read/written when num_groups >= 1; may be NULL otherwise):
 *   group_counts[G], group_offsets[G+1]   rows per group and their prefix sum
 *   grow[T*K]          grouped row carrying (t,k): group_offsets[g] + number
 *                      of tokens t' < t hitting group g; -1 if masked
 *   row_src[row_capacity]                 source token of each grouped row
 *   row_topk_idx[row_capacity*K]          per row, per k: the expert's index
 *                      inside the row's group if (t,k) is valid and in that
 *                      group, else -1
 *   row_topk_weights[row_capacity*K]      fp32: topk_weights[t,k] under the
 *                      same condition, else 0
 *   row_capacity       rows the three lists hold; if R exceeds it the lists
 *                      are not written and EP_STATUS_LIST_OVERFLOW is set.
 * Stale-layout guard (host field, not a device pointer):
 *   generation         set by every ep_layout to a value unique in the
 *                      process (never 0), which it also stamps into the
 *                      device word EP_STATUS_GENERATION in stream order.  A
 *                      copy of this struct taken after ep_layout is a cached
 *                      handle to that layout: ep_dispatch, ep_combine and
 *                      ep_expert_gemm compare the copy's generation with the
 *                      device word and, if a later ep_layout has rewritten
 *                      the buffers, write nothing and set EP_STATUS_STALE
 *                      (the PR's cached handle= dispatch, rejected once the
 *                      buffer's _layout_generation has moved on; commit
 *                      adding the cached-layout dispatch).  A zeroed struct
 *                      that no ep_layout has stamped fails the check. */
typedef struct ep_layout {
  int32_t* counts;
  int32_t* offsets;
  int32_t* slot;
  int32_t* status;
  int32_t* group_counts;
  int32_t* group_offsets;
  int32_t* grow;
  int32_t* row_src;
  int32_t* row_topk_idx;
  float* row_topk_weights;
  int64_t row_capacity;
  int32_t* expert_row_src;
  int64_t expert_row_capacity;
  uint32_t* recv_stats;
  uint32_t generation;
} ep_layout_t;

/* Bytes of one packed fp8 row: H bytes of E4M3FN payload, then H/128
 * little-endian fp32 scales, zero-padded to a multiple of 16 bytes
 * (hidden 7168 -> 7392, hidden 128 -> 144).  Returns -1 if hidden <= 0 or
 * hidden % 128 != 0.  Host only; no device work.
 * Defined by: TileScale PR #68, commit packing the fp8 payload and its
 * scales into one row (row = payload, then scales, 16-byte padded). */
int64_t ep_fp8_row_bytes(int32_t hidden);

/* Bytes of device workspace ep_layout needs for this problem (per-block
 * tallies and per-chunk totals; at most 2,230,528 bytes for any accepted
 * problem).  Returns 0 for an invalid problem.  Host only.
 * Defined by: TileScale PR #68, Design section (per-block counts that a
 * prefix sum turns into bases). */
size_t ep_layout_workspace_bytes(const ep_problem_t* p);

/* Layout: phase 1 (count per expert, and per group), phase 2 (exclusive
 * scan into bases) and phase 3 (slots and grouped rows) for topk_idx int64
 * [T*K] row-major.  topk_weights fp32 [T*K] is read only to fill
 * row_topk_weights and may be NULL when num_groups == 0.  `workspace` must
 * hold ep_layout_workspace_bytes(p) bytes, 16-byte aligned (contents need
 * no initialisation and are clobbered).  Writes every output of `L` listed above and every
 * status word (EP_STATUS_COMBINE_OOB, _DISPATCH_OVERFLOW and _STALE as 0),
 * and sets L->generation (host field) to a fresh value that it also stamps
 * into EP_STATUS_GENERATION.  Placement is deterministic: identical inputs
 * give identical bytes.
 * Defined by: TileScale PR #68, Design section (count, exclusive prefix
 * sum, slot claimed under the base); commit adding DeepEP's do_expand (the
 * destination is the expert, segments expert-major, expert_alignment,
 * -1 entries skipped); commit on masked topk_idx; commit adding the
 * expanded combine (per-row local expert ids and weights, recv_topk_idx). */
int ep_layout(const ep_problem_t* p, const int64_t* topk_idx, const float* topk_weights,
              ep_layout_t* L, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ep_layout without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Identical outputs to ep_layout; the
 * per-block tallies live instead in a library-owned device array of
 * EP_LAYOUT_SCRATCH_BYTES, one per GPU, held until the process ends.  The
 * call allocates and frees nothing.  The array covers every problem the
 * library accepts (the largest ep_layout_workspace_bytes over all shapes is
 * 2,230,528 bytes); EP_ESCRATCH, with nothing enqueued, guards a problem
 * whose workspace would exceed it.  EP_EHIP if the array's device
 * address cannot be found on the current device.  Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (two
 * streams, or two host threads) race and must be ordered by the caller.
 * Nothing in the array needs to start at zero (the tallies are written
 * before they are read). */
int ep_layout_noalloc(const ep_problem_t* p, const int64_t* topk_idx, const float* topk_weights,
                      ep_layout_t* L, hipStream_t stream);

/* Dispatch: scatter every token row of x (bf16 [T*H]) to the receive rows
 * the layout assigned it (with EP_FLAG_ZERO_PADDING also zero the expert
 * alignment padding rows).
 *   rows == EP_ROWS_EXPERT: recv row slot[t,k] for each valid (t,k);
 *   rows == EP_ROWS_GROUP:  recv row grow[t,k] once per distinct row.
 *   format == EP_FORMAT_BF16: a receive row is the token's H bf16 values
 *     (2*H bytes);
 *   format == EP_FORMAT_FP8_PACKED: a receive row is the packed fp8 row of
 *     ep_fp8_row_bytes(H) bytes, quantised per 128-element group j as
 *     s_j = amax_j / 448 and q = E4M3FN(x / s_j) (both fp32 IEEE divisions,
 *     round to nearest even, saturating at 448; s_j == 0 gives q = 0);
 *     requires H % 128 == 0 and H <= 32768.
 * Receive row r starts at byte r * recv_row_stride of recv; recv_row_stride
 * == 0 means the row size itself (rows packed back to back).  A larger
 * stride pads each row to an aligned pitch (for the fp8 row at hidden 7168,
 * 7424 bytes puts every row on a 128-byte boundary, which MI355X writes
 * markedly faster than the packed 7392).  For the fp8 format with recv and
 * the stride both multiples of 128 bytes, each row written is followed by
 * zero bytes up to the next 128-byte boundary (at most 112 bytes, never
 * past the stride), so every 128-byte line is written whole: at hidden
 * 7168 and the 7424-byte pitch that measured 99 against 107 us.  Otherwise
 * the bytes between a row's end and the next row are never written.  recv
 * must hold capacity_rows rows.
 * Each source row is read once and written once per destination row.  If
 * the rows needed (status word EP_STATUS_ROWS_EXPERT or _GROUP) exceed
 * capacity_rows the call writes no row and sets EP_STATUS_DISPATCH_OVERFLOW
 * to 1 (else it sets it to 0): an overflow is known before any payload
 * moves.  Rows at or beyond the rows needed are never touched.  If L's
 * generation is not the one stamped on its buffers, the call writes nothing
 * but EP_STATUS_STALE = 1.
 * Base pointers of x and recv, and the stride, must be 16-byte aligned for
 * the fp8 format; for bf16 any 2-byte alignment works (wider alignment is
 * faster).
 * Defined by: TileScale PR #68, summary and Design section (each row
 * written once, at its final compact index); commit adding DeepEP's
 * do_expand (expert-major rows, expand_overflow, zero_padding); commit
 * packing the fp8 payload and scales into one row; PR description,
 * Testing section (per-token, per-128 fp8 cast). */
int ep_dispatch(const ep_problem_t* p, const ep_layout_t* L, const void* x, void* recv,
                int64_t capacity_rows, int64_t recv_row_stride, int32_t rows, int32_t format,
                hipStream_t stream);

/* Combine: out[t] (bf16 [T*H]) = bf16_rne of the fp32 sum over the token's
 * valid selections of topk_weights[t,k] * y[slot[t,k]], with y bf16
 * [y_rows * H] in expert-major receive order (y row r is the expert output
 * for receive row r).  Each product and each sum is one fp32 rounding (no
 * fused multiply-add).
 *   order == EP_COMBINE_FLAT:    ascending k;
 *   order == EP_COMBINE_GROUPED: per group in ascending k, then the group
 *     partials in ascending group order (needs num_groups >= 1 and
 *     topk_idx int64 [T*K]; topk_idx may be NULL for the flat order).
 * The accumulator starts at +0, or at the bias: bias0 and bias1 (bf16
 * [T*H], either may be NULL) seed it as fl32(bias0 + bias1) (or the one
 * given) instead of being added afterwards, so a token with no valid
 * selection returns its bias, and +0 without one (the PR's combine bias,
 * commit adding receive stats and combine bias).  In the grouped order the
 * bias seeds the cross-group total.  A slot >= y_rows is skipped and sets
 * status word EP_STATUS_COMBINE_OOB.  Every one of the T output rows is
 * written, unless L's generation is not the one stamped on its buffers:
 * then the call writes nothing but EP_STATUS_STALE = 1.
 * Defined by: TileScale PR #68, summary and Design section (one reduce per
 * source token over its gathered rows); commit on masked topk_idx (-1
 * skipped, a fully masked token gives zero); commit adding the expanded
 * combine, kDoExpandedSend (sum within the group first); commit adding
 * receive stats and combine bias. */
int ep_combine(const ep_problem_t* p, const ep_layout_t* L, const int64_t* topk_idx,
               const float* topk_weights, const void* y, int64_t y_rows, const void* bias0,
               const void* bias1, void* out, int32_t order, hipStream_t stream);

/* Grouped GEMM over the expert-major segments (the consumer of dispatch;
 * the mKernel article's MoE dispatch + grouped GEMM, one-GPU consumer
 * half): for every expert e and receive row r in [offsets[e],
 * offsets[e] + counts[e]),
 *   y[r, n] = bf16_rne( sum over h < H of x[r, h] * w[e, n, h] ),  n < n_out,
 * summed in fp32 in the matrix cores' order (so results agree with an exact
 * sum within 2^-8 |y| + H 2^-24 sum |x w|, not bit for bit).
 *   x  bf16 receive rows (ep_dispatch's bf16 output), row r at element
 *      r * x_row_stride (0 = H);
 *   w  bf16 [E, n_out, H]: expert e's n_out output rows, each H long;
 *   y  bf16 output rows, row r at element r * y_row_stride (0 = n_out).
 * Rows outside every expert's selections (alignment padding, rows past the
 * layout) are not written.
 * With EP_FLAG_GATHER_ROWS in p->flags, x is instead the token matrix
 * (bf16 [T, H], row t at element t * x_row_stride) and expert row r reads
 * x row expert_row_src[r]: the dispatch's scatter folded into the GEMM's
 * operand loads, as the mKernel article's fused MoE dispatch + grouped GEMM
 * runs the GEMM on rows as they arrive, with no staging copy.  L must then
 * carry expert_row_src (from ep_layout) with expert_row_capacity covering
 * every expert row; the result equals the unfused dispatch + GEMM bit for
 * bit.  With EP_FLAG_PACKED_WEIGHTS, w is the packed copy
 * ep_pack_expert_weights made of the [E, n_out, H] weights (same E, n_out
 * and H); the result equals the unpacked GEMM bit for bit.
 * Requires H % 64 == 0 and n_out % 128 == 0, and
 * at most 2^31 - 1 output tiles of 320 x 256 (EP_ENOTSUP otherwise), 16-byte
 * aligned x, w and y, x_row_stride a multiple of 8 and y_row_stride a
 * multiple of 4.  If L's generation is not the one stamped on its buffers,
 * the call writes nothing but EP_STATUS_STALE = 1.
 * Defined by: the mKernel article ("Introducing mKernel"), its table of
 * fused kernels (MoE dispatch + grouped GEMM). */
int ep_expert_gemm(const ep_problem_t* p, const ep_layout_t* L, const void* x,
                   int64_t x_row_stride, const void* w, int32_t n_out, void* y,
                   int64_t y_row_stride, hipStream_t stream);

/* Weights packed once for the grouped GEMM.  Not from the pages: a layout
 * of this library.  Each 256-column tile of an expert's weights is stored
 * as H/32 blocks of 256 rows x 32 elements, so every reduction step of a
 * GEMM tile reads one contiguous 16 KiB block instead of 64 bytes from each
 * of 256 rows 2H bytes apart; static weights are packed once and reused.
 *   packed[e][j][k][r][c] = w[e, 256 j + r, 32 k + c]  if 256 j + r < n_out,
 *                           0                          otherwise,
 * for j < ceil(n_out / 256), k < H / 32, r < 256, c < 32 (bf16).
 * ep_expert_weights_packed_bytes gives the size, E * ceil(n_out/256) * 256
 * * H * 2 bytes, or -1 if E < 1, n_out < 1, H < 1, n_out % 128 != 0 or
 * H % 64 != 0 (host only, no device work).  ep_pack_expert_weights writes
 * the packed copy of w (bf16 [E, n_out, H], 16-byte aligned) to w_packed
 * (caller-owned, that many bytes, 16-byte aligned, not overlapping w) on
 * the stream; EP_EINVAL for null, misaligned or overlapping pointers or
 * invalid sizes. */
int64_t ep_expert_weights_packed_bytes(int32_t num_experts, int32_t n_out, int32_t hidden);
int ep_pack_expert_weights(const void* w, int32_t num_experts, int32_t n_out, int32_t hidden,
                           void* w_packed, hipStream_t stream);

/* Static description of a return code.  Not from the pages. */
const char* ep_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* EP_MI355X_H */
