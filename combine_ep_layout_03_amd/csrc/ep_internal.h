// Internal launch interface between the C-ABI entry points and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ep {

// Geometry of the layout kernels.  Place block b handles entries
// [b * rounds * 256, (b + 1) * rounds * 256) of the flattened (t,k) order;
// count block c tallies the `chunk` consecutive place blocks
// [c * chunk, (c + 1) * chunk).
struct LayoutGeom {
  int nblocks;  // place blocks, >= 1
  int rounds;   // entries per place-block thread (a power of two)
  int span_shift;  // log2 of a place block's entries, 8 + log2(rounds)
  int half;     // count-block tallies in 16-bit halves (span <= 32768)
  int ncols;    // E + G + 1 tally columns (last column: invalid ids)
  int chunk;    // place blocks per count block, >= 1
  int ncount;   // count blocks, ceil(nblocks / chunk)
};

LayoutGeom layout_geom(int64_t n_entries, int E, int G);
size_t layout_workspace_bytes(const LayoutGeom& g);

struct LayoutArgs {
  const int64_t* idx;
  const float* w;
  uint32_t n;  // T * K
  int K, E, G, epg;
  int32_t* counts;
  int32_t* offsets;
  int32_t* slot;
  int32_t* status;
  int32_t* gcounts;
  int32_t* goffsets;
  int32_t* grow;
  int32_t* row_src;
  int32_t* row_idx;
  float* row_w;
  int64_t row_cap;
  int align;  // expert segment alignment (1 = none)
  int32_t* expert_row_src;  // optional
  int64_t expert_row_cap;
  uint32_t* recv_stats;  // optional, accumulated
  int32_t* partials;  // workspace
  uint32_t generation;  // stamped into status[EP_STATUS_GENERATION]
};
hipError_t launch_layout(const LayoutArgs& a, const LayoutGeom& g, hipStream_t s);

// Stale-layout guard shared by dispatch, combine and the GEMM: the kernels
// run only if the layout buffers still carry the generation the caller's
// handle was taken at (device word status[kStatusGeneration]); otherwise
// they write nothing and set status[kStatusStale].
constexpr int kStatusDispatchOverflow = 7;
constexpr int kStatusGeneration = 8;
constexpr int kStatusStale = 9;

// A status word read through the vector memory path.  Scalar loads return
// out of order, so any later wait for a kernel argument would also wait for
// this word; vector loads retire in order, so the loads issued after it
// (a wave's first indices) stay in flight while it is checked.
__device__ __forceinline__ int32_t status_word(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Is the layout behind `status` still the one the caller's handle names?
// `word` is status[kStatusGeneration] as the wave read it (the scatters load
// it together with their first destination rows, so the check costs them no
// round trip of its own).  On a stale handle the grid's first lane sets the
// sticky stale flag; the caller's kernel then returns.
__device__ __forceinline__ bool layout_current(int32_t* status, int32_t word,
                                               uint32_t generation) {
  const bool cur = static_cast<uint32_t>(word) == generation;
  if (!cur && blockIdx.x == 0 && threadIdx.x == 0) status[kStatusStale] = 1;
  return cur;
}
__device__ __forceinline__ bool layout_current(int32_t* status, uint32_t generation) {
  return layout_current(status, status[kStatusGeneration], generation);
}

struct ScatterArgs {
  const void* x;
  void* recv;
  const int32_t* dest;  // [T*K] slot or grow
  const int32_t* rows_needed;  // device word
  int32_t* status;             // layout status words
  uint32_t generation;         // the caller's handle
  int64_t T;
  int K;
  int H;
  int64_t capacity;
  int64_t stride;  // bytes from one receive row to the next
  bool dedup;  // several k may name one row (grouped rows)
  // alignment padding rows to zero (expert rows only): [offsets[e] + counts[e], offsets[e+1])
  const int32_t* counts;
  const int32_t* offsets;
  int E;
};
// bf16 rows; `vec_bytes` in {16, 8, 4, 2} divides the row size, the stride
// and both base alignments.
hipError_t launch_scatter_bf16(const ScatterArgs& a, int vec_bytes, hipStream_t s);

// The two device words a dispatch kernel checks before its first store,
// loaded together and early (the loads of the first token's destination
// rows follow without waiting for them).
struct DispatchGate {
  int32_t generation;
  int32_t rows_needed;
};
__device__ __forceinline__ DispatchGate dispatch_gate(const ScatterArgs& a) {
  return {status_word(a.status + kStatusGeneration), status_word(a.rows_needed)};
}
// May a dispatch kernel write?  Only if the layout is current and its rows
// fit the capacity (an overflow writes no row).  The grid's first lane
// records the overflow verdict of a current call (1 or 0).  Every wave
// calls this before any store.
__device__ __forceinline__ bool dispatch_may_write(const ScatterArgs& a, const DispatchGate& g) {
  if (!layout_current(a.status, g.generation, a.generation)) return false;
  const bool fits = static_cast<int64_t>(g.rows_needed) <= a.capacity;
  if (blockIdx.x == 0 && threadIdx.x == 0) a.status[kStatusDispatchOverflow] = fits ? 0 : 1;
  return fits;
}
__device__ __forceinline__ bool dispatch_may_write(const ScatterArgs& a) {
  return dispatch_may_write(a, dispatch_gate(a));
}
// packed fp8 rows; H % 128 == 0, H <= 32768, 16-byte aligned bases and stride.
hipError_t launch_scatter_fp8(const ScatterArgs& a, int64_t row_bytes, hipStream_t s);
// zero the first row_bytes bytes of every alignment padding row; `vec_bytes`
// divides row_bytes, the stride and the base alignment.
hipError_t launch_zero_padding(const ScatterArgs& a, int64_t row_bytes, int vec_bytes,
                               hipStream_t s);

struct CombineArgs {
  const void* y;
  int64_t y_rows;
  const int32_t* slot;
  const float* w;
  const int64_t* idx;  // grouped order only
  int epg;
  int E;
  int64_t T;
  int K;
  int H;
  const void* bias0;  // optional bf16 [T*H]
  const void* bias1;  // optional bf16 [T*H]
  void* out;
  int32_t* status;
  uint32_t generation;
  bool grouped;
};
// `vec_elems` in {8, 4, 2, 1} divides H and both base alignments (in bf16 elements).
hipError_t launch_combine(const CombineArgs& a, int vec_elems, hipStream_t s);

struct GemmArgs {
  const uint16_t* x;  // bf16 receive rows, row stride ldx elements
  int64_t ldx;
  const uint16_t* w;  // bf16 [E, N, H], or (packed) the tile order below
  uint16_t* y;        // bf16 output rows, row stride ldy elements
  int64_t ldy;
  const int32_t* counts;
  const int32_t* offsets;
  int E, H, N;
  int ntn;  // column tiles, ceil(N / 256)
  // null: x holds the expert rows; else x holds token rows and expert row r
  // reads x row row_src[r]
  const int32_t* row_src;
  // w packed by launch_pack_expert_weights: [E][ntn][H/32][256][32], each
  // (expert, column tile, 32-wide reduction step) block 16 KiB contiguous,
  // rows past N zero
  bool packed;
  int32_t* status;
  uint32_t generation;
};
// H % 64 == 0, N % 128 == 0, E <= 1024, 16-byte aligned x / w / y and strides
// (ldx % 8 == 0, ldy % 4 == 0); max_rows bounds the expert-major rows.
// upper bound on the grouped GEMM's tiles for max_rows receive rows
int64_t expert_gemm_max_tiles(int64_t max_rows, int E, int N);
hipError_t launch_expert_gemm(const GemmArgs& a, int64_t max_rows, hipStream_t s);
// w bf16 [E, N, H] -> the packed tile order of GemmArgs::w (H % 32 == 0)
hipError_t launch_pack_expert_weights(const uint16_t* w, int E, int N, int H, uint16_t* packed,
                                      hipStream_t s);

}  // namespace ep
