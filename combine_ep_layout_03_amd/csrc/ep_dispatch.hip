// Dispatch: scatter each token row straight to its final receive rows.
//
// Each row is stored once, at the expert-major destination the layout gave
// it (base of its destination + claimed slot), so no compaction pass runs
// afterwards (TileScale PR #68, "EP v2 intranode dispatch/combine": PR
// summary and Design section).  Here a token row is cut into chunks; the
// grid's waves take the (token, chunk) items cyclically, read each chunk of
// the source row once and store it once per destination row.  Receive rows
// are written with non-temporal stores: they are not read again by this
// step and streaming them past the caches measured about 15-20% faster on
// MI355X than ordinary stores.  Vectors are 16 bytes when the row size and
// base alignment allow, otherwise the widest vector dividing both, so there
// is no remainder to drop (the pages' copy-tail fix, commit on
// cp_warp_impl).
//
// The fp8 variant fuses DeepEP's per-token, per-128-element cast into the
// same pass and writes payload, scales and padding of the packed row in one
// sweep per destination (commit packing payload and scales into one row).
#include "ep_device.h"
#include "ep_internal.h"
#include "ep_launch.h"

namespace ep {

namespace {

// Destination rows of token t, wave-uniform (scalar registers).  With
// `dedup`, later k that repeat an earlier row are dropped.  dest_lane issues
// the load (lane k holds row k); spread_dests waits for it and spreads it.
__device__ __forceinline__ int dest_lane(const ScatterArgs& a, int64_t t, int lane) {
  return lane < a.K ? a.dest[t * a.K + lane] : -1;
}
template <int KMAX>
__device__ __forceinline__ void spread_dests(const ScatterArgs& a, int dl, int (&d)[KMAX]) {
#pragma unroll
  for (int j = 0; j < KMAX; ++j) d[j] = readlane(dl, j);
  if (a.dedup) {
#pragma unroll
    for (int j = 1; j < KMAX; ++j) {
#pragma unroll
      for (int jj = 0; jj < j; ++jj)
        if (d[j] == d[jj]) d[j] = -1;
    }
  }
}
template <int KMAX>
__device__ __forceinline__ void load_dests(const ScatterArgs& a, int64_t t, int lane,
                                           int (&d)[KMAX]) {
  spread_dests<KMAX>(a, dest_lane(a, t, lane), d);
}

// Has the token any destination row?  (Wave-uniform: d is.)  A token
// without one is not read at all.
template <int KMAX>
__device__ __forceinline__ bool any_dest(const int (&d)[KMAX]) {
  bool any = false;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) any = any || d[j] >= 0;
  return any;
}

template <int KMAX, int VB, int U>
__global__ __launch_bounds__(kBlock) void k_scatter_bf16(ScatterArgs a, int nchunks,
                                                         int64_t items) {
  using V = typename VecOf<VB>::type;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t nw = grid_waves();
  const int64_t row_bytes = static_cast<int64_t>(a.H) * 2;
  const int nvec = static_cast<int>(row_bytes / VB);
  char* rbase = static_cast<char*>(a.recv);
  int d[KMAX];
  int64_t loaded = -1;
  bool any = false;
  // The first token's destination rows and the gate words load together.
  const int64_t it0 = global_wave();
  const int64_t t0 = it0 < items ? it0 / nchunks : 0;
  const int dl0 = it0 < items ? dest_lane(a, t0, lane) : -1;
  if (!dispatch_may_write(a, dispatch_gate(a))) return;  // stale layout or overflow: write nothing
  if (it0 < items) {
    spread_dests<KMAX>(a, dl0, d);
    any = any_dest<KMAX>(d);
    loaded = t0;
  }
  for (int64_t it = it0; it < items; it += nw) {
    const int64_t t = it / nchunks;
    const int c = static_cast<int>(it - t * nchunks);
    if (t != loaded) {
      load_dests<KMAX>(a, t, lane, d);
      any = any_dest<KMAX>(d);
      loaded = t;
    }
    if (!any) continue;
    const V* src = reinterpret_cast<const V*>(static_cast<const char*>(a.x) + t * row_bytes);
    const int vb = c * (kWave * U);
    V val[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int vi = vb + u * kWave + lane;
      val[u] = vi < nvec ? src[vi] : V{};
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (d[j] < 0) continue;
      V* dst = reinterpret_cast<V*>(rbase + static_cast<int64_t>(d[j]) * a.stride);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int vi = vb + u * kWave + lane;
        if (vi < nvec) nt_store(val[u], dst + vi);
      }
    }
  }
}

// Packed fp8 row, per 128-element group j of the token:
//   a_j = max |x| (exact), s_j = a_j / 448 (IEEE fp32 division),
//   q = E4M3FN_rne_sat(x / s_j) (IEEE fp32 division), or q = 0 when s_j == 0;
// bytes: q[0..H) | s_0 .. s_{H/128-1} (fp32, little-endian) | zeros to row_bytes
// (row_bytes: the packed row, or more when the launcher extends the zeros to
// a 128-byte line end).
// A wave owns whole tokens, taken cyclically.  Each lane converts 16
// consecutive elements per step, so 8 lanes form one group and a step covers
// 1024 elements (H % 128 == 0 keeps every group's 8 lanes together and
// active).  A step's source elements are loaded one step ahead (the first
// step of the wave's next token during the last step of a token), so the
// loads fly while a step converts.  A token without a destination row is
// skipped unread.
// The group scales stay in registers (group g in lane g % 64, slot g / 64).
// With ROWBUF (H <= 8192) the token's whole payload stays in registers too,
// and each destination row is then written in one burst: payload, scales,
// padding.  Otherwise each step's payload is stored as it is made and the
// scales follow the last step (the launcher picks by row pitch).  Writing
// the scales piecewise per step, or at the packed 7392-byte pitch instead of
// a 128-byte aligned one, measured 20-45% slower at hidden 7168.
template <int KMAX, bool ROWBUF>
__global__ __launch_bounds__(kBlock) void k_scatter_fp8(ScatterArgs a, int64_t row_bytes) {
  constexpr int kMaxScaleSlots = 4;  // H <= 4 * 64 * 128
  constexpr int kRowSteps = 8;       // ROWBUF: H <= 8 * 1024
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t nw = grid_waves();
  int64_t t = global_wave();
  // the first token's destination rows and the gate words load together
  const int dl0 = t < a.T ? dest_lane(a, t, lane) : -1;
  if (!dispatch_may_write(a, dispatch_gate(a)) || t >= a.T) return;
  int d[KMAX];
  spread_dests<KMAX>(a, dl0, d);
  const int H = a.H;
  const int ngroups = H / 128;
  const int nsteps = (H + kWave * 16 - 1) / (kWave * 16);
  const int pad_words = static_cast<int>((row_bytes - H - 4 * ngroups) / 4);
  const uint16_t* const x = static_cast<const uint16_t*>(a.x);
  char* rbase = static_cast<char*>(a.recv);
  u32x4 nx0 = {0u, 0u, 0u, 0u}, nx1 = {0u, 0u, 0u, 0u};
  auto load_step = [&](int64_t tt, int c) {
    const int el = c * (kWave * 16) + lane * 16;
    if (el < H) {
      const uint16_t* src = x + tt * H + el;
      nx0 = *reinterpret_cast<const u32x4*>(src);
      nx1 = *reinterpret_cast<const u32x4*>(src + 8);
    }
  };
  // convert step c of token t (inputs already in nx0/nx1), start the next
  // load, and file the step's group scales; returns the step's 16 codes
  float my_sc[kMaxScaleSlots];
  auto convert_step = [&](int64_t tt, int c) -> u32x4 {
    const int el = c * (kWave * 16) + lane * 16;
    const bool act = el < H;
    const u32x4 in0 = act ? nx0 : u32x4{0u, 0u, 0u, 0u};
    const u32x4 in1 = act ? nx1 : u32x4{0u, 0u, 0u, 0u};
    if (c + 1 < nsteps) load_step(tt, c + 1);
    else if (tt + nw < a.T) load_step(tt + nw, 0);
    float f[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_lo(in0[i]);
      f[2 * i + 1] = bf16_hi(in0[i]);
      f[8 + 2 * i] = bf16_lo(in1[i]);
      f[8 + 2 * i + 1] = bf16_hi(in1[i]);
    }
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(f[i]));
    am = fmaxf(am, __shfl_xor(am, 1, kWave));
    am = fmaxf(am, __shfl_xor(am, 2, kWave));
    am = fmaxf(am, __shfl_xor(am, 4, kWave));
    const float s = am / 448.0f;
    u32x4 q = {0u, 0u, 0u, 0u};
    if (s != 0.0f) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t lo = e4m3fn_sat_pair(f[4 * i] / s, f[4 * i + 1] / s);
        const uint32_t hi = e4m3fn_sat_pair(f[4 * i + 2] / s, f[4 * i + 3] / s);
        q[i] = lo | (hi << 16);
      }
    }
    // this step's groups are c*8 .. c*8+7; group c*8+g goes to lane
    // (c*8+g) % 64, which is lane (c%8)*8 + g, register slot c/8
    const float sc = __shfl(s, (lane & 7) * 8, kWave);
    const bool keep = (lane >> 3) == (c & 7);
#pragma unroll
    for (int r = 0; r < kMaxScaleSlots; ++r)
      if (keep && r == (c >> 3)) my_sc[r] = sc;
    return q;
  };
  bool have0 = false;  // step 0 of token t is loaded (by the previous token's last step)
  for (bool first = true; t < a.T; t += nw, first = false) {
    if (!first) load_dests<KMAX>(a, t, lane, d);
    if (!any_dest<KMAX>(d)) {
      have0 = false;
      continue;
    }
    if (!have0) load_step(t, 0);
#pragma unroll
    for (int r = 0; r < kMaxScaleSlots; ++r) my_sc[r] = 0.0f;
    u32x4 qrow[ROWBUF ? kRowSteps : 1];
    if constexpr (ROWBUF) {
#pragma unroll
      for (int c = 0; c < kRowSteps; ++c)
        if (c < nsteps) qrow[c] = convert_step(t, c);
    } else {
      for (int c = 0; c < nsteps; ++c) {
        const u32x4 q = convert_step(t, c);
        const int el = c * (kWave * 16) + lane * 16;
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
          if (d[j] < 0) continue;
          if (el < H) nt_store(q, reinterpret_cast<u32x4*>(rbase + static_cast<int64_t>(d[j]) * a.stride + el));
        }
      }
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (d[j] < 0) continue;
      char* row = rbase + static_cast<int64_t>(d[j]) * a.stride;
      if constexpr (ROWBUF) {
#pragma unroll
        for (int c = 0; c < kRowSteps; ++c) {
          const int el = c * (kWave * 16) + lane * 16;
          if (c < nsteps && el < H) nt_store(qrow[c], reinterpret_cast<u32x4*>(row + el));
        }
      }
      char* tail = row + H;
      // the scales, then the zero words to row_bytes, as one run of 4-byte
      // words: one store per 64 words (separate scale and padding stores
      // measured 104 against 99 us at hidden 7168)
#pragma unroll
      for (int r = 0; r <= kMaxScaleSlots; ++r) {
        const int i = r * kWave + lane;
        const uint32_t v = r < kMaxScaleSlots && i < ngroups ? __float_as_uint(my_sc[r < kMaxScaleSlots ? r : 0]) : 0u;
        if (i < ngroups + pad_words) nt_store(v, reinterpret_cast<uint32_t*>(tail) + i);
      }
    }
    have0 = t + nw < a.T;  // the last step loaded the next token's step 0
  }
}

// Zero the alignment padding rows [offsets[e] + counts[e], offsets[e+1]) of
// every expert: the PR's zero_padding, so each expert's A-aligned block
// holds its rows followed by zeros.  Blocks take experts in turn.
template <int VB>
__global__ __launch_bounds__(kBlock) void k_zero_padding(ScatterArgs a, int64_t row_bytes) {
  using V = typename VecOf<VB>::type;
  if (!dispatch_may_write(a)) return;
  const int nvec = static_cast<int>(row_bytes / VB);
  char* rbase = static_cast<char*>(a.recv);
  for (int e = blockIdx.x; e < a.E; e += gridDim.x) {
    const int r0 = a.offsets[e] + a.counts[e];
    const int r1 = a.offsets[e + 1];
    const int64_t n = static_cast<int64_t>(r1 - r0) * nvec;
    for (int64_t q = threadIdx.x; q < n; q += kBlock) {
      const int64_t r = r0 + q / nvec;
      const int v = static_cast<int>(q % nvec);
      nt_store(V{}, reinterpret_cast<V*>(rbase + r * a.stride) + v);
    }
  }
}

template <int KMAX, int VB>
hipError_t scatter_bf16_v(const ScatterArgs& a, hipStream_t s) {
  // One vector per lane per chunk and one wave per chunk: at hidden 7168,
  // top-8 of 256 this measured 185 us against 188 us for four vectors per
  // lane on the resident grid (and 1100 against 1170 us for the 65,536-token
  // grouped rows).
  constexpr int U = 1;
  const int nvec = static_cast<int>(static_cast<int64_t>(a.H) * 2 / VB);
  const int nchunks = (nvec + kWave * U - 1) / (kWave * U);
  const int64_t items = a.T * nchunks;
  // At most 6 blocks on a CU: each asks for 24 KiB of LDS it does not use,
  // so 6 fit in a CU's 160 KiB and 7 do not.  The 65,536-token grouped rows
  // took 946 us at 6 waves per SIMD against 1102 us at the 8 its registers
  // allow (994 at 5, 1119 at 4); 8192 tokens measured 186 against 187 us.
  constexpr size_t kOccupancyLds = 24576;
  k_scatter_bf16<KMAX, VB, U><<<wave_per_item_blocks(items), kBlock, kOccupancyLds, s>>>(a, nchunks, items);
  return hipGetLastError();
}

template <int KMAX>
hipError_t scatter_bf16_k(const ScatterArgs& a, int vb, hipStream_t s) {
  switch (vb) {
    case 16: return scatter_bf16_v<KMAX, 16>(a, s);
    case 8: return scatter_bf16_v<KMAX, 8>(a, s);
    case 4: return scatter_bf16_v<KMAX, 4>(a, s);
    default: return scatter_bf16_v<KMAX, 2>(a, s);
  }
}

// The row burst pays where rows share 128-byte lines with their neighbours
// (a pitch that is not a multiple of 128: each row starts and ends inside a
// line, and writing a whole row at once lets those partial lines combine);
// at a line-aligned pitch the step-by-step stores keep more waves resident
// and measured faster (hidden 7168: 126 vs 146 us at the packed 7392-byte
// pitch, 118 vs 112 us at 7424).
// One wave per token: at hidden 7168 the resident grid (six blocks per CU)
// left a third of its waves a second token, 109 us against 108 us.
template <int KMAX, bool ROWBUF>
void kern_launch_fp8(const ScatterArgs& a, int64_t row_bytes, hipStream_t s) {
  k_scatter_fp8<KMAX, ROWBUF><<<wave_per_item_blocks(a.T), kBlock, 0, s>>>(a, row_bytes);
}

template <int KMAX>
hipError_t scatter_fp8_k(const ScatterArgs& a, int64_t row_bytes, hipStream_t s) {
  if (a.H <= 8 * kWave * 16 && a.stride % 128 != 0) {
    kern_launch_fp8<KMAX, true>(a, row_bytes, s);
  } else {
    kern_launch_fp8<KMAX, false>(a, row_bytes, s);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scatter_bf16(const ScatterArgs& a, int vec_bytes, hipStream_t s) {
  if (a.K <= 1) return scatter_bf16_k<1>(a, vec_bytes, s);
  if (a.K <= 2) return scatter_bf16_k<2>(a, vec_bytes, s);
  if (a.K <= 4) return scatter_bf16_k<4>(a, vec_bytes, s);
  if (a.K <= 8) return scatter_bf16_k<8>(a, vec_bytes, s);
  if (a.K <= 16) return scatter_bf16_k<16>(a, vec_bytes, s);
  return scatter_bf16_k<32>(a, vec_bytes, s);
}

hipError_t launch_zero_padding(const ScatterArgs& a, int64_t row_bytes, int vec_bytes,
                               hipStream_t s) {
  const unsigned grid = static_cast<unsigned>(a.E < 1024 ? a.E : 1024);
  switch (vec_bytes) {
    case 16: k_zero_padding<16><<<grid, kBlock, 0, s>>>(a, row_bytes); break;
    case 8: k_zero_padding<8><<<grid, kBlock, 0, s>>>(a, row_bytes); break;
    case 4: k_zero_padding<4><<<grid, kBlock, 0, s>>>(a, row_bytes); break;
    default: k_zero_padding<2><<<grid, kBlock, 0, s>>>(a, row_bytes); break;
  }
  return hipGetLastError();
}

hipError_t launch_scatter_fp8(const ScatterArgs& a, int64_t row_bytes, hipStream_t s) {
  if (a.K <= 1) return scatter_fp8_k<1>(a, row_bytes, s);
  if (a.K <= 2) return scatter_fp8_k<2>(a, row_bytes, s);
  if (a.K <= 4) return scatter_fp8_k<4>(a, row_bytes, s);
  if (a.K <= 8) return scatter_fp8_k<8>(a, row_bytes, s);
  if (a.K <= 16) return scatter_fp8_k<16>(a, row_bytes, s);
  return scatter_fp8_k<32>(a, row_bytes, s);
}

}  // namespace ep
