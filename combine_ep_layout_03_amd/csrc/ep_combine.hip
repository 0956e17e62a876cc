// Combine: gather each source token's expert-output rows and reduce them,
// the one-block-per-source-token local reduce of TileScale PR #68 (PR
// summary; Design section).  Rows are found through the forward map
// slot[t,k] the layout wrote, so no inverse bucketing is needed on one GPU.
//
// Arithmetic (exactly what the reduction order defines, no fused
// multiply-add): acc starts at +0, each term is fl32(w * y) and each sum is
// fl32(acc + term).  Flat order: ascending k.  Grouped order: the token's
// rows inside one expert group are summed first in ascending k, then the
// group partials in ascending group order: the order of the expanded
// combine, which adds up the rows a token has on one destination's experts
// before that destination's single row goes out (commit adding
// kDoExpandedSend).  Masked entries (-1) are skipped, so a fully
// masked token gives +0 (commit on masked topk_idx).  An optional bias (one
// or two bf16 rows per token) seeds the accumulator instead of +0, so a fully
// masked token returns its bias (commit adding receive stats and combine
// bias); in the grouped order it seeds the cross-group total.
//
// Work split: a token row is cut into chunks of 64 vectors (one per lane),
// and the grid's waves take the (token, chunk) items cyclically, so the tokens in
// flight at any moment are neighbours and their rows inside each expert
// segment are neighbours too.  The grid gives every item its own wave: the
// hardware then starts blocks in item order as others finish, which keeps
// the window of tokens in flight tightest.  Measured on MI355X at hidden
// 7168, top-8 of 256: 200 us with contiguous per-wave ranges on a resident
// grid (concurrent reads span the whole expert-output buffer), 195 us with
// the cyclic walk on that grid, 183.5 us with one wave per item.
// Expert-output rows are read exactly once, with non-temporal buffer loads,
// and output rows are written with non-temporal stores: with the
// token-ordered window this measured the same for the flat order and 5-9%
// faster for the grouped order (1569 -> 1435 us at 65,536 tokens).
#include <limits.h>

#include "ep_device.h"
#include "ep_internal.h"
#include "ep_launch.h"

namespace ep {

namespace {

template <int VE>
struct BfVec;
template <>
struct BfVec<8> {
  using V = u32x4;
  __device__ static float get(const V& v, int e) {
    return (e & 1) ? bf16_hi(v[e >> 1]) : bf16_lo(v[e >> 1]);
  }
  __device__ static V pack(const float (&f)[8]) {
    V r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    return r;
  }
};
template <>
struct BfVec<4> {
  using V = u32x2;
  __device__ static float get(const V& v, int e) {
    return (e & 1) ? bf16_hi(v[e >> 1]) : bf16_lo(v[e >> 1]);
  }
  __device__ static V pack(const float (&f)[4]) {
    V r;
    r[0] = pack_bf16x2(f[0], f[1]);
    r[1] = pack_bf16x2(f[2], f[3]);
    return r;
  }
};
template <>
struct BfVec<2> {
  using V = uint32_t;
  __device__ static float get(const V& v, int e) { return e ? bf16_hi(v) : bf16_lo(v); }
  __device__ static V pack(const float (&f)[2]) { return pack_bf16x2(f[0], f[1]); }
};
template <>
struct BfVec<1> {
  using V = uint16_t;
  __device__ static float get(const V& v, int) { return bf16_to_f32(v); }
  __device__ static V pack(const float (&f)[1]) {
    return static_cast<uint16_t>(f32_to_bf16_bits(f[0]));
  }
};

// A token's valid selections in summation order, wave-uniform.
template <int KMAX>
struct Sel {
  int nv;           // number of valid selections
  int os[KMAX];     // receive rows; entries past nv repeat a valid row
  float ow[KMAX];   // weights
  bool newg[KMAX];  // position i starts a new group (never position 0)
};

template <int KMAX, bool GROUPED>
__device__ __forceinline__ void load_sel(const CombineArgs& a, int64_t t, int lane, Sel<KMAX>& m) {
  const int K = a.K;
  int s = -1;
  float wt = 0.0f;
  int g = 0;
  if (lane < K) {
    s = a.slot[t * K + lane];
    if (s >= 0 && static_cast<int64_t>(s) >= a.y_rows) {
      a.status[4] = 1;  // out-of-range row: skipped, reported
      s = -1;
    }
    wt = a.w[t * K + lane];
    if (GROUPED && s >= 0) g = static_cast<int>(a.idx[t * K + lane]) / a.epg;
  }
  const bool valid = s >= 0;
  const uint64_t vmask = ballot(valid);
  m.nv = __popcll(vmask);
  // rank of each valid selection in summation order: (group, k) ascending
  int rank;
  if (GROUPED) {
    rank = 0;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      const int gj = __shfl(g, j, kWave);
      const bool vj = (vmask >> j) & 1ull;
      if (vj && (gj < g || (gj == g && j < lane))) ++rank;
    }
  } else {
    rank = __popcll(vmask & lanemask_lt());
  }
  int gprev = INT_MIN;
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    const uint64_t mk = ballot(valid && rank == (i < m.nv ? i : 0));
    const int L = mk ? static_cast<int>(__builtin_ctzll(mk)) : 0;
    m.os[i] = readlane(s, L);
    m.ow[i] = __int_as_float(readlane(__float_as_int(wt), L));
    const int gi = readlane(g, L);
    m.newg[i] = i > 0 && gi != gprev;
    gprev = gi;
  }
}

// The accumulator's starting value for element e of a vector: +0, or the
// bias (one or two bf16 rows, summed in fp32).
template <int VE, int NB>
__device__ __forceinline__ float bias_seed(const typename BfVec<VE>::V (&b)[2], int e) {
  using B = BfVec<VE>;
  if (NB == 0) return 0.0f;
  if (NB == 1) return B::get(b[0], e);
  return __fadd_rn(B::get(b[0], e), B::get(b[1], e));
}

template <int VE, int NB>
__device__ __forceinline__ void load_bias(const CombineArgs& a, int64_t t, int nvec, int vi,
                                          typename BfVec<VE>::V (&b)[2]) {
  using V = typename BfVec<VE>::V;
  const int64_t off = t * nvec + vi;
  b[0] = NB >= 1 ? static_cast<const V*>(a.bias0 ? a.bias0 : a.bias1)[off] : V{};
  b[1] = NB >= 2 ? static_cast<const V*>(a.bias1)[off] : V{};
}

// One chunk: U vectors per lane of the token's output row.
template <int KMAX, int VE, bool GROUPED, int U, bool FULL, int NB>
__device__ __forceinline__ void reduce_chunk(const CombineArgs& a, int64_t t,
                                             const typename BfVec<VE>::V* __restrict__ yv,
                                             typename BfVec<VE>::V* __restrict__ outv, int nvec,
                                             int vb, int lane, const Sel<KMAX>& m) {
  using B = BfVec<VE>;
  using V = typename B::V;
  V in[U][KMAX];
  V bias[U][2];
  // Each row is a buffer resource with a wave-uniform base (scalar
  // registers); the in-row byte offset is one 32-bit vector register shared
  // by all K loads.  A row is H * 2 < 2^32 bytes.  A position past the valid
  // count gets a zero-length resource: its load returns zeros without a
  // memory access, and the reduction never reads it.
  const uint32_t row_bytes = static_cast<uint32_t>(nvec) * static_cast<uint32_t>(sizeof(V));
  __amdgpu_buffer_rsrc_t rows[KMAX];
#pragma unroll
  for (int i = 0; i < KMAX; ++i)
    rows[i] = buffer_rsrc(reinterpret_cast<const char*>(yv) + static_cast<int64_t>(m.os[i]) * row_bytes,
                          FULL || i < m.nv ? row_bytes : 0u);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int vi = min(vb + u * kWave + lane, nvec - 1);
    if (NB > 0) load_bias<VE, NB>(a, t, nvec, vi, bias[u]);
    const uint32_t boff = static_cast<uint32_t>(vi) * static_cast<uint32_t>(sizeof(V));
#pragma unroll
    for (int i = 0; i < KMAX; ++i) in[u][i] = buffer_load_nt<V>(rows[i], boff);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float res[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      // flat: acc = seed, then acc += w*y;  grouped: tot = seed, P per group
      float tot = bias_seed<VE, NB>(bias[u], e);
      float P = GROUPED ? 0.0f : tot;
#pragma unroll
      for (int i = 0; i < KMAX; ++i) {
        if (FULL || i < m.nv) {
          if (GROUPED && m.newg[i]) {
            tot = __fadd_rn(tot, P);
            P = 0.0f;
          }
          P = __fadd_rn(P, __fmul_rn(m.ow[i], B::get(in[u][i], e)));
        }
      }
      res[e] = GROUPED ? __fadd_rn(tot, P) : P;
    }
    const int vi = vb + u * kWave + lane;
    if (vi < nvec) nt_store(B::pack(res), outv + vi);
  }
}

// A token with no valid selection: the bias seed (grouped: seed + 0, as the
// cross-group total adds the empty partials), or +0 without a bias.
template <int VE, bool GROUPED, int U, int NB>
__device__ __forceinline__ void empty_chunk(const CombineArgs& a, int64_t t,
                                            typename BfVec<VE>::V* __restrict__ outv, int nvec,
                                            int vb, int lane) {
  using B = BfVec<VE>;
  using V = typename B::V;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int vi = vb + u * kWave + lane;
    if (vi >= nvec) continue;
    V bias[2];
    if (NB > 0) load_bias<VE, NB>(a, t, nvec, vi, bias);
    float res[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      const float seed = bias_seed<VE, NB>(bias, e);
      res[e] = GROUPED ? __fadd_rn(seed, 0.0f) : seed;
    }
    nt_store(B::pack(res), outv + vi);
  }
}

// BT threads per block (256, or 64: one wave per block).
template <int KMAX, int VE, bool GROUPED, int U, int NB, int BT>
__global__ __launch_bounds__(BT) void k_combine(CombineArgs a, int nchunks, int64_t items) {
  using B = BfVec<VE>;
  using V = typename B::V;
  // The generation check, the slot load and the weight load run in sequence.
  // Issuing all three at once (two round trips fewer per wave) measured
  // slower at hidden 7168, top-8 of 256: flat 177 -> 182 us, grouped order
  // over 65,536 tokens 1442 -> 1571 us.
  if (!layout_current(a.status, a.generation)) return;  // stale handle: write nothing
  constexpr int kWaves = BT / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t nw = static_cast<int64_t>(gridDim.x) * kWaves;
  const int nvec = a.H / VE;
  const V* yv = static_cast<const V*>(a.y);
  Sel<KMAX> m;
  int64_t loaded = -1;
  const int64_t w0 = static_cast<int64_t>(blockIdx.x) * kWaves +
                     (kWaves == 1 ? 0 : __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave));
  for (int64_t it = w0; it < items; it += nw) {
    const int64_t t = it / nchunks;
    const int c = static_cast<int>(it - t * nchunks);
    if (t != loaded) {
      load_sel<KMAX, GROUPED>(a, t, lane, m);
      loaded = t;
    }
    V* outv = static_cast<V*>(a.out) + t * nvec;
    const int vb = c * (kWave * U);
    if (m.nv == KMAX) {
      reduce_chunk<KMAX, VE, GROUPED, U, true, NB>(a, t, yv, outv, nvec, vb, lane, m);
    } else if (m.nv > 0) {
      reduce_chunk<KMAX, VE, GROUPED, U, false, NB>(a, t, yv, outv, nvec, vb, lane, m);
    } else {
      empty_chunk<VE, GROUPED, U, NB>(a, t, outv, nvec, vb, lane);
    }
  }
}

template <int KMAX, int VE, bool GROUPED, int NB>
hipError_t combine_v(const CombineArgs& a, hipStream_t s) {
  // one vector per lane per row: 2 per lane measured 186 against 183.5 us
  // (hidden 7168, top-8 of 256)
  constexpr int U = 1;
  const int nvec = a.H / VE;
  const int nchunks = (nvec + kWave * U - 1) / (kWave * U);
  const int64_t items = a.T * nchunks;
  // With 8 or more rows per token the flat order runs best with at most 5
  // waves per SIMD: hidden 7168, top-8 of 256: 178.5 us at 5, 181.5 at 6,
  // 183.2 at the 8 its registers allow.  The cap is unused LDS, and the
  // blocks are single waves (8000 bytes each, 20 to a CU), so a finished
  // wave frees its place at once instead of waiting for its block's other
  // waves: 174.9 against 176.7 us with 4-wave blocks of 29 KiB, two biases
  // 185.1 against 188.0 us.  At 4 waves per SIMD (16 blocks of 10 KiB) the
  // bench shape gains another 1.0 us but the skewed, masked routing loses
  // 4.6 us (162.9 against 158.3), so 5 it stays.  With fewer rows per token
  // fewer rows are open per wave, and the cap costs: hidden 4096, top-4 of
  // 64, 4096 tokens, cold caches: 35.7 us capped, 33.0 uncapped.  The
  // grouped order is best uncapped in 4-wave blocks (4 waves per SIMD: 1528
  // against 1437 us at 65,536 tokens; single-wave blocks 1474 us).
  if (!GROUPED && a.K >= 8) {
    constexpr auto kern = k_combine<KMAX, VE, GROUPED, U, NB, kWave>;
    kern<<<wave_per_item_blocks(items, 1), kWave, 8000, s>>>(a, nchunks, items);
  } else {
    constexpr auto kern = k_combine<KMAX, VE, GROUPED, U, NB, kBlock>;
    kern<<<wave_per_item_blocks(items), kBlock, 0, s>>>(a, nchunks, items);
  }
  return hipGetLastError();
}

template <int KMAX, int VE, bool GROUPED>
hipError_t combine_b(const CombineArgs& a, hipStream_t s) {
  const int nb = (a.bias0 ? 1 : 0) + (a.bias1 ? 1 : 0);
  if (nb == 0) return combine_v<KMAX, VE, GROUPED, 0>(a, s);
  if (nb == 1) return combine_v<KMAX, VE, GROUPED, 1>(a, s);
  return combine_v<KMAX, VE, GROUPED, 2>(a, s);
}

template <int KMAX, bool GROUPED>
hipError_t combine_k(const CombineArgs& a, int ve, hipStream_t s) {
  switch (ve) {
    case 8: return combine_b<KMAX, 8, GROUPED>(a, s);
    case 4: return combine_b<KMAX, 4, GROUPED>(a, s);
    case 2: return combine_b<KMAX, 2, GROUPED>(a, s);
    default: return combine_b<KMAX, 1, GROUPED>(a, s);
  }
}

template <bool GROUPED>
hipError_t combine_g(const CombineArgs& a, int ve, hipStream_t s) {
  if (a.K <= 1) return combine_k<1, GROUPED>(a, ve, s);
  if (a.K <= 2) return combine_k<2, GROUPED>(a, ve, s);
  if (a.K <= 4) return combine_k<4, GROUPED>(a, ve, s);
  if (a.K <= 8) return combine_k<8, GROUPED>(a, ve, s);
  if (a.K <= 16) return combine_k<16, GROUPED>(a, ve, s);
  return combine_k<32, GROUPED>(a, ve, s);
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, int vec_elems, hipStream_t s) {
  return a.grouped ? combine_g<true>(a, vec_elems, s) : combine_g<false>(a, vec_elems, s);
}

}  // namespace ep
