// Combine: one wave per source token gathers the token's expert-output rows
// and reduces them, the one-block-per-source-token local reduce of TileScale
// PR #68 (PR summary; Design section).  Rows are found through the forward
// map slot[t,k] the layout wrote, so no inverse bucketing is needed on one
// GPU.
//
// Arithmetic (exactly what the reduction order defines, no fused
// multiply-add): acc starts at +0, each term is fl32(w * y) and each sum is
// fl32(acc + term).  Flat order: ascending k.  Grouped order: the token's
// rows inside one expert group are summed first in ascending k, then the
// group partials in ascending group order, as the expanded combine sums a
// token's local-expert rows before one row per destination is sent (commit
// adding kDoExpandedSend).  Masked entries (-1) are skipped, so a fully
// masked token gives +0 (commit on masked topk_idx).
#include <limits.h>

#include "ep_device.h"
#include "ep_internal.h"

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

template <int KMAX, int VE, bool GROUPED, int U>
__global__ __launch_bounds__(kBlock) void k_combine(CombineArgs a) {
  using B = BfVec<VE>;
  using V = typename B::V;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave;
  if (t >= a.T) return;
  const int K = a.K;

  // Per-lane selection k = lane.
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
  const int nv = __popcll(vmask);

  // Rank of each valid selection in summation order: (group, k) ascending.
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

  // The ordered list, wave-uniform.  Positions past nv repeat the first row
  // (loads stay in bounds and branch-free) and are never accumulated.
  int os[KMAX];
  float ow[KMAX];
  bool newg[KMAX];
  int gprev = INT_MIN;
#pragma unroll
  for (int i = 0; i < KMAX; ++i) {
    const uint64_t m = ballot(valid && rank == (i < nv ? i : 0));
    const int L = m ? static_cast<int>(__builtin_ctzll(m)) : 0;
    os[i] = readlane(s, L);
    ow[i] = __int_as_float(readlane(__float_as_int(wt), L));
    const int gi = readlane(g, L);
    newg[i] = i > 0 && gi != gprev;
    gprev = gi;
  }

  const int nvec = a.H / VE;
  const V* yv = static_cast<const V*>(a.y);
  V* outv = static_cast<V*>(a.out) + t * nvec;
  if (nv == 0) {
    const float zf[VE] = {};
    const V z = B::pack(zf);
    for (int vi = lane; vi < nvec; vi += kWave) outv[vi] = z;
    return;
  }
  for (int v0 = 0; v0 < nvec; v0 += kWave * U) {
    V in[U][KMAX];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int vi = min(v0 + u * kWave + lane, nvec - 1);
#pragma unroll
      for (int i = 0; i < KMAX; ++i) in[u][i] = yv[static_cast<int64_t>(os[i]) * nvec + vi];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float res[VE];
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        float tot = 0.0f, P = 0.0f;
#pragma unroll
        for (int i = 0; i < KMAX; ++i) {
          if (i < nv) {
            if (GROUPED && newg[i]) {
              tot = __fadd_rn(tot, P);
              P = 0.0f;
            }
            P = __fadd_rn(P, __fmul_rn(ow[i], B::get(in[u][i], e)));
          }
        }
        res[e] = GROUPED ? __fadd_rn(tot, P) : P;
      }
      const int vi = v0 + u * kWave + lane;
      if (vi < nvec) outv[vi] = B::pack(res);
    }
  }
}

template <int KMAX, bool GROUPED>
hipError_t combine_k(const CombineArgs& a, int ve, dim3 grid, hipStream_t s) {
  // two row chunks in flight per lane while the K loads stay within registers
  constexpr int U = KMAX <= 8 ? 2 : 1;
  switch (ve) {
    case 8: k_combine<KMAX, 8, GROUPED, U><<<grid, kBlock, 0, s>>>(a); break;
    case 4: k_combine<KMAX, 4, GROUPED, U><<<grid, kBlock, 0, s>>>(a); break;
    case 2: k_combine<KMAX, 2, GROUPED, U><<<grid, kBlock, 0, s>>>(a); break;
    default: k_combine<KMAX, 1, GROUPED, U><<<grid, kBlock, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

template <bool GROUPED>
hipError_t combine_g(const CombineArgs& a, int ve, dim3 grid, hipStream_t s) {
  if (a.K <= 1) return combine_k<1, GROUPED>(a, ve, grid, s);
  if (a.K <= 2) return combine_k<2, GROUPED>(a, ve, grid, s);
  if (a.K <= 4) return combine_k<4, GROUPED>(a, ve, grid, s);
  if (a.K <= 8) return combine_k<8, GROUPED>(a, ve, grid, s);
  if (a.K <= 16) return combine_k<16, GROUPED>(a, ve, grid, s);
  return combine_k<32, GROUPED>(a, ve, grid, s);
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, int vec_elems, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((a.T + kWavesPerBlock - 1) / kWavesPerBlock));
  return a.grouped ? combine_g<true>(a, vec_elems, grid, s)
                   : combine_g<false>(a, vec_elems, grid, s);
}

}  // namespace ep
