// Dispatch: scatter each token row straight to its final receive rows.
//
// TileScale PR #68 ("EP v2 intranode dispatch/combine") writes every row at
// send_base[d] + slot, its final compact index, so there is no copy
// epilogue (PR summary; Design section).  One wave moves one token: the row
// is read from HBM once into registers and stored once per destination row,
// in 16-byte vectors when the row size and base alignment allow, otherwise
// in the widest vector that divides both, so no remainder tail can be
// dropped (the pages' copy-tail fix in the commit on cp_warp_impl).
//
// The fp8 variant fuses DeepEP's per-token, per-128-element cast into the
// same pass and writes payload, scales and padding of the packed row in one
// sweep per destination (commit packing payload and scales into one row).
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {

namespace {

// Destination rows of token t, wave-uniform (scalar registers).  With
// `dedup`, later k that repeat an earlier row are dropped.
template <int KMAX>
__device__ __forceinline__ void load_dests(const ScatterArgs& a, int64_t t, int lane,
                                           int (&d)[KMAX]) {
  const int dl = lane < a.K ? a.dest[t * a.K + lane] : -1;
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

template <int KMAX, int VB, int U>
__global__ __launch_bounds__(kBlock) void k_scatter_bf16(ScatterArgs a) {
  using V = typename VecOf<VB>::type;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave;
  if (t >= a.T) return;
  if (static_cast<int64_t>(*a.rows_needed) > a.capacity) return;  // overflow: write nothing

  int d[KMAX];
  load_dests<KMAX>(a, t, lane, d);

  const int64_t row_bytes = static_cast<int64_t>(a.H) * 2;
  const int nvec = static_cast<int>(row_bytes / VB);
  const V* src = reinterpret_cast<const V*>(static_cast<const char*>(a.x) + t * row_bytes);
  char* rbase = static_cast<char*>(a.recv);
  for (int v0 = 0; v0 < nvec; v0 += kWave * U) {
    V val[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int vi = v0 + u * kWave + lane;
      val[u] = vi < nvec ? src[vi] : V{};
    }
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (d[j] < 0) continue;
      V* dst = reinterpret_cast<V*>(rbase + static_cast<int64_t>(d[j]) * row_bytes);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int vi = v0 + u * kWave + lane;
        if (vi < nvec) dst[vi] = val[u];
      }
    }
  }
}

// Packed fp8 row, per 128-element group j of the token:
//   a_j = max |x| (exact), s_j = a_j / 448 (IEEE fp32 division),
//   q = E4M3FN_rne_sat(x / s_j) (IEEE fp32 division), or q = 0 when s_j == 0;
// bytes: q[0..H) | s_0 .. s_{H/128-1} (fp32, little-endian) | zeros to row_bytes.
// Each lane owns 16 consecutive elements, so 8 lanes form one group and a
// wave covers 1024 elements per step; H % 128 == 0 keeps every group's 8
// lanes together and active.
template <int KMAX>
__global__ __launch_bounds__(kBlock) void k_scatter_fp8(ScatterArgs a, int64_t row_bytes) {
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave;
  if (t >= a.T) return;
  if (static_cast<int64_t>(*a.rows_needed) > a.capacity) return;

  int d[KMAX];
  load_dests<KMAX>(a, t, lane, d);

  const int H = a.H;
  const uint16_t* xr = static_cast<const uint16_t*>(a.x) + t * H;
  char* rbase = static_cast<char*>(a.recv);
  for (int e0 = 0; e0 < H; e0 += kWave * 16) {
    const int el = e0 + lane * 16;
    const bool act = el < H;
    u32x4 in0 = {0u, 0u, 0u, 0u}, in1 = {0u, 0u, 0u, 0u};
    if (act) {
      in0 = *reinterpret_cast<const u32x4*>(xr + el);
      in1 = *reinterpret_cast<const u32x4*>(xr + el + 8);
    }
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
      for (int i = 0; i < 16; ++i) q[i >> 2] |= f32_to_e4m3fn_sat(f[i] / s) << (8 * (i & 3));
    }
    const bool scale_lane = act && (lane & 7) == 0;
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (d[j] < 0) continue;
      char* row = rbase + static_cast<int64_t>(d[j]) * row_bytes;
      if (act) *reinterpret_cast<u32x4*>(row + el) = q;
      if (scale_lane) *reinterpret_cast<float*>(row + H + 4 * (el / 128)) = s;
    }
  }
  // zero padding after the scales (a multiple of 4 bytes, under 16)
  const int pad_words = static_cast<int>((row_bytes - H - 4 * (H / 128)) / 4);
  if (lane < pad_words) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      if (d[j] < 0) continue;
      char* row = rbase + static_cast<int64_t>(d[j]) * row_bytes;
      reinterpret_cast<uint32_t*>(row + H + 4 * (H / 128))[lane] = 0u;
    }
  }
}

template <int KMAX>
hipError_t scatter_bf16_k(const ScatterArgs& a, int vb, dim3 grid, hipStream_t s) {
  switch (vb) {
    case 16: k_scatter_bf16<KMAX, 16, 4><<<grid, kBlock, 0, s>>>(a); break;
    case 8: k_scatter_bf16<KMAX, 8, 4><<<grid, kBlock, 0, s>>>(a); break;
    case 4: k_scatter_bf16<KMAX, 4, 4><<<grid, kBlock, 0, s>>>(a); break;
    default: k_scatter_bf16<KMAX, 2, 4><<<grid, kBlock, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scatter_bf16(const ScatterArgs& a, int vec_bytes, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((a.T + kWavesPerBlock - 1) / kWavesPerBlock));
  if (a.K <= 1) return scatter_bf16_k<1>(a, vec_bytes, grid, s);
  if (a.K <= 2) return scatter_bf16_k<2>(a, vec_bytes, grid, s);
  if (a.K <= 4) return scatter_bf16_k<4>(a, vec_bytes, grid, s);
  if (a.K <= 8) return scatter_bf16_k<8>(a, vec_bytes, grid, s);
  if (a.K <= 16) return scatter_bf16_k<16>(a, vec_bytes, grid, s);
  return scatter_bf16_k<32>(a, vec_bytes, grid, s);
}

hipError_t launch_scatter_fp8(const ScatterArgs& a, int64_t row_bytes, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((a.T + kWavesPerBlock - 1) / kWavesPerBlock));
  if (a.K <= 1) k_scatter_fp8<1><<<grid, kBlock, 0, s>>>(a, row_bytes);
  else if (a.K <= 2) k_scatter_fp8<2><<<grid, kBlock, 0, s>>>(a, row_bytes);
  else if (a.K <= 4) k_scatter_fp8<4><<<grid, kBlock, 0, s>>>(a, row_bytes);
  else if (a.K <= 8) k_scatter_fp8<8><<<grid, kBlock, 0, s>>>(a, row_bytes);
  else if (a.K <= 16) k_scatter_fp8<16><<<grid, kBlock, 0, s>>>(a, row_bytes);
  else k_scatter_fp8<32><<<grid, kBlock, 0, s>>>(a, row_bytes);
  return hipGetLastError();
}

}  // namespace ep
