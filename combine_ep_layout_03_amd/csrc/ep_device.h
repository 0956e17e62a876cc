// Device helpers shared by the dispatch / combine kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ep {

constexpr int kWave = 64;
constexpr int kBlock = 256;  // threads per block for every kernel here
constexpr int kWavesPerBlock = kBlock / kWave;

// ---------------------------------------------------------------- bf16 / fp32
__device__ __forceinline__ float bf16_lo(uint32_t two) {  // element 0 of a packed pair
  return __uint_as_float(two << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t two) {  // element 1 of a packed pair
  return __uint_as_float(two & 0xFFFF0000u);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, round to nearest, ties to even.  Adding 0x7FFF plus the
// lowest kept bit to the pattern carries into the kept half exactly when the
// dropped half exceeds one half ulp, or equals it with an odd kept half.
// Finite inputs only (the sums here are finite); overflow yields infinity.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// ---------------------------------------------------------------- E4M3FN
// fp32 -> OCP E4M3FN code, round to nearest even, saturating at 448.
//   |v| >= 448             -> 0x7E (largest finite; the format has no inf)
//   |v| <  2^-6 (subnormal) -> round(|v| * 2^9) to an integer k in [0, 8];
//                              k is the code (k = 8 is 2^-6, the first normal)
//   otherwise               -> keep 3 mantissa bits, rounding on the 20
//                              dropped bits, and rebias the exponent 127 -> 7
// The sign bit is copied, so negative values rounding to zero give 0x80.
// NaN is outside the domain.
__device__ __forceinline__ uint32_t f32_to_e4m3fn_sat(float v) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t sign = (b >> 24) & 0x80u;
  const uint32_t m = b & 0x7FFFFFFFu;
  // all three candidates, then a select (no divergent branches); the
  // subnormal candidate is only chosen below 2^-6, where |v| * 2^9 < 8, and
  // the clamp keeps the conversion defined everywhere else
  const uint32_t sub =
      static_cast<uint32_t>(__builtin_rintf(fminf(__uint_as_float(m) * 512.0f, 16.0f)));
  const uint32_t nrm = ((m + 0x7FFFFu + ((m >> 20) & 1u)) >> 20) - (120u << 3);
  uint32_t code = m < 0x3C800000u ? sub : nrm;  // 2^-6
  code = m >= 0x43E00000u ? 0x7Eu : code;       // 448.0f
  return code | sign;
}

// Hardware conversion of two fp32 values to E4M3FN codes (gfx950
// v_cvt_pk_fp8_f32, round to nearest even, OCP encoding).  Magnitudes are
// clamped to 448 first (keeping the sign, also of -0.0), which gives the
// saturating conversion above for every non-NaN input; an exhaustive test
// over all 2^32 fp32 patterns checks this against f32_to_e4m3fn_sat.
__device__ __forceinline__ uint32_t e4m3fn_sat_pair(float a, float b) {
  const float ca = __builtin_copysignf(fminf(fabsf(a), 448.0f), a);
  const float cb = __builtin_copysignf(fminf(fabsf(b), 448.0f), b);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(ca, cb, 0, false)) & 0xFFFFu;
}

// ---------------------------------------------------------------- wave utils
__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

__device__ __forceinline__ int readlane(int v, int l) { return __builtin_amdgcn_readlane(v, l); }

template <typename T>
__device__ __forceinline__ T nt_load(const T* p) {
  return __builtin_nontemporal_load(p);
}
template <typename T>
__device__ __forceinline__ void nt_store(T v, T* p) {
  __builtin_nontemporal_store(v, p);
}

// Cyclic work split: wave w of the grid's nw waves takes items w, w + nw,
// w + 2 nw, ...  At any moment the grid works on a window of about nw
// consecutive items, so the rows that tokens next to each other read or
// write (neighbours inside each expert segment) are in flight together.
// The wave index is read from the first lane so the compiler knows it is
// wave-uniform: items, tokens and row bases derived from it then live in
// scalar registers.
__device__ __forceinline__ int64_t global_wave() {
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  return static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + w;
}
__device__ __forceinline__ int64_t grid_waves() {
  return static_cast<int64_t>(gridDim.x) * kWavesPerBlock;
}

// Vectors used for row copies (clang extended vectors: one global
// load/store instruction each).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Raw buffer resource over `bytes` bytes at `p` (byte offsets, no stride;
// word 3 selects 32-bit data format, as gfx9-family raw loads expect).  A
// wave-uniform base lives in four scalar registers, so K loads from K rows
// share one 32-bit vector offset instead of K 64-bit vector addresses.
// Loads at offsets past `bytes` return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes),
                                           0x00020000);
}

// Non-temporal buffer loads of 16, 8, 4 and 2 bytes at byte offset `off`.
template <typename T>
__device__ __forceinline__ T buffer_load_nt(__amdgpu_buffer_rsrc_t r, uint32_t off);
template <>
__device__ __forceinline__ u32x4 buffer_load_nt<u32x4>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 2);
}
template <>
__device__ __forceinline__ u32x2 buffer_load_nt<u32x2>(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, static_cast<int>(off), 0, 2);
}
template <>
__device__ __forceinline__ uint32_t buffer_load_nt<uint32_t>(__amdgpu_buffer_rsrc_t r,
                                                             uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(off), 0, 2);
}
template <>
__device__ __forceinline__ uint16_t buffer_load_nt<uint16_t>(__amdgpu_buffer_rsrc_t r,
                                                             uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, static_cast<int>(off), 0, 2);
}

template <int N>
struct VecOf;
template <>
struct VecOf<16> {
  using type = u32x4;
};
template <>
struct VecOf<8> {
  using type = u32x2;
};
template <>
struct VecOf<4> {
  using type = uint32_t;
};
template <>
struct VecOf<2> {
  using type = uint16_t;
};

// Exclusive scan of a[0..n) in LDS, n <= 1024, by a block of NT threads
// (NT a multiple of 64 dividing 1024).  tmp holds NT / 64 ints.  Returns the
// total.  Every thread of the block must call it: it contains barriers.
template <int NT = kBlock>
__device__ __forceinline__ int block_exclusive_scan(int* a, int n, int* tmp) {
  constexpr int kItems = 1024 / NT;
  constexpr int kWaves = NT / kWave;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int i0 = tid * kItems;
  int v[kItems];
  int s = 0;
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    v[j] = (i0 + j < n) ? a[i0 + j] : 0;
    s += v[j];
  }
  int x = s;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  if (lane == kWave - 1) tmp[wave] = x;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const int t = tmp[w];
    if (w < wave) before += t;
    total += t;
  }
  int run = before + x - s;
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    if (i0 + j < n) {
      a[i0 + j] = run;
      run += v[j];
    }
  }
  __syncthreads();
  return total;
}

}  // namespace ep
