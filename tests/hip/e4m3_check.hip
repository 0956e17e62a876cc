// Test-only library: exposes the product's two E4M3FN encoders (the
// hardware pair conversion used by the fp8 dispatch, and the software
// round-to-nearest-even saturating encoder it is checked against) so the
// GPU tests can compare them exhaustively and against the CPU oracle.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ep_device.h"

namespace {

// Every fp32 bit pattern except NaN: thread i checks patterns [64 i, 64 i + 64).
__global__ void k_exhaustive(unsigned long long* nbad, uint32_t* first) {
  const uint64_t tid = blockIdx.x * static_cast<uint64_t>(blockDim.x) + threadIdx.x;
  for (int j = 0; j < 64; j += 2) {
    const uint32_t b0 = static_cast<uint32_t>(tid * 64 + j);
    const uint32_t b1 = b0 + 1;
    const float v0 = __uint_as_float(b0), v1 = __uint_as_float(b1);
    const uint32_t hw = ep::e4m3fn_sat_pair(v0, v1);
    const bool nan0 = (b0 & 0x7FFFFFFFu) > 0x7F800000u;
    const bool nan1 = (b1 & 0x7FFFFFFFu) > 0x7F800000u;
    const uint32_t s0 = ep::f32_to_e4m3fn_sat(v0), s1 = ep::f32_to_e4m3fn_sat(v1);
    if (!nan0 && (hw & 0xFFu) != s0) {
      const unsigned long long k = atomicAdd(nbad, 1ull);
      if (k < 8) first[k] = b0;
    }
    if (!nan1 && (hw >> 8) != s1) {
      const unsigned long long k = atomicAdd(nbad, 1ull);
      if (k < 8) first[k] = b1;
    }
  }
}

__global__ void k_convert(const float* in, uint8_t* out, int64_t n) {
  const int64_t i = (blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x) * 2;
  if (i + 1 < n) {
    const uint32_t c = ep::e4m3fn_sat_pair(in[i], in[i + 1]);
    out[i] = static_cast<uint8_t>(c & 0xFFu);
    out[i + 1] = static_cast<uint8_t>(c >> 8);
  } else if (i < n) {
    out[i] = static_cast<uint8_t>(ep::e4m3fn_sat_pair(in[i], 0.0f) & 0xFFu);
  }
}

}  // namespace

extern "C" {

// Count the fp32 patterns (NaN excluded) where the two encoders differ;
// *nbad must be zeroed by the caller, first[8] receives the first patterns.
int e4m3_check_exhaustive(unsigned long long* nbad, uint32_t* first, hipStream_t s) {
  // 2^32 patterns / 64 per thread / 256 threads = 262144 blocks
  k_exhaustive<<<262144, 256, 0, s>>>(nbad, first);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

// out[i] = hardware E4M3FN code of in[i] (magnitude clamped to 448).
int e4m3_convert_hw(const float* in, uint8_t* out, int64_t n, hipStream_t s) {
  if (n <= 0) return 0;
  const int64_t threads = (n + 1) / 2;
  k_convert<<<static_cast<unsigned>((threads + 255) / 256), 256, 0, s>>>(in, out, n);
  return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // extern "C"
