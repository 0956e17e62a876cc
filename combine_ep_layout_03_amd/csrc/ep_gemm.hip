// Grouped GEMM over the expert-major segments: the consumer of dispatch.
//
// The mKernel article (its table of fusion kernels: MoE dispatch + grouped
// GEMM) runs each expert's GEMM over the tokens routed to it; on one GPU the
// consumer half is a grouped GEMM over the contiguous blocks the expert-major
// layout produced: for every expert e and receive row r in
// [offsets[e], offsets[e] + counts[e]),
//     y[r, n] = bf16_rne( sum_h x[r, h] * w[e, n, h] )
// with the sum in fp32 (MFMA accumulation order).
//
// Tiling for gfx950: a 256-thread block computes a 128-row x 128-column tile
// of one expert, stepping the reduction 64 at a time through LDS (rows padded
// to 72 elements so the 16-byte operand reads of 32 consecutive rows hit
// distinct banks), with the next step's global loads in flight during the
// MFMAs.  Each wave owns a 64 x 64 quarter as 2 x 2 v_mfma_f32_32x32x16_bf16
// tiles; the weight rows are the MFMA's A operand and the receive rows its B
// operand, so each lane ends with 16 outputs of one receive row and writes
// them as 8-byte runs along n.
//
// Work: tile t of Σ_e ceil(counts[e]/128) * (N/128) tiles (per expert,
// n-tile major, m-tile minor).  Blocks are dealt to the 8 XCDs round-robin
// by block index, so each XCD takes a contiguous run of tiles: the m-tiles
// sharing a weight slice, and the n-tiles sharing an expert's rows, then
// meet in one L2.
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128;       // receive rows per tile
constexpr int kBN = 128;       // output columns per tile
constexpr int kBK = 64;        // reduction step
constexpr int kLD = kBK + 8;   // padded LDS row, bf16 elements (144 bytes)
constexpr int kXcds = 8;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__global__ __launch_bounds__(kBlock) void k_expert_gemm(GemmArgs a) {
  __shared__ __align__(16) uint16_t sX[kBM * kLD];
  __shared__ __align__(16) uint16_t sW[kBN * kLD];
  __shared__ int sTiles[1024 + 1];
  __shared__ int sTmp[kWavesPerBlock];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int E = a.E;

  // tiles per expert, then their exclusive prefix (same in every block)
  for (int e = tid; e < E; e += kBlock) sTiles[e] = ((a.counts[e] + kBM - 1) / kBM) * a.ntn;
  __syncthreads();
  const int total = block_exclusive_scan(sTiles, E, sTmp);
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int xcd = static_cast<int>(blockIdx.x % kXcds);
  const int seat = static_cast<int>(blockIdx.x / kXcds);
  if (seat >= per_xcd) return;
  const int tile = xcd * per_xcd + seat;
  if (tile >= total) return;
  // owning expert: the last e with sTiles[e] <= tile (empty experts repeat
  // the prefix of the next one and are skipped)
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (sTiles[mid] <= tile) lo = mid;
    else hi = mid - 1;
  }
  const int e = lo;
  const int cnt = a.counts[e];
  const int mt = (cnt + kBM - 1) / kBM;
  const int local = tile - sTiles[e];
  const int im = local % mt;
  const int jn = local / mt;
  const int row0 = a.offsets[e] + im * kBM;
  const int row_end = a.offsets[e] + cnt;
  const int n0 = jn * kBN;

  // global -> register staging: thread t moves vectors t + 256 q (q < 4) of
  // each 128 x 64 tile; vector v is row v / 8, columns (v % 8) * 8 .. +8
  const uint16_t* wbase = a.w + (static_cast<int64_t>(e) * a.N + n0) * a.H;
  u32x4 rx[4], rw[4];
  int srow[4], scol[4];
  const uint16_t* xrow[4];
  const uint16_t* wrow[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int v = tid + kBlock * q;
    srow[q] = v >> 3;
    scol[q] = (v & 7) * 8;
    const int gr = min(row0 + srow[q], row_end - 1);  // rows past the segment: any valid row, never stored
    xrow[q] = a.x + static_cast<int64_t>(gr) * a.ldx + scol[q];
    wrow[q] = wbase + static_cast<int64_t>(srow[q]) * a.H + scol[q];
  }
  auto gload = [&](int k0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      rx[q] = *reinterpret_cast<const u32x4*>(xrow[q] + k0);
      rw[q] = nt_load(reinterpret_cast<const u32x4*>(wrow[q] + k0));
    }
  };

  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int lr = lane & 31;          // operand row within a 32-row tile
  const int lk = (lane >> 5) * 8;    // operand k offset within a 16-step
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int nk = a.H / kBK;
  gload(0);
  for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      *reinterpret_cast<u32x4*>(&sX[srow[q] * kLD + scol[q]]) = rx[q];
      *reinterpret_cast<u32x4*>(&sW[srow[q] * kLD + scol[q]]) = rw[q];
    }
    __syncthreads();
    if (kt + 1 < nk) gload((kt + 1) * kBK);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      bf16x8 av[2], bv[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        av[t] = as_bf16x8(*reinterpret_cast<const u32x4*>(&sW[(wn * 64 + t * 32 + lr) * kLD + kk * 16 + lk]));
        bv[t] = as_bf16x8(*reinterpret_cast<const u32x4*>(&sX[(wm * 64 + t * 32 + lr) * kLD + kk * 16 + lk]));
      }
#pragma unroll
      for (int tm = 0; tm < 2; ++tm)
#pragma unroll
        for (int tn = 0; tn < 2; ++tn)
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[tn], bv[tm], acc[tm][tn], 0, 0, 0);
    }
    __syncthreads();
  }

  // D[n][m] of each 32 x 32 tile: lane -> receive row m = lane % 32, outputs
  // n = (i / 4) * 8 + (lane / 32) * 4 + i % 4 for i < 16
#pragma unroll
  for (int tm = 0; tm < 2; ++tm) {
    const int r = row0 + wm * 64 + tm * 32 + lr;
    if (r >= row_end) continue;
    uint16_t* yrow = a.y + static_cast<int64_t>(r) * a.ldy + n0;
#pragma unroll
    for (int tn = 0; tn < 2; ++tn) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int nb = wn * 64 + tn * 32 + g * 8 + (lane >> 5) * 4;
        u32x2 pk;
        pk[0] = pack_bf16x2(acc[tm][tn][4 * g], acc[tm][tn][4 * g + 1]);
        pk[1] = pack_bf16x2(acc[tm][tn][4 * g + 2], acc[tm][tn][4 * g + 3]);
        *reinterpret_cast<u32x2*>(yrow + nb) = pk;
      }
    }
  }
}

}  // namespace

int64_t expert_gemm_max_tiles(int64_t max_rows, int E, int N) {
  return ((max_rows + kBM - 1) / kBM + E) * (N / kBN);
}

hipError_t launch_expert_gemm(const GemmArgs& a, int64_t max_rows, hipStream_t s) {
  const int64_t tiles = expert_gemm_max_tiles(max_rows, a.E, a.N);
  const int64_t grid = (tiles + kXcds - 1) / kXcds * kXcds;
  k_expert_gemm<<<static_cast<unsigned>(grid), kBlock, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace ep
