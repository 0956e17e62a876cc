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
// Tiling for gfx950: a 512-thread block computes up to 256 rows x 256
// columns of one expert.  The reduction runs 32 at a time through a 4-stage
// LDS ring filled by LDS-direct loads (global_load_lds_dwordx4: each lane's
// 16 bytes land in LDS without passing through registers), issued three
// steps ahead, so three 32 KiB stages are in flight while the MFMAs consume
// the fourth.  A stage holds 256 rows of 4 16-byte k-vectors per operand;
// vector kv of row r sits in slot r*4 + (kv ^ ((r >> 2) & 3)), which keeps
// the 16-byte operand reads of 16 consecutive rows on distinct banks.
//
// Each of the 8 waves owns 64 rows x 128 columns as 2 x 4
// v_mfma_f32_32x32x16_bf16 tiles; the weight rows are the MFMA's A operand
// and the receive rows its B operand, so each lane ends with outputs of one
// receive row and writes them as 8-byte runs along n.  An expert's rows are
// split evenly over ceil(count/256) row tiles (in 32-row steps), so with
// ~256 rows per expert its weights stream once.  Every lane loads a full
// stage share (rows past the tile, or past N, re-read a valid row and are
// never stored), which keeps the number of loads in flight per wave exact:
// waiting until at most 4 * (stages still ahead) remain marks the current
// stage complete.  The LDS operand reads are issued as inline ds_read_b128
// with explicit lgkmcnt waits tied to their registers, so the compiler's
// wait-count pass, which cannot tell the ring stages apart, does not drain
// every outstanding load before them.  32-row sub-tiles without a valid row
// skip their MFMAs.
//
// Work: tile t of sum_e ceil(counts[e]/256) * ceil(N/256) tiles (per
// expert, column-tile major, row-tile minor).  Blocks are dealt to the 8
// XCDs round-robin by block index, so each XCD takes a contiguous run of
// tiles: the row tiles sharing a weight slice, and the column tiles sharing
// an expert's rows, then meet in one L2.
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 512;   // 8 waves: 4 (rows) x 2 (columns), 64 x 128 each
constexpr int kBM = 256;        // receive rows per tile (at most)
constexpr int kBN = 256;        // output columns per tile
constexpr int kBK = 32;         // reduction step
constexpr int kStages = 4;      // LDS ring depth
constexpr int kStageElems = kBM * kBK;  // bf16 elements of one operand stage (16 KiB)
constexpr int kXcds = 8;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 16-byte slot of k-vector kv (0..3) of row r within a stage
__device__ __forceinline__ int slot_of(int r, int kv) { return r * 4 + (kv ^ ((r >> 2) & 3)); }

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p));
}

// 16-byte LDS read, ordered by lgkm_wait below rather than by the compiler
__device__ __forceinline__ u32x4 lds_read16(uint32_t addr) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(addr));
  return r;
}

// wait until at most N LDS reads are outstanding; the registers of the reads
// that must have landed are operands, so their uses cannot move above it
template <int N>
__device__ __forceinline__ void lgkm_wait(u32x4& a0, u32x4& a1, u32x4& a2, u32x4& a3, u32x4& b0,
                                          u32x4& b1) {
  asm volatile("s_waitcnt lgkmcnt(%6)"
               : "+v"(a0), "+v"(a1), "+v"(a2), "+v"(a3), "+v"(b0), "+v"(b1)
               : "n"(N));
}

// wait until at most n (0, 4 or 8) vector-memory loads of this wave are
// outstanding; expcnt and lgkmcnt are left unconstrained
__device__ __forceinline__ void wait_vm(int n) {
  if (n >= 8) __builtin_amdgcn_s_waitcnt(0xF70 | 8);
  else if (n >= 4) __builtin_amdgcn_s_waitcnt(0xF70 | 4);
  else __builtin_amdgcn_s_waitcnt(0xF70);
}

__global__ __launch_bounds__(kThreads) void k_expert_gemm(GemmArgs a) {
  __shared__ __align__(16) uint16_t sX[kStages * kStageElems];
  __shared__ __align__(16) uint16_t sW[kStages * kStageElems];
  __shared__ int sTiles[1024 + 1];
  __shared__ int sTmp[kThreads / kWave];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int E = a.E;

  // tiles per expert: ceil(count / 256) row tiles x ceil(N / 256) column
  // tiles, then their exclusive prefix (the same in every block)
  for (int e = tid; e < E; e += kThreads) sTiles[e] = ((a.counts[e] + kBM - 1) / kBM) * a.ntn;
  __syncthreads();
  const int total = block_exclusive_scan<kThreads>(sTiles, E, sTmp);
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
  // the expert's rows split evenly over its row tiles, in 32-row steps
  const int per = ((cnt + mt - 1) / mt + 31) / 32 * 32;
  const int row0 = a.offsets[e] + im * per;
  const int nrows = min(per, cnt - im * per);  // valid rows of this tile, > 0
  const int n0 = jn * kBN;

  // Each wave fills 2 of the 16 1-KiB chunks of a stage, per operand: lane l
  // of chunk j fills slot s = j*64 + l, i.e. row s/4, k-vector
  // (s % 4) ^ ((row >> 2) & 3).
  const uint16_t* xsrc[2];
  const uint16_t* wsrc[2];
  int dst[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int j = wave * 2 + q;
    const int s = j * 64 + lane;
    const int r = s >> 2;
    const int kv = (s & 3) ^ ((r >> 2) & 3);
    const int xr = r < nrows ? r : 0;
    const int wr = n0 + r < a.N ? r : 0;  // the last column tile may be half valid
    xsrc[q] = a.x + static_cast<int64_t>(row0 + xr) * a.ldx + kv * 8;
    wsrc[q] = a.w + (static_cast<int64_t>(e) * a.N + n0 + wr) * a.H + kv * 8;
    dst[q] = j * 64 * 8;
  }
  auto issue = [&](int kt) {
    const int st = kt % kStages;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(xsrc[q] + kt * kBK),
          (__attribute__((address_space(3))) void*)(sX + st * kStageElems + dst[q]), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(wsrc[q] + kt * kBK),
          (__attribute__((address_space(3))) void*)(sW + st * kStageElems + dst[q]), 16, 0, 0);
    }
  };

  const int wm = wave >> 1;          // 64-row slab
  const int wn = wave & 1;           // 128-column slab
  const int lr = lane & 31;          // operand row within a 32-row tile
  const int lkv = lane >> 5;         // operand k-vector within a 16-step
  // 32-row sub-tiles of this wave holding at least one valid row (none if
  // the wave's 128 columns lie past N)
  const int live = n0 + wn * 128 < a.N ? min(2, max(0, (nrows - wm * 64 + 31) / 32)) : 0;
  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  // operand byte offsets within a stage, per 16-step kk of the 32-step
  uint32_t aoff[2][4], boff[2][2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
    for (int t = 0; t < 4; ++t) aoff[kk][t] = slot_of(wn * 128 + t * 32 + lr, kk * 2 + lkv) * 16;
#pragma unroll
    for (int t = 0; t < 2; ++t) boff[kk][t] = slot_of(wm * 64 + t * 32 + lr, kk * 2 + lkv) * 16;
  }
  const uint32_t xbase = lds_addr(sX);
  const uint32_t wbase = lds_addr(sW);

  const int nk = a.H / kBK;
  for (int kt = 0; kt < kStages - 1 && kt < nk; ++kt) issue(kt);
  for (int kt = 0; kt < nk; ++kt) {
    // stage kt landed (for this wave), then for every wave; the barrier also
    // ends all reads of the stage the next issue overwrites
    wait_vm(4 * min(kStages - 2, nk - 1 - kt));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (kt + kStages - 1 < nk) issue(kt + kStages - 1);
    if (live > 0) {
      const uint32_t so = static_cast<uint32_t>((kt % kStages) * kStageElems * 2);
      u32x4 av[2][4], bv[2][2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int t = 0; t < 4; ++t) av[kk][t] = lds_read16(wbase + so + aoff[kk][t]);
#pragma unroll
        for (int t = 0; t < 2; ++t) bv[kk][t] = lds_read16(xbase + so + boff[kk][t]);
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        if (kk == 0) lgkm_wait<6>(av[0][0], av[0][1], av[0][2], av[0][3], bv[0][0], bv[0][1]);
        else lgkm_wait<0>(av[1][0], av[1][1], av[1][2], av[1][3], bv[1][0], bv[1][1]);
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) {
          acc[0][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av[kk][tn]),
                                                               as_bf16x8(bv[kk][0]), acc[0][tn], 0, 0, 0);
          if (live > 1)
            acc[1][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                as_bf16x8(av[kk][tn]), as_bf16x8(bv[kk][1]), acc[1][tn], 0, 0, 0);
        }
      }
    }
  }

  // D[n][m] of each 32 x 32 tile: lane -> receive row m = lane % 32, outputs
  // n = (i / 4) * 8 + (lane / 32) * 4 + i % 4 for i < 16
#pragma unroll
  for (int tm = 0; tm < 2; ++tm) {
    const int rl = wm * 64 + tm * 32 + lr;
    if (rl >= nrows || n0 + wn * 128 >= a.N) continue;
    uint16_t* yrow = a.y + static_cast<int64_t>(row0 + rl) * a.ldy + n0;
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int nb = wn * 128 + tn * 32 + g * 8 + (lane >> 5) * 4;
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
  return ((max_rows + kBM - 1) / kBM + E) * ((N + kBN - 1) / kBN);
}

hipError_t launch_expert_gemm(const GemmArgs& a, int64_t max_rows, hipStream_t s) {
  const int64_t tiles = expert_gemm_max_tiles(max_rows, a.E, a.N);
  const int64_t grid = (tiles + kXcds - 1) / kXcds * kXcds;
  k_expert_gemm<<<static_cast<unsigned>(grid), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace ep
