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
// Tiling for gfx950: a 512-thread block computes up to 320 rows x 256
// columns of one expert, so an expert of up to 320 receive rows (all of them
// at the 8192-token, top-8-of-256 shape) streams each weight slice through
// one CU only.  The reduction runs 32 at a time (one step) through two LDS
// rings (144 KiB) filled by LDS-direct loads (global_load_lds_dwordx4: each
// lane's 16 bytes land in LDS without passing through registers).  Weight
// stages are one step wide, 4 of them, issued three steps ahead.
// Receive-row stages are two steps wide, 2 of them, one stage ahead: a
// receive row's 64 elements of a stage are one whole 128-byte line, which the
// 8 column tiles of an expert read from L2 (whole lines measured 1.5% faster
// than half lines).  Vector kv of row r sits in slot r*4 + (kv ^ ((r >> 2) &
// 3)) of a weight stage and r*8 + (kv ^ ((r >> 1) & 7)) of a receive-row
// stage, which keeps the 16-byte operand reads of 16 consecutive rows on
// distinct banks.  Waves 0-3 fill the receive-row stage (10 KiB each), waves
// 4-7 the weight stage (4 KiB each).
//
// The 8 waves form 2 (rows) x 4 (columns).  A wave owns 64 columns and the
// 32-row sub-tiles wm, wm+2, ..., wm+8 (interleaved, so a tile of any height
// splits its MFMA work evenly between the two row waves of each SIMD), as
// 5 x 2 v_mfma_f32_32x32x16_bf16 tiles; the weight rows are the MFMA's A
// operand and the receive rows its B operand, so each lane ends with outputs
// of one receive row and writes them as 8-byte runs along n.  An expert's
// rows are split evenly over ceil(count/320) row tiles, in 32-row steps.
// Every lane loads a full stage share (rows past the tile, or past N,
// re-read a valid row and are never stored), which keeps the number of
// loads in flight per wave exact: waiting until at most (loads per stage) *
// (younger stages issued) remain marks the stage a step reads complete.  The LDS
// operand reads are issued as inline ds_read_b128 with explicit lgkmcnt
// waits tied to their registers, so the compiler's wait-count pass, which
// cannot tell the ring stages apart, does not drain every outstanding load
// before them.  Sub-tiles without a valid row skip their MFMAs.  The two
// waves of each SIMD (one per row half) run half a step apart, so one reads
// its operands from LDS while the other issues MFMAs (see the main loop).
//
// Work: tile t of sum_e ceil(counts[e]/320) * ceil(N/256) tiles (per
// expert, column-tile major, row-tile minor).  Blocks are dealt to the 8
// XCDs round-robin by block index, so each XCD takes a contiguous run of
// tiles: the column tiles sharing an expert's rows then meet in one L2.
//
// With rows gathered, x is the token matrix and each expert row's operand is
// loaded from the token the layout recorded for it, so the dispatch's scatter
// happens inside the GEMM's loads (the mKernel article's fused MoE dispatch
// and grouped GEMM): no receive buffer is written or read.
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 512;   // 8 waves: 2 (rows) x 4 (columns)
constexpr int kBM = 320;        // receive rows per tile (at most)
constexpr int kBN = 256;        // output columns per tile
constexpr int kBK = 32;         // reduction step
constexpr int kXStages = 2;     // receive-row ring: 64-wide stages (whole 128-B lines), one ahead
constexpr int kWStages = 4;     // weight ring: 32-wide stages, three ahead
constexpr int kXBK = 2 * kBK;   // reduction width of a receive-row stage
constexpr int kXElems = kBM * kXBK;  // bf16 elements of a receive-row stage (40 KiB)
constexpr int kWElems = kBN * kBK;   // bf16 elements of a weight stage (16 KiB)
constexpr int kXcds = 8;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 16-byte slot of k-vector kv of row r within a weight stage (kv 0..3) or a
// receive-row stage (kv 0..7); the XOR keeps the operand reads of 16
// consecutive rows at one kv on distinct banks
__device__ __forceinline__ int slot_w(int r, int kv) { return r * 4 + (kv ^ ((r >> 2) & 3)); }
__device__ __forceinline__ int slot_x(int r, int kv) { return r * 8 + (kv ^ ((r >> 1) & 7)); }

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
__device__ __forceinline__ void lgkm_wait(u32x4& a0, u32x4& a1, u32x4& b0, u32x4& b1, u32x4& b2,
                                          u32x4& b3, u32x4& b4) {
  asm volatile("s_waitcnt lgkmcnt(%7)"
               : "+v"(a0), "+v"(a1), "+v"(b0), "+v"(b1), "+v"(b2), "+v"(b3), "+v"(b4)
               : "n"(N));
}

// wait until at most n (0, 4, 8 or 10) vector-memory loads of this wave are
// outstanding; expcnt and lgkmcnt are left unconstrained
__device__ __forceinline__ void wait_vm(int n) {
  if (n >= 10) __builtin_amdgcn_s_waitcnt(0xF70 | 10);
  else if (n >= 8) __builtin_amdgcn_s_waitcnt(0xF70 | 8);
  else if (n >= 4) __builtin_amdgcn_s_waitcnt(0xF70 | 4);
  else __builtin_amdgcn_s_waitcnt(0xF70);
}

__global__ __launch_bounds__(kThreads) void k_expert_gemm(GemmArgs a) {
  __shared__ __align__(16) uint16_t sX[kXStages * kXElems];
  __shared__ __align__(16) uint16_t sW[kWStages * kWElems];
  // tile table (E + 1 ints) and scan scratch, in the ring until the first load
  static_assert((1024 + 1 + 16 + kThreads / kWave) * sizeof(int) <= sizeof(sW), "tile table fits");
  int* const sTiles = reinterpret_cast<int*>(sW);
  int* const sTmp = sTiles + 1024 + 16;

  // a stale layout handle: the whole grid returns before any barrier
  if (!layout_current(a.status, a.generation)) return;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  // wave-uniform for the compiler too, so branches on it are scalar
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int E = a.E;

  // tiles per expert: ceil(count / 320) row tiles x ceil(N / 256) column
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
  // the expert's rows split evenly over its row tiles, in 32-row steps; as
  // per <= 320 and (mt - 1) * 320 < cnt, every tile holds at least one row
  const int per = ((cnt + mt - 1) / mt + 31) / 32 * 32;
  const int row0 = a.offsets[e] + im * per;
  const int nrows = min(per, cnt - im * per);
  const int n0 = jn * kBN;
  __syncthreads();  // every read of the tile table precedes the ring's first load

  // Waves 0-3 fill the receive-row stage (40 chunks of 64 slots, 10 each):
  // lane l of chunk j fills slot s = j*64 + l, row s/8, k-vector
  // (s % 8) ^ ((row >> 1) & 7), so one load instruction covers 8 whole
  // 128-byte lines of 8 receive rows.  Waves 4-7 fill the weight stage (16
  // chunks, 4 each): row s/4, k-vector (s % 4) ^ ((row >> 2) & 3).
  const bool xwave = wave < 4;
  const uint16_t* src[10];
  int dst[10];
#pragma unroll
  for (int q = 0; q < 10; ++q) {
    if (xwave) {
      const int j = wave * 10 + q;
      const int s = j * 64 + lane;
      const int r = s >> 3;
      const int kv = (s & 7) ^ ((r >> 1) & 7);
      const int xr = r < nrows ? r : 0;
      // expert row -> the x row holding its operand: itself, or (rows
      // gathered) the token it came from
      const int64_t xrow = a.row_src ? a.row_src[row0 + xr] : row0 + xr;
      src[q] = a.x + xrow * a.ldx + kv * 8;
      dst[q] = j * 64 * 8;
    } else {
      const int j = (wave - 4) * 4 + (q < 4 ? q : 3);
      const int s = j * 64 + lane;
      const int r = s >> 2;
      const int kv = (s & 3) ^ ((r >> 2) & 3);
      if (a.packed) {
        // the (expert, column tile) block; rows past N are zero there
        src[q] = a.w + (static_cast<int64_t>(e) * a.ntn + jn) * (static_cast<int64_t>(a.H) * kBN) +
                 r * kBK + kv * 8;
      } else {
        const int wr = n0 + r < a.N ? r : 0;  // the last column tile may be half valid
        src[q] = a.w + (static_cast<int64_t>(e) * a.N + n0 + wr) * a.H + kv * 8;
      }
      dst[q] = j * 64 * 8;
    }
  }
  // elements between consecutive weight stages of one row: the next 32 of
  // the row, or the next 16 KiB block of the packed order
  const int64_t wstep = a.packed ? kBN * kBK : kBK;
  const int nk = a.H / kBK;  // 32-wide steps; H % 64 == 0, so nk is even
  const int nsx = nk / 2;    // receive-row stages
  auto issue_x = [&](int sx) __attribute__((always_inline)) {
    uint16_t* base = sX + (sx % kXStages) * kXElems;
#pragma unroll
    for (int q = 0; q < 10; ++q)
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(src[q] + sx * kXBK),
          (__attribute__((address_space(3))) void*)(base + dst[q]), 16, 0, 0);
  };
  // Packed weight stages are whole lines read once, so they load
  // non-temporal (2.342 against 2.389 ms at 65,536 rows x 7168 -> 2048); the
  // plain order reads half lines whose other halves the next step needs, and
  // non-temporal loads there refetch them (2.73 against 2.44 ms).
  auto issue_w = [&](int kt) __attribute__((always_inline)) {
    uint16_t* base = sW + (kt % kWStages) * kWElems;
    if (a.packed) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(src[q] + kt * wstep),
            (__attribute__((address_space(3))) void*)(base + dst[q]), 16, 0, 2);
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        __builtin_amdgcn_global_load_lds(
            (const __attribute__((address_space(1))) void*)(src[q] + kt * wstep),
            (__attribute__((address_space(3))) void*)(base + dst[q]), 16, 0, 0);
    }
  };
  // this wave's loads of the stages step kt reads have landed.  Receive-row
  // stage kt/2: stages 0 and 1 are issued up front and stage s + 1 at step
  // 2s (s >= 1), so before even steps only stage 1 at step 0 is younger, and
  // before odd steps stage kt/2 + 1 (10 loads each).  Weight stage kt:
  // stages kt + 1 and kt + 2 are younger (4 loads each).
  auto wait_own = [&](int kt) __attribute__((always_inline)) {
    if (xwave) {
      const int sx = kt >> 1;
      const int issued = min(nsx - 1, (kt & 1) ? sx + 1 : max(sx, 1));
      wait_vm(10 * (issued - sx));
    } else {
      wait_vm(4 * min(kWStages - 2, nk - 1 - kt));
    }
  };
  // after step kt's first barrier: on even steps kt = 2s >= 2 receive-row
  // stage s + 1 (its slot held stage s - 1), and weight stage kt + 3 (its
  // slot held stage kt - 1); both were read by both halves before that
  // barrier
  auto issue_next = [&](int kt) __attribute__((always_inline)) {
    if (xwave) {
      if (!(kt & 1) && kt >= 2 && (kt >> 1) + 1 < nsx) issue_x((kt >> 1) + 1);
    } else if (kt + kWStages - 1 < nk) {
      issue_w(kt + kWStages - 1);
    }
  };

  const int wm = wave >> 2;          // row half: sub-tiles wm, wm+2, ..., wm+8
  const int wn = wave & 3;           // 64-column slab
  const int lr = lane & 31;          // operand row within a 32-row tile
  const int lkv = lane >> 5;         // operand k-vector within a 16-step
  // sub-tiles of this wave holding at least one valid row (none if the
  // wave's 64 columns lie past N)
  int live = 0;
#pragma unroll
  for (int i = 0; i < 5; ++i) live += (2 * i + wm) * 32 < nrows ? 1 : 0;
  if (n0 + wn * 64 >= a.N) live = 0;
  f32x16 acc[5][2];
#pragma unroll
  for (int i = 0; i < 5; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const uint32_t xbase = lds_addr(sX);
  const uint32_t wbase = lds_addr(sW);
  // one stage's operands: 2 reduction halves x (2 weight, 5 receive-row) vectors
  u32x4 av[2][2], bv[2][5];
  auto read_stage = [&](int kt) __attribute__((always_inline)) {
    const uint32_t xs = xbase + static_cast<uint32_t>(((kt >> 1) % kXStages) * kXElems * 2);
    const uint32_t ws = wbase + static_cast<uint32_t>((kt % kWStages) * kWElems * 2);
    const int xk = (kt & 1) * 4;  // this step's k-vectors inside the receive-row stage
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
        av[kk][t] = lds_read16(ws + slot_w(wn * 64 + t * 32 + lr, kk * 2 + lkv) * 16);
#pragma unroll
      for (int i = 0; i < 5; ++i)
        bv[kk][i] = lds_read16(xs + slot_x((2 * i + wm) * 32 + lr, xk + kk * 2 + lkv) * 16);
    }
    lgkm_wait<7>(av[0][0], av[0][1], bv[0][0], bv[0][1], bv[0][2], bv[0][3], bv[0][4]);
    lgkm_wait<0>(av[1][0], av[1][1], bv[1][0], bv[1][1], bv[1][2], bv[1][3], bv[1][4]);
  };
  auto mfma_stage = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        if (i < live) {
#pragma unroll
          for (int t = 0; t < 2; ++t)
            acc[i][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                as_bf16x8(av[kk][t]), as_bf16x8(bv[kk][i]), acc[i][t], 0, 0, 0);
        }
      }
    }
  };
  auto block_sync = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  // Ping-pong: each SIMD runs one wave of each row half.  A step has two
  // phases split by barriers; in the first the row-half-0 waves read stage
  // kt from LDS while the row-half-1 waves run the MFMAs of step kt - 1, in
  // the second the roles swap, so the LDS reads of one wave overlap the
  // MFMAs of the other instead of all eight waves doing each in turn.  The
  // stage the next issue overwrites was read by both halves before the
  // step's first barrier, and each wave's wait for its own loads of stage kt
  // before that barrier makes the stage complete for all.
  // The two halves run separate loops with the same barriers in the same
  // order.
  if (xwave) {
    issue_x(0);
    if (nsx > 1) issue_x(1);
  } else {
    for (int kt = 0; kt < kWStages - 1 && kt < nk; ++kt) issue_w(kt);
  }
  if (wm == 0) {
    for (int kt = 0; kt < nk; ++kt) {
      wait_own(kt);
      block_sync();
      issue_next(kt);
      if (live > 0) read_stage(kt);
      block_sync();
      if (live > 0) mfma_stage();
    }
  } else {
    for (int kt = 0; kt < nk; ++kt) {
      wait_own(kt);
      block_sync();
      issue_next(kt);
      if (kt > 0 && live > 0) mfma_stage();
      block_sync();
      if (live > 0) read_stage(kt);
    }
    if (live > 0) mfma_stage();
  }

  // D[n][m] of each 32 x 32 tile: lane -> receive row m = lane % 32, outputs
  // n = (i / 4) * 8 + (lane / 32) * 4 + i % 4 for i < 16
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int rl = (2 * i + wm) * 32 + lr;
    if (rl >= nrows || n0 + wn * 64 >= a.N) continue;
    uint16_t* yrow = a.y + static_cast<int64_t>(row0 + rl) * a.ldy + n0;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int nb = wn * 64 + t * 32 + g * 8 + (lane >> 5) * 4;
        u32x2 pk;
        pk[0] = pack_bf16x2(acc[i][t][4 * g], acc[i][t][4 * g + 1]);
        pk[1] = pack_bf16x2(acc[i][t][4 * g + 2], acc[i][t][4 * g + 3]);
        *reinterpret_cast<u32x2*>(yrow + nb) = pk;
      }
    }
  }
}

// One 16-byte chunk per thread of the packed order: chunk c is k-vector
// c % 4 of row (c / 4) % 256 of block c / 1024, block = (expert, column
// tile, reduction step) in that order of significance.
__global__ __launch_bounds__(256) void k_pack_expert_weights(const uint16_t* __restrict__ w, int N,
                                                             int H, int ntn, int64_t chunks,
                                                             uint16_t* __restrict__ packed) {
  const int nk = H / kBK;
  for (int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; c < chunks;
       c += static_cast<int64_t>(gridDim.x) * 256) {
    const int kv = static_cast<int>(c & 3);
    const int r = static_cast<int>((c >> 2) & (kBN - 1));
    const int64_t blk = c >> 10;
    const int kt = static_cast<int>(blk % nk);
    const int64_t et = blk / nk;  // expert * ntn + column tile
    const int e = static_cast<int>(et / ntn);
    const int n = static_cast<int>(et % ntn) * kBN + r;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (n < N) v = *reinterpret_cast<const u32x4*>(w + (static_cast<int64_t>(e) * N + n) * H + kt * kBK + kv * 8);
    *reinterpret_cast<u32x4*>(packed + c * 8) = v;
  }
}

}  // namespace

hipError_t launch_pack_expert_weights(const uint16_t* w, int E, int N, int H, uint16_t* packed,
                                      hipStream_t s) {
  const int ntn = (N + kBN - 1) / kBN;
  const int64_t chunks = static_cast<int64_t>(E) * ntn * (H / kBK) * kBN * 4;
  const int64_t blocks = (chunks + 255) / 256;
  k_pack_expert_weights<<<static_cast<unsigned>(blocks < 65536 ? blocks : 65536), 256, 0, s>>>(
      w, N, H, ntn, chunks, packed);
  return hipGetLastError();
}

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
