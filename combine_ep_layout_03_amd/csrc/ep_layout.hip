// Layout kernels: the three dispatch phases of TileScale PR #68 ("EP v2
// intranode dispatch/combine"; Design section and the commit adding DeepEP's
// do_expand) on one GPU.
//   phase 1  k_layout_count   per-block tallies per destination (expert, and
//                             group when grouped rows are asked for)
//   phase 2  k_layout_colscan exclusive scan of the tallies over blocks; on
//                             one GPU the cross-rank count exchange reduces
//                             to this scan
//   phase 3  k_layout_place   base + locally claimed slot for every entry
// The pages claim slots in whatever order lanes arrive; here the claim order
// is the (t,k) order, so placement is deterministic: inside a wave the rank
// comes from a match mask built with LDS bit-or (gfx950 has no match-any
// instruction), across the block's waves from running counters updated wave
// by wave, across blocks from the scanned tallies.
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {

namespace {

// Is (t,k) the first valid entry of token t inside expert group g?  The
// grouped layout sends one row per (token, group hit); the row is claimed by
// this entry.
__device__ __forceinline__ bool first_in_group(const int64_t* __restrict__ idx, uint32_t t, int k,
                                               int K, int E, int epg, int g) {
  const int64_t* row = idx + static_cast<size_t>(t) * K;
  for (int kk = 0; kk < k; ++kk) {
    const int64_t v = row[kk];
    if (v >= 0 && v < E && static_cast<int>(v) / epg == g) return false;
  }
  return true;
}

// The same test from the neighbouring lanes, when K divides the wave size:
// every block, round and wave starts at an entry index that is a multiple of
// 64, so lanes (lane & ~(K-1)) .. + K-1 hold one token's K entries in k
// order.  g is this entry's group, or -1 when it is not valid.  Every lane of
// the wave must call this (the shuffles read the other lanes).
__device__ __forceinline__ bool first_in_group_lanes(int g, int K, int lane) {
  const int base = lane & ~(K - 1);
  bool first = g >= 0;
  for (int j = 0; j < K; ++j) {
    const int gj = __shfl(g, base + j, kWave);
    if (base + j < lane && gj == g) first = false;
  }
  return first;
}

template <bool GROUPED>
__global__ __launch_bounds__(kBlock) void k_layout_count(const int64_t* __restrict__ idx,
                                                         uint32_t n, int K, int E, int epg,
                                                         int ncols, int rounds,
                                                         int* __restrict__ partials) {
  extern __shared__ int cnt[];  // [ncols]
  for (int c = threadIdx.x; c < ncols; c += kBlock) cnt[c] = 0;
  __syncthreads();
  const uint32_t base = blockIdx.x * static_cast<uint32_t>(rounds) * kBlock;
  const bool lanes = GROUPED && kWave % K == 0;  // a token's entries in neighbouring lanes
  const int lane = threadIdx.x & (kWave - 1);
  // each round's id is loaded one round ahead
  int64_t v_next = base + threadIdx.x < n ? idx[base + threadIdx.x] : -1;
  for (int r = 0; r < rounds; ++r) {
    const uint32_t i = base + static_cast<uint32_t>(r) * kBlock + threadIdx.x;
    const int64_t v = v_next;
    if (r + 1 < rounds) {
      const uint32_t i2 = i + kBlock;
      v_next = i2 < n ? idx[i2] : -1;
    }
    const bool valid = v >= 0 && v < E;
    const int e = valid ? static_cast<int>(v) : -1;
    if (valid) atomicAdd(&cnt[e], 1);
    else if (v != -1) atomicAdd(&cnt[ncols - 1], 1);
    if (GROUPED) {
      if (lanes) {
        const int g = valid ? e / epg : -1;
        if (first_in_group_lanes(g, K, lane)) atomicAdd(&cnt[E + g], 1);
      } else if (valid) {
        const uint32_t t = i / static_cast<uint32_t>(K);
        const int k = static_cast<int>(i - t * static_cast<uint32_t>(K));
        const int g = e / epg;
        if (first_in_group(idx, t, k, K, E, epg, g)) atomicAdd(&cnt[E + g], 1);
      }
    }
  }
  __syncthreads();
  int* dst = partials + static_cast<size_t>(blockIdx.x) * ncols;
  for (int c = threadIdx.x; c < ncols; c += kBlock) dst[c] = cnt[c];
}

// In-place exclusive scan of each column over the nblocks rows; the column
// totals go to row nblocks.  Block = 64 columns x 16 row slices; a slice
// holds at most kScanRows rows (nblocks <= 16 * kScanRows), loaded at once
// and kept in registers for the write-back.
constexpr int kScanRows = 16;

__global__ __launch_bounds__(1024) void k_layout_colscan(int* __restrict__ partials, int nblocks,
                                                         int ncols) {
  __shared__ int s[16][kWave + 1];
  const int cl = threadIdx.x & (kWave - 1);
  const int rl = threadIdx.x / kWave;
  const int c = blockIdx.x * kWave + cl;
  const int chunk = (nblocks + 15) / 16;
  const int b0 = rl * chunk;
  int v[kScanRows];
  int sum = 0;
#pragma unroll
  for (int j = 0; j < kScanRows; ++j) {
    const int b = b0 + j;
    v[j] = (j < chunk && b < nblocks && c < ncols) ? partials[static_cast<size_t>(b) * ncols + c] : 0;
    sum += v[j];
  }
  s[rl][cl] = sum;
  __syncthreads();
  if (rl == 0) {
    int run = 0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int x = s[j][cl];
      s[j][cl] = run;
      run += x;
    }
    if (c < ncols) partials[static_cast<size_t>(nblocks) * ncols + c] = run;
  }
  __syncthreads();
  int run = s[rl][cl];
#pragma unroll
  for (int j = 0; j < kScanRows; ++j) {
    const int b = b0 + j;
    if (j < chunk && b < nblocks && c < ncols) {
      partials[static_cast<size_t>(b) * ncols + c] = run;
      run += v[j];
    }
  }
}

// The same scan for 257 to 2048 rows: block = 16 columns x 64 row slices of
// at most kScanRowsWide rows; the slice sums of a column are scanned in
// log2(64) steps across the slices rather than one after another.
constexpr int kScanColsWide = 16;
constexpr int kScanSlicesWide = 64;
constexpr int kScanRowsWide = 32;

__global__ __launch_bounds__(1024) void k_layout_colscan_wide(int* __restrict__ partials,
                                                              int nblocks, int ncols) {
  __shared__ int s[kScanSlicesWide][kScanColsWide + 1];
  const int cl = threadIdx.x % kScanColsWide;
  const int rl = threadIdx.x / kScanColsWide;
  const int c = blockIdx.x * kScanColsWide + cl;
  const int chunk = (nblocks + kScanSlicesWide - 1) / kScanSlicesWide;
  const int b0 = rl * chunk;
  int v[kScanRowsWide];
  int sum = 0;
#pragma unroll
  for (int j = 0; j < kScanRowsWide; ++j) {
    const int b = b0 + j;
    v[j] = (j < chunk && b < nblocks && c < ncols) ? partials[static_cast<size_t>(b) * ncols + c] : 0;
    sum += v[j];
  }
  s[rl][cl] = sum;
  __syncthreads();
  // inclusive scan over the slices (Hillis-Steele), then this slice's base
  for (int off = 1; off < kScanSlicesWide; off <<= 1) {
    const int add = rl >= off ? s[rl - off][cl] : 0;
    __syncthreads();
    s[rl][cl] += add;
    __syncthreads();
  }
  if (rl == kScanSlicesWide - 1 && c < ncols)
    partials[static_cast<size_t>(nblocks) * ncols + c] = s[rl][cl];
  int run = s[rl][cl] - sum;
#pragma unroll
  for (int j = 0; j < kScanRowsWide; ++j) {
    const int b = b0 + j;
    if (j < chunk && b < nblocks && c < ncols) {
      partials[static_cast<size_t>(b) * ncols + c] = run;
      run += v[j];
    }
  }
}

template <bool GROUPED>
__global__ __launch_bounds__(kBlock) void k_layout_place(LayoutArgs a, int ncols, int rounds,
                                                         int nblocks) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int E = a.E;
  const int nkeys = E + (GROUPED ? a.G : 0);
  uint64_t* bm = reinterpret_cast<uint64_t*>(smem);  // [kWavesPerBlock][nkeys]
  int* sbase = reinterpret_cast<int*>(bm + kWavesPerBlock * nkeys);  // [nkeys]
  int* run = sbase + nkeys;                                          // [nkeys]
  int* tmp = run + nkeys;                                            // [kWavesPerBlock]

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid & (kWave - 1);
  const int* tot = a.partials + static_cast<size_t>(nblocks) * ncols;
  const int* mine = a.partials + static_cast<size_t>(blockIdx.x) * ncols;
  const uint32_t base = blockIdx.x * static_cast<uint32_t>(rounds) * kBlock;
  // the first round's id, loaded early so its latency overlaps the scans
  int64_t v_next = (base + tid < a.n) ? a.idx[base + tid] : -1;
  // this thread's keys' totals and this block's tallies, loaded together
  // up front (keys tid, tid + kBlock, ...; at most EP_MAX_KEYS + 1 columns)
  constexpr int kKeysPerThread = (1024 + kBlock - 1) / kBlock + 1;
  int my_tot[kKeysPerThread], my_part[kKeysPerThread];
#pragma unroll
  for (int q = 0; q < kKeysPerThread; ++q) {
    const int c = tid + q * kBlock;
    my_tot[q] = c < nkeys ? tot[c] : 0;
    my_part[q] = c < nkeys ? mine[c] : 0;
  }

  // Segment bases: exclusive prefix sums over the experts of their counts
  // rounded up to the alignment, and (separately) over the groups.  The raw
  // expert counts are scanned too, for the number of selections.
  const int A = a.align;
#pragma unroll
  for (int q = 0; q < kKeysPerThread; ++q) {
    const int c = tid + q * kBlock;
    if (c < E) run[c] = my_tot[q];
    if (c < nkeys) sbase[c] = c < E ? (my_tot[q] + A - 1) / A * A : my_tot[q];
  }
  __syncthreads();
  const int n_sel = A > 1 ? block_exclusive_scan(run, E, tmp) : 0;
  const int n_rows_e = block_exclusive_scan(sbase, E, tmp);
  int n_rows = 0;
  if (GROUPED) n_rows = block_exclusive_scan(sbase + E, a.G, tmp);
  const bool lists_ok = !GROUPED || static_cast<int64_t>(n_rows) <= a.row_cap;
  const bool erows_ok =
      a.expert_row_src != nullptr && static_cast<int64_t>(n_rows_e) <= a.expert_row_cap;

  if (blockIdx.x == 0) {
    for (int e = tid; e < E; e += kBlock) {
      a.counts[e] = tot[e];
      a.offsets[e] = sbase[e];
      if (a.recv_stats) a.recv_stats[e] += static_cast<uint32_t>(tot[e]);
    }
    if (GROUPED) {
      for (int g = tid; g < a.G; g += kBlock) {
        a.gcounts[g] = tot[E + g];
        a.goffsets[g] = sbase[E + g];
      }
    }
    if (tid == 0) {
      a.offsets[E] = n_rows_e;
      if (GROUPED) a.goffsets[a.G] = n_rows;
      a.status[0] = tot[ncols - 1];
      a.status[1] = n_rows_e;
      a.status[2] = n_rows;
      a.status[3] = lists_ok ? 0 : 1;
      a.status[4] = 0;
      a.status[5] = (a.expert_row_src != nullptr && !erows_ok) ? 1 : 0;
      a.status[6] = A > 1 ? n_sel : n_rows_e;
      a.status[kStatusDispatchOverflow] = 0;
      a.status[kStatusGeneration] = static_cast<int32_t>(a.generation);
      a.status[kStatusStale] = 0;
      for (int w = kStatusStale + 1; w < 16; ++w) a.status[w] = 0;
    }
  }
  // alignment padding rows are marked unoccupied (-1); experts are spread
  // over the blocks
  if (A > 1 && erows_ok) {
    for (int e = blockIdx.x; e < E; e += gridDim.x) {
      const int r0 = sbase[e] + tot[e];
      const int r1 = sbase[e] + (tot[e] + A - 1) / A * A;
      for (int r = r0 + tid; r < r1; r += kBlock) a.expert_row_src[r] = -1;
    }
  }
  __syncthreads();  // run[] is reused below

  // This block's base per key: segment base + entries of earlier blocks.
#pragma unroll
  for (int q = 0; q < kKeysPerThread; ++q) {
    const int c = tid + q * kBlock;
    if (c < nkeys) {
      sbase[c] += my_part[q];
      run[c] = 0;
    }
  }
  for (int c = tid; c < kWavesPerBlock * nkeys; c += kBlock) bm[c] = 0;
  __syncthreads();

  uint64_t* wbm = bm + wave * nkeys;
  const uint64_t bit = 1ull << lane;
  const uint64_t lt = lanemask_lt();
  const bool lanes = GROUPED && kWave % a.K == 0;  // a token's entries in neighbouring lanes
  // the lanes path loads each round's weights one round ahead, with the ids
  const bool want_w = lanes && lists_ok && a.row_cap > 0 && a.w != nullptr;
  float w_next = want_w && base + tid < a.n ? a.w[base + tid] : 0.0f;
  for (int r = 0; r < rounds; ++r) {
    const uint32_t i = base + static_cast<uint32_t>(r) * kBlock + tid;
    const bool in = i < a.n;
    const int64_t v = v_next;
    const float w_cur = w_next;
    if (r + 1 < rounds) {
      const uint32_t i2 = i + kBlock;
      v_next = i2 < a.n ? a.idx[i2] : -1;
      if (want_w) w_next = i2 < a.n ? a.w[i2] : 0.0f;
    }
    const bool valid = in && v >= 0 && v < E;
    const int e = valid ? static_cast<int>(v) : -1;
    int kg = -1, g = 0;
    uint32_t t = 0;
    if (GROUPED && lanes) {
      g = valid ? e / a.epg : -1;
      t = i / static_cast<uint32_t>(a.K);
      if (first_in_group_lanes(g, a.K, lane)) kg = E + g;
    } else if (GROUPED && valid) {
      t = i / static_cast<uint32_t>(a.K);
      const int k = static_cast<int>(i - t * static_cast<uint32_t>(a.K));
      g = e / a.epg;
      if (first_in_group(a.idx, t, k, a.K, E, a.epg, g)) kg = E + g;
    }
    // Lanes of this wave holding the same key: bit-or into the wave's map,
    // read it back, and let the lowest such lane clear it again.
    if (e >= 0) atomicOr(reinterpret_cast<unsigned long long*>(&wbm[e]), bit);
    if (kg >= 0) atomicOr(reinterpret_cast<unsigned long long*>(&wbm[kg]), bit);
    __syncthreads();
    const uint64_t mE = e >= 0 ? wbm[e] : 0ull;
    const uint64_t mG = kg >= 0 ? wbm[kg] : 0ull;
    __syncthreads();
    const bool leadE = e >= 0 && (mE & lt) == 0;
    const bool leadG = kg >= 0 && (mG & lt) == 0;
    if (leadE) wbm[e] = 0ull;
    if (leadG) wbm[kg] = 0ull;
    // Claim slots wave by wave so earlier waves (earlier entries) rank first.
    int rankE = 0, rankG = 0;
    for (int w2 = 0; w2 < kWavesPerBlock; ++w2) {
      __syncthreads();
      if (wave == w2) {
        if (e >= 0) rankE = run[e] + __popcll(mE & lt);
        if (kg >= 0) rankG = run[kg] + __popcll(mG & lt);
        if (leadE) run[e] = rankE + __popcll(mE);
        if (leadG) run[kg] = rankG + __popcll(mG);
      }
    }
    if (in) a.slot[i] = e >= 0 ? sbase[e] + rankE : -1;
    if (erows_ok && e >= 0) a.expert_row_src[sbase[e] + rankE] = static_cast<int>(i / static_cast<uint32_t>(a.K));
    if (GROUPED && lanes) {
      // The token's K lanes share the rows its first-in-group lanes claimed:
      // each lane writes its own grow entry and its own position k of every
      // row of its token (coalesced across the K lanes).
      const int row = kg >= 0 ? sbase[kg] + rankG : -1;
      const int tb = lane & ~(a.K - 1);
      const int k = lane - tb;
      const int loc = valid ? e - g * a.epg : -1;
      const float wv = valid ? w_cur : 0.0f;
      int myrow = -1;
      for (int j = 0; j < a.K; ++j) {
        const int rj = __shfl(row, tb + j, kWave);  // row claimed by entry j, or -1
        const int gj = __shfl(g, tb + j, kWave);
        if (rj >= 0) {
          const bool same = valid && gj == g;
          if (same) myrow = rj;
          if (lists_ok) {
            const size_t rk = static_cast<size_t>(rj) * a.K + k;
            a.row_idx[rk] = same ? loc : -1;
            a.row_w[rk] = same ? wv : 0.0f;
          }
        }
      }
      if (in) a.grow[i] = myrow;
      if (kg >= 0 && lists_ok) a.row_src[row] = static_cast<int>(t);
    } else if (GROUPED && in) {
      if (!valid) a.grow[i] = -1;
      if (kg >= 0) {
        const int row = sbase[kg] + rankG;
        const size_t tk = static_cast<size_t>(t) * a.K;
        const size_t rk = static_cast<size_t>(row) * a.K;
        for (int kk = 0; kk < a.K; ++kk) {
          const int64_t v2 = a.idx[tk + kk];
          const bool same = v2 >= 0 && v2 < E && static_cast<int>(v2) / a.epg == g;
          if (same) a.grow[tk + kk] = row;
          if (lists_ok) {
            a.row_idx[rk + kk] = same ? static_cast<int>(v2) - g * a.epg : -1;
            a.row_w[rk + kk] = same ? a.w[tk + kk] : 0.0f;
          }
        }
        if (lists_ok) a.row_src[row] = static_cast<int>(t);
      }
    }
  }
}

}  // namespace

LayoutGeom layout_geom(int64_t n_entries, int E, int G) {
  LayoutGeom g;
  // One entry per thread on up to 256 blocks (the narrow scan's limit,
  // 16 * kScanRows); beyond that up to 2048 blocks (the wide scan's limit,
  // kScanSlicesWide * kScanRowsWide), each thread taking `rounds` entries.
  const int64_t max_blocks = n_entries <= static_cast<int64_t>(kBlock) * 16 * kScanRows
                                 ? 16 * kScanRows
                                 : kScanSlicesWide * kScanRowsWide;
  const int64_t per_round = static_cast<int64_t>(kBlock) * max_blocks;
  int64_t rounds = (n_entries + per_round - 1) / per_round;
  if (rounds < 1) rounds = 1;
  g.rounds = static_cast<int>(rounds);
  const int64_t chunk = rounds * kBlock;
  int64_t nb = (n_entries + chunk - 1) / chunk;
  if (nb < 1) nb = 1;
  g.nblocks = static_cast<int>(nb);
  g.ncols = E + G + 1;
  return g;
}

size_t layout_workspace_bytes(const LayoutGeom& g) {
  const size_t b = static_cast<size_t>(g.nblocks + 1) * g.ncols * sizeof(int32_t);
  return (b + 255) / 256 * 256;
}

hipError_t launch_layout(const LayoutArgs& a, const LayoutGeom& geo, hipStream_t s) {
  const bool grouped = a.G > 0;
  const size_t count_lds = static_cast<size_t>(geo.ncols) * sizeof(int);
  if (grouped)
    k_layout_count<true><<<geo.nblocks, kBlock, count_lds, s>>>(
        a.idx, a.n, a.K, a.E, a.epg, geo.ncols, geo.rounds, a.partials);
  else
    k_layout_count<false><<<geo.nblocks, kBlock, count_lds, s>>>(
        a.idx, a.n, a.K, a.E, a.epg, geo.ncols, geo.rounds, a.partials);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  if (geo.nblocks <= 16 * kScanRows)
    k_layout_colscan<<<(geo.ncols + kWave - 1) / kWave, 1024, 0, s>>>(a.partials, geo.nblocks,
                                                                      geo.ncols);
  else
    k_layout_colscan_wide<<<(geo.ncols + kScanColsWide - 1) / kScanColsWide, 1024, 0, s>>>(
        a.partials, geo.nblocks, geo.ncols);
  err = hipGetLastError();
  if (err != hipSuccess) return err;

  const int nkeys = a.E + (grouped ? a.G : 0);
  const size_t place_lds = static_cast<size_t>(kWavesPerBlock) * nkeys * sizeof(uint64_t) +
                           static_cast<size_t>(2 * nkeys + kWavesPerBlock) * sizeof(int);
  if (grouped)
    k_layout_place<true><<<geo.nblocks, kBlock, place_lds, s>>>(a, geo.ncols, geo.rounds,
                                                                geo.nblocks);
  else
    k_layout_place<false><<<geo.nblocks, kBlock, place_lds, s>>>(a, geo.ncols, geo.rounds,
                                                                 geo.nblocks);
  return hipGetLastError();
}

}  // namespace ep
