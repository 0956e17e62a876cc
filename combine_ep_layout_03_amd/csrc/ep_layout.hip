// Layout kernels: the three dispatch phases of TileScale PR #68 ("EP v2
// intranode dispatch/combine"; Design section and the commit adding DeepEP's
// do_expand) on one GPU, in two launches.
//   phase 1  k_layout_count   tallies per destination (expert, and group
//                             when grouped rows are asked for).  A count
//                             block covers `chunk` consecutive place blocks
//                             and writes, per place block, the tallies of
//                             the chunk's entries before it, and the chunk's
//                             totals
//   phase 2  (prologue of k_layout_place) every place block sums the chunk
//                             totals into the per-destination totals and the
//                             entries of earlier chunks, and scans the totals
//                             into segment bases; on one GPU the cross-rank
//                             count exchange reduces to this
//   phase 3  k_layout_place   base + locally claimed slot for every entry
// Up to kFusedRounds * 256 entries, one k_layout_place block runs all three
// phases in one launch: it tallies every entry itself (the count phase) and
// has no earlier blocks, so neither the count launch nor the workspace is
// used (128 tokens x top-2: 6.1 -> 3.1 us of GPU time per layout).
// The pages claim slots in whatever order lanes arrive; here the claim order
// is the (t,k) order, so placement is deterministic: inside a wave the rank
// comes from a match mask built with LDS bit-or (gfx950 has no match-any
// instruction), across the block's waves from running counters updated wave
// by wave, across blocks from the tallies.
//
// Workspace (int32, 16-byte aligned): [nblocks][ncols] per-place-block
// tallies of the earlier entries of its chunk, padded to a multiple of four
// ints, then the chunk totals in groups of four chunks,
// [ceil(ncount / 4)][ncols][4], so a place block reads four chunks' totals of
// a column with one 16-byte load.  Columns: E experts, G groups, invalid ids.
#include "ep_device.h"
#include "ep_internal.h"

namespace ep {

namespace {

constexpr int kCountThreads = 1024;  // threads per count block
constexpr int kCountBatch = 8;       // ids a count thread loads together
constexpr int kMaxCount = 32;        // count blocks (chunk-total rows) at most

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

// Value of lane (lane - J) when it lies in the same 16-lane row, else 0: the
// DPP row_shr:J move.
template <int J>
__device__ __forceinline__ int row_shr(int v) {
  return __builtin_amdgcn_update_dpp(0, v, 0x110 | J, 0xF, 0xF, false);
}

// The same test from the neighbouring lanes, when K divides the wave size:
// every block, round and wave starts at an entry index that is a multiple of
// 64, so lanes (lane & ~(K-1)) .. + K-1 hold one token's K entries in k
// order.  g is this entry's group, or -1 when it is not valid.  Every lane of
// the wave must call this.  For K <= 16 a token's lanes share one 16-lane
// row, and the earlier entries' groups arrive by DPP row shifts; wider
// tokens use LDS permutes.
__device__ __forceinline__ bool first_in_group_lanes(int g, int K, int lane, bool small_g) {
  bool first = g >= 0;
  const int kl = lane & (K - 1);  // k of this lane's entry
  if (K == 1) return first;
  if (K <= 16 && small_g) {
    // groups below 32: OR of the group bits of the token's earlier entries
    // (inclusive prefix OR in log2(K) row shifts, then one more shift)
    const int bit = first ? (1 << g) : 0;
    int inc = bit;
    int y = row_shr<1>(inc);
    inc |= kl >= 1 ? y : 0;
    if (K > 2) {
      y = row_shr<2>(inc);
      inc |= kl >= 2 ? y : 0;
    }
    if (K > 4) {
      y = row_shr<4>(inc);
      inc |= kl >= 4 ? y : 0;
    }
    if (K > 8) {
      y = row_shr<8>(inc);
      inc |= kl >= 8 ? y : 0;
    }
    y = row_shr<1>(inc);
    const int before = kl >= 1 ? y : 0;
    return first && (before & bit) == 0;
  }
  if (K <= 16) {
#define EP_SHR_TEST(J) \
    if (J < K) {       \
      const int gj = row_shr<J>(g); \
      if (kl >= J && gj == g) first = false; \
    }
    EP_SHR_TEST(1) EP_SHR_TEST(2) EP_SHR_TEST(3) EP_SHR_TEST(4) EP_SHR_TEST(5)
    EP_SHR_TEST(6) EP_SHR_TEST(7) EP_SHR_TEST(8) EP_SHR_TEST(9) EP_SHR_TEST(10)
    EP_SHR_TEST(11) EP_SHR_TEST(12) EP_SHR_TEST(13) EP_SHR_TEST(14) EP_SHR_TEST(15)
#undef EP_SHR_TEST
    return first;
  }
  const int base = lane - kl;
  for (int j = 0; j < K; ++j) {
    const int gj = __shfl(g, base + j, kWave);
    if (j < kl && gj == g) first = false;
  }
  return first;
}

// e / epg for 0 <= e < 1024 and 1 <= epg <= 1024, from a float reciprocal
// inv = fl(1 / epg): (e + 1/2) / epg lies at least 1/(2 epg) >= 2^-11 from an
// integer, while the two roundings move the float product by at most
// 1024 * 2^-23 = 2^-13, so truncation gives the exact quotient.
__device__ __forceinline__ int group_of(int e, float inv_epg) {
  return static_cast<int>((static_cast<float>(e) + 0.5f) * inv_epg);
}

// Tally one entry (global index i, id v) into the histogram h: its expert,
// or the invalid column, and (grouped) its group when it is the token's first
// entry in that group.  Every lane of the wave must call it (the lanes test
// reads the other lanes).
// Add one to column col of the histogram at word offset base (16-bit halves
// with HALF).
template <bool HALF>
__device__ __forceinline__ void hist_add(int* h, int base, int col) {
  const int x = base + col;
  if (HALF) atomicAdd(&h[x >> 1], 1 << ((x & 1) << 4));
  else atomicAdd(&h[x], 1);
}

// Tally one entry (global index i, id v) into the histogram at offset base:
// its expert, or the invalid column, and (grouped) its group when it is the
// token's first entry in that group.  Every lane of the wave must call it
// (the lanes test reads the other lanes).
template <bool GROUPED, bool HALF>
__device__ __forceinline__ void tally_entry(int* h, int base, const int64_t* __restrict__ idx,
                                            uint32_t i, int64_t v, int K, int E, int epg,
                                            float inv_epg, int ncols, bool lanes, bool small_g,
                                            int lane) {
  const bool valid = v >= 0 && v < E;
  const int e = valid ? static_cast<int>(v) : -1;
  const int col = valid ? e : (v != -1 ? ncols - 1 : -1);
  if (col >= 0) hist_add<HALF>(h, base, col);
  if (GROUPED) {
    if (lanes) {
      const int g = valid ? group_of(e, inv_epg) : -1;
      if (first_in_group_lanes(g, K, lane, small_g)) hist_add<HALF>(h, base, E + g);
    } else if (valid) {
      const uint32_t t = i / static_cast<uint32_t>(K);
      const int k = static_cast<int>(i - t * static_cast<uint32_t>(K));
      const int g = group_of(e, inv_epg);
      if (first_in_group(idx, t, k, K, E, epg, g)) hist_add<HALF>(h, base, E + g);
    }
  }
}

// Count block c: one LDS histogram per place block of its chunk, filled in
// parallel; then, per column, the running sum over the chunk's place blocks
// (workspace row b: the chunk's entries before place block b) and the chunk
// total (packed by fours, see above).  With HALF, a place block's tallies
// (at most its 2^span_shift <= 32768 entries) are 16-bit halves of the LDS
// words, so twice as many place blocks fit a count block.
template <bool GROUPED, bool HALF>
__global__ __launch_bounds__(kCountThreads) void k_layout_count(
    const int64_t* __restrict__ idx, uint32_t n, int K, int E, int epg, int ncols, int span_shift,
    int chunk, int nblocks, int packed_off, int* __restrict__ partials) {
  extern __shared__ int hist[];  // [chunk][ncols] ints, or halves of them with HALF
  const int pb0 = blockIdx.x * chunk;
  const int nsub = min(chunk, nblocks - pb0);
  const int nwords = HALF ? (nsub * ncols + 1) / 2 : nsub * ncols;
  const bool lanes = GROUPED && kWave % K == 0;  // a token's entries in neighbouring lanes
  const bool small_g = E / epg <= 32;
  const float inv_epg = 1.0f / static_cast<float>(epg);
  const int lane = threadIdx.x & (kWave - 1);
  // entry j of this thread is i = first + j * kCountThreads + tid; a place
  // block spans 2^span_shift entries (a multiple of the wave size, so a
  // wave's 64 entries never straddle two place blocks)
  const uint32_t first = static_cast<uint32_t>(pb0) << span_shift;
  const uint32_t count = static_cast<uint32_t>(nsub) << span_shift;  // may pass n
  const int per = n == 0 ? 0 : static_cast<int>((count + kCountThreads - 1) / kCountThreads);
  // all loads of a batch first (out-of-range lanes read index 0), the
  // out-of-range test only where the value is used, so no load waits for
  // the one before it; the first batch is in flight while the histograms
  // are cleared (the barrier waits for LDS work only)
  int64_t v[kCountBatch];
  auto load_batch = [&](int j0) {
#pragma unroll
    for (int u = 0; u < kCountBatch; ++u) {
      v[u] = -1;
      if (j0 + u < per) {  // block-uniform
        const uint32_t off = static_cast<uint32_t>(j0 + u) * kCountThreads + threadIdx.x;
        const bool ok = off < count && first + off < n;
        v[u] = idx[ok ? first + off : 0];  // n >= 1: index 0 is in bounds
      }
    }
  };
  load_batch(0);
  for (int c = threadIdx.x; c < nwords; c += kCountThreads) hist[c] = 0;
  __syncthreads();
  for (int j0 = 0; j0 < per; j0 += kCountBatch) {
    if (j0 > 0) load_batch(j0);
#pragma unroll
    for (int u = 0; u < kCountBatch; ++u) {
      if (j0 + u < per) {  // block-uniform
        const uint32_t off = static_cast<uint32_t>(j0 + u) * kCountThreads + threadIdx.x;
        const bool ok = off < count && first + off < n;
        const uint32_t sub = off < count ? off >> span_shift : 0;
        tally_entry<GROUPED, HALF>(hist, static_cast<int>(sub) * ncols, idx, first + off,
                                   ok ? v[u] : -1, K, E, epg, inv_epg, ncols, lanes, small_g, lane);
      }
    }
  }
  __syncthreads();
  int* packed = partials + packed_off;  // [ceil(ncount / 4)][nkeys][4], then invalid[ncount]
  const int nkeys = ncols - 1;
  const int grp = blockIdx.x >> 2, slot4 = blockIdx.x & 3;
  const int ngroups = (static_cast<int>(gridDim.x) + 3) / 4;
  // each column's running sum over the chunk's place blocks, eight LDS
  // reads in flight at a time
  constexpr int kEpiBatch = 8;
  for (int c = threadIdx.x; c < ncols; c += kCountThreads) {
    int run = 0;
    for (int s0 = 0; s0 < nsub; s0 += kEpiBatch) {
      int t[kEpiBatch];
#pragma unroll
      for (int u = 0; u < kEpiBatch; ++u) {
        const int x = (s0 + u) * ncols + c;
        t[u] = 0;
        if (s0 + u < nsub)  // block-uniform
          t[u] = HALF ? (static_cast<uint32_t>(hist[x >> 1]) >> ((x & 1) << 4)) & 0xFFFFu : hist[x];
      }
#pragma unroll
      for (int u = 0; u < kEpiBatch; ++u) {
        if (s0 + u < nsub) {
          partials[static_cast<size_t>(pb0 + s0 + u) * ncols + c] = run;
          run += t[u];
        }
      }
    }
    if (c < nkeys) packed[(static_cast<size_t>(grp) * nkeys + c) * 4 + slot4] = run;
    else packed[static_cast<size_t>(ngroups) * nkeys * 4 + blockIdx.x] = run;  // invalid ids
  }
}

// A place block reads, per key column it owns, the kChunkGroups int4 groups
// of chunk totals (four chunks each; groups past the last one re-read group
// 0 and are dropped), with a fixed load count so the first round's id load,
// issued before them, can be waited for alone.
constexpr int kChunkGroups = kMaxCount / 4;

struct ColumnChunks {
  int4 r[kChunkGroups];
};

__device__ __forceinline__ void column_load(const int4* __restrict__ packed, int nkeys, int c,
                                            int ngroups, ColumnChunks& b) {
  const int cc = c < nkeys ? c : 0;
#pragma unroll
  for (int q = 0; q < kChunkGroups; ++q)
    b.r[q] = packed[static_cast<size_t>(q < ngroups ? q : 0) * nkeys + cc];
}

// The column's total over every chunk, and over the chunks before my_chunk.
__device__ __forceinline__ void column_sum(const ColumnChunks& b, int ncount, int my_chunk,
                                           int& tot, int& pre) {
  tot = 0;
  pre = 0;
#pragma unroll
  for (int q = 0; q < kChunkGroups; ++q) {
    const int a[4] = {b.r[q].x, b.r[q].y, b.r[q].z, b.r[q].w};
#pragma unroll
    for (int l = 0; l < 4; ++l) {
      const int j = q * 4 + l;
      if (j < ncount) {
        tot += a[l];
        if (j < my_chunk) pre += a[l];
      }
    }
  }
}

// One round of a place block: the entry's key(s) and its ranks inside the
// block (rank phase), then its slot, grouped row and list writes (write
// phase, which needs the block's bases).
struct PlaceEntry {
  uint32_t i, t;
  bool in, valid;
  int e, kg, g;
  float w;
  int rankE, rankG;
};

// FUSED: one place block holds every entry (at most kFusedRounds rounds) and
// tallies them itself, so the count launch and the workspace are not used.
constexpr int kFusedRounds = 8;

template <bool GROUPED, int KS, bool FUSED>
__global__ __launch_bounds__(kBlock) void k_layout_place(LayoutArgs a, int ncols, int rounds,
                                                         int chunk, int ncount, int packed_off) {
  // KS key columns per thread: keys tid, tid + kBlock, ... (E + G <= KS * kBlock)
  extern __shared__ __align__(16) unsigned char smem[];
  const int E = a.E;
  const int nkeys = E + (GROUPED ? a.G : 0);
  uint64_t* bm = reinterpret_cast<uint64_t*>(smem);  // [kWavesPerBlock][nkeys]
  int* sbase = reinterpret_cast<int*>(bm + kWavesPerBlock * nkeys);  // [nkeys]
  int* run = sbase + nkeys;                                          // [nkeys]
  int* claim = run + nkeys;                                          // [nkeys]
  int* stot = claim + nkeys;                                         // [nkeys]
  int* tmp = stot + nkeys;                                           // [kWavesPerBlock]
  int* tally = tmp + kWavesPerBlock;  // FUSED: [ncols] tallies of all entries

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid & (kWave - 1);
  const int4* packed = reinterpret_cast<const int4*>(a.partials + packed_off);
  const int* mine = a.partials + static_cast<size_t>(blockIdx.x) * ncols;
  const int my_chunk = static_cast<int>(blockIdx.x) / chunk;
  const uint32_t base = blockIdx.x * static_cast<uint32_t>(rounds) * kBlock;
  const bool lanes = GROUPED && kWave % a.K == 0;  // a token's entries in neighbouring lanes
  const bool small_g = a.G <= 32;
  const float inv_epg = 1.0f / static_cast<float>(a.epg);
  const int k_shift = 31 - __builtin_clz(static_cast<unsigned>(a.K));  // log2 K when lanes
  // the lanes path loads each round's weights one round ahead, with the ids
  const bool want_w = lanes && a.row_cap > 0 && a.w != nullptr;

  // The first round's id (and weight), then this thread's columns of the
  // chunk totals, its invalid-id chunk count and this block's own tallies:
  // a fixed number of loads, all in flight together, and still in flight
  // while the first round ranks its entries in LDS.
  // (loads past the entries read the last one: whether an entry is in range
  // is decided where it is used, so no load waits for the test; a.n == 0 is
  // the one case with nothing to read)
  const uint32_t last = a.n ? a.n - 1 : 0;
  const uint32_t i0 = base + tid < a.n ? base + tid : last;
  int64_t v_next = a.n ? a.idx[i0] : -1;
  float w_next = want_w && a.n ? a.w[i0] : 0.0f;
  const int ngroups = (ncount + 3) / 4;
  ColumnChunks cols[KS];
  int inv_v = 0;
  int mine_v[KS];
  int64_t vf[FUSED ? kFusedRounds : 1];
  if constexpr (FUSED) {
    // every round's id at once (out-of-range rounds and entries read the last)
#pragma unroll
    for (int r = 0; r < kFusedRounds; ++r) {
      const uint32_t i = static_cast<uint32_t>(r) * kBlock + tid;
      vf[r] = r < rounds && a.n ? a.idx[i < a.n ? i : last] : -1;
    }
  } else {
#pragma unroll
    for (int q = 0; q < KS; ++q) column_load(packed, nkeys, tid + q * kBlock, ngroups, cols[q]);
    const int* invalid_chunk = a.partials + packed_off + static_cast<size_t>(ngroups) * nkeys * 4;
    inv_v = invalid_chunk[tid < ncount ? tid : 0];
#pragma unroll
    for (int q = 0; q < KS; ++q) {
      const int c = tid + q * kBlock;
      mine_v[q] = mine[c < nkeys ? c : 0];
    }
  }

  for (int c = tid; c < nkeys; c += kBlock) claim[c] = 0;
  for (int c = tid; c < kWavesPerBlock * nkeys; c += kBlock) bm[c] = 0;
  if (FUSED)
    for (int c = tid; c < ncols; c += kBlock) tally[c] = 0;
  __syncthreads();
  if constexpr (FUSED) {
    // the count phase, on this block's own entries (all of them)
#pragma unroll
    for (int r = 0; r < kFusedRounds; ++r) {
      if (r < rounds) {  // block-uniform
        const uint32_t i = static_cast<uint32_t>(r) * kBlock + tid;
        tally_entry<GROUPED, false>(tally, 0, a.idx, i, i < a.n ? vf[r] : -1, a.K, E, a.epg,
                                    inv_epg, ncols, lanes, small_g, lane);
      }
    }
    // rank_phase(0) below starts with a barrier-separated LDS pass, after
    // which every tally is complete
  }

  uint64_t* wbm = bm + wave * nkeys;
  const uint64_t bit = 1ull << lane;
  const uint64_t lt = lanemask_lt();

  // Rank phase of round r: keys, match masks, ranks in (t,k) order.
  auto rank_phase = [&](int r) {
    PlaceEntry q;
    q.i = base + static_cast<uint32_t>(r) * kBlock + tid;
    q.in = q.i < a.n;
    const int64_t v = v_next;
    q.w = w_next;
    if (r + 1 < rounds) {
      const uint32_t i2 = q.i + kBlock;
      v_next = a.idx[i2 < a.n ? i2 : last];  // rounds > 1: a.n > 0
      if (want_w) w_next = a.w[i2 < a.n ? i2 : last];
    }
    q.valid = q.in && v >= 0 && v < E;
    q.e = q.valid ? static_cast<int>(v) : -1;
    q.kg = -1;
    q.g = 0;
    q.t = 0;
    if (GROUPED && lanes) {
      q.g = q.valid ? group_of(q.e, inv_epg) : -1;
      q.t = q.i >> k_shift;  // K is a power of two here
      if (first_in_group_lanes(q.g, a.K, lane, small_g)) q.kg = E + q.g;
    } else if (GROUPED && q.valid) {
      q.t = q.i / static_cast<uint32_t>(a.K);
      const int k = static_cast<int>(q.i - q.t * static_cast<uint32_t>(a.K));
      q.g = group_of(q.e, inv_epg);
      if (first_in_group(a.idx, q.t, k, a.K, E, a.epg, q.g)) q.kg = E + q.g;
    }
    // Lanes of this wave holding the same key: bit-or into the wave's map,
    // read it back, and let the lowest such lane clear it again.
    if (q.e >= 0) atomicOr(reinterpret_cast<unsigned long long*>(&wbm[q.e]), bit);
    if (q.kg >= 0) atomicOr(reinterpret_cast<unsigned long long*>(&wbm[q.kg]), bit);
    __syncthreads();
    const uint64_t mE = q.e >= 0 ? wbm[q.e] : 0ull;
    const uint64_t mG = q.kg >= 0 ? wbm[q.kg] : 0ull;
    __syncthreads();
    const bool leadE = q.e >= 0 && (mE & lt) == 0;
    const bool leadG = q.kg >= 0 && (mG & lt) == 0;
    if (leadE) wbm[q.e] = 0ull;
    if (leadG) wbm[q.kg] = 0ull;
    // Claim ranks wave by wave so earlier waves (earlier entries) rank first.
    q.rankE = 0;
    q.rankG = 0;
    for (int w2 = 0; w2 < kWavesPerBlock; ++w2) {
      __syncthreads();
      if (wave == w2) {
        if (q.e >= 0) q.rankE = claim[q.e] + __popcll(mE & lt);
        if (q.kg >= 0) q.rankG = claim[q.kg] + __popcll(mG & lt);
        if (leadE) claim[q.e] = q.rankE + __popcll(mE);
        if (leadG) claim[q.kg] = q.rankG + __popcll(mG);
      }
    }
    return q;
  };

  PlaceEntry first = rank_phase(0);

  // Per key: the total over every chunk, and this block's entries-before =
  // the earlier chunks' totals + the tallies of its own chunk before it.
  int my_tot[KS], my_part[KS];
#pragma unroll
  for (int q = 0; q < KS; ++q) {
    const int c = tid + q * kBlock;
    int t = 0, p = 0;
    if constexpr (FUSED) t = tally[c < nkeys ? c : 0];
    else column_sum(cols[q], ncount, my_chunk, t, p);
    my_tot[q] = c < nkeys ? t : 0;
    my_part[q] = c < nkeys ? (FUSED ? 0 : p + mine_v[q]) : 0;
  }
  // invalid ids (block 0 only reports them): the chunk counts summed by wave 0
  int invalid_ids = 0;
  if (FUSED) {
    invalid_ids = tally[ncols - 1];
  } else if (wave == 0) {
    int x = tid < ncount ? inv_v : 0;
    x += __shfl_xor(x, 1, kWave);
    x += __shfl_xor(x, 2, kWave);
    x += __shfl_xor(x, 4, kWave);
    x += __shfl_xor(x, 8, kWave);
    x += __shfl_xor(x, 16, kWave);
    invalid_ids = x;  // kMaxCount = 32 chunks: lanes 0..31 hold the sum
  }

  // Segment bases: exclusive prefix sums over the experts of their counts
  // rounded up to the alignment, and (separately) over the groups.  The raw
  // expert counts are scanned too, for the number of selections.
  const int A = a.align;
#pragma unroll
  for (int q = 0; q < KS; ++q) {
    const int c = tid + q * kBlock;
    if (c < E) run[c] = my_tot[q];
    if (c < nkeys) {
      stot[c] = my_tot[q];
      sbase[c] = c < E ? (my_tot[q] + A - 1) / A * A : my_tot[q];
    }
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
      a.counts[e] = stot[e];
      a.offsets[e] = sbase[e];
      if (a.recv_stats) a.recv_stats[e] += static_cast<uint32_t>(stot[e]);
    }
    if (GROUPED) {
      for (int g = tid; g < a.G; g += kBlock) {
        a.gcounts[g] = stot[E + g];
        a.goffsets[g] = sbase[E + g];
      }
    }
    if (tid == 0) {
      a.offsets[E] = n_rows_e;
      if (GROUPED) a.goffsets[a.G] = n_rows;
      a.status[0] = invalid_ids;  // thread 0 is in wave 0
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
      const int r0e = sbase[e] + stot[e];
      const int r1e = sbase[e] + (stot[e] + A - 1) / A * A;
      for (int r = r0e + tid; r < r1e; r += kBlock) a.expert_row_src[r] = -1;
    }
  }
  __syncthreads();  // every thread has read sbase as a segment base

  // This block's base per key: segment base + entries of earlier blocks.
#pragma unroll
  for (int q = 0; q < KS; ++q) {
    const int c = tid + q * kBlock;
    if (c < nkeys) sbase[c] += my_part[q];
  }
  __syncthreads();

  // Write phase: slot, expert row source, grouped row and row lists.
  auto write_phase = [&](const PlaceEntry& q) {
    if (q.in) a.slot[q.i] = q.e >= 0 ? sbase[q.e] + q.rankE : -1;
    if (erows_ok && q.e >= 0)
      a.expert_row_src[sbase[q.e] + q.rankE] = static_cast<int>(q.i / static_cast<uint32_t>(a.K));
    if (GROUPED && lanes) {
      // The token's K lanes share the rows its first-in-group lanes claimed:
      // each lane writes its own grow entry and its own position k of every
      // row of its token (coalesced across the K lanes).
      const int row = q.kg >= 0 ? sbase[q.kg] + q.rankG : -1;
      const int tb = lane & ~(a.K - 1);
      const int k = lane - tb;
      const int loc = q.valid ? q.e - q.g * a.epg : -1;
      const float wv = q.valid ? q.w : 0.0f;
      int myrow = -1;
      for (int j = 0; j < a.K; ++j) {
        const int rj = __shfl(row, tb + j, kWave);  // row claimed by entry j, or -1
        const int gj = __shfl(q.g, tb + j, kWave);
        if (rj >= 0) {
          const bool same = q.valid && gj == q.g;
          if (same) myrow = rj;
          if (lists_ok) {
            const size_t rk = static_cast<size_t>(rj) * a.K + k;
            a.row_idx[rk] = same ? loc : -1;
            a.row_w[rk] = same ? wv : 0.0f;
          }
        }
      }
      if (q.in) a.grow[q.i] = myrow;
      if (q.kg >= 0 && lists_ok) a.row_src[row] = static_cast<int>(q.t);
    } else if (GROUPED && q.in) {
      if (!q.valid) a.grow[q.i] = -1;
      if (q.kg >= 0) {
        const int row = sbase[q.kg] + q.rankG;
        const size_t tk = static_cast<size_t>(q.t) * a.K;
        const size_t rk = static_cast<size_t>(row) * a.K;
        for (int kk = 0; kk < a.K; ++kk) {
          const int64_t v2 = a.idx[tk + kk];
          const bool same = v2 >= 0 && v2 < E && static_cast<int>(v2) / a.epg == q.g;
          if (same) a.grow[tk + kk] = row;
          if (lists_ok) {
            a.row_idx[rk + kk] = same ? static_cast<int>(v2) - q.g * a.epg : -1;
            a.row_w[rk + kk] = same ? a.w[tk + kk] : 0.0f;
          }
        }
        if (lists_ok) a.row_src[row] = static_cast<int>(q.t);
      }
    }
  };

  write_phase(first);
  for (int r = 1; r < rounds; ++r) write_phase(rank_phase(r));
}

}  // namespace

// LDS ints a count block's histograms may take (64 KiB), and place blocks at
// most.
constexpr int kCountLdsInts = 16384;
constexpr int kMaxPlaceBlocks = 512;

LayoutGeom layout_geom(int64_t n_entries, int E, int G) {
  LayoutGeom g;
  g.ncols = E + G + 1;
  // Place blocks of 256 * rounds entries (rounds a power of two), as many as
  // kMaxPlaceBlocks and the count blocks' LDS allow: kMaxCount count blocks
  // of at most by_lds place blocks each, whose tallies take 16-bit halves of
  // the LDS words while a place block spans at most 32768 entries.
  // 32-bit tallies when they reach kMaxPlaceBlocks (adding 1 to a 16-bit half
  // costs a little more), halves when that lets more place blocks in
  const int full_blocks = kMaxCount * (kCountLdsInts / g.ncols);
  for (int half = full_blocks >= kMaxPlaceBlocks ? 0 : 1; half >= 0; --half) {
    const int by_lds = kCountLdsInts * (half ? 2 : 1) / g.ncols;
    int64_t max_blocks = static_cast<int64_t>(kMaxCount) * by_lds;
    if (max_blocks > kMaxPlaceBlocks) max_blocks = kMaxPlaceBlocks;
    int shift = 8;  // log2 of the place-block span
    while ((static_cast<int64_t>(1) << shift) * max_blocks < n_entries) ++shift;
    if (half && shift > 15) continue;  // halves hold at most 32768 entries' tallies
    g.half = half;
    g.rounds = 1 << (shift - 8);
    g.span_shift = shift;
    const int64_t span = static_cast<int64_t>(1) << shift;
    int64_t nb = (n_entries + span - 1) / span;
    if (nb < 1) nb = 1;
    g.nblocks = static_cast<int>(nb);
    int chunk = (g.nblocks + kMaxCount - 1) / kMaxCount;  // <= by_lds by the choice of span
    if (chunk < 1) chunk = 1;
    g.chunk = chunk;
    g.ncount = (g.nblocks + chunk - 1) / chunk;
    break;
  }
  return g;
}

// Ints before the packed chunk totals: the per-place-block rows, rounded up
// so the packed groups start on a 16-byte boundary.
static int64_t packed_offset(const LayoutGeom& g) {
  return (static_cast<int64_t>(g.nblocks) * g.ncols + 3) / 4 * 4;
}

size_t layout_workspace_bytes(const LayoutGeom& g) {
  const size_t ints = static_cast<size_t>(packed_offset(g)) +
                      static_cast<size_t>((g.ncount + 3) / 4) * 4 * (g.ncols - 1) + g.ncount;
  const size_t b = ints * sizeof(int32_t);
  return (b + 255) / 256 * 256;
}

hipError_t launch_layout(const LayoutArgs& a, const LayoutGeom& geo, hipStream_t s) {
  const bool grouped = a.G > 0;
  if (a.n <= static_cast<uint32_t>(kFusedRounds * kBlock)) {
    // Small problems: one block tallies and places every entry, one launch.
    int rounds = 1;
    while (static_cast<uint32_t>(rounds * kBlock) < a.n) rounds *= 2;
    const int nkeys = a.E + (grouped ? a.G : 0);
    const size_t lds = static_cast<size_t>(kWavesPerBlock) * nkeys * sizeof(uint64_t) +
                       static_cast<size_t>(4 * nkeys + kWavesPerBlock + geo.ncols) * sizeof(int);
    const int ks = nkeys <= kBlock ? 1 : nkeys <= 2 * kBlock ? 2 : 4;
#define EP_FUSED(GR, KS) \
  k_layout_place<GR, KS, true><<<1, kBlock, lds, s>>>(a, geo.ncols, rounds, 1, 1, 0)
    if (grouped) {
      if (ks == 1) EP_FUSED(true, 1);
      else if (ks == 2) EP_FUSED(true, 2);
      else EP_FUSED(true, 4);
    } else {
      if (ks == 1) EP_FUSED(false, 1);
      else if (ks == 2) EP_FUSED(false, 2);
      else EP_FUSED(false, 4);
    }
#undef EP_FUSED
    return hipGetLastError();
  }
  // the geometry guarantees both
  const int64_t words = geo.half ? (static_cast<int64_t>(geo.chunk) * geo.ncols + 1) / 2
                                 : static_cast<int64_t>(geo.chunk) * geo.ncols;
  if (geo.ncount > kMaxCount || words > kCountLdsInts) return hipErrorInvalidValue;
  const int poff = static_cast<int>(packed_offset(geo));
  const size_t count_lds = static_cast<size_t>(words) * sizeof(int);
#define EP_COUNT(GR, HF)                                                                   \
  k_layout_count<GR, HF><<<geo.ncount, kCountThreads, count_lds, s>>>(                   \
      a.idx, a.n, a.K, a.E, a.epg, geo.ncols, geo.span_shift, geo.chunk, geo.nblocks, poff, \
      a.partials)
  if (grouped) {
    if (geo.half) EP_COUNT(true, true);
    else EP_COUNT(true, false);
  } else {
    if (geo.half) EP_COUNT(false, true);
    else EP_COUNT(false, false);
  }
#undef EP_COUNT
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  const int nkeys = a.E + (grouped ? a.G : 0);
  const size_t place_lds = static_cast<size_t>(kWavesPerBlock) * nkeys * sizeof(uint64_t) +
                           static_cast<size_t>(4 * nkeys + kWavesPerBlock + geo.ncols) * sizeof(int);
  const int ks = nkeys <= kBlock ? 1 : nkeys <= 2 * kBlock ? 2 : 4;
#define EP_PLACE(GR, KS)                                                                        \
  k_layout_place<GR, KS, false><<<geo.nblocks, kBlock, place_lds, s>>>(a, geo.ncols, geo.rounds, \
                                                                        geo.chunk, geo.ncount, poff)
  if (grouped) {
    if (ks == 1) EP_PLACE(true, 1);
    else if (ks == 2) EP_PLACE(true, 2);
    else EP_PLACE(true, 4);
  } else {
    if (ks == 1) EP_PLACE(false, 1);
    else if (ks == 2) EP_PLACE(false, 2);
    else EP_PLACE(false, 4);
  }
#undef EP_PLACE
  return hipGetLastError();
}

}  // namespace ep
