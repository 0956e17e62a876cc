/*
 * The C ABI used from plain C (C99, built with gcc): layout, bf16 and fp8
 * dispatch, flat and grouped combine, grouped rows and the grouped GEMM on
 * one GPU, checked against closed forms rather than an oracle.
 *
 * Routing: T tokens pick K distinct experts (e = (7t + 5k) mod E); some
 * entries are masked (-1) and one id is out of range (counted in the
 * invalid-id status word and treated as -1).  Token rows hold integers in
 * [-7, 7], so the combine of the dispatched rows with unit weights must
 * return every token as exactly K_eff * x (fp32 sums of small integers are
 * exact, and so is their bf16 rounding).
 *
 * The fp8 dispatch of the same rows: every 128-element group holds the values
 * -7..7 (period 15 along h), so its amax is 7, its scale 7/448 = 2^-6 exactly,
 * and every payload byte is the E4M3FN code of 64 * x, an exactly
 * representable value (64 .. 448), so the packed row is known byte for byte.
 *
 * Grouped rows (G = 4 groups of 4 experts): every selection's group row holds
 * its token's row, the row lists name the token and its local experts, and
 * the grouped-order combine of the expert rows is again K_eff * x.
 *
 * The grouped GEMM then multiplies the dispatched rows by weights in
 * {-1, 0, 1} (N = 128), once with the weights as given and once packed by
 * ep_pack_expert_weights: every partial sum is an exact fp32 integer, so
 * both must equal the bf16 rounding (nearest, ties to even) of the exact
 * sum, computed here on the host.
 *
 * A dispatch one row short of capacity must write nothing and set the
 * overflow status word; a copy of the layout struct taken before a later
 * ep_layout on the same buffers (a stale cached handle) must make dispatch
 * and combine write nothing and set the stale word.
 *
 * Prints "OK" and exits 0 on success; prints the first mismatch and exits
 * 1 otherwise.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ep_mi355x.h"

#define T 512
#define H 256
#define K 4
#define E 16
#define N 128

#define CHECK_HIP(x)                                                          \
  do {                                                                        \
    hipError_t e_ = (x);                                                      \
    if (e_ != hipSuccess) {                                                   \
      printf("HIP error %d at line %d\n", (int)e_, __LINE__);                 \
      return 1;                                                               \
    }                                                                         \
  } while (0)

#define CHECK_EP(x)                                                           \
  do {                                                                        \
    int r_ = (x);                                                             \
    if (r_ != EP_OK) {                                                        \
      printf("ep error %d (%s) at line %d\n", r_, ep_strerror(r_), __LINE__); \
      return 1;                                                               \
    }                                                                         \
  } while (0)

static uint16_t bf16_of_int(int v) {
  float f = (float)v;
  uint32_t b;
  memcpy(&b, &f, 4);
  return (uint16_t)(b >> 16); /* exact for small integers */
}

/* bf16 of an exactly representable fp32 value, round to nearest even */
static uint16_t bf16_rne_of_int(int v) {
  float f = (float)v;
  uint32_t b;
  memcpy(&b, &f, 4);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

/* E4M3FN code of 64 * v for an integer v in [-7, 7]: 2^6 .. 1.75 * 2^8 */
static uint8_t e4m3_of_64x(int v) {
  static const uint8_t mag[8] = {0x00, 0x68, 0x70, 0x74, 0x78, 0x7A, 0x7C, 0x7E};
  return (uint8_t)(mag[v < 0 ? -v : v] | (v < 0 ? 0x80 : 0x00));
}

static int gemm_weight(int e, int n, int h) { return (e + n * 5 + h * 7) % 3 - 1; }

static int int_of_bf16(uint16_t h) {
  uint32_t b = (uint32_t)h << 16;
  float f;
  memcpy(&f, &b, 4);
  return (int)f;
}

int main(void) {
  static int64_t idx[T * K];
  static float w[T * K];
  static uint16_t x[T * H], out[T * H];
  static int32_t slot[T * K], counts[E], status[EP_STATUS_WORDS];
  int keff[T];
  int t, k, h, e;
  int n_sel = 0, n_invalid = 0;

  for (t = 0; t < T; ++t) {
    keff[t] = 0;
    for (k = 0; k < K; ++k) {
      int64_t id = (7 * t + 5 * k) % E;
      if (t % 9 == 0 && k == 3) id = -1;    /* masked */
      if (t % 31 == 0 && k == 1) id = -1;   /* masked */
      if (t == 7 && k == 2) id = E + 5;     /* out of range: invalid */
      idx[t * K + k] = id;
      w[t * K + k] = 1.0f;
      if (id >= 0 && id < E) {
        ++keff[t];
        ++n_sel;
      } else if (id != -1) {
        ++n_invalid;
      }
    }
    for (h = 0; h < H; ++h) x[t * H + h] = bf16_of_int((t * 13 + h * 7) % 15 - 7);
  }

  ep_problem_t p;
  memset(&p, 0, sizeof p);
  p.num_tokens = T;
  p.hidden = H;
  p.topk = K;
  p.num_experts = E;

  /* host-side checks that need no device */
  if (ep_fp8_row_bytes(7168) != 7392 || ep_fp8_row_bytes(100) != -1) {
    printf("ep_fp8_row_bytes disagrees with the packed-row size\n");
    return 1;
  }
  const size_t ws_bytes = ep_layout_workspace_bytes(&p);
  if (ws_bytes == 0) {
    printf("ep_layout_workspace_bytes returned 0\n");
    return 1;
  }

  hipStream_t s;
  CHECK_HIP(hipStreamCreate(&s));
  int64_t* d_idx;
  float* d_w;
  uint16_t *d_x, *d_recv, *d_out;
  int32_t *d_counts, *d_offsets, *d_slot, *d_status;
  void* d_ws;
  CHECK_HIP(hipMalloc((void**)&d_idx, sizeof idx));
  CHECK_HIP(hipMalloc((void**)&d_w, sizeof w));
  CHECK_HIP(hipMalloc((void**)&d_x, sizeof x));
  CHECK_HIP(hipMalloc((void**)&d_recv, (size_t)T * K * H * 2));
  CHECK_HIP(hipMalloc((void**)&d_out, sizeof out));
  CHECK_HIP(hipMalloc((void**)&d_counts, E * 4));
  CHECK_HIP(hipMalloc((void**)&d_offsets, (E + 1) * 4));
  CHECK_HIP(hipMalloc((void**)&d_slot, T * K * 4));
  CHECK_HIP(hipMalloc((void**)&d_status, EP_STATUS_WORDS * 4));
  CHECK_HIP(hipMalloc(&d_ws, ws_bytes));
  CHECK_HIP(hipMemcpy(d_idx, idx, sizeof idx, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_w, w, sizeof w, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(d_x, x, sizeof x, hipMemcpyHostToDevice));

  ep_layout_t L;
  memset(&L, 0, sizeof L);
  L.counts = d_counts;
  L.offsets = d_offsets;
  L.slot = d_slot;
  L.status = d_status;

  /* an fp8 dispatch of a hidden size that is not a multiple of 128 is
     refused on the host, before anything is enqueued */
  {
    ep_problem_t q = p;
    q.hidden = 100;
    if (ep_dispatch(&q, &L, d_x, d_recv, T * K, 0, EP_ROWS_EXPERT, EP_FORMAT_FP8_PACKED, s) !=
        EP_ENOTSUP) {
      printf("fp8 dispatch with hidden 100 was not refused\n");
      return 1;
    }
  }

  CHECK_EP(ep_layout(&p, d_idx, d_w, &L, d_ws, ws_bytes, s));
  CHECK_EP(ep_dispatch(&p, &L, d_x, d_recv, T * K, 0, EP_ROWS_EXPERT, EP_FORMAT_BF16, s));
  CHECK_EP(ep_combine(&p, &L, NULL, d_w, d_recv, T * K, NULL, NULL, d_out, EP_COMBINE_FLAT, s));
  CHECK_HIP(hipStreamSynchronize(s));
  CHECK_HIP(hipMemcpy(slot, d_slot, sizeof slot, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(counts, d_counts, sizeof counts, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(status, d_status, sizeof status, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(out, d_out, sizeof out, hipMemcpyDeviceToHost));

  if (status[EP_STATUS_INVALID_IDS] != n_invalid || status[EP_STATUS_SELECTIONS] != n_sel ||
      status[EP_STATUS_ROWS_EXPERT] != n_sel) {
    printf("status words %d %d %d, expected %d %d %d\n", status[EP_STATUS_INVALID_IDS],
           status[EP_STATUS_SELECTIONS], status[EP_STATUS_ROWS_EXPERT], n_invalid, n_sel, n_sel);
    return 1;
  }
  {
    int sum = 0;
    for (e = 0; e < E; ++e) sum += counts[e];
    if (sum != n_sel) {
      printf("counts sum to %d, expected %d\n", sum, n_sel);
      return 1;
    }
  }
  /* slots of the valid selections are a permutation of [0, n_sel) */
  {
    static unsigned char seen[T * K];
    memset(seen, 0, sizeof seen);
    for (t = 0; t < T * K; ++t) {
      const int64_t id = idx[t];
      const int valid = id >= 0 && id < E;
      if (!valid) {
        if (slot[t] != -1) {
          printf("entry %d: no selection but slot %d\n", t, slot[t]);
          return 1;
        }
        continue;
      }
      if (slot[t] < 0 || slot[t] >= n_sel || seen[slot[t]]) {
        printf("entry %d: slot %d out of range or repeated\n", t, slot[t]);
        return 1;
      }
      seen[slot[t]] = 1;
    }
  }
  for (t = 0; t < T; ++t)
    for (h = 0; h < H; ++h) {
      const int want = keff[t] * ((t * 13 + h * 7) % 15 - 7);
      const int got = int_of_bf16(out[t * H + h]);
      if (got != want) {
        printf("token %d element %d: combine gave %d, expected %d\n", t, h, got, want);
        return 1;
      }
    }

  /* fp8 dispatch: payload, scales and padding of every packed row */
  {
    const int64_t rb = ep_fp8_row_bytes(H);
    static uint8_t recv8[(size_t)T * K * 272];
    uint8_t* d_recv8;
    if (rb != 272) {
      printf("fp8 row bytes %lld, expected 272\n", (long long)rb);
      return 1;
    }
    CHECK_HIP(hipMalloc((void**)&d_recv8, (size_t)T * K * rb));
    CHECK_EP(ep_dispatch(&p, &L, d_x, d_recv8, T * K, 0, EP_ROWS_EXPERT, EP_FORMAT_FP8_PACKED, s));
    CHECK_HIP(hipStreamSynchronize(s));
    CHECK_HIP(hipMemcpy(recv8, d_recv8, (size_t)n_sel * rb, hipMemcpyDeviceToHost));
    for (t = 0; t < T * K; ++t) {
      if (slot[t] < 0) continue;
      const uint8_t* row = recv8 + (size_t)slot[t] * rb;
      const int tok = t / K;
      for (h = 0; h < H; ++h)
        if (row[h] != e4m3_of_64x((tok * 13 + h * 7) % 15 - 7)) {
          printf("fp8 row of entry %d, byte %d: %02x, expected %02x\n", t, h, row[h],
                 e4m3_of_64x((tok * 13 + h * 7) % 15 - 7));
          return 1;
        }
      for (h = H; h < rb; ++h) {
        /* scales 2^-6 = 0x3C800000 little-endian, then zero padding */
        const int i = h - H;
        const uint8_t want = i < 4 * (H / 128) ? (uint8_t[]){0x00, 0x00, 0x80, 0x3C}[i % 4] : 0;
        if (row[h] != want) {
          printf("fp8 row of entry %d, tail byte %d: %02x, expected %02x\n", t, i, row[h], want);
          return 1;
        }
      }
    }
    hipFree(d_recv8);
  }

  /* Dispatch overflow and the stale-layout guard.  A capacity one row short
     writes no row and raises EP_STATUS_DISPATCH_OVERFLOW; a copy of the
     layout struct taken before a later ep_layout on the same buffers is a
     stale handle: dispatch and combine then write nothing and raise the
     sticky EP_STATUS_STALE, which the next ep_layout clears. */
  {
    const size_t nbytes = (size_t)T * K * H * 2;
    static uint8_t poison[(size_t)T * K * H * 2];
    uint8_t* d_poison;
    uint16_t* d_out2;
    size_t i;
    CHECK_HIP(hipMalloc((void**)&d_poison, nbytes));
    CHECK_HIP(hipMalloc((void**)&d_out2, sizeof out));
    CHECK_HIP(hipMemset(d_poison, 0xAB, nbytes));
    CHECK_HIP(hipMemset(d_out2, 0xCD, sizeof out));
    CHECK_EP(ep_dispatch(&p, &L, d_x, d_poison, n_sel - 1, 0, EP_ROWS_EXPERT, EP_FORMAT_BF16, s));
    CHECK_HIP(hipStreamSynchronize(s));
    CHECK_HIP(hipMemcpy(status, d_status, sizeof status, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(poison, d_poison, nbytes, hipMemcpyDeviceToHost));
    if (status[EP_STATUS_DISPATCH_OVERFLOW] != 1 || status[EP_STATUS_STALE] != 0) {
      printf("capacity n_sel - 1: overflow word %d, stale word %d, expected 1, 0\n",
             status[EP_STATUS_DISPATCH_OVERFLOW], status[EP_STATUS_STALE]);
      return 1;
    }
    for (i = 0; i < nbytes; ++i)
      if (poison[i] != 0xAB) {
        printf("overflowing dispatch wrote byte %zu\n", i);
        return 1;
      }
    CHECK_EP(ep_dispatch(&p, &L, d_x, d_poison, n_sel, 0, EP_ROWS_EXPERT, EP_FORMAT_BF16, s));
    CHECK_HIP(hipStreamSynchronize(s));
    CHECK_HIP(hipMemcpy(status, d_status, sizeof status, hipMemcpyDeviceToHost));
    if (status[EP_STATUS_DISPATCH_OVERFLOW] != 0) {
      printf("capacity n_sel: overflow word %d, expected 0\n", status[EP_STATUS_DISPATCH_OVERFLOW]);
      return 1;
    }

    const ep_layout_t old = L; /* a cached handle to this layout */
    if (L.generation == 0 || (uint32_t)status[EP_STATUS_GENERATION] != L.generation) {
      printf("generation %u, device stamp %d\n", L.generation, status[EP_STATUS_GENERATION]);
      return 1;
    }
    CHECK_EP(ep_layout(&p, d_idx, d_w, &L, d_ws, ws_bytes, s)); /* same buffers rewritten */
    if (L.generation == old.generation) {
      printf("ep_layout did not advance the generation\n");
      return 1;
    }
    CHECK_HIP(hipMemset(d_poison, 0xAB, nbytes));
    CHECK_EP(ep_dispatch(&p, &old, d_x, d_poison, T * K, 0, EP_ROWS_EXPERT, EP_FORMAT_BF16, s));
    CHECK_EP(ep_combine(&p, &old, NULL, d_w, d_recv, T * K, NULL, NULL, d_out2, EP_COMBINE_FLAT, s));
    CHECK_HIP(hipStreamSynchronize(s));
    CHECK_HIP(hipMemcpy(status, d_status, sizeof status, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(poison, d_poison, nbytes, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(out, d_out2, sizeof out, hipMemcpyDeviceToHost));
    if (status[EP_STATUS_STALE] != 1) {
      printf("stale handle: stale word %d, expected 1\n", status[EP_STATUS_STALE]);
      return 1;
    }
    for (i = 0; i < nbytes; ++i)
      if (poison[i] != 0xAB) {
        printf("dispatch with a stale handle wrote byte %zu\n", i);
        return 1;
      }
    for (i = 0; i < (size_t)T * H; ++i)
      if (out[i] != 0xCDCD) {
        printf("combine with a stale handle wrote element %zu\n", i);
        return 1;
      }
    /* the current handle works, and the next layout clears the flag */
    CHECK_EP(ep_combine(&p, &L, NULL, d_w, d_recv, T * K, NULL, NULL, d_out2, EP_COMBINE_FLAT, s));
    CHECK_HIP(hipStreamSynchronize(s));
    CHECK_HIP(hipMemcpy(out, d_out2, sizeof out, hipMemcpyDeviceToHost));
    for (t = 0; t < T; ++t)
      for (h = 0; h < H; ++h)
        if (int_of_bf16(out[t * H + h]) != keff[t] * ((t * 13 + h * 7) % 15 - 7)) {
          printf("combine with the current handle: token %d element %d wrong\n", t, h);
          return 1;
        }
    CHECK_EP(ep_layout(&p, d_idx, d_w, &L, d_ws, ws_bytes, s));
    CHECK_HIP(hipStreamSynchronize(s));
    CHECK_HIP(hipMemcpy(status, d_status, sizeof status, hipMemcpyDeviceToHost));
    if (status[EP_STATUS_STALE] != 0 || (uint32_t)status[EP_STATUS_GENERATION] != L.generation) {
      printf("after a new layout: stale word %d, stamp %d (generation %u)\n", status[EP_STATUS_STALE],
             status[EP_STATUS_GENERATION], L.generation);
      return 1;
    }
    hipFree(d_poison);
    hipFree(d_out2);
  }

  /* grouped rows and the grouped combine order */
  {
    enum { G = 4, EPG = E / G };
    ep_problem_t pg = p;
    pg.num_groups = G;
    static int32_t grow[T * K], rsrc[T * G], ridx[T * G * K], gcounts[G];
    static float rw[T * G * K];
    static uint16_t recvg[T * G * H], outg[T * H];
    int32_t *d_gcounts, *d_goffsets, *d_grow, *d_rsrc, *d_ridx;
    float* d_rw;
    uint16_t *d_recvg, *d_outg;
    void* d_wsg;
    const size_t wsg_bytes = ep_layout_workspace_bytes(&pg);
    CHECK_HIP(hipMalloc((void**)&d_gcounts, G * 4));
    CHECK_HIP(hipMalloc((void**)&d_goffsets, (G + 1) * 4));
    CHECK_HIP(hipMalloc((void**)&d_grow, T * K * 4));
    CHECK_HIP(hipMalloc((void**)&d_rsrc, T * G * 4));
    CHECK_HIP(hipMalloc((void**)&d_ridx, T * G * K * 4));
    CHECK_HIP(hipMalloc((void**)&d_rw, T * G * K * 4));
    CHECK_HIP(hipMalloc((void**)&d_recvg, sizeof recvg));
    CHECK_HIP(hipMalloc((void**)&d_outg, sizeof outg));
    CHECK_HIP(hipMalloc(&d_wsg, wsg_bytes));
    ep_layout_t Lg = L;
    Lg.group_counts = d_gcounts;
    Lg.group_offsets = d_goffsets;
    Lg.grow = d_grow;
    Lg.row_src = d_rsrc;
    Lg.row_topk_idx = d_ridx;
    Lg.row_topk_weights = d_rw;
    Lg.row_capacity = T * G;
    CHECK_EP(ep_layout(&pg, d_idx, d_w, &Lg, d_wsg, wsg_bytes, s));
    CHECK_EP(ep_dispatch(&pg, &Lg, d_x, d_recvg, T * G, 0, EP_ROWS_GROUP, EP_FORMAT_BF16, s));
    CHECK_EP(ep_combine(&pg, &Lg, d_idx, d_w, d_recv, T * K, NULL, NULL, d_outg, EP_COMBINE_GROUPED, s));
    CHECK_HIP(hipStreamSynchronize(s));
    CHECK_HIP(hipMemcpy(status, d_status, sizeof status, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(gcounts, d_gcounts, sizeof gcounts, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(grow, d_grow, sizeof grow, hipMemcpyDeviceToHost));
    const int R = status[EP_STATUS_ROWS_GROUP];
    CHECK_HIP(hipMemcpy(rsrc, d_rsrc, (size_t)R * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(ridx, d_ridx, (size_t)R * K * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(rw, d_rw, (size_t)R * K * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(recvg, d_recvg, (size_t)R * H * 2, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(outg, d_outg, sizeof outg, hipMemcpyDeviceToHost));
    {
      int hits = 0, sum = 0, g;
      for (t = 0; t < T; ++t)
        for (g = 0; g < G; ++g) {
          int hit = 0;
          for (k = 0; k < K; ++k) {
            const int64_t id = idx[t * K + k];
            if (id >= 0 && id < E && id / EPG == g) hit = 1;
          }
          hits += hit;
        }
      for (g = 0; g < G; ++g) sum += gcounts[g];
      if (R != hits || sum != hits || status[EP_STATUS_LIST_OVERFLOW] != 0) {
        printf("grouped rows %d (group counts sum %d), expected %d\n", R, sum, hits);
        return 1;
      }
    }
    for (t = 0; t < T * K; ++t) {
      const int64_t id = idx[t];
      const int tok = t / K;
      if (!(id >= 0 && id < E)) {
        if (grow[t] != -1) {
          printf("entry %d: no selection but group row %d\n", t, grow[t]);
          return 1;
        }
        continue;
      }
      const int r = grow[t];
      if (r < 0 || r >= R || rsrc[r] != tok) {
        printf("entry %d: group row %d of token %d\n", t, r, r >= 0 && r < R ? rsrc[r] : -1);
        return 1;
      }
      for (k = 0; k < K; ++k) {
        const int64_t id2 = idx[tok * K + k];
        const int same = id2 >= 0 && id2 < E && id2 / EPG == id / EPG;
        if (ridx[r * K + k] != (same ? (int)(id2 - (id / EPG) * EPG) : -1) ||
            rw[r * K + k] != (same ? w[tok * K + k] : 0.0f)) {
          printf("row %d list entry %d: %d %g\n", r, k, ridx[r * K + k], rw[r * K + k]);
          return 1;
        }
      }
      for (h = 0; h < H; ++h)
        if (recvg[(size_t)r * H + h] != x[tok * H + h]) {
          printf("group row %d element %d differs from token %d\n", r, h, tok);
          return 1;
        }
    }
    for (t = 0; t < T; ++t)
      for (h = 0; h < H; ++h)
        if (int_of_bf16(outg[t * H + h]) != keff[t] * ((t * 13 + h * 7) % 15 - 7)) {
          printf("grouped combine, token %d element %d: %d\n", t, h, int_of_bf16(outg[t * H + h]));
          return 1;
        }
    hipFree(d_gcounts);
    hipFree(d_goffsets);
    hipFree(d_grow);
    hipFree(d_rsrc);
    hipFree(d_ridx);
    hipFree(d_rw);
    hipFree(d_recvg);
    hipFree(d_outg);
    hipFree(d_wsg);
  }

  /* grouped GEMM over the expert-major rows, plain and packed weights */
  {
    static uint16_t wg[E * N * H];
    static uint16_t y[T * K * N], yp[T * K * N];
    static int row_t[T * K], row_e[T * K];
    int n, r;
    for (e = 0; e < E; ++e)
      for (n = 0; n < N; ++n)
        for (h = 0; h < H; ++h) wg[(e * N + n) * H + h] = bf16_of_int(gemm_weight(e, n, h));
    for (t = 0; t < T * K; ++t) {
      const int64_t id = idx[t];
      if (id >= 0 && id < E) {
        row_t[slot[t]] = t / K;
        row_e[slot[t]] = (int)id;
      }
    }
    const int64_t packed_bytes = ep_expert_weights_packed_bytes(E, N, H);
    if (packed_bytes != (int64_t)E * 256 * H * 2 || ep_expert_weights_packed_bytes(E, 100, H) != -1) {
      printf("ep_expert_weights_packed_bytes gave %lld\n", (long long)packed_bytes);
      return 1;
    }
    uint16_t *d_wg, *d_wp, *d_y, *d_yp;
    CHECK_HIP(hipMalloc((void**)&d_wg, sizeof wg));
    CHECK_HIP(hipMalloc((void**)&d_wp, (size_t)packed_bytes));
    CHECK_HIP(hipMalloc((void**)&d_y, sizeof y));
    CHECK_HIP(hipMalloc((void**)&d_yp, sizeof yp));
    CHECK_HIP(hipMemcpy(d_wg, wg, sizeof wg, hipMemcpyHostToDevice));
    /* the grouped layout above rewrote these buffers (it shares them), so
       the flat layout is computed again for a current handle */
    CHECK_EP(ep_layout(&p, d_idx, d_w, &L, d_ws, ws_bytes, s));
    CHECK_EP(ep_expert_gemm(&p, &L, d_recv, 0, d_wg, N, d_y, 0, s));
    CHECK_EP(ep_pack_expert_weights(d_wg, E, N, H, d_wp, s));
    {
      ep_problem_t q = p;
      q.flags = EP_FLAG_PACKED_WEIGHTS;
      CHECK_EP(ep_expert_gemm(&q, &L, d_recv, 0, d_wp, N, d_yp, 0, s));
    }
    CHECK_HIP(hipStreamSynchronize(s));
    CHECK_HIP(hipMemcpy(y, d_y, sizeof y, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(yp, d_yp, sizeof yp, hipMemcpyDeviceToHost));
    for (r = 0; r < n_sel; ++r)
      for (n = 0; n < N; ++n) {
        int sum = 0;
        for (h = 0; h < H; ++h)
          sum += ((row_t[r] * 13 + h * 7) % 15 - 7) * gemm_weight(row_e[r], n, h);
        const uint16_t want = bf16_rne_of_int(sum);
        if (y[r * N + n] != want || yp[r * N + n] != want) {
          printf("gemm row %d column %d: got %04x / packed %04x, expected %04x (sum %d)\n", r, n,
                 y[r * N + n], yp[r * N + n], want, sum);
          return 1;
        }
      }
    hipFree(d_wg);
    hipFree(d_wp);
    hipFree(d_y);
    hipFree(d_yp);
  }

  /* the allocation-free layout (no workspace argument) gives the same
     counts, offsets, slots and status words as ep_layout */
  {
    int32_t *d_counts2, *d_offsets2, *d_slot2, *d_status2;
    static int32_t counts2[E], offsets[E + 1], offsets2[E + 1], slot2[T * K], st1[EP_STATUS_WORDS],
        st2[EP_STATUS_WORDS];
    ep_layout_t L2;
    CHECK_HIP(hipMalloc((void**)&d_counts2, E * 4));
    CHECK_HIP(hipMalloc((void**)&d_offsets2, (E + 1) * 4));
    CHECK_HIP(hipMalloc((void**)&d_slot2, T * K * 4));
    CHECK_HIP(hipMalloc((void**)&d_status2, EP_STATUS_WORDS * 4));
    memset(&L2, 0, sizeof L2);
    L2.counts = d_counts2;
    L2.offsets = d_offsets2;
    L2.slot = d_slot2;
    L2.status = d_status2;
    memset(&L, 0, sizeof L);
    L.counts = d_counts;
    L.offsets = d_offsets;
    L.slot = d_slot;
    L.status = d_status;
    CHECK_EP(ep_layout(&p, d_idx, d_w, &L, d_ws, ws_bytes, s));
    CHECK_EP(ep_layout_noalloc(&p, d_idx, d_w, &L2, s));
    CHECK_HIP(hipStreamSynchronize(s));
    CHECK_HIP(hipMemcpy(counts, d_counts, sizeof counts, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(counts2, d_counts2, sizeof counts2, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(offsets, d_offsets, sizeof offsets, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(offsets2, d_offsets2, sizeof offsets2, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(slot, d_slot, sizeof slot, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(slot2, d_slot2, sizeof slot2, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(st1, d_status, sizeof st1, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(st2, d_status2, sizeof st2, hipMemcpyDeviceToHost));
    if (memcmp(counts, counts2, sizeof counts) || memcmp(offsets, offsets2, sizeof offsets) ||
        memcmp(slot, slot2, sizeof slot)) {
      printf("ep_layout_noalloc differs from ep_layout\n");
      return 1;
    }
    for (e = 0; e < EP_STATUS_WORDS; ++e)
      if (e != EP_STATUS_GENERATION && st1[e] != st2[e]) {
        printf("ep_layout_noalloc status word %d: %d, ep_layout %d\n", e, st2[e], st1[e]);
        return 1;
      }
    hipFree(d_counts2);
    hipFree(d_offsets2);
    hipFree(d_slot2);
    hipFree(d_status2);
  }

  hipFree(d_idx);
  hipFree(d_w);
  hipFree(d_x);
  hipFree(d_recv);
  hipFree(d_out);
  hipFree(d_counts);
  hipFree(d_offsets);
  hipFree(d_slot);
  hipFree(d_status);
  hipFree(d_ws);
  hipStreamDestroy(s);
  printf("OK: %d selections, %d invalid ids, combine of the dispatched rows = K_eff * x, "
         "fp8 rows exact, overflow and stale handles write nothing and are flagged, "
         "grouped rows, lists and grouped combine exact, "
         "grouped GEMM exact (plain and packed weights), allocation-free layout identical\n",
         n_sel, n_invalid);
  return 0;
}
