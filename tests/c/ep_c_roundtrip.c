/*
 * The C ABI used from plain C (C99, built with gcc): layout, bf16 dispatch
 * and combine on one GPU, checked against closed forms rather than an
 * oracle.
 *
 * Routing: T tokens pick K distinct experts (e = (7t + 5k) mod E); some
 * entries are masked (-1) and one id is out of range (counted in the
 * invalid-id status word and treated as -1).  Token rows hold small
 * integers, so the combine of the dispatched rows with unit weights must
 * return every token as exactly K_eff * x (fp32 sums of small integers are
 * exact, and so is their bf16 rounding).
 *
 * The grouped GEMM then multiplies the dispatched rows by weights in
 * {-1, 0, 1} (N = 128), once with the weights as given and once packed by
 * ep_pack_expert_weights: every partial sum is an exact fp32 integer, so
 * both must equal the bf16 rounding (nearest, ties to even) of the exact
 * sum, computed here on the host.
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
    for (h = 0; h < H; ++h) x[t * H + h] = bf16_of_int((t * 13 + h * 7) % 17 - 8);
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
      const int want = keff[t] * ((t * 13 + h * 7) % 17 - 8);
      const int got = int_of_bf16(out[t * H + h]);
      if (got != want) {
        printf("token %d element %d: combine gave %d, expected %d\n", t, h, got, want);
        return 1;
      }
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
          sum += ((row_t[r] * 13 + h * 7) % 17 - 8) * gemm_weight(row_e[r], n, h);
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
         "grouped GEMM exact (plain and packed weights)\n",
         n_sel, n_invalid);
  return 0;
}
