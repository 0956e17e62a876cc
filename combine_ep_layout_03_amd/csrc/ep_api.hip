// C-ABI entry points: argument checks, launch shapes, error codes.
// Semantics of every call are documented in include/ep_mi355x.h.
#include <limits.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "ep_internal.h"
#include "ep_mi355x.h"

// Layout scratch of ep_layout_noalloc: one array per GPU, in the code
// object, zero at load and held until the process ends.  Host code never
// passes `scratch` itself to a kernel (on the host it only names the
// symbol); it passes the device address scratch_on_current_device() looks up.
static __device__ __align__(256) unsigned char scratch[EP_LAYOUT_SCRATCH_BYTES];

namespace {

static_assert(EP_STATUS_DISPATCH_OVERFLOW == ep::kStatusDispatchOverflow &&
                  EP_STATUS_GENERATION == ep::kStatusGeneration &&
                  EP_STATUS_STALE == ep::kStatusStale && EP_STATUS_WORDS == 16,
              "status word numbering");

// Layout generations, unique in the process (never 0, so a zeroed
// ep_layout_t that no ep_layout has stamped never matches).
uint32_t next_generation() {
  static std::atomic<uint32_t> counter{0};
  uint32_t g;
  do {
    g = counter.fetch_add(1, std::memory_order_relaxed) + 1;
  } while (g == 0);
  return g;
}

constexpr int kMaxDevices = 64;

// The current device's address of `scratch`, looked up once per device
// (with that device current) and kept; null if the lookup fails.
void* scratch_on_current_device() {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    addr[dev] = ptr;
  }
  return addr[dev];
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Basic shape checks shared by every call.
int check_problem(const ep_problem_t* p) {
  if (!p) return EP_EINVAL;
  if (p->num_tokens < 0 || p->hidden < 1 || p->topk < 1 || p->num_experts < 1 ||
      p->num_groups < 0)
    return EP_EINVAL;
  if (p->num_groups > 0 && p->num_experts % p->num_groups != 0) return EP_EINVAL;
  if (p->expert_alignment < 0 || p->expert_alignment > (1 << 20)) return EP_EINVAL;
  if (p->flags & ~(EP_FLAG_ZERO_PADDING | EP_FLAG_GATHER_ROWS | EP_FLAG_PACKED_WEIGHTS)) return EP_EINVAL;
  if (p->topk > EP_MAX_TOPK) return EP_ENOTSUP;
  if (static_cast<int64_t>(p->num_experts) + p->num_groups > EP_MAX_KEYS) return EP_ENOTSUP;
  // slots and rows are int32: every (t,k) row, padding included, must index below 2^31
  const int64_t pad = static_cast<int64_t>(p->num_experts) *
                      (p->expert_alignment > 1 ? p->expert_alignment - 1 : 0);
  if (p->num_tokens > (static_cast<int64_t>(INT32_MAX) - pad) / p->topk) return EP_ENOTSUP;
  return EP_OK;
}

// Widest vector (bytes) that divides `row_bytes` and the alignment of both bases.
int vec_bytes_for(int64_t row_bytes, const void* a, const void* b) {
  for (int v = 16; v > 2; v >>= 1)
    if (row_bytes % v == 0 && aligned(a, v) && aligned(b, v)) return v;
  return 2;
}

}  // namespace

extern "C" {

int64_t ep_fp8_row_bytes(int32_t hidden) {
  if (hidden <= 0 || hidden % 128 != 0) return -1;
  const int64_t raw = static_cast<int64_t>(hidden) + 4 * (hidden / 128);
  return (raw + 15) / 16 * 16;
}

size_t ep_layout_workspace_bytes(const ep_problem_t* p) {
  if (check_problem(p) != EP_OK) return 0;
  const ep::LayoutGeom g =
      ep::layout_geom(p->num_tokens * p->topk, p->num_experts, p->num_groups);
  return ep::layout_workspace_bytes(g);
}

int ep_layout(const ep_problem_t* p, const int64_t* topk_idx, const float* topk_weights,
              ep_layout_t* L, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int rc = check_problem(p);
  if (rc != EP_OK) return rc;
  if (!L || !L->counts || !L->offsets || !L->status || !workspace) return EP_EINVAL;
  const int64_t T = p->num_tokens;
  const bool grouped = p->num_groups > 0;
  if (T > 0 && (!topk_idx || !L->slot)) return EP_EINVAL;
  if (grouped) {
    if (!L->group_counts || !L->group_offsets || (T > 0 && !L->grow)) return EP_EINVAL;
    if (L->row_capacity < 0) return EP_EINVAL;
    if (L->row_capacity > 0 && T > 0 &&
        (!L->row_src || !L->row_topk_idx || !L->row_topk_weights || !topk_weights))
      return EP_EINVAL;
  }
  if (L->expert_row_src && L->expert_row_capacity < 0) return EP_EINVAL;
  if (!aligned(topk_idx, 8) || !aligned(workspace, 16)) return EP_EINVAL;

  const ep::LayoutGeom g = ep::layout_geom(T * p->topk, p->num_experts, p->num_groups);
  if (workspace_bytes < ep::layout_workspace_bytes(g)) return EP_EWORKSPACE;

  ep::LayoutArgs a;
  a.idx = topk_idx;
  a.w = topk_weights;
  a.n = static_cast<uint32_t>(T * p->topk);
  a.K = p->topk;
  a.E = p->num_experts;
  a.G = p->num_groups;
  a.epg = grouped ? p->num_experts / p->num_groups : 1;
  a.counts = L->counts;
  a.offsets = L->offsets;
  a.slot = L->slot;
  a.status = L->status;
  a.gcounts = L->group_counts;
  a.goffsets = L->group_offsets;
  a.grow = L->grow;
  a.row_src = L->row_src;
  a.row_idx = L->row_topk_idx;
  a.row_w = L->row_topk_weights;
  a.row_cap = grouped ? L->row_capacity : 0;
  a.align = p->expert_alignment > 1 ? p->expert_alignment : 1;
  a.expert_row_src = L->expert_row_src;
  a.expert_row_cap = L->expert_row_src ? L->expert_row_capacity : 0;
  a.recv_stats = L->recv_stats;
  a.partials = static_cast<int32_t*>(workspace);
  a.generation = next_generation();
  if (ep::launch_layout(a, g, stream) != hipSuccess) return EP_EHIP;
  L->generation = a.generation;
  return EP_OK;
}

int ep_layout_noalloc(const ep_problem_t* p, const int64_t* topk_idx, const float* topk_weights,
                      ep_layout_t* L, hipStream_t stream) {
  const int rc = check_problem(p);
  if (rc != EP_OK) return rc;
  const ep::LayoutGeom g = ep::layout_geom(p->num_tokens * p->topk, p->num_experts, p->num_groups);
  if (ep::layout_workspace_bytes(g) > EP_LAYOUT_SCRATCH_BYTES) return EP_ESCRATCH;
  void* ws = scratch_on_current_device();
  if (!ws) return EP_EHIP;
  return ep_layout(p, topk_idx, topk_weights, L, ws, EP_LAYOUT_SCRATCH_BYTES, stream);
}

int ep_dispatch(const ep_problem_t* p, const ep_layout_t* L, const void* x, void* recv,
                int64_t capacity_rows, int64_t recv_row_stride, int32_t rows, int32_t format,
                hipStream_t stream) {
  int rc = check_problem(p);
  if (rc != EP_OK) return rc;
  if (!L || !L->status || capacity_rows < 0 || recv_row_stride < 0) return EP_EINVAL;
  if (rows != EP_ROWS_EXPERT && rows != EP_ROWS_GROUP) return EP_EINVAL;
  if (format != EP_FORMAT_BF16 && format != EP_FORMAT_FP8_PACKED) return EP_EINVAL;
  if (rows == EP_ROWS_GROUP && p->num_groups < 1) return EP_EINVAL;
  int64_t row_bytes = static_cast<int64_t>(p->hidden) * 2;
  if (format == EP_FORMAT_FP8_PACKED) {
    row_bytes = ep_fp8_row_bytes(p->hidden);
    if (row_bytes < 0 || p->hidden > 32768) return EP_ENOTSUP;
  }
  const int64_t stride = recv_row_stride == 0 ? row_bytes : recv_row_stride;
  if (stride < row_bytes) return EP_EINVAL;
  if (p->num_tokens == 0) return EP_OK;
  const int32_t* dest = rows == EP_ROWS_EXPERT ? L->slot : L->grow;
  if (!dest || !x || (!recv && capacity_rows > 0)) return EP_EINVAL;
  if (!aligned(x, 2) || !aligned(recv, 2) || stride % 2 != 0) return EP_EINVAL;

  ep::ScatterArgs a;
  a.x = x;
  a.recv = recv;
  a.dest = dest;
  a.rows_needed = L->status + (rows == EP_ROWS_EXPERT ? EP_STATUS_ROWS_EXPERT : EP_STATUS_ROWS_GROUP);
  a.status = L->status;
  a.generation = L->generation;
  a.T = p->num_tokens;
  a.K = p->topk;
  a.H = p->hidden;
  a.capacity = capacity_rows;
  a.stride = stride;
  a.dedup = rows == EP_ROWS_GROUP;
  a.counts = L->counts;
  a.offsets = L->offsets;
  a.E = p->num_experts;
  const bool zero_pad =
      (p->flags & EP_FLAG_ZERO_PADDING) && rows == EP_ROWS_EXPERT && p->expert_alignment > 1;
  if (zero_pad && (!L->counts || !L->offsets)) return EP_EINVAL;
  hipError_t err;
  int vb = 16;
  if (format == EP_FORMAT_FP8_PACKED) {
    if (!aligned(x, 16) || !aligned(recv, 16) || stride % 16 != 0) return EP_EINVAL;
    // Rows on 128-byte lines: extend each row with zeros to its line end, so
    // no line is written in part (the row format's own zero padding, longer).
    if (aligned(recv, 128) && stride % 128 == 0)
      row_bytes = std::min(stride, (row_bytes + 127) / 128 * 128);
    err = ep::launch_scatter_fp8(a, row_bytes, stream);
  } else {
    vb = vec_bytes_for(row_bytes, x, recv);
    while (stride % vb != 0) vb >>= 1;
    err = ep::launch_scatter_bf16(a, vb, stream);
  }
  if (err == hipSuccess && zero_pad) err = ep::launch_zero_padding(a, row_bytes, vb, stream);
  return err == hipSuccess ? EP_OK : EP_EHIP;
}

int ep_combine(const ep_problem_t* p, const ep_layout_t* L, const int64_t* topk_idx,
               const float* topk_weights, const void* y, int64_t y_rows, const void* bias0,
               const void* bias1, void* out, int32_t order, hipStream_t stream) {
  int rc = check_problem(p);
  if (rc != EP_OK) return rc;
  if (!L || !L->status || y_rows < 0) return EP_EINVAL;
  if (order != EP_COMBINE_FLAT && order != EP_COMBINE_GROUPED) return EP_EINVAL;
  const bool grouped = order == EP_COMBINE_GROUPED;
  if (grouped && p->num_groups < 1) return EP_EINVAL;
  if (p->num_tokens == 0) return EP_OK;
  if (!L->slot || !topk_weights || !out || (grouped && !topk_idx)) return EP_EINVAL;
  if (!y && y_rows > 0) return EP_EINVAL;
  if (!aligned(y, 2) || !aligned(out, 2) || !aligned(topk_weights, 4) ||
      !aligned(topk_idx, 8) || !aligned(bias0, 2) || !aligned(bias1, 2))
    return EP_EINVAL;

  ep::CombineArgs a;
  a.y = y;
  a.y_rows = y_rows;
  a.slot = L->slot;
  a.w = topk_weights;
  a.idx = topk_idx;
  a.E = p->num_experts;
  a.epg = grouped ? p->num_experts / p->num_groups : 1;
  a.T = p->num_tokens;
  a.K = p->topk;
  a.H = p->hidden;
  a.bias0 = bias0;
  a.bias1 = bias1;
  a.out = out;
  a.status = L->status;
  a.generation = L->generation;
  a.grouped = grouped;
  int ve = vec_bytes_for(static_cast<int64_t>(p->hidden) * 2, y ? y : out, out) / 2;
  while (ve > 1 && (!aligned(bias0, 2 * ve) || !aligned(bias1, 2 * ve))) ve >>= 1;
  return ep::launch_combine(a, ve, stream) == hipSuccess ? EP_OK : EP_EHIP;
}

int ep_expert_gemm(const ep_problem_t* p, const ep_layout_t* L, const void* x,
                   int64_t x_row_stride, const void* w, int32_t n_out, void* y,
                   int64_t y_row_stride, hipStream_t stream) {
  int rc = check_problem(p);
  if (rc != EP_OK) return rc;
  if (!L || !L->counts || !L->offsets || !L->status || x_row_stride < 0 || y_row_stride < 0 ||
      n_out < 1)
    return EP_EINVAL;
  if (p->hidden % 64 != 0 || n_out % 128 != 0) return EP_ENOTSUP;
  const int64_t ldx = x_row_stride == 0 ? p->hidden : x_row_stride;
  const int64_t ldy = y_row_stride == 0 ? n_out : y_row_stride;
  if (ldx < p->hidden || ldy < n_out || ldx % 8 != 0 || ldy % 4 != 0) return EP_EINVAL;
  if (p->num_tokens == 0) return EP_OK;
  if (!x || !w || !y || !aligned(x, 16) || !aligned(w, 16) || !aligned(y, 16)) return EP_EINVAL;
  ep::GemmArgs a;
  a.x = static_cast<const uint16_t*>(x);
  a.ldx = ldx;
  a.w = static_cast<const uint16_t*>(w);
  a.y = static_cast<uint16_t*>(y);
  a.ldy = ldy;
  a.counts = L->counts;
  a.offsets = L->offsets;
  a.E = p->num_experts;
  a.H = p->hidden;
  a.N = n_out;
  a.ntn = (n_out + 255) / 256;
  a.status = L->status;
  a.generation = L->generation;
  const int64_t pad = static_cast<int64_t>(p->num_experts) *
                      (p->expert_alignment > 1 ? p->expert_alignment - 1 : 0);
  const int64_t max_rows = p->num_tokens * p->topk + pad;
  a.row_src = nullptr;
  a.packed = (p->flags & EP_FLAG_PACKED_WEIGHTS) != 0;
  if (p->flags & EP_FLAG_GATHER_ROWS) {
    // token rows gathered through the layout's expert-row map, which must
    // cover every expert row the layout can produce
    if (!L->expert_row_src || L->expert_row_capacity < max_rows) return EP_EINVAL;
    a.row_src = L->expert_row_src;
  }
  // the kernel numbers its tiles in int32
  if (ep::expert_gemm_max_tiles(max_rows, p->num_experts, n_out) > INT32_MAX) return EP_ENOTSUP;
  return ep::launch_expert_gemm(a, max_rows, stream) == hipSuccess ? EP_OK : EP_EHIP;
}

int64_t ep_expert_weights_packed_bytes(int32_t num_experts, int32_t n_out, int32_t hidden) {
  if (num_experts < 1 || n_out < 1 || hidden < 1 || n_out % 128 != 0 || hidden % 64 != 0) return -1;
  return static_cast<int64_t>(num_experts) * ((n_out + 255) / 256) * 256 * hidden * 2;
}

int ep_pack_expert_weights(const void* w, int32_t num_experts, int32_t n_out, int32_t hidden,
                           void* w_packed, hipStream_t stream) {
  const int64_t packed_bytes = ep_expert_weights_packed_bytes(num_experts, n_out, hidden);
  if (packed_bytes < 0) return EP_EINVAL;
  if (!w || !w_packed || !aligned(w, 16) || !aligned(w_packed, 16)) return EP_EINVAL;
  // the copy reads w while writing w_packed: the two must not overlap
  const uintptr_t w0 = reinterpret_cast<uintptr_t>(w);
  const uintptr_t p0 = reinterpret_cast<uintptr_t>(w_packed);
  const uintptr_t w_bytes = static_cast<uintptr_t>(num_experts) * n_out * hidden * 2;
  if (w0 < p0 + static_cast<uintptr_t>(packed_bytes) && p0 < w0 + w_bytes) return EP_EINVAL;
  return ep::launch_pack_expert_weights(static_cast<const uint16_t*>(w), num_experts, n_out, hidden,
                                        static_cast<uint16_t*>(w_packed), stream) == hipSuccess
             ? EP_OK
             : EP_EHIP;
}

const char* ep_strerror(int code) {
  switch (code) {
    case EP_OK: return "ok";
    case EP_EINVAL: return "invalid argument (null pointer, bad size or misaligned base)";
    case EP_ENOTSUP:
      return "unsupported (fp8 needs hidden % 128 == 0 and hidden <= 32768; K <= 32; E + G <= 1024)";
    case EP_EHIP: return "HIP launch failed";
    case EP_EWORKSPACE: return "workspace smaller than ep_layout_workspace_bytes()";
    case EP_ESCRATCH:
      return "problem needs more layout scratch than EP_LAYOUT_SCRATCH_BYTES (use ep_layout with a workspace)";
    default: return "unknown error code";
  }
}

}  // extern "C"
