// libmoe C ABI: argument validation, workspace layout, path choice, launches.
// Every entry point validates on the host before enqueuing anything and never
// synchronises or reads device memory.
#include "libmoe.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <atomic>
#include <functional>
#include <mutex>

#include "moe_internal.hpp"

namespace {

using moe::Shape;

static_assert(moe::kMaxExperts == MOE_MAX_EXPERTS, "one expert limit for every kernel");
static_assert(moe::kTileM == MOE_TILE_M, "one segment granule");
static_assert(moe::kStreamMaxTokens == MOE_STREAM_MAX_TOKENS, "one streaming limit");

constexpr size_t kAlign = 256;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape checks shared by every entry point.  Returns MOE_OK and fills `s`.
moe_status_t check_problem(const moe_problem_t* p, Shape* s) {
  if (!p) return MOE_EINVAL;
  if (p->tokens < 0 || p->dim <= 0 || p->hidden <= 0 || p->n_experts <= 0 || p->top_k <= 0)
    return MOE_EINVAL;
  if (p->top_k > p->n_experts) return MOE_EINVAL;
  if (p->dim % 8 != 0 || p->hidden % 8 != 0) return MOE_EINVAL;
  if (p->out_dtype != MOE_F32 && p->out_dtype != MOE_BF16) return MOE_EINVAL;
  if (p->path != MOE_PATH_AUTO && p->path != MOE_PATH_STREAM && p->path != MOE_PATH_TILED)
    return MOE_EINVAL;
  if (p->path == MOE_PATH_STREAM && p->tokens > moe::kStreamMaxTokens) return MOE_ENOTSUP;
  if (p->n_experts > MOE_MAX_EXPERTS) return MOE_ENOTSUP;
  const int64_t P = int64_t(p->tokens) * p->top_k;
  const int64_t cap =
      (P + int64_t(p->n_experts) * (MOE_TILE_M - 1) + MOE_TILE_M - 1) / MOE_TILE_M * MOE_TILE_M;
  // row indices and element offsets inside one expert are int32 on the device
  if (cap >= (int64_t(1) << 31)) return MOE_ENOTSUP;
  // buffer resources address x, one expert's weight matrix and one row tile
  // of h with 32-bit byte offsets
  if (int64_t(p->dim) * p->hidden * 2 >= (int64_t(1) << 31)) return MOE_ENOTSUP;
  if (int64_t(p->tokens) * p->dim * 2 >= (int64_t(1) << 31)) return MOE_ENOTSUP;
  if (int64_t(MOE_TILE_M) * p->hidden * 2 >= (int64_t(1) << 31)) return MOE_ENOTSUP;
  s->T = p->tokens;
  s->D = p->dim;
  s->H = p->hidden;
  s->n = p->n_experts;
  s->K = p->top_k;
  s->cap = cap;
  s->stream = p->path == MOE_PATH_STREAM ||
              (p->path == MOE_PATH_AUTO && p->tokens <= moe::kDecodeMaxTokens);
  return MOE_OK;
}

// Workspace carve-up (each piece 256-byte aligned):
//   topk_idx  int32 [T*K]     topk_gate fp32 [T*K]
//   count     int32 [n]       offset    int32 [n+1]
//   row_slot  int32 [cap]     slot_row  int32 [T*K]
//   h         bf16  [cap][H]  y_rows    fp32  [S][cap][D] (split partials: S = 2, or
//                                           up to 8 on the weight-streaming path)
// With the weight-streaming path the h region holds that path's first-product
// results instead (bf16 h or fp32 a and b per token-slot; decode_scratch_bytes).  The router's partial logits
// (route_scratch_bytes) use the start of the y_rows region, which is written
// only after the router has finished with them; so do the tiled first
// product's split last-round halves (grouped_up_scratch_bytes), consumed
// before the second product writes there.
struct Carve {
  size_t idx, gate, count, offset, row_slot, slot_row, h, y, total;
};

// Contraction partials of the second product the y_rows region holds.
int y_planes(const Shape& s) {
  return s.stream ? std::max(2, moe::decode_down_splits(s)) : 2;
}

Carve carve(const Shape& s) {
  Carve c{};
  const size_t P = size_t(s.T) * s.K;
  size_t o = 0;
  c.idx = o;      o = align_up(o + P * 4, kAlign);
  c.gate = o;     o = align_up(o + P * 4, kAlign);
  c.count = o;    o = align_up(o + size_t(s.n) * 4, kAlign);
  c.offset = o;   o = align_up(o + size_t(s.n + 1) * 4, kAlign);
  c.row_slot = o; o = align_up(o + size_t(s.cap) * 4, kAlign);
  c.slot_row = o; o = align_up(o + P * 4, kAlign);
  size_t h_bytes = size_t(s.cap) * s.H * 2;
  if (s.stream) h_bytes = std::max(h_bytes, moe::decode_scratch_bytes(s));
  c.h = o;        o = align_up(o + h_bytes, kAlign);
  c.y = o;
  o = align_up(o + std::max({size_t(y_planes(s)) * s.cap * s.D * 4, moe::route_scratch_bytes(s),
                             s.stream ? size_t(0) : moe::grouped_up_scratch_bytes(s)}),
               kAlign);
  c.total = o;
  return c;
}

moe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

// ---------------------------------------------------------------------------
// Allocation-free forward (moe_forward_noalloc): its intermediates live in
// `scratch`, a library-owned array that every GPU the library runs on holds
// from module load until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: kernels only ever get the address
// hipGetSymbolAddress returns for the current device.
// ---------------------------------------------------------------------------
constexpr size_t kStaticScratchBytes = size_t(MOE_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

// Device address of `scratch` on the calling thread's current device, looked
// up once per device (devices 0..63) and kept; nullptr if the lookup fails.
uint8_t* static_scratch(int dev) {
  constexpr int kDevices = 64;
  static std::atomic<void*> addr[kDevices];
  static std::mutex mu;
  if (dev < 0 || dev >= kDevices) return nullptr;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(mu);
    p = addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
      addr[dev].store(p, std::memory_order_release);
    }
  }
  return static_cast<uint8_t*>(p);
}

// Layout of the weight-streaming path without a permute pass, rows indexed
// by slot (P = T*K rows per plane): routing, the fp32 first products and the
// second product's partials (the router's partial logits, when it needs
// them, at the start of the y region, consumed before y is written).
struct CompactCarve {
  size_t idx, gate, ab, y, total;
  int planes;
};

CompactCarve compact_carve(const Shape& s) {
  CompactCarve c{};
  const size_t P = size_t(s.T) * s.K;
  size_t o = 0;
  c.idx = o;  o = align_up(o + P * 4, kAlign);
  c.gate = o; o = align_up(o + P * 4, kAlign);
  c.ab = o;   o = align_up(o + moe::decode_scratch_bytes(s), kAlign);
  c.planes = moe::decode_down_splits(s);
  c.y = o;
  o = align_up(o + std::max(size_t(c.planes) * P * s.D * 4, moe::route_scratch_bytes(s)), kAlign);
  c.total = o;
  return c;
}

bool use_decode(const Shape& s) { return s.stream; }

// `mark(i)`, when given, records stage event i (3 after the first product, 4
// after the second).
using MarkFn = std::function<hipError_t(int)>;

// Expert products into y_rows (partial 0) and, when the second product is
// split, y_part (partial 1); returns the number of partials in *nsplit.
// With `topk_idx` (weight-streaming path only) the experts' token-slots are
// read from the routing and the rows land at the slot index; otherwise the
// permuted layout (count, offset, row_slot) gives them.
// part_stride: floats between consecutive partials of the streaming path's
// second product (partial p >= 1 at y_part + (p - 1) * part_stride).
// up_scratch: workspace the second product has not yet written, for the tiled
// first product's split last round (may be null).
moe_status_t run_ffn(const Shape& s, const void* x, const int32_t* count, const int32_t* offset,
                     const int32_t* row_slot, const int32_t* topk_idx, const void* w1,
                     const void* w3, const void* w2, float* y_rows, float* y_part,
                     size_t part_stride, int* nsplit, uint16_t* h, void* up_scratch,
                     size_t up_scratch_bytes, hipStream_t st, const MarkFn& mark = nullptr) {
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const uint16_t* w1b = static_cast<const uint16_t*>(w1);
  const uint16_t* w3b = static_cast<const uint16_t*>(w3);
  const uint16_t* w2b = static_cast<const uint16_t*>(w2);
  hipError_t e;
  if (use_decode(s)) {  // first products in the h region (decode_scratch_bytes)
    e = moe::launch_decode_up(s, xb, count, offset, row_slot, topk_idx, w1b, w3b, h, st);
  } else {
    e = moe::launch_grouped_up(s, xb, count, offset, row_slot, w1b, w3b, h, up_scratch,
                               up_scratch_bytes, st);
  }
  if (e != hipSuccess || (mark && mark(3) != hipSuccess)) return MOE_EHIP;
  *nsplit = 1;
  if (use_decode(s)) {
    *nsplit = y_part ? moe::decode_down_splits(s) : 1;
    e = moe::launch_decode_down(s, count, offset, row_slot, topk_idx, h, w2b, y_rows, y_part,
                                *nsplit, part_stride, st);
  } else {
    *nsplit = y_part ? moe::grouped_down_splits(s) : 1;
    e = moe::launch_grouped_down(s, count, offset, h, w2b, y_rows, *nsplit, y_part, st);
  }
  if (e != hipSuccess || (mark && mark(4) != hipSuccess)) return MOE_EHIP;
  return MOE_OK;
}


// LIBMOE_LOG set to anything but "" or "0": every call that enqueues work
// prints one line to stderr (entry point, shape, the expert-product path the
// shape selects, returned status).  Read once; off costs one atomic load.
bool log_enabled() {
  static std::atomic<int> state{-1};
  int v = state.load(std::memory_order_relaxed);
  if (v < 0) {
    const char* e = std::getenv("LIBMOE_LOG");
    v = (e && e[0] && !(e[0] == '0' && e[1] == 0)) ? 1 : 0;
    state.store(v, std::memory_order_relaxed);
  }
  return v == 1;
}

moe_status_t logged(const char* fn, const moe_problem_t* p, moe_status_t st) {
  if (!log_enabled()) return st;
  if (!p) {
    std::fprintf(stderr, "libmoe: %s problem=null -> %d\n", fn, int(st));
    return st;
  }
  Shape s;
  const bool ok = check_problem(p, &s) == MOE_OK;
  std::fprintf(stderr, "libmoe: %s T=%d D=%d H=%d n=%d K=%d out=%s path=%s -> %d (%s)\n", fn,
               p->tokens, p->dim, p->hidden, p->n_experts, p->top_k,
               p->out_dtype == MOE_BF16 ? "bf16" : "f32",
               !ok ? "-" : (s.stream ? "stream" : "tiled"), int(st),
               st == MOE_OK ? "ok" : st == MOE_EINVAL ? "invalid argument"
               : st == MOE_ENOTSUP ? "unsupported shape"
               : st == MOE_EWORKSPACE ? "workspace missing or too small"
               : st == MOE_EHIP ? "HIP launch failed" : "unknown status");
  return st;
}

}  // namespace

extern "C" {

int64_t moe_capacity_rows(const moe_problem_t* p) {
  Shape s;
  if (check_problem(p, &s) != MOE_OK) return -1;
  return s.cap;
}

size_t moe_workspace_bytes(const moe_problem_t* p) {
  Shape s;
  if (check_problem(p, &s) != MOE_OK) return 0;
  return carve(s).total;
}

const char* moe_status_string(int32_t status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_ENOTSUP: return "unsupported shape";
    case MOE_EWORKSPACE: return "workspace missing or too small";
    case MOE_EHIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int32_t moe_decode_max_tokens(void) { return moe::kDecodeMaxTokens; }

size_t moe_route_workspace_bytes(const moe_problem_t* p) {
  Shape s;
  if (check_problem(p, &s) != MOE_OK) return 0;
  return moe::route_scratch_bytes(s);
}

static moe_status_t moe_route_impl(const moe_problem_t* p, const void* x, const void* w_gate,
                       int32_t* topk_idx, float* topk_gate, float* logits, void* ws,
                       size_t ws_bytes, void* stream) {
  Shape s;
  moe_status_t st = check_problem(p, &s);
  if (st != MOE_OK) return st;
  if (s.T == 0) return MOE_OK;
  if (!x || !w_gate || !topk_idx || !topk_gate) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(w_gate) || !aligned16(topk_idx) || !aligned16(topk_gate) ||
      (logits && !aligned16(logits)) || (ws && !aligned16(ws)))
    return MOE_EINVAL;
  const size_t need = moe::route_scratch_bytes(s);
  if (need && (!ws || ws_bytes < need)) return MOE_EWORKSPACE;
  return hip_status(moe::launch_route(s, static_cast<const uint16_t*>(x),
                                      static_cast<const uint16_t*>(w_gate), topk_idx, topk_gate,
                                      logits, static_cast<float*>(ws),
                                      static_cast<hipStream_t>(stream)));
}

static moe_status_t moe_permute_impl(const moe_problem_t* p, const int32_t* topk_idx, int32_t* expert_count,
                         int32_t* expert_offset, int32_t* row_slot, int32_t* slot_row,
                         void* stream) {
  Shape s;
  moe_status_t st = check_problem(p, &s);
  if (st != MOE_OK) return st;
  if (s.T == 0) return MOE_OK;
  if (!topk_idx || !expert_count || !expert_offset || !row_slot || !slot_row) return MOE_EINVAL;
  if (!aligned16(topk_idx) || !aligned16(expert_count) || !aligned16(expert_offset) ||
      !aligned16(row_slot) || !aligned16(slot_row))
    return MOE_EINVAL;
  return hip_status(moe::launch_permute(s, topk_idx, expert_count, expert_offset, row_slot,
                                        slot_row, static_cast<hipStream_t>(stream)));
}

static moe_status_t moe_grouped_ffn_impl(const moe_problem_t* p, const void* x, const int32_t* expert_count,
                             const int32_t* expert_offset, const int32_t* row_slot,
                             const void* w1, const void* w3, const void* w2, float* y_rows,
                             void* ws, size_t ws_bytes, void* stream) {
  Shape s;
  moe_status_t st = check_problem(p, &s);
  if (st != MOE_OK) return st;
  if (s.T == 0) return MOE_OK;
  if (!x || !expert_count || !expert_offset || !row_slot || !w1 || !w3 || !w2 || !y_rows)
    return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(expert_count) || !aligned16(expert_offset) ||
      !aligned16(row_slot) || !aligned16(w1) || !aligned16(w3) || !aligned16(w2) ||
      !aligned16(y_rows))
    return MOE_EINVAL;
  const Carve c = carve(s);
  if (!ws || ws_bytes < c.total) return MOE_EWORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0) return MOE_EINVAL;
  uint8_t* base = static_cast<uint8_t*>(ws);
  float* y_part = reinterpret_cast<float*>(base + c.y);
  int nsplit = 1;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  // a split second product leaves its partials beyond the first in the
  // workspace; they are added into y_rows in order
  st = run_ffn(s, x, expert_count, expert_offset, row_slot, nullptr, w1, w3, w2, y_rows, y_part,
               size_t(s.cap) * s.D, &nsplit, reinterpret_cast<uint16_t*>(base + c.h), y_part,
               c.total - c.y, hs);
  if (st != MOE_OK || nsplit == 1) return st;
  return hip_status(moe::launch_add_rows(s, expert_count, expert_offset, y_rows, y_part,
                                         nsplit - 1, size_t(s.cap) * s.D, hs));
}

static moe_status_t moe_combine_impl(const moe_problem_t* p, const float* y_rows, const int32_t* slot_row,
                         const float* topk_gate, void* out, void* stream) {
  Shape s;
  moe_status_t st = check_problem(p, &s);
  if (st != MOE_OK) return st;
  if (s.T == 0) return MOE_OK;
  if (!y_rows || !slot_row || !topk_gate || !out) return MOE_EINVAL;
  if (!aligned16(y_rows) || !aligned16(slot_row) || !aligned16(topk_gate) || !aligned16(out))
    return MOE_EINVAL;
  return hip_status(moe::launch_combine(s, y_rows, 1, 0, slot_row, nullptr, topk_gate, out,
                                        p->out_dtype == MOE_BF16,
                                        static_cast<hipStream_t>(stream)));
}

static moe_status_t moe_route_stats_impl(const moe_problem_t* p, const int32_t* topk_idx, int32_t* counts,
                             void* stream) {
  Shape s;
  moe_status_t st = check_problem(p, &s);
  if (st != MOE_OK) return st;
  if (!counts || (s.T > 0 && !topk_idx)) return MOE_EINVAL;
  if (!aligned16(counts) || (topk_idx && !aligned16(topk_idx))) return MOE_EINVAL;
  return hip_status(moe::launch_route_stats(s, topk_idx, counts, static_cast<hipStream_t>(stream)));
}

static moe_status_t moe_forward_timed_impl(const moe_problem_t* p, const void* x,
                                           const void* w_gate, const void* w1, const void* w3,
                                           const void* w2, void* out, int32_t* topk_idx,
                                           float* topk_gate, void* ws, size_t ws_bytes,
                                           void* stream, void* const* events);

moe_status_t moe_forward(const moe_problem_t* p, const void* x, const void* w_gate,
                         const void* w1, const void* w3, const void* w2, void* out,
                         int32_t* topk_idx, float* topk_gate, void* ws, size_t ws_bytes,
                         void* stream) {
  return logged("moe_forward", p,
                moe_forward_timed_impl(p, x, w_gate, w1, w3, w2, out, topk_idx, topk_gate, ws,
                                       ws_bytes, stream, nullptr));
}

static moe_status_t moe_forward_timed_impl(const moe_problem_t* p, const void* x, const void* w_gate,
                               const void* w1, const void* w3, const void* w2, void* out,
                               int32_t* topk_idx, float* topk_gate, void* ws, size_t ws_bytes,
                               void* stream, void* const* events) {
  Shape s;
  moe_status_t st = check_problem(p, &s);
  if (st != MOE_OK) return st;
  if (s.T == 0) return MOE_OK;
  if (!x || !w_gate || !w1 || !w3 || !w2 || !out) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(w_gate) || !aligned16(w1) || !aligned16(w3) ||
      !aligned16(w2) || !aligned16(out) || (topk_idx && !aligned16(topk_idx)) ||
      (topk_gate && !aligned16(topk_gate)))
    return MOE_EINVAL;
  const Carve c = carve(s);
  if (!ws || ws_bytes < c.total) return MOE_EWORKSPACE;
  if ((reinterpret_cast<uintptr_t>(ws) & (kAlign - 1)) != 0) return MOE_EINVAL;
  uint8_t* base = static_cast<uint8_t*>(ws);
  int32_t* idx = topk_idx ? topk_idx : reinterpret_cast<int32_t*>(base + c.idx);
  float* gate = topk_gate ? topk_gate : reinterpret_cast<float*>(base + c.gate);
  int32_t* count = reinterpret_cast<int32_t*>(base + c.count);
  int32_t* offset = reinterpret_cast<int32_t*>(base + c.offset);
  int32_t* row_slot = reinterpret_cast<int32_t*>(base + c.row_slot);
  int32_t* slot_row = reinterpret_cast<int32_t*>(base + c.slot_row);
  uint16_t* h = reinterpret_cast<uint16_t*>(base + c.h);
  float* y = reinterpret_cast<float*>(base + c.y);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  auto mark = [&](int i) {
    return events && events[i] ? hipEventRecord(static_cast<hipEvent_t>(events[i]), hs)
                               : hipSuccess;
  };

  if (mark(0) != hipSuccess) return MOE_EHIP;
  if (moe::launch_route(s, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_gate),
                        idx, gate, nullptr, y, hs) != hipSuccess || mark(1) != hipSuccess)
    return MOE_EHIP;
  // The weight-streaming path finds each expert's token-slots in the routing
  // itself (at most MOE_STREAM_MAX_TOKENS tokens), so it needs no permute pass; its rows of y
  // are then indexed by slot.
  const bool scan = use_decode(s);
  if ((!scan && moe::launch_permute(s, idx, count, offset, row_slot, slot_row, hs) != hipSuccess) ||
      mark(2) != hipSuccess)
    return MOE_EHIP;
  const size_t part_stride = size_t(s.cap) * s.D;
  int nsplit = 1;
  st = run_ffn(s, x, count, offset, row_slot, scan ? idx : nullptr, w1, w3, w2, y,
               y + part_stride, part_stride, &nsplit, h, y, c.total - c.y, hs,
               events ? MarkFn(mark) : MarkFn());
  if (st != MOE_OK) return st;
  if (moe::launch_combine(s, y, nsplit, part_stride, scan ? nullptr : slot_row, idx, gate, out,
                          p->out_dtype == MOE_BF16, hs) != hipSuccess ||
      mark(5) != hipSuccess)
    return MOE_EHIP;
  return MOE_OK;
}

static moe_status_t moe_forward_noalloc_impl(const moe_problem_t* p, const void* x, const void* w_gate,
                                 const void* w1, const void* w3, const void* w2, void* out,
                                 int32_t* topk_idx, float* topk_gate, void* stream) {
  Shape s;
  moe_status_t st = check_problem(p, &s);
  if (st != MOE_OK) return st;
  if (s.T == 0) return MOE_OK;
  if (!x || !w_gate || !w1 || !w3 || !w2 || !out) return MOE_EINVAL;
  if (!aligned16(x) || !aligned16(w_gate) || !aligned16(w1) || !aligned16(w3) ||
      !aligned16(w2) || !aligned16(out) || (topk_idx && !aligned16(topk_idx)) ||
      (topk_gate && !aligned16(topk_gate)))
    return MOE_EINVAL;
  // only the weight-streaming path, whose intermediates are small
  if (!s.stream) return MOE_ENOTSUP;
  const CompactCarve c = compact_carve(s);
  if (c.total > kStaticScratchBytes) return MOE_ENOTSUP;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  int dev = -1, sdev = -1;
  if (hipGetDevice(&dev) != hipSuccess || hipStreamGetDevice(hs, &sdev) != hipSuccess)
    return MOE_EHIP;
  if (sdev != dev) return MOE_EINVAL;  // the array's address is the current device's
  uint8_t* base = static_scratch(dev);
  if (!base) return MOE_EHIP;
  int32_t* idx = topk_idx ? topk_idx : reinterpret_cast<int32_t*>(base + c.idx);
  float* gate = topk_gate ? topk_gate : reinterpret_cast<float*>(base + c.gate);
  float* ab = reinterpret_cast<float*>(base + c.ab);
  float* y = reinterpret_cast<float*>(base + c.y);
  const size_t part_stride = size_t(s.T) * s.K * s.D;
  if (moe::launch_route(s, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_gate),
                        idx, gate, nullptr, y, hs) != hipSuccess)
    return MOE_EHIP;
  int nsplit = 1;
  st = run_ffn(s, x, nullptr, nullptr, nullptr, idx, w1, w3, w2, y, y + part_stride, part_stride,
               &nsplit, reinterpret_cast<uint16_t*>(ab), nullptr, 0, hs);
  if (st != MOE_OK) return st;
  // nsplit == c.planes: the second product's partials fill the y planes
  return hip_status(moe::launch_combine(s, y, nsplit, part_stride, nullptr, idx, gate, out,
                                        p->out_dtype == MOE_BF16, hs));
}

moe_status_t moe_route(const moe_problem_t* p, const void* x, const void* w_gate,
                       int32_t* topk_idx, float* topk_gate, float* logits, void* ws,
                       size_t ws_bytes, void* stream) {
  return logged("moe_route", p, moe_route_impl(p, x, w_gate, topk_idx, topk_gate, logits, ws,
                                               ws_bytes, stream));
}

moe_status_t moe_permute(const moe_problem_t* p, const int32_t* topk_idx, int32_t* expert_count,
                         int32_t* expert_offset, int32_t* row_slot, int32_t* slot_row,
                         void* stream) {
  return logged("moe_permute", p, moe_permute_impl(p, topk_idx, expert_count, expert_offset,
                                                   row_slot, slot_row, stream));
}

moe_status_t moe_grouped_ffn(const moe_problem_t* p, const void* x, const int32_t* expert_count,
                             const int32_t* expert_offset, const int32_t* row_slot,
                             const void* w1, const void* w3, const void* w2, float* y_rows,
                             void* ws, size_t ws_bytes, void* stream) {
  return logged("moe_grouped_ffn", p,
                moe_grouped_ffn_impl(p, x, expert_count, expert_offset, row_slot, w1, w3, w2,
                                     y_rows, ws, ws_bytes, stream));
}

moe_status_t moe_combine(const moe_problem_t* p, const float* y_rows, const int32_t* slot_row,
                         const float* topk_gate, void* out, void* stream) {
  return logged("moe_combine", p, moe_combine_impl(p, y_rows, slot_row, topk_gate, out, stream));
}

moe_status_t moe_route_stats(const moe_problem_t* p, const int32_t* topk_idx, int32_t* counts,
                             void* stream) {
  return logged("moe_route_stats", p, moe_route_stats_impl(p, topk_idx, counts, stream));
}

moe_status_t moe_forward_timed(const moe_problem_t* p, const void* x, const void* w_gate,
                               const void* w1, const void* w3, const void* w2, void* out,
                               int32_t* topk_idx, float* topk_gate, void* ws, size_t ws_bytes,
                               void* stream, void* const* events) {
  return logged("moe_forward_timed", p,
                moe_forward_timed_impl(p, x, w_gate, w1, w3, w2, out, topk_idx, topk_gate, ws,
                                       ws_bytes, stream, events));
}

moe_status_t moe_forward_noalloc(const moe_problem_t* p, const void* x, const void* w_gate,
                                 const void* w1, const void* w3, const void* w2, void* out,
                                 int32_t* topk_idx, float* topk_gate, void* stream) {
  return logged("moe_forward_noalloc", p,
                moe_forward_noalloc_impl(p, x, w_gate, w1, w3, w2, out, topk_idx, topk_gate,
                                         stream));
}

}  // extern "C"
