// Internal interface between the C ABI (moe_api.cpp) and the HIP kernels.
// Nothing here is exported; every launcher enqueues on `stream` and returns
// the launch status without synchronising.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Permuted-layout granule (rows per expert segment step); equals MOE_TILE_M.
constexpr int kTileM = 256;
// Largest number of experts; equals MOE_MAX_EXPERTS.
constexpr int kMaxExperts = 256;
// Largest T the weight-streaming (decode) expert path supports (equals
// MOE_STREAM_MAX_TOKENS): every expert then holds at most 128 token rows,
// taken in passes of 32 or 64 rows.
constexpr int kStreamMaxTokens = 128;
// Largest T for which the automatic path choice streams: the small-batch sweep
// (Mixtral shape) measures streaming faster up to T = 80 (478-488 against
// 495-497 us on two boxes), the two paths within 3% of each other at T = 96
// (489-505 against 499 us), and the tiled path faster from T = 112.
constexpr int kDecodeMaxTokens = 80;
// Token rows handled together by one decode pass (one 16x16 MFMA column block).
constexpr int kDecodeRows = 16;

struct Shape {
  int T, D, H, n, K;
  int64_t cap;  // rows of the permuted layout
  bool stream;  // expert products by weight streaming (else tiled)
};

// Router and gate.  With more than 16 experts the logits run on the matrix
// cores in contraction slices whose fp32 partial sums go through `scratch`
// (route_scratch_bytes; 0 and unused otherwise).
size_t route_scratch_bytes(const Shape& s);
hipError_t launch_route(const Shape& s, const uint16_t* x, const uint16_t* w_gate,
                        int32_t* topk_idx, float* topk_gate, float* logits, float* scratch,
                        hipStream_t stream);

hipError_t launch_permute(const Shape& s, const int32_t* topk_idx, int32_t* expert_count,
                          int32_t* expert_offset, int32_t* row_slot, int32_t* slot_row,
                          hipStream_t stream);

// Tiled matrix-core path: h = silu(x w1) * (x w3) per expert segment, then
// y_rows = h w2.  h is bf16 [cap][H] in the workspace.  Experts with at most
// 128 slots run as one tile of 128 or 64 rows (chosen from expert_count on
// the device), larger ones as full 256-row tiles.  `scratch` (may be null)
// holds the fp32 halves of a split last round of first-product tiles; it is
// only read and written between the two launches of this call.
hipError_t launch_grouped_up(const Shape& s, const uint16_t* x, const int32_t* expert_count,
                             const int32_t* expert_offset, const int32_t* row_slot,
                             const uint16_t* w1, const uint16_t* w3, uint16_t* h, void* scratch,
                             size_t scratch_bytes, hipStream_t stream);
// Scratch that lets launch_grouped_up split its last round (0: never splits).
size_t grouped_up_scratch_bytes(const Shape& s);
// The second product may be split along its contraction into nsplit = 2
// partial sums (see grouped_down_splits): partial 0 at y_rows, partial 1 at
// y_part (unused, may be null, when nsplit = 1).
int grouped_down_splits(const Shape& s);
// Rows past an expert's slots (padding) are not written.
hipError_t launch_grouped_down(const Shape& s, const int32_t* expert_count,
                               const int32_t* expert_offset, const uint16_t* h,
                               const uint16_t* w2, float* y_rows, int nsplit, float* y_part,
                               hipStream_t stream);

// Weight-streaming path for small T (every touched expert's weights read once).
// The first product writes into `scratch` (decode_scratch_bytes) either
// h = bf16(silu(x w1) * (x w3)) per token-slot ([T*K][H], wide experts with
// many tokens) or fp32 a = x w1 and b = x w3 ([S][2][T*K][H], S contraction
// partials), from which the second product forms h on the fly.  The second
// product may split its contraction into `nsplit` partial sums
// (decode_down_splits, at most 8): partial 0 at y_rows, partial ks >= 1 at
// y_part + (ks-1) * part_stride.
// Each expert's token-slots come from the permuted layout (expert_count,
// expert_offset, row_slot; y rows at the permuted row) or, when topk_idx is
// given, from scanning the routing (the others may be null; y rows at the
// slot index t*K + k).
size_t decode_scratch_bytes(const Shape& s);
int decode_down_splits(const Shape& s);
// launch_decode_up writes a and b; launch_decode_down forms h in the scratch
// (one pass over the slots) and runs the second product.
hipError_t launch_decode_up(const Shape& s, const uint16_t* x, const int32_t* expert_count,
                            const int32_t* expert_offset, const int32_t* row_slot,
                            const int32_t* topk_idx, const uint16_t* w1, const uint16_t* w3,
                            void* scratch, hipStream_t stream);
hipError_t launch_decode_down(const Shape& s, const int32_t* expert_count,
                              const int32_t* expert_offset, const int32_t* row_slot,
                              const int32_t* topk_idx, void* scratch, const uint16_t* w2,
                              float* y_rows, float* y_part, int nsplit, size_t part_stride,
                              hipStream_t stream);

// out[t] = sum_k gate[t][k] * (sum_p y_rows[p * split_stride + row(t,k)]),
// partials p summed first, in order.  row(t,k) = slot_row[t*K + k] (-1: the
// slot contributes nothing) or, with slot_row null, the slot index t*K + k
// itself for slots whose topk_idx names an expert in [0, n).
hipError_t launch_combine(const Shape& s, const float* y_rows, int nsplit, size_t split_stride,
                          const int32_t* slot_row, const int32_t* topk_idx,
                          const float* topk_gate, void* out, bool out_bf16, hipStream_t stream);

// Routing diagnostics: counts [2n + 2] (see moe_route_stats).
hipError_t launch_route_stats(const Shape& s, const int32_t* topk_idx, int32_t* counts,
                              hipStream_t stream);

// y_rows[r] += y_part[p * part_stride + r] for p = 0 .. nparts-1 in order, for
// the rows that hold token-slots (offset[e] <= r < offset[e] + count[e]).
hipError_t launch_add_rows(const Shape& s, const int32_t* expert_count,
                           const int32_t* expert_offset, float* y_rows, const float* y_part,
                           int nparts, size_t part_stride, hipStream_t stream);

}  // namespace moe
