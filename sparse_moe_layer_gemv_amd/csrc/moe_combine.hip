// Gate-weighted combine of the expert outputs.
// "Mixtral of Experts", section 2.1, first display equation: the layer output
// is the sum over experts of G(x)_i * E_i(x); with TopK gating only the K
// chosen experts contribute.  out[t] = sum_k gate[t][k] * y_rows[slot_row[t*K+k]],
// summed in slot order k = 0, 1, ... (a gather, no atomics, so it is
// deterministic).  Bound by HBM: reads K fp32 rows and writes one row per token.
#include <algorithm>

#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kCombineThreads = 256;
constexpr int kCols = kCombineThreads * 4;  // columns per workgroup

// Every expert row is read once and every output row written once, so both
// bypass the caches' retention (non-temporal): at fine_prefill (537 MB of
// rows) the combine went from 120 to 104 us alone, 63% to 73% of HBM.
__device__ __forceinline__ f32x4 load_once(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}

template <bool OUT_BF16>
__device__ __forceinline__ void store_out(void* out, size_t at, const f32x4& acc) {
  if constexpr (OUT_BF16) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 pk = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
    __builtin_nontemporal_store(pk, reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + at));
  } else {
    __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(static_cast<float*>(out) + at));
  }
}

// Row of y_rows holding slot i: slot_row[i], or (slot_row null) the slot
// itself when its expert index is in range; -1 when the slot contributes
// nothing.
__device__ __forceinline__ int slot_source(const int32_t* __restrict__ slot_row,
                                           const int32_t* __restrict__ topk_idx, int n,
                                           size_t i) {
  if (slot_row) return slot_row[i];
  const int e = topk_idx[i];
  return (e >= 0 && e < n) ? int(i) : -1;
}

// One workgroup per (token, 1024-column block); each thread owns 4 columns.
// The token's slots and gates are read once and all K (x nsplit partial) row
// fragments are loaded before they are summed, so a small batch is one round
// of loads deep.  KMAX bounds K for this register copy of the slots.
template <bool OUT_BF16, int KMAX>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const float* __restrict__ y_rows, int nsplit, size_t split_stride,
    const int32_t* __restrict__ slot_row, const int32_t* __restrict__ topk_idx, int n,
    const float* __restrict__ gate, int D, int K, int ncb, void* __restrict__ out) {
  const int t = blockIdx.x / ncb;
  const int d = (blockIdx.x - t * ncb) * kCols + threadIdx.x * 4;
  if (d >= D) return;
  int r[KMAX];
  float g[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    r[k] = k < K ? slot_source(slot_row, topk_idx, n, size_t(t) * K + k) : -1;
    g[k] = k < K ? gate[size_t(t) * K + k] : 0.f;
  }
  f32x4 v[KMAX];
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    v[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (r[k] >= 0) {
      v[k] = load_once(y_rows + size_t(r[k]) * D + d);
      for (int p = 1; p < nsplit; ++p) v[k] += load_once(y_rows + p * split_stride + size_t(r[k]) * D + d);
    }
  }
  // slot order; the partials of one slot were added first
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    if (r[k] < 0) continue;
    acc[0] = fmaf(g[k], v[k][0], acc[0]);
    acc[1] = fmaf(g[k], v[k][1], acc[1]);
    acc[2] = fmaf(g[k], v[k][2], acc[2]);
    acc[3] = fmaf(g[k], v[k][3], acc[3]);
  }
  store_out<OUT_BF16>(out, size_t(t) * D + d, acc);
}

// K beyond the register copy: the slots are walked in order from memory.
template <bool OUT_BF16>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel_any_k(
    const float* __restrict__ y_rows, int nsplit, size_t split_stride,
    const int32_t* __restrict__ slot_row, const int32_t* __restrict__ topk_idx, int n,
    const float* __restrict__ gate, int D, int K, int ncb, void* __restrict__ out) {
  const int t = blockIdx.x / ncb;
  const int d = (blockIdx.x - t * ncb) * kCols + threadIdx.x * 4;
  if (d >= D) return;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < K; ++k) {
    const int r = slot_source(slot_row, topk_idx, n, size_t(t) * K + k);
    if (r < 0) continue;
    const float g = gate[size_t(t) * K + k];
    f32x4 v = load_once(y_rows + size_t(r) * D + d);
    for (int p = 1; p < nsplit; ++p) v += load_once(y_rows + p * split_stride + size_t(r) * D + d);
    acc[0] = fmaf(g, v[0], acc[0]);
    acc[1] = fmaf(g, v[1], acc[1]);
    acc[2] = fmaf(g, v[2], acc[2]);
    acc[3] = fmaf(g, v[3], acc[3]);
  }
  store_out<OUT_BF16>(out, size_t(t) * D + d, acc);
}

template <bool OUT_BF16>
hipError_t launch_combine_t(const Shape& s, const float* y_rows, int nsplit, size_t split_stride,
                            const int32_t* slot_row, const int32_t* topk_idx,
                            const float* topk_gate, void* out, hipStream_t stream) {
  const int ncb = (s.D + kCols - 1) / kCols;
  const dim3 grid(unsigned(s.T) * unsigned(ncb));
  if (s.K <= 2)
    hipLaunchKernelGGL((combine_kernel<OUT_BF16, 2>), grid, dim3(kCombineThreads), 0, stream,
                       y_rows, nsplit, split_stride, slot_row, topk_idx, s.n, topk_gate, s.D, s.K,
                       ncb, out);
  else if (s.K <= 8)
    hipLaunchKernelGGL((combine_kernel<OUT_BF16, 8>), grid, dim3(kCombineThreads), 0, stream,
                       y_rows, nsplit, split_stride, slot_row, topk_idx, s.n, topk_gate, s.D, s.K,
                       ncb, out);
  else
    hipLaunchKernelGGL((combine_kernel_any_k<OUT_BF16>), grid, dim3(kCombineThreads), 0, stream,
                       y_rows, nsplit, split_stride, slot_row, topk_idx, s.n, topk_gate, s.D, s.K,
                       ncb, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const Shape& s, const float* y_rows, int nsplit, size_t split_stride,
                          const int32_t* slot_row, const int32_t* topk_idx,
                          const float* topk_gate, void* out, bool out_bf16, hipStream_t stream) {
  if (s.T == 0) return hipSuccess;
  return out_bf16 ? launch_combine_t<true>(s, y_rows, nsplit, split_stride, slot_row, topk_idx,
                                           topk_gate, out, stream)
                  : launch_combine_t<false>(s, y_rows, nsplit, split_stride, slot_row, topk_idx,
                                            topk_gate, out, stream);
}

// Partials added in order, as the combine adds them: (y + p1) + p2 + ...
// Only the rows that hold token-slots (offset[e] .. offset[e] + count[e] of
// each expert) are touched; padding rows are left as they were.  Workgroups
// (x, e) stride over expert e's rows (blockIdx.y = expert).
__global__ __launch_bounds__(kCombineThreads) void add_rows_kernel(
    const int32_t* __restrict__ expert_count, const int32_t* __restrict__ expert_offset, int D,
    float* __restrict__ y, const float* __restrict__ y_part, int nparts, size_t part_stride) {
  const int e = blockIdx.y;
  const size_t first = size_t(expert_offset[e]) * D / 4;
  const size_t total = size_t(expert_count[e]) * D / 4;
  for (size_t i = size_t(blockIdx.x) * kCombineThreads + threadIdx.x; i < total;
       i += size_t(gridDim.x) * kCombineThreads) {
    f32x4 a = reinterpret_cast<f32x4*>(y)[first + i];
    for (int p = 0; p < nparts; ++p)
      a += reinterpret_cast<const f32x4*>(y_part + p * part_stride)[first + i];
    reinterpret_cast<f32x4*>(y)[first + i] = a;
  }
}

hipError_t launch_add_rows(const Shape& s, const int32_t* expert_count,
                           const int32_t* expert_offset, float* y_rows, const float* y_part,
                           int nparts, size_t part_stride, hipStream_t stream) {
  // about 1024 workgroups over all experts
  const int per_expert = std::max(1, 1024 / s.n);
  hipLaunchKernelGGL(add_rows_kernel, dim3(per_expert, s.n), dim3(kCombineThreads), 0, stream,
                     expert_count, expert_offset, s.D, y_rows, y_part, nparts, part_stride);
  return hipGetLastError();
}

}  // namespace moe
