// Router and gate: logits = x . W_g, G(x) = Softmax(TopK(logits)).
// "Mixtral of Experts", section 2.1 (garden.houmin.site translation): the gate
// is the softmax of the Top-K logits of a linear layer; logits outside the
// top K are set to -inf, so they get a gate of exactly zero.
//
// A workgroup of 256 threads owns TPW consecutive tokens and splits the dim
// axis between its threads: thread i reads the 16-byte steps 8*i + 2048*j, so
// each token row is read as coalesced 1 KiB segments, and every W_g row is
// loaded once per step and reused for the TPW tokens.  The TPW*NE partial sums
// of the 256 threads are reduced through LDS in two fixed-order stages (no
// atomics, deterministic), then thread t picks the top K of token t (strict
// ">" so the lower expert index wins a tie) and writes the softmax over the
// kept logits.  The kernel is bound by reading x from HBM (n = 8 multiply-adds
// per 2-byte element) and by its latency at small batches, so it is kept
// short: no unrolled cross-lane shuffles, one compact epilogue.
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kRouterThreads = 256;

// NE: compile-time upper bound on n; VEC: n == NE == 8k, W_g rows loaded as uint4.
template <int NE, int TPW, bool VEC>
__global__ __launch_bounds__(kRouterThreads) void router_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg, int T, int D, int n,
    int K, int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate,
    float* __restrict__ logits) {
  constexpr int R = TPW * NE;                 // values per workgroup: (token, expert)
  constexpr int TPR = kRouterThreads / R;     // threads per value in the first stage
  static_assert(kRouterThreads % R == 0, "values must divide the threads");
  __shared__ float part[kRouterThreads][R + 1];   // +1: spread the column reads over banks
  __shared__ float stage1[R][TPR];
  __shared__ float total[R];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * TPW;

  float acc[TPW][NE];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[t][e] = 0.f;

  for (int k = tid * 8; k < D; k += kRouterThreads * 8) {
    uint4 xv[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
      xv[t] = (t0 + t < T) ? *reinterpret_cast<const uint4*>(x + size_t(t0 + t) * D + k)
                           : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float w[NE];
      if constexpr (VEC) {
#pragma unroll
        for (int q = 0; q < NE / 8; ++q) {
          const uint4 wv = *reinterpret_cast<const uint4*>(wg + size_t(k + j) * NE + q * 8);
          w[q * 8 + 0] = bf16_lo(wv.x); w[q * 8 + 1] = bf16_hi(wv.x);
          w[q * 8 + 2] = bf16_lo(wv.y); w[q * 8 + 3] = bf16_hi(wv.y);
          w[q * 8 + 4] = bf16_lo(wv.z); w[q * 8 + 5] = bf16_hi(wv.z);
          w[q * 8 + 6] = bf16_lo(wv.w); w[q * 8 + 7] = bf16_hi(wv.w);
        }
      } else {
#pragma unroll
        for (int e = 0; e < NE; ++e)
          w[e] = (e < n) ? bf16_to_f32(wg[size_t(k + j) * n + e]) : 0.f;
      }
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        const uint32_t word = (j >> 1) == 0 ? xv[t].x : (j >> 1) == 1 ? xv[t].y
                            : (j >> 1) == 2 ? xv[t].z : xv[t].w;
        const float xj = (j & 1) ? bf16_hi(word) : bf16_lo(word);
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[t][e] = fmaf(xj, w[e], acc[t][e]);
      }
    }
  }

  // reduction: part[thread][value]; stage 1 sums TPR contiguous runs of
  // threads per value, stage 2 sums the runs, both in increasing order
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int e = 0; e < NE; ++e) part[tid][t * NE + e] = acc[t][e];
  __syncthreads();
  {
    const int v = tid / TPR, c = tid - v * TPR;
    constexpr int RUN = kRouterThreads / TPR;
    float sum = 0.f;
    for (int i = 0; i < RUN; ++i) sum += part[c * RUN + i][v];
    stage1[v][c] = sum;
  }
  __syncthreads();
  if (tid < R) {
    float sum = 0.f;
    for (int c = 0; c < TPR; ++c) sum += stage1[tid][c];
    total[tid] = sum;
  }
  __syncthreads();
  if (tid >= TPW || t0 + tid >= T) return;

  const int tok = t0 + tid;
  float l[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) l[e] = total[tid * NE + e];
  if (logits)
    for (int e = 0; e < n; ++e) logits[size_t(tok) * n + e] = l[e];
  // Top-K by repeated selection: strictly larger wins, so ties keep the lower
  // index, and slot order is decreasing logit.  Softmax over the kept logits
  // (exp(-inf) = 0 for the rest), shifted by the largest, which is slot 0.
  uint64_t taken = 0;
  float top = 0.f, sum = 0.f;
  for (int s = 0; s < K; ++s) {
    int bi = -1;
    float bv = 0.f;
#pragma unroll
    for (int e = 0; e < NE; ++e)
      if (e < n && !((taken >> e) & 1ull) && (bi < 0 || l[e] > bv)) {
        bi = e;
        bv = l[e];
      }
    taken |= 1ull << bi;
    if (s == 0) top = bv;
    const float ex = __expf(bv - top);
    sum += ex;
    topk_idx[size_t(tok) * K + s] = bi;
    topk_gate[size_t(tok) * K + s] = ex;
  }
  const float inv = 1.f / sum;
  for (int s = 0; s < K; ++s) topk_gate[size_t(tok) * K + s] *= inv;
}

template <int NE, int TPW, bool VEC>
hipError_t launch_router_t(const Shape& s, const uint16_t* x, const uint16_t* wg, int32_t* idx,
                           float* gate, float* logits, hipStream_t stream) {
  const int blocks = (s.T + TPW - 1) / TPW;
  hipLaunchKernelGGL((router_kernel<NE, TPW, VEC>), dim3(blocks), dim3(kRouterThreads), 0,
                     stream, x, wg, s.T, s.D, s.n, s.K, idx, gate, logits);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const Shape& s, const uint16_t* x, const uint16_t* w_gate,
                        int32_t* topk_idx, float* topk_gate, float* logits,
                        hipStream_t stream) {
  if (s.T == 0) return hipSuccess;
  if (s.n == 8) return launch_router_t<8, 4, true>(s, x, w_gate, topk_idx, topk_gate, logits, stream);
  if (s.n == 16) return launch_router_t<16, 2, true>(s, x, w_gate, topk_idx, topk_gate, logits, stream);
  if (s.n <= 8) return launch_router_t<8, 4, false>(s, x, w_gate, topk_idx, topk_gate, logits, stream);
  if (s.n <= 16) return launch_router_t<16, 2, false>(s, x, w_gate, topk_idx, topk_gate, logits, stream);
  if (s.n <= 32) return launch_router_t<32, 1, false>(s, x, w_gate, topk_idx, topk_gate, logits, stream);
  return launch_router_t<64, 1, false>(s, x, w_gate, topk_idx, topk_gate, logits, stream);
}

}  // namespace moe
