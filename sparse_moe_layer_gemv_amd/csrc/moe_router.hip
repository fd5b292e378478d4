// Router and gate: logits = x . W_g, G(x) = Softmax(TopK(logits)).
// "Mixtral of Experts", section 2.1 (garden.houmin.site translation): the gate
// is the softmax of the Top-K logits of a linear layer; logits outside the
// top K are set to -inf, so they get a gate of exactly zero.
//
// A workgroup of 4 wavefronts owns TPW consecutive tokens and splits the dim
// axis between its waves: lane l of wave w reads the 16-byte steps
// 8*(64*w + l) + 2048*i, so each token row is read as coalesced 1 KiB
// segments, and every W_g row is loaded once per step and reused for the TPW
// tokens.  The n partial sums per token are reduced across each wave with a
// butterfly and across the 4 waves through LDS in a fixed order; then lane t
// of wave 0 picks the top K of token t in registers (strict ">" so the lower
// expert index wins a tie) and writes the softmax over the kept logits.
// The kernel is bound by reading x from HBM (n = 8 multiply-adds per 2-byte
// element); splitting the dim axis over 4 waves keeps small batches (decode)
// from being one long dependent chain of loads.
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
  constexpr int kWaves = kRouterThreads / 64;
  __shared__ float red[kWaves][TPW][NE];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * TPW;

  float acc[TPW][NE];
#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[t][e] = 0.f;

  for (int k = (wave * 64 + lane) * 8; k < D; k += kRouterThreads * 8) {
    uint4 xv[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      if (t0 + t < T)
        xv[t] = *reinterpret_cast<const uint4*>(x + size_t(t0 + t) * D + k);
      else
        xv[t] = make_uint4(0, 0, 0, 0);
    }
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

#pragma unroll
  for (int t = 0; t < TPW; ++t)
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const float v = wave_sum(acc[t][e]);
      if (lane == 0) red[wave][t][e] = v;
    }
  __syncthreads();
  if (wave != 0) return;

#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int tok = t0 + t;
    if (lane != t || tok >= T) continue;
    float l[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      float v = red[0][t][e];
#pragma unroll
      for (int w = 1; w < kWaves; ++w) v += red[w][t][e];
      l[e] = v;
    }
    if (logits) {
#pragma unroll
      for (int e = 0; e < NE; ++e)
        if (e < n) logits[size_t(tok) * n + e] = l[e];
    }
    // Top-K by repeated selection: strictly larger wins, so ties keep the
    // lower index, and slot order is decreasing logit.
    uint64_t taken = 0;
    float kept[NE];
    int kidx[NE];
#pragma unroll
    for (int s = 0; s < NE; ++s) {
      kept[s] = 0.f;
      kidx[s] = 0;
      if (s < K) {
        int bi = -1;
        float bv = 0.f;
#pragma unroll
        for (int e = 0; e < NE; ++e) {
          if (e < n && !((taken >> e) & 1ull) && (bi < 0 || l[e] > bv)) {
            bi = e;
            bv = l[e];
          }
        }
        taken |= 1ull << bi;
        kept[s] = bv;
        kidx[s] = bi;
      }
    }
    // Softmax over the kept logits (exp(-inf) = 0 for the rest), shifted by
    // the largest, which is slot 0.
    float ex[NE];
    float sum = 0.f;
#pragma unroll
    for (int s = 0; s < NE; ++s) {
      ex[s] = (s < K) ? __expf(kept[s] - kept[0]) : 0.f;
      sum += ex[s];
    }
#pragma unroll
    for (int s = 0; s < NE; ++s) {
      if (s < K) {
        topk_idx[size_t(tok) * K + s] = kidx[s];
        topk_gate[size_t(tok) * K + s] = ex[s] / sum;
      }
    }
  }
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
