// Routing diagnostics over the chosen experts ("Mixtral of Experts",
// section 5, Routing analysis: Figure 7 and Figure 9 count the share of
// tokens assigned to each expert, as first choice and as either choice;
// Table 5 counts consecutive tokens t, t+1 that share the first-choice expert,
// or that share any chosen expert).
//
// One workgroup of 1024 threads walks the tokens (the topk_idx stream is small:
// T*K int32), keeps the per-expert histograms in LDS with integer atomics and
// the two repeat counts in registers, then reduces those through LDS.  Integer
// counts are order-independent, so the result is exact and deterministic.
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kStatThreads = 1024;

// counts layout: [0, n) first-choice slots per expert; [n, 2n) slots per
// expert over all K choices; [2n] tokens t < T-1 whose first choice equals
// that of t+1; [2n+1] tokens t < T-1 sharing any chosen expert with t+1.
// Expert ids outside [0, n) are not counted and match nothing.
__global__ __launch_bounds__(kStatThreads) void route_stats_kernel(
    const int32_t* __restrict__ idx, int T, int K, int n, int32_t* __restrict__ counts) {
  __shared__ int hist_first[kMaxExperts];
  __shared__ int hist_any[kMaxExperts];
  __shared__ int rep[2];
  const int tid = threadIdx.x;
  for (int e = tid; e < n; e += kStatThreads) {
    hist_first[e] = 0;
    hist_any[e] = 0;
  }
  if (tid < 2) rep[tid] = 0;
  __syncthreads();

  int rep_first = 0, rep_either = 0;
  for (int t = tid; t < T; t += kStatThreads) {
    const int32_t* cur = idx + size_t(t) * K;
    const int e0 = cur[0];
    if (e0 >= 0 && e0 < n) atomicAdd(&hist_first[e0], 1);
    for (int k = 0; k < K; ++k) {
      const int e = cur[k];
      if (e >= 0 && e < n) atomicAdd(&hist_any[e], 1);
    }
    if (t + 1 < T) {
      const int32_t* nxt = cur + K;
      const bool v0 = e0 >= 0 && e0 < n;
      rep_first += (v0 && nxt[0] == e0) ? 1 : 0;
      bool any = false;
      for (int a = 0; a < K && !any; ++a) {
        const int ea = cur[a];
        if (ea < 0 || ea >= n) continue;
        for (int b = 0; b < K; ++b) any = any || nxt[b] == ea;
      }
      rep_either += any ? 1 : 0;
    }
  }
  if (rep_first) atomicAdd(&rep[0], rep_first);
  if (rep_either) atomicAdd(&rep[1], rep_either);
  __syncthreads();
  for (int e = tid; e < n; e += kStatThreads) {
    counts[e] = hist_first[e];
    counts[n + e] = hist_any[e];
  }
  if (tid < 2) counts[2 * n + tid] = rep[tid];
}

}  // namespace

hipError_t launch_route_stats(const Shape& s, const int32_t* topk_idx, int32_t* counts,
                              hipStream_t stream) {
  hipLaunchKernelGGL(route_stats_kernel, dim3(1), dim3(kStatThreads), 0, stream, topk_idx, s.T,
                     s.K, s.n, counts);
  return hipGetLastError();
}

}  // namespace moe
