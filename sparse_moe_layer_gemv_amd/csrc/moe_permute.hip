// Group token-slots by expert.
// "Mixtral of Experts", section 2.1: experts whose gate is zero are skipped,
// so each expert processes only the tokens routed to it, and different experts
// receive unequal numbers of tokens.  This kernel builds that grouping: a
// counting sort of the T*K slots by expert, stable in slot order, with each
// expert's segment padded to a multiple of kTileM rows so the grouped GEMM can
// tile every segment without crossing into the next expert.
//
// One workgroup of 1024 threads: an LDS histogram, a scan of the padded
// counts, then rounds of 1024 slots in which each wavefront ranks its lanes
// per expert with ballots and the waves' counts are prefix-summed in LDS.
// The work is integer-only and tiny (T*K int32 read once); a single workgroup
// keeps the result deterministic without atomics on global memory.
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / 64;

__global__ __launch_bounds__(kPermThreads) void permute_kernel(
    const int32_t* __restrict__ topk_idx, int P, int n, int64_t cap,
    int32_t* __restrict__ expert_count, int32_t* __restrict__ expert_offset,
    int32_t* __restrict__ row_slot, int32_t* __restrict__ slot_row) {
  __shared__ int s_cnt[64];
  __shared__ int s_off[65];
  __shared__ int s_run[64];
  __shared__ int s_wcnt[kPermWaves][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const uint64_t lanes_below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));

  if (tid < 64) {
    s_cnt[tid] = 0;
    s_run[tid] = 0;
  }
  __syncthreads();

  // 1. histogram of valid slots
  for (int s = tid; s < P; s += kPermThreads) {
    const int e = topk_idx[s];
    if (e >= 0 && e < n) atomicAdd(&s_cnt[e], 1);
  }
  __syncthreads();

  // 2. padded exclusive scan
  if (tid == 0) {
    int off = 0;
    for (int e = 0; e < n; ++e) {
      s_off[e] = off;
      off += (s_cnt[e] + kTileM - 1) / kTileM * kTileM;
    }
    s_off[n] = off;
  }
  __syncthreads();
  if (tid < n) expert_count[tid] = s_cnt[tid];
  if (tid <= n) expert_offset[tid] = s_off[tid];

  // 3. stable scatter, 1024 slots per round
  int e_next = (tid < P) ? topk_idx[tid] : -1;
  for (int base = 0; base < P; base += kPermThreads) {
    const int s = base + tid;
    int e = e_next;
    if (s < P && (e < 0 || e >= n)) {
      slot_row[s] = -1;
      e = -1;
    }
    if (s >= P) e = -1;
    e_next = (s + kPermThreads < P) ? topk_idx[s + kPermThreads] : -1;

    int rank = 0;
    for (int x = 0; x < n; ++x) {
      const uint64_t m = __ballot(e == x);
      if (e == x) rank = __popcll(m & lanes_below);
      if (lane == 0) s_wcnt[wave][x] = __popcll(m);
    }
    __syncthreads();
    if (e >= 0) {
      int before = s_run[e];
      for (int w = 0; w < wave; ++w) before += s_wcnt[w][e];
      const int pos = s_off[e] + before + rank;
      row_slot[pos] = s;
      slot_row[s] = pos;
    }
    __syncthreads();
    if (tid < n) {
      int add = 0;
      for (int w = 0; w < kPermWaves; ++w) add += s_wcnt[w][tid];
      s_run[tid] += add;
    }
    __syncthreads();
  }

  // 4. padding rows of each segment, and the unused tail of the capacity
  for (int e = 0; e < n; ++e)
    for (int r = s_off[e] + s_cnt[e] + tid; r < s_off[e + 1]; r += kPermThreads) row_slot[r] = -1;
  for (int64_t r = s_off[n] + tid; r < cap; r += kPermThreads) row_slot[r] = -1;
}

}  // namespace

hipError_t launch_permute(const Shape& s, const int32_t* topk_idx, int32_t* expert_count,
                          int32_t* expert_offset, int32_t* row_slot, int32_t* slot_row,
                          hipStream_t stream) {
  hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermThreads), 0, stream, topk_idx,
                     s.T * s.K, s.n, s.cap, expert_count, expert_offset, row_slot, slot_row);
  return hipGetLastError();
}

}  // namespace moe
