// Group token-slots by expert.
// "Mixtral of Experts", section 2.1: experts whose gate is zero are skipped,
// so each expert processes only the tokens routed to it, and different experts
// receive unequal numbers of tokens.  This kernel builds that grouping: a
// counting sort of the T*K slots by expert, stable in slot order, with each
// expert's segment padded to a multiple of kTileM rows so the grouped GEMM can
// tile every segment without crossing into the next expert.
//
// The slots are taken in rounds of 1024, one slot per thread; the rounds are
// split into contiguous runs over up to kPermMaxBlocks workgroups.  Every
// workgroup histograms the whole batch in LDS (integer atomics, so the counts
// are exact) and with it the slots before its first round, scans the padded
// counts itself, and then places its own rounds: inside a wavefront a slot's
// rank among the lanes of its expert comes from a ballot per distinct expert
// present in the wave (at most 64, usually far fewer than n), and the waves'
// counts are prefix-summed in LDS.  No workgroup waits for another, nothing
// goes through global scratch, and the result is deterministic.
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kPermThreads = 1024;
constexpr int kPermWaves = kPermThreads / 64;
constexpr int kPermMaxBlocks = 64;
static_assert(kMaxExperts <= 4 * 64, "the offset scan gives each lane 4 experts");

__device__ __forceinline__ int padded(int c) { return (c + kTileM - 1) / kTileM * kTileM; }

__global__ __launch_bounds__(kPermThreads) void permute_kernel(
    const int32_t* __restrict__ topk_idx, int P, int n, int64_t cap, int rounds_per_block,
    int32_t* __restrict__ expert_count, int32_t* __restrict__ expert_offset,
    int32_t* __restrict__ row_slot, int32_t* __restrict__ slot_row) {
  __shared__ int s_cnt[kMaxExperts];    // slots per expert in the batch
  __shared__ int s_run[kMaxExperts];    // slots per expert before the current round
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_wcnt[kPermWaves][kMaxExperts];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const uint64_t lanes_below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int first = blockIdx.x * rounds_per_block * kPermThreads;  // first slot of this block
  const int last = min(P, first + rounds_per_block * kPermThreads);

  if (tid < n) {
    s_cnt[tid] = 0;
    s_run[tid] = 0;
  }
  __syncthreads();

  // 1. histogram of the valid slots: all of them, and those before `first`;
  //    the thread keeps the value of slot `first + tid` (its slot in this
  //    block's first round) so that round need not read it again
  int own = -1;
  for (int s0 = 0; s0 < P; s0 += 4 * kPermThreads) {
    int e[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int s = s0 + u * kPermThreads + tid;
      e[u] = s < P ? topk_idx[s] : -1;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int s = s0 + u * kPermThreads + tid;
      if (s == first + tid) own = e[u];
      if (e[u] >= 0 && e[u] < n) {
        atomicAdd(&s_cnt[e[u]], 1);
        if (s < first) atomicAdd(&s_run[e[u]], 1);
      }
    }
  }
  __syncthreads();

  // 2. padded exclusive scan over the experts: wave 0, 4 experts per lane
  if (wave == 0) {
    int pc[4], local = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane * 4 + j;
      pc[j] = e < n ? padded(s_cnt[e]) : 0;
      local += pc[j];
    }
    int inc = local;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(inc, d, 64);
      if (lane >= d) inc += y;
    }
    int off = inc - local;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane * 4 + j;
      if (e < n) s_off[e] = off;
      off += pc[j];
    }
    if (lane == 63) s_off[n] = inc;
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    if (tid < n) expert_count[tid] = s_cnt[tid];
    if (tid <= n) expert_offset[tid] = s_off[tid];
  }

  // 3. stable placement of this block's rounds
  for (int base = first; base < last; base += kPermThreads) {
    const int s = base + tid;
    int e = -1;
    if (s < P) {
      e = base == first ? own : topk_idx[s];
      if (e < 0 || e >= n) {
        slot_row[s] = -1;
        e = -1;
      }
    }
    for (int x = lane; x < n; x += 64) s_wcnt[wave][x] = 0;
    int rank = 0;
    uint64_t todo = __ballot(e >= 0);
    while (todo) {
      const int lead = __builtin_ctzll(todo);
      const int x = __builtin_amdgcn_readlane(e, lead);
      const uint64_t m = __ballot(e == x);
      if (e == x) rank = __popcll(m & lanes_below);
      if (lane == 0) s_wcnt[wave][x] = __popcll(m);
      todo &= ~m;
    }
    __syncthreads();
    if (e >= 0) {
      int pos = s_off[e] + s_run[e] + rank;
      for (int w = 0; w < wave; ++w) pos += s_wcnt[w][e];
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

  // 4. padding rows of the segments and the unused tail of the capacity,
  //    shared out over the workgroups
  const int nb = gridDim.x;
  for (int x = blockIdx.x * kPermWaves + wave; x < n; x += nb * kPermWaves)
    for (int r = s_off[x] + s_cnt[x] + lane; r < s_off[x + 1]; r += 64) row_slot[r] = -1;
  const int64_t tail0 = s_off[n];
  const int64_t per = (cap - tail0 + nb - 1) / nb;
  const int64_t r0 = tail0 + int64_t(blockIdx.x) * per;
  const int64_t r1 = min(cap, r0 + per);
  for (int64_t r = r0 + tid; r < r1; r += kPermThreads) row_slot[r] = -1;
}

}  // namespace

hipError_t launch_permute(const Shape& s, const int32_t* topk_idx, int32_t* expert_count,
                          int32_t* expert_offset, int32_t* row_slot, int32_t* slot_row,
                          hipStream_t stream) {
  const int P = s.T * s.K;
  const int rounds = (P + kPermThreads - 1) / kPermThreads;
  const int per_block = max(1, (rounds + kPermMaxBlocks - 1) / kPermMaxBlocks);
  const int blocks = max(1, (rounds + per_block - 1) / per_block);
  hipLaunchKernelGGL(permute_kernel, dim3(blocks), dim3(kPermThreads), 0, stream, topk_idx, P,
                     s.n, s.cap, per_block, expert_count, expert_offset, row_slot, slot_row);
  return hipGetLastError();
}

}  // namespace moe
