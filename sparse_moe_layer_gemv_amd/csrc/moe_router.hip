// Router and gate: logits = x . W_g, G(x) = Softmax(TopK(logits)).
// "Mixtral of Experts", section 2.1 (garden.houmin.site translation): the gate
// is the softmax of the Top-K logits of a linear layer; logits outside the
// top K are set to -inf, so they get a gate of exactly zero.
//
// Up to 64 experts: a workgroup of 256 threads owns TPW consecutive tokens and splits the dim
// axis between its threads: thread i reads the 16-byte steps 8*i + 2048*j, so
// each token row is read as coalesced 1 KiB segments, and every W_g row is
// loaded once per step and reused for the TPW tokens.  The TPW*NE partial sums
// of the 256 threads are reduced through LDS in two fixed-order stages (no
// atomics, deterministic), then thread t picks the top K of token t (strict
// ">" so the lower expert index wins a tie) and writes the softmax over the
// kept logits.  The kernel is bound by reading x from HBM (n = 8 multiply-adds
// per 2-byte element) and by its latency at small batches, so it is kept
// short: no unrolled cross-lane shuffles, one compact epilogue.
#include <algorithm>

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

// Many experts (n > 16, up to the fine-grained layout).  The logits are then
// a genuine matrix product, [T x D] . [D x n], and run on the matrix cores, in
// two launches so that many workgroups share the reading of W_g even for a
// handful of tokens.
//
// router_partial_kernel: a workgroup of 4 waves owns 16*RG tokens, 128
// experts and one slice of the contraction; its waves take the slice's
// 32-deep steps in turn.  Per step a lane loads an 8 x 8 block of W_g (8
// contraction rows, 8 experts), transposes it in registers into 8 operands
// whose rows are 16 experts strided by 8, and runs 8
// v_mfma_f32_16x16x32_bf16 per 16-token group against that group's x
// fragment.  The waves' sums are added in a fixed tree through LDS and the
// slice's partial logits are written as fp32 rows [slice][token][expert].
//
// router_select_kernel: one wave per token adds the slices' partials in
// slice order (deterministic), then selects the top K: each lane holds the
// logits of experts lane, lane+64, ... and a butterfly argmax (larger value,
// then lower index) picks each slot in turn.
constexpr int kRpWaves = 4;
constexpr int kRpThreads = kRpWaves * 64;
constexpr int kRpCols = 128;      // experts per workgroup
constexpr int kRpTarget = 1024;   // workgroups to aim for (4 per compute unit)
static_assert(kMaxExperts <= 4 * 64, "a lane holds at most 4 logits of a token");

struct RouterSplit {
  int rg;       // 16-token groups per workgroup (1 or 2)
  int tiles;    // token tiles of 16*rg
  int cblocks;  // expert blocks of 128
  int S;        // contraction slices
  int kc;       // slice length (a multiple of 32)
};

RouterSplit router_split(const Shape& s) {
  RouterSplit r;
  r.rg = s.T <= 16 ? 1 : 2;
  r.tiles = (s.T + 16 * r.rg - 1) / (16 * r.rg);
  r.cblocks = (s.n + kRpCols - 1) / kRpCols;
  const int base = r.tiles * r.cblocks;
  const int ksteps = (s.D + 31) / 32;
  int S = (kRpTarget + base - 1) / base;
  S = std::max(1, std::min(S, ksteps / kRpWaves));  // every wave gets a step
  const int steps = (ksteps + S - 1) / S;
  r.kc = steps * 32;
  r.S = (s.D + r.kc - 1) / r.kc;
  return r;
}

bool uses_matrix_router(const Shape& s) { return s.n > 16; }

template <int RG, bool VEC>
__global__ __launch_bounds__(kRpThreads) void router_partial_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg, int T, int D, int n, int S,
    int kc, int cblocks, float* __restrict__ part) {
  constexpr int NV = RG * 8 * 4;                  // accumulator floats per lane
  constexpr int TOK = 16 * RG;
  __shared__ float red[kRpWaves / 2][NV * 64];    // tree buffers; then the output tile
  float(*tile)[kRpCols] = reinterpret_cast<float(*)[kRpCols]>(&red[0][0]);
  static_assert(sizeof(red) >= sizeof(float) * TOK * kRpCols, "output tile fits");

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int kg = lane >> 4;          // contraction group of 8
  const int c16 = lane & 15;         // token column (B) and expert row block (A)
  const int sl = blockIdx.x % S;
  const int rest = blockIdx.x / S;
  const int cb = rest % cblocks;
  const int t0 = (rest / cblocks) * TOK;
  const int kbeg = sl * kc;
  const int kend = min(D, kbeg + kc);
  const int col = cb * kRpCols + c16 * 8;

  const uint16_t* xrow[RG];
  bool tok_ok[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    const int t = t0 + 16 * g + c16;
    tok_ok[g] = t < T;
    xrow[g] = x + size_t(tok_ok[g] ? t : 0) * D;
  }

  f32x4 acc[RG][8];
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[g][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = kbeg + wave * 32; k0 < kend; k0 += kRpWaves * 32) {
    const int kk = k0 + kg * 8;
    const bool kval = kk < kend;  // kend is a multiple of 8: a group is all in or all out
    uint4 wv[8];
    if constexpr (VEC) {
      const bool ok = kval && col < n;  // n is a multiple of 8 here
#pragma unroll
      for (int i = 0; i < 8; ++i)
        wv[i] = ok ? *reinterpret_cast<const uint4*>(wg + size_t(kk + i) * n + col)
                   : make_uint4(0, 0, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t h[8];
#pragma unroll
        for (int c = 0; c < 8; ++c)
          h[c] = (kval && col + c < n) ? uint32_t(wg[size_t(kk + i) * n + col + c]) : 0u;
        wv[i] = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                           h[6] | (h[7] << 16));
      }
    }
    uint4 xv[RG];
#pragma unroll
    for (int g = 0; g < RG; ++g)
      xv[g] = (kval && tok_ok[g]) ? *reinterpret_cast<const uint4*>(xrow[g] + kk)
                                  : make_uint4(0, 0, 0, 0);
    uint4 wt[8];
    transpose8x8_bf16(wv, wt);
#pragma unroll
    for (int g = 0; g < RG; ++g)
#pragma unroll
      for (int c = 0; c < 8; ++c)
        acc[g][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wt[c]), as_bf16x8(xv[g]),
                                                            acc[g][c], 0, 0, 0);
  }

  // fixed-order tree over the waves: (w0 + w2) + (w1 + w3)
#pragma unroll
  for (int half = kRpWaves / 2; half >= 1; half >>= 1) {
    if (wave >= half && wave < 2 * half) {
      float* dst = red[wave - half];
#pragma unroll
      for (int g = 0; g < RG; ++g)
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
          for (int i = 0; i < 4; ++i) dst[((g * 8 + c) * 4 + i) * 64 + lane] = acc[g][c][i];
    }
    __syncthreads();
    if (wave < half) {
      const float* src = red[wave];
#pragma unroll
      for (int g = 0; g < RG; ++g)
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[g][c][i] += src[((g * 8 + c) * 4 + i) * 64 + lane];
    }
    __syncthreads();
  }
  // wave 0 holds the slice's sums: acc[g][c][i] is expert cb*128 + (4*kg + i)*8 + c
  // of token t0 + 16*g + c16; stage them as [token][expert] rows
  if (wave == 0) {
#pragma unroll
    for (int g = 0; g < RG; ++g)
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) tile[16 * g + c16][(4 * kg + i) * 8 + c] = acc[g][c][i];
  }
  __syncthreads();
  const int ncols = min(kRpCols, n - cb * kRpCols);
  for (int q = threadIdx.x; q < TOK * kRpCols; q += kRpThreads) {
    const int r = q / kRpCols, e = q - r * kRpCols;
    const int t = t0 + r;
    if (t < T && e < ncols) part[(size_t(sl) * T + t) * n + cb * kRpCols + e] = tile[r][e];
  }
}

__global__ __launch_bounds__(256) void router_select_kernel(
    const float* __restrict__ part, int S, int T, int n, int K, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_gate, float* __restrict__ logits) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  // the slices' partials are loaded 16 slices at a time (64 loads in flight
  // per lane) and added in slice order: p0 + p1 + p2 + ...
  float v[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += 16) {
    float pv[4][16];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int e = lane + 64 * j;
        pv[j][u] = (e < n && s0 + u < S) ? part[(size_t(s0 + u) * T + t) * n + e] : 0.f;
      }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (s0 + u < S) v[j] = (s0 + u == 0) ? pv[j][u] : v[j] + pv[j][u];
  }
  if (logits)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      if (e < n) logits[size_t(t) * n + e] = v[j];
    }
  // Top-K by repeated selection.  Within a lane the experts rise with j, so a
  // strict ">" keeps the lower index; across lanes equal values go to the
  // lower index.  Slot s's expert and e^(l - top) stay in lane s % 64.
  bool taken[4] = {false, false, false, false};
  int my_idx[4] = {0, 0, 0, 0};
  float my_ex[4] = {0.f, 0.f, 0.f, 0.f};
  float top = 0.f, sum = 0.f;
  for (int s = 0; s < K; ++s) {
    int bi = -1;
    float bv = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      if (e < n && !taken[j] && (bi < 0 || v[j] > bv)) {
        bi = e;
        bv = v[j];
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const float ov = __shfl_xor(bv, m, 64);
      const int oi = __shfl_xor(bi, m, 64);
      if (oi >= 0 && (bi < 0 || ov > bv || (ov == bv && oi < bi))) {
        bv = ov;
        bi = oi;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (bi == lane + 64 * j) taken[j] = true;
    if (s == 0) top = bv;
    const float ex = __expf(bv - top);
    sum += ex;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (s == q * 64 + lane) {
        my_idx[q] = bi;
        my_ex[q] = ex;
      }
  }
  const float inv = 1.f / sum;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int s = q * 64 + lane;
    if (s < K) {
      topk_idx[size_t(t) * K + s] = my_idx[q];
      topk_gate[size_t(t) * K + s] = my_ex[q] * inv;
    }
  }
}

template <int RG, bool VEC>
void launch_partial_t(const Shape& s, const RouterSplit& r, const uint16_t* x, const uint16_t* wg,
                      float* part, hipStream_t stream) {
  const unsigned blocks = unsigned(r.tiles) * r.cblocks * r.S;
  hipLaunchKernelGGL((router_partial_kernel<RG, VEC>), dim3(blocks), dim3(kRpThreads), 0, stream,
                     x, wg, s.T, s.D, s.n, r.S, r.kc, r.cblocks, part);
}

template <bool VEC>
void launch_partial(const Shape& s, const RouterSplit& r, const uint16_t* x, const uint16_t* wg,
                    float* part, hipStream_t stream) {
  if (r.rg == 1) launch_partial_t<1, VEC>(s, r, x, wg, part, stream);
  else launch_partial_t<2, VEC>(s, r, x, wg, part, stream);
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

size_t route_scratch_bytes(const Shape& s) {
  if (s.T == 0 || !uses_matrix_router(s)) return 0;
  const RouterSplit r = router_split(s);
  return size_t(r.S) * s.T * s.n * sizeof(float);
}

hipError_t launch_route(const Shape& s, const uint16_t* x, const uint16_t* w_gate,
                        int32_t* topk_idx, float* topk_gate, float* logits, float* scratch,
                        hipStream_t stream) {
  if (s.T == 0) return hipSuccess;
  if (s.n == 8) return launch_router_t<8, 4, true>(s, x, w_gate, topk_idx, topk_gate, logits, stream);
  if (s.n == 16) return launch_router_t<16, 2, true>(s, x, w_gate, topk_idx, topk_gate, logits, stream);
  if (s.n <= 8) return launch_router_t<8, 4, false>(s, x, w_gate, topk_idx, topk_gate, logits, stream);
  if (s.n <= 16) return launch_router_t<16, 2, false>(s, x, w_gate, topk_idx, topk_gate, logits, stream);
  const RouterSplit r = router_split(s);
  if (s.n % 8 == 0) launch_partial<true>(s, r, x, w_gate, scratch, stream);
  else launch_partial<false>(s, r, x, w_gate, scratch, stream);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(router_select_kernel, dim3((s.T + 3) / 4), dim3(256), 0, stream, scratch, r.S,
                     s.T, s.n, s.K, topk_idx, topk_gate, logits);
  return hipGetLastError();
}

}  // namespace moe
