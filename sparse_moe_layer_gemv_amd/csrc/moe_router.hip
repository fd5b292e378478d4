// Router and gate: logits = x . W_g, G(x) = Softmax(TopK(logits)).
// "Mixtral of Experts", section 2.1 (garden.houmin.site translation): the gate
// is the softmax of the Top-K logits of a linear layer; logits outside the
// top K are set to -inf, so they get a gate of exactly zero.
//
// Up to 16 experts (router_kernel): a workgroup of 256 threads owns TPW
// consecutive tokens and splits the dim axis between its threads: thread i
// reads the 16-byte steps 8*i + 2048*j, so
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
constexpr int kRingMinTokens = 2048;  // up to 16 experts: the matrix-core path from here

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
// handful of tokens: a first kernel writes fp32 partial logits per
// contraction slice, [slice][token][expert]; router_select_kernel adds them.
//
// router_ring_kernel (n a multiple of 4): a workgroup of 4 waves owns 64 or
// 128 tokens (16 or 32 per wave) and one contraction slice.  The slice's 32-deep steps
// of W_g (32 consecutive rows: one contiguous byte range) and of x pass
// through a ring of kRingStages LDS stages filled by direct-to-LDS loads,
// issued kRingStages-1 steps ahead.  Per step a wave reads its x fragment
// (the A operand: 16 tokens x 32) and, per 16 experts, two transposing reads
// of the W_g rows (16 experts x 32), one v_mfma_f32_16x16x32_bf16 per 16
// tokens, W_g as the A operand so that a lane's results are 4 consecutive
// experts of one token, stored as one 16-byte write.  Each wave's tokens are its own, so
// no reduction across waves is needed.
//
// router_partial_kernel (any n): the same split with per-lane loads of 8 x 8
// W_g blocks transposed in registers, for widths whose rows are not 8-byte
// aligned.
//
// router_select_kernel: 16 lanes per token add the slices' partials in slice
// order (deterministic), then select the top K: each lane holds the logits of
// 4 consecutive experts per 64, and a butterfly argmax over the 16 lanes
// (larger value, then lower index) picks each slot in turn.
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

// Up to 16 experts the vector kernel is faster while the batch is small: it
// is one launch, and its cost is latency.  From about 2048 tokens it re-reads
// W_g from L2 once per 4 tokens and a matrix-core path takes over (measured
// with the caches flushed, n = 8, D = 4096: 16.8 vs 15.8 us at T = 2048, 26.0
// vs 21.5 us at T = 4096 for the slice kernel below; at T <= 1024 the vector
// kernel wins): the one-launch router_fused_kernel when W_g fits its LDS copy
// (uses_fused_router, checked first), else the slice kernel and its selection
// pass.  The matrix-core paths need n to be a multiple of 4 below 17 experts.
bool uses_matrix_router(const Shape& s) {
  return s.n > 16 || (s.n % 4 == 0 && s.T >= kRingMinTokens);
}

template <int RG>
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
    // element-wise: W_g rows of these widths are not 16-byte aligned
    uint4 wv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t h[8];
#pragma unroll
      for (int c = 0; c < 8; ++c)
        h[c] = (kval && col + c < n) ? uint32_t(wg[size_t(kk + i) * n + col + c]) : 0u;
      wv[i] = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                         h[6] | (h[7] << 16));
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

constexpr int kRingWaves = 4;
constexpr int kRingStages = 4;
constexpr int kRingTarget = 256;  // workgroups to aim for
constexpr int kRingMaxSlices = 16;  // the selection reads every slice's partials

struct RingSplit {
  int rg;     // 16-token groups per wave (1, or 2 above 64 tokens)
  int tiles;  // token tiles of 16 * rg * kRingWaves
  int S;      // contraction slices
  int kc;     // slice length (a multiple of 32)
};

RingSplit ring_split(const Shape& s) {
  RingSplit r;
  r.rg = s.T > 16 * kRingWaves ? 2 : 1;
  const int tok = 16 * r.rg * kRingWaves;
  r.tiles = (s.T + tok - 1) / tok;
  const int ksteps = (s.D + 31) / 32;
  int S = (kRingTarget + r.tiles - 1) / r.tiles;
  S = std::max(1, std::min({S, ksteps / kRingStages, kRingMaxSlices}));
  const int steps = (ksteps + S - 1) / S;
  r.kc = steps * 32;
  r.S = (s.D + r.kc - 1) / r.kc;
  return r;
}

// NT: 16-expert column tiles (even, >= n/16); RG: 16-token groups per wave,
// each W_g fragment feeding RG matrix-core products; CW: 1 KiB W_g loads per
// wave per stage (a stage holds 32 rows = 64*n bytes of W_g, padded to 4*CW
// KiB, and RG KiB of x per wave).
template <int NT, int RG>
struct Ring {
  static constexpr int CW = (NT + 3) / 4;
  static constexpr int WB = CW * kRingWaves * 1024;  // W_g bytes per stage
  static constexpr int XB = kRingWaves * RG * 1024;  // x bytes per stage
  static constexpr int SB = WB + XB;
  static constexpr int TOK = 16 * RG * kRingWaves;
  static constexpr int WAIT = (kRingStages - 1) * (CW + RG);  // loads issued after a step's
};
static_assert(kRingStages == 4, "the stages are four distinct LDS objects");

struct RingLane {
  __amdgpu_buffer_rsrc_t rw, rx;
  uint32_t row_bytes;  // 2 n
  uint32_t b_off;      // transposing-read offset within a stage
  int wave, lane, kbeg, kend, nsteps, wchunks;
};

// Step i of the slice into stage `st`.  Loads past the slice (issued to keep
// the per-step load count uniform) and past the W_g piece read as zeros.  A
// step never crosses the slice end except at D, where the rows read as zeros.
template <int NT, int RG>
__device__ __forceinline__ void ring_issue(const RingLane& c, const uint32_t (&x_lane)[RG],
                                           uint8_t* st, int i) {
  using R = Ring<NT, RG>;
  const int g = c.lane >> 4;
  const int kw = c.kbeg + 32 * i;
  const bool live = i < c.nsteps;
  const uint32_t wbase = uint32_t(kw) * c.row_bytes;
#pragma unroll
  for (int cc = 0; cc < R::CW; ++cc) {
    const int j = c.wave + kRingWaves * cc;
    dma16(c.rw, lds(st) + j * 1024, live && j < c.wchunks ? wbase + j * 1024 + c.lane * 16 : kOOB,
          0);
  }
#pragma unroll
  for (int u = 0; u < RG; ++u) {
    const bool xin = live && x_lane[u] != kOOB && kw + 8 * g < c.kend;
    dma16(c.rx, lds(st) + R::WB + (c.wave * RG + u) * 1024,
          xin ? x_lane[u] + uint32_t(kw) * 2 : kOOB, 0);
  }
}

template <int NT, int RG>
__device__ __forceinline__ void ring_compute(const RingLane& c, uint8_t* st,
                                             f32x4 (&acc)[RG][NT]) {
  using R = Ring<NT, RG>;
  bf16x8 a[RG];
#pragma unroll
  for (int u = 0; u < RG; ++u)
    a[u] = as_bf16x8(
        *reinterpret_cast<const uint4*>(st + R::WB + (c.wave * RG + u) * 1024 + c.lane * 16));
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
#pragma unroll
  for (int q = 0; q < NT; ++q) {
    const uint32_t off = c.b_off + uint32_t(32 * q);
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds(st) + off));
    const v4i16 hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds(st) + off + 4 * c.row_bytes));
    const bf16x8 b =
        __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    // W_g rows as the A operand and x as B: the product is [expert][token],
    // so each lane ends with 4 consecutive experts of one token
#pragma unroll
    for (int u = 0; u < RG; ++u)
      acc[u][q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, a[u], acc[u][q], 0, 0, 0);
  }
}

// One step: stage `cur` is computed while the loads of 3 steps later go into
// stage `nxt` (the one computed in the previous step).
template <int NT, int RG>
__device__ __forceinline__ void ring_step(const RingLane& c, const uint32_t (&x_lane)[RG],
                                          uint8_t* cur, uint8_t* nxt, int i,
                                          f32x4 (&acc)[RG][NT]) {
  wait_lgkmcnt0();                                   // this wave's reads of `nxt` are done
  stage_barrier();                                   // ... and every other wave's
  ring_issue<NT, RG>(c, x_lane, nxt, i + kRingStages - 1);
  wait_vmcnt<Ring<NT, RG>::WAIT>();                  // this wave's loads of step i landed
  stage_barrier();                                   // ... and every other wave's loads
  ring_compute<NT, RG>(c, cur, acc);
}

template <int NT, int RG>
__global__ __launch_bounds__(kRingWaves * 64) void router_ring_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg, int T, int D, int n, int S,
    int kc, float* __restrict__ part) {
  using R = Ring<NT, RG>;
  // four stage objects, so the compiler can tell the loads into one stage
  // from the reads of another
  __shared__ __attribute__((aligned(1024))) uint8_t st0[R::SB];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[R::SB];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[R::SB];
  __shared__ __attribute__((aligned(1024))) uint8_t st3[R::SB];

  RingLane c;
  c.lane = threadIdx.x & 63;
  c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = c.lane >> 4;     // contraction group of 8 (A and B), row group of 4 (C)
  const int j16 = c.lane & 15;   // token (A row) and expert (B and C column)
  const int sl = blockIdx.x % S;
  const int t0 = (blockIdx.x / S) * R::TOK + 16 * RG * c.wave;  // this wave's first token
  c.kbeg = sl * kc;
  c.kend = min(D, c.kbeg + kc);
  c.nsteps = (c.kend - c.kbeg + 31) / 32;
  c.row_bytes = uint32_t(n) * 2;
  c.wchunks = (64 * n + 1023) / 1024;  // 1 KiB pieces of a step's W_g rows
  c.rw = make_rsrc(wg, uint32_t(D) * c.row_bytes);
  c.rx = make_rsrc(x, uint32_t(T) * uint32_t(D) * 2);
  // rows 8g + (j16 >> 2) (+4 for the second read), columns 16q + 4 (j16 & 3) .. +4
  c.b_off = uint32_t(8 * g + (j16 >> 2)) * c.row_bytes + uint32_t(4 * (j16 & 3)) * 2;
  uint32_t x_lane[RG];
#pragma unroll
  for (int u = 0; u < RG; ++u) {
    const int tok = t0 + 16 * u + j16;
    x_lane[u] = tok < T ? (uint32_t(tok) * uint32_t(D) + 8 * g) * 2 : kOOB;
  }

  f32x4 acc[RG][NT];
#pragma unroll
  for (int u = 0; u < RG; ++u)
#pragma unroll
    for (int q = 0; q < NT; ++q) acc[u][q] = f32x4{0.f, 0.f, 0.f, 0.f};

  ring_issue<NT, RG>(c, x_lane, st0, 0);
  ring_issue<NT, RG>(c, x_lane, st1, 1);
  ring_issue<NT, RG>(c, x_lane, st2, 2);
  // whole rounds of four steps: steps past the slice read zero-filled stages
  // and add exact zeros, and a branch-free loop body keeps the compiler's
  // own load tracking from waiting for the whole ring
  for (int i = 0; i < c.nsteps; i += 4) {
    ring_step<NT, RG>(c, x_lane, st0, st3, i, acc);
    ring_step<NT, RG>(c, x_lane, st1, st0, i + 1, acc);
    ring_step<NT, RG>(c, x_lane, st2, st1, i + 2, acc);
    ring_step<NT, RG>(c, x_lane, st3, st2, i + 3, acc);
  }
  wait_vmcnt<0>();  // the trailing zero-fill loads must land before the workgroup ends

  // acc[u][q][r]: expert 16 q + 4 g + r of token t0 + 16 u + j16; n is a
  // multiple of 4, so a lane's 4 experts are all inside or all outside
#pragma unroll
  for (int u = 0; u < RG; ++u) {
    const int t = t0 + 16 * u + j16;
#pragma unroll
    for (int q = 0; q < NT; ++q) {
      const int e = 16 * q + 4 * g;
      if (t < T && e < n)
        *reinterpret_cast<f32x4*>(part + (size_t(sl) * T + t) * n + e) = acc[u][q];
    }
  }
}

// (bv, bi) <- the better of itself and the lane R places further round its
// 16-lane row: larger value, then lower index; bi < 0 marks "none".
template <int R>
__device__ __forceinline__ void row_argmax(float& bv, int& bi) {
  constexpr int kRowRor = 0x120 + R;  // DPP row_ror:R
  const float ov = __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(bv), kRowRor, 0xF, 0xF, false));
  const int oi = __builtin_amdgcn_update_dpp(0, bi, kRowRor, 0xF, 0xF, false);
  // selects, not a branch: every lane of the row takes part in the next step
  const bool take = (oi >= 0) & ((bi < 0) | (ov > bv) | ((ov == bv) & (oi < bi)));
  bv = take ? ov : bv;
  bi = take ? oi : bi;
}

// 16 lanes per token, 16 tokens per 256-thread workgroup; lane j16 of a token
// holds the logits of experts 64 m + 4 j16 + c (c = 0..3, m = 0..NM-1), read
// as 16-byte vectors when n is a multiple of 4.  KQ: slots a lane keeps (slot
// s in lane s % 16): 1 for K <= 16, else 16.
template <int NM, bool VEC4, int KQ>
__global__ __launch_bounds__(256) void router_select_kernel(
    const float* __restrict__ part, int S, int T, int n, int K, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_gate, float* __restrict__ logits) {
  const int j16 = threadIdx.x & 15;
  const int t = blockIdx.x * 16 + (threadIdx.x >> 4);
  const bool tok_ok = t < T;
  const int tc = tok_ok ? t : 0;  // every lane takes part in the shuffles
  auto load4 = [&](int sl, int m) -> f32x4 {
    const float* row = part + (size_t(sl) * T + tc) * n;
    const int e = 64 * m + 4 * j16;
    if constexpr (VEC4) {
      return *reinterpret_cast<const f32x4*>(row + min(e, n - 4));
    } else {
      f32x4 r;
#pragma unroll
      for (int c = 0; c < 4; ++c) r[c] = row[min(e + c, n - 1)];
      return r;
    }
  };
  // the slices' partials, loaded SB slices at a time and added in slice order
  constexpr int SB = 8;
  f32x4 v[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) v[m] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < S; s0 += SB) {
    f32x4 pv[SB][NM];
#pragma unroll
    for (int u = 0; u < SB; ++u)
#pragma unroll
      for (int m = 0; m < NM; ++m) pv[u][m] = load4(min(s0 + u, S - 1), m);
#pragma unroll
    for (int u = 0; u < SB; ++u)
#pragma unroll
      for (int m = 0; m < NM; ++m)
        if (s0 + u < S) v[m] = (s0 + u == 0) ? pv[u][m] : v[m] + pv[u][m];
  }
  if (logits && tok_ok)
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int e = 64 * m + 4 * j16 + c;
        if (e < n) logits[size_t(t) * n + e] = v[m][c];
      }
  // Top-K by repeated selection.  Within a lane the experts rise with (m, c),
  // so a strict ">" keeps the lower index; across the 16 lanes equal values
  // go to the lower index.  Slot s's expert and e^(l - top) stay in lane
  // s % 16.
  uint32_t taken = 0;  // bit 4 m + c
  int my_idx[KQ];
  float my_ex[KQ];
#pragma unroll
  for (int q = 0; q < KQ; ++q) {
    my_idx[q] = 0;
    my_ex[q] = 0.f;
  }
  float top = 0.f, sum = 0.f;
  for (int s = 0; s < K; ++s) {
    int bi = -1;
    float bv = 0.f;
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int e = 64 * m + 4 * j16 + c;
        const bool better = (e < n) & !((taken >> (4 * m + c)) & 1u) & ((bi < 0) | (v[m][c] > bv));
        bi = better ? e : bi;
        bv = better ? v[m][c] : bv;
      }
    // all-reduce over the 16 lanes of a row by rotations of 8, 4, 2, 1 (the
    // order (value, then lower index) is total, so any combining order gives
    // the same winner); DPP moves, no LDS round trips
    row_argmax<8>(bv, bi);
    row_argmax<4>(bv, bi);
    row_argmax<2>(bv, bi);
    row_argmax<1>(bv, bi);
    if (((bi >> 2) & 15) == j16) taken |= 1u << (4 * (bi >> 6) + (bi & 3));
    if (s == 0) top = bv;
    const float ex = __expf(bv - top);
    sum += ex;
#pragma unroll
    for (int q = 0; q < KQ; ++q)
      if (s == 16 * q + j16) {
        my_idx[q] = bi;
        my_ex[q] = ex;
      }
  }
  if (!tok_ok) return;
  const float inv = 1.f / sum;
#pragma unroll
  for (int q = 0; q < KQ; ++q) {
    const int s = 16 * q + j16;
    if (s < K) {
      topk_idx[size_t(t) * K + s] = my_idx[q];
      topk_gate[size_t(t) * K + s] = my_ex[q] * inv;
    }
  }
}

// The same selection with one wavefront per token (4 tokens per 256-thread
// workgroup), for K <= 64: lane l holds the logits of experts l + 64 m
// (m = 0..NM-1), so a top-K round scans NM values per lane instead of 4 NM,
// and the lanes' candidates meet in the row rotations above plus two
// butterfly exchanges across the four rows.  Partials are added in slice
// order and the gates formed exactly as in router_select_kernel, so both give
// the same bits.
template <int R>
__device__ __forceinline__ void xor_argmax(float& bv, int& bi) {
  const float ov = __shfl_xor(bv, R, 64);
  const int oi = __shfl_xor(bi, R, 64);
  const bool take = (oi >= 0) & ((bi < 0) | (ov > bv) | ((ov == bv) & (oi < bi)));
  bv = take ? ov : bv;
  bi = take ? oi : bi;
}

template <int NM>
__global__ __launch_bounds__(256) void router_select_wave_kernel(
    const float* __restrict__ part, int S, int T, int n, int K, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_gate, float* __restrict__ logits) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;  // the whole wavefront
  constexpr int SB = 8;
  float v[NM];
#pragma unroll
  for (int m = 0; m < NM; ++m) v[m] = 0.f;
  for (int s0 = 0; s0 < S; s0 += SB) {
    float pv[SB][NM];
#pragma unroll
    for (int u = 0; u < SB; ++u)
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const int e = lane + 64 * m;
        pv[u][m] = e < n ? part[(size_t(min(s0 + u, S - 1)) * T + t) * n + e] : 0.f;
      }
#pragma unroll
    for (int u = 0; u < SB; ++u)
#pragma unroll
      for (int m = 0; m < NM; ++m)
        if (s0 + u < S) v[m] = (s0 + u == 0) ? pv[u][m] : v[m] + pv[u][m];
  }
  if (logits)
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int e = lane + 64 * m;
      if (e < n) logits[size_t(t) * n + e] = v[m];
    }
  // Top-K by repeated selection; within a lane the experts rise with m, so a
  // strict ">" keeps the lower index, and across lanes equal values go to the
  // lower index.  Slot s's expert and e^(l - top) stay in lane s.
  uint32_t taken = 0;  // bit m
  int my_idx = 0;
  float my_ex = 0.f;
  float top = 0.f, sum = 0.f;
  for (int s = 0; s < K; ++s) {
    int bi = -1;
    float bv = 0.f;
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      const int e = lane + 64 * m;
      const bool better = (e < n) & !((taken >> m) & 1u) & ((bi < 0) | (v[m] > bv));
      bi = better ? e : bi;
      bv = better ? v[m] : bv;
    }
    row_argmax<8>(bv, bi);
    row_argmax<4>(bv, bi);
    row_argmax<2>(bv, bi);
    row_argmax<1>(bv, bi);
    xor_argmax<16>(bv, bi);
    xor_argmax<32>(bv, bi);
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (s == 0) top = bv;
    const float ex = __expf(bv - top);
    sum += ex;
    if (s == lane) {
      my_idx = bi;
      my_ex = ex;
    }
  }
  const float inv = 1.f / sum;
  if (lane < K) {
    topk_idx[size_t(t) * K + lane] = my_idx;
    topk_gate[size_t(t) * K + lane] = my_ex * inv;
  }
}

template <int NM>
void launch_select_t(const Shape& s, int S, const float* part, int32_t* idx, float* gate,
                     float* logits, hipStream_t stream) {
  const dim3 grid((s.T + 15) / 16), block(256);
  if (s.n % 4 == 0 && s.K <= 16)
    hipLaunchKernelGGL((router_select_kernel<NM, true, 1>), grid, block, 0, stream, part, S, s.T,
                       s.n, s.K, idx, gate, logits);
  else if (s.n % 4 == 0)
    hipLaunchKernelGGL((router_select_kernel<NM, true, 16>), grid, block, 0, stream, part, S, s.T,
                       s.n, s.K, idx, gate, logits);
  else if (s.K <= 16)
    hipLaunchKernelGGL((router_select_kernel<NM, false, 1>), grid, block, 0, stream, part, S, s.T,
                       s.n, s.K, idx, gate, logits);
  else
    hipLaunchKernelGGL((router_select_kernel<NM, false, 16>), grid, block, 0, stream, part, S,
                       s.T, s.n, s.K, idx, gate, logits);
}

void launch_select(const Shape& s, int S, const float* part, int32_t* idx, float* gate,
                   float* logits, hipStream_t stream) {
  const int nm = (s.n + 63) / 64;  // 64-expert groups
  // a wavefront per token below 2048 tokens (route time with the slice kernel,
  // n = 160, K = 8, D = 4096: 12.8 -> 11.2 us at T = 16, 22.1 -> 19.7 at
  // 1024, even at 2048, 23.3 -> 25.7 at 4096), 16 lanes per token above
  if (s.K <= 64 && s.T < 2048) {
    const dim3 grid((s.T + 3) / 4), block(256);
    auto kern = nm <= 1 ? router_select_wave_kernel<1>
              : nm <= 2 ? router_select_wave_kernel<2>
              : nm <= 3 ? router_select_wave_kernel<3> : router_select_wave_kernel<4>;
    hipLaunchKernelGGL(kern, grid, block, 0, stream, part, S, s.T, s.n, s.K, idx, gate, logits);
    return;
  }
  if (nm <= 1) launch_select_t<1>(s, S, part, idx, gate, logits, stream);
  else if (nm <= 2) launch_select_t<2>(s, S, part, idx, gate, logits, stream);
  else if (nm <= 3) launch_select_t<3>(s, S, part, idx, gate, logits, stream);
  else launch_select_t<4>(s, S, part, idx, gate, logits, stream);
}

template <int RG>
void launch_partial_t(const Shape& s, const RouterSplit& r, const uint16_t* x, const uint16_t* wg,
                      float* part, hipStream_t stream) {
  const unsigned blocks = unsigned(r.tiles) * r.cblocks * r.S;
  hipLaunchKernelGGL((router_partial_kernel<RG>), dim3(blocks), dim3(kRpThreads), 0, stream, x,
                     wg, s.T, s.D, s.n, r.S, r.kc, r.cblocks, part);
}

void launch_partial(const Shape& s, const RouterSplit& r, const uint16_t* x, const uint16_t* wg,
                    float* part, hipStream_t stream) {
  if (r.rg == 1) launch_partial_t<1>(s, r, x, wg, part, stream);
  else launch_partial_t<2>(s, r, x, wg, part, stream);
}

// Up to 16 experts (a multiple of 4) from kFusedMinTokens tokens, with W_g
// (rows rounded up to whole 32-row steps) at most kFusedWBytes: the logits on
// the matrix cores in one launch, with no partial sums in memory.
// - A workgroup of kFusedWaves waves owns 16 tokens and splits the contraction
//   between its waves: wave w takes the w-th share of the 32-deep steps.
// - W_g is copied once into LDS in its own row-major layout (plain buffer
//   loads, zeros past its end, and LDS stores), so the transposing reads the
//   ring kernel uses turn each 32-row step into the A operand of
//   v_mfma_f32_16x16x32_bf16: 16 expert columns, where the columns past n read
//   the next rows (or zeros past the end) and their products are dropped.
// - x goes straight from memory into the B operand (lane: token j16,
//   contraction elements 8 g .. 8 g + 7 of the step), all of a wave's steps in
//   flight at once.  Tokens past T read row T-1 and elements past D read
//   element D-8; their products reach only dropped outputs or zero W_g rows.
// - The waves' [expert][token] sums are added in wave order through LDS (in the
//   bytes W_g used), then one lane per token selects the top K exactly as
//   router_kernel does: strict ">", so the lower index wins a tie, and the
//   softmax over the kept logits.
// Measured alone (n = 8, D = 4096, rotating 1 GiB of x, graph replays): 9.0 /
// 10.6 / 16.3 us at T = 2048 / 4096 / 8192, against 10.3 / 12.9 / 21.3 us for
// the slice kernel and its selection pass.  Every call costs ~7.5 us even for
// one workgroup (the vector kernel takes 5 us at T = 16 and 8.2 us at 1024),
// so smaller batches keep the vector kernel.  4 and 16 waves per workgroup
// measured the same or slower.
constexpr int kFusedWaves = 8;
constexpr int kFusedTokens = 16;
constexpr int kFusedMinTokens = 2048;
constexpr int kFusedWBytes = 64 * 1024;        // W_g bytes (whole steps) the LDS copy holds
constexpr int kFusedFill = kFusedWBytes + 64;  // plus the bytes the last step's reads run past
constexpr int kFusedThreads = kFusedWaves * 64;
constexpr int kFusedCopy = (kFusedFill / 16 + kFusedThreads - 1) / kFusedThreads;  // 16 B rounds
constexpr int kFusedCh = 128 / kFusedWaves;    // x steps a wave holds at once (D = 4096: all)

bool uses_fused_router(const Shape& s) {
  const size_t wbytes = size_t((s.D + 31) / 32) * 32 * s.n * 2;
  return s.n % 4 == 0 && s.n <= 16 && s.T >= kFusedMinTokens && wbytes <= size_t(kFusedWBytes);
}

__global__ __launch_bounds__(kFusedThreads) void router_fused_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg, int T, int D, int n, int K,
    int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate, float* __restrict__ logits) {
  // W_g; after the steps, the waves' sums and the logits in the same bytes
  __shared__ __attribute__((aligned(16))) uint8_t wl[kFusedFill];
  static_assert(kFusedWaves * 64 * sizeof(f32x4) + kFusedTokens * 17 * sizeof(float) <= kFusedFill,
                "the sums fit where W_g was");
  f32x4(*red)[64] = reinterpret_cast<f32x4(*)[64]>(wl);
  float(*lg)[17] = reinterpret_cast<float(*)[17]>(wl + kFusedWaves * 64 * sizeof(f32x4));
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, j16 = lane & 15;
  const int t0 = blockIdx.x * kFusedTokens;
  const uint32_t row_bytes = uint32_t(n) * 2;
  const uint32_t wbytes = uint32_t(D) * row_bytes;
  const int ksteps = (D + 31) / 32;
  const int spw = (ksteps + kFusedWaves - 1) / kFusedWaves;
  const int s0 = min(ksteps, wave * spw), s1 = min(ksteps, s0 + spw);
  const uint16_t* xrow = x + size_t(min(t0 + j16, T - 1)) * D;

  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(wg, wbytes);
  u32x4 wv[kFusedCopy];
#pragma unroll
  for (int i = 0; i < kFusedCopy; ++i)
    wv[i] = __builtin_amdgcn_raw_buffer_load_b128(
        rw, int((uint32_t(i) * kFusedThreads + threadIdx.x) * 16), 0, 0);
  // steps past the wave's share hold zeros, so the step loop below runs
  // without branches and its LDS reads can be issued ahead
  uint4 xa[kFusedCh];
  auto load_round = [&](int r0) {
#pragma unroll
    for (int j = 0; j < kFusedCh; ++j) {
      const int kk = min(32 * (r0 + j) + 8 * g, D - 8);
      const uint4 v = *reinterpret_cast<const uint4*>(xrow + kk);
      xa[j] = r0 + j < s1 ? v : make_uint4(0, 0, 0, 0);
    }
  };
  load_round(s0);
#pragma unroll
  for (int i = 0; i < kFusedCopy; ++i) {
    const uint32_t o = (uint32_t(i) * kFusedThreads + threadIdx.x) * 16;
    if (i + 1 < kFusedCopy || o < uint32_t(kFusedFill)) *reinterpret_cast<u32x4*>(wl + o) = wv[i];
  }
  __syncthreads();

  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  // rows 8 g + (j16 >> 2) and + 4, expert columns 4 (j16 & 3) .. + 3 of a step
  const uint32_t b_off = uint32_t(8 * g + (j16 >> 2)) * row_bytes + uint32_t(8 * (j16 & 3));
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int r0 = s0; r0 < s1; r0 += kFusedCh) {
    if (r0 != s0) load_round(r0);
#pragma unroll
    for (int j = 0; j < kFusedCh; ++j) {
      // a step past the end reads the last step's (finite) rows against zeros
      const uint32_t off = uint32_t(min(r0 + j, ksteps - 1)) * 32 * row_bytes + b_off;
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds(wl) + off));
      const v4i16 hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds(wl) + off + 4 * row_bytes));
      const bf16x8 b =
          __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(b, as_bf16x8(xa[j]), acc, 0, 0, 0);
    }
  }

  // acc[r]: expert 4 g + r of token t0 + j16, over this wave's share
  __syncthreads();  // every wave is past its W_g reads
  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    f32x4 v = red[0][lane];
#pragma unroll
    for (int w = 1; w < kFusedWaves; ++w) v += red[w][lane];
#pragma unroll
    for (int r = 0; r < 4; ++r) lg[j16][4 * g + r] = v[r];
  }
  __syncthreads();
  const int tid = threadIdx.x;
  if (tid >= kFusedTokens || t0 + tid >= T) return;
  const int tok = t0 + tid;
  if (logits)
    for (int e = 0; e < n; ++e) logits[size_t(tok) * n + e] = lg[tid][e];
  uint32_t taken = 0;
  float top = 0.f, sum = 0.f;
  for (int s = 0; s < K; ++s) {
    int bi = -1;
    float bv = 0.f;
    for (int e = 0; e < n; ++e)
      if (!((taken >> e) & 1u) && (bi < 0 || lg[tid][e] > bv)) {
        bi = e;
        bv = lg[tid][e];
      }
    taken |= 1u << bi;
    if (s == 0) top = bv;
    const float ex = __expf(bv - top);
    sum += ex;
    topk_idx[size_t(tok) * K + s] = bi;
    topk_gate[size_t(tok) * K + s] = ex;
  }
  const float inv = 1.f / sum;
  for (int s = 0; s < K; ++s) topk_gate[size_t(tok) * K + s] *= inv;
}

hipError_t launch_fused(const Shape& s, const uint16_t* x, const uint16_t* wg, int32_t* idx,
                        float* gate, float* logits, hipStream_t stream) {
  hipLaunchKernelGGL(router_fused_kernel, dim3((s.T + kFusedTokens - 1) / kFusedTokens),
                     dim3(kFusedThreads), 0, stream, x, wg, s.T, s.D, s.n, s.K, idx, gate, logits);
  return hipGetLastError();
}

template <int NE, int TPW, bool VEC>
hipError_t launch_router_t(const Shape& s, const uint16_t* x, const uint16_t* wg, int32_t* idx,
                           float* gate, float* logits, hipStream_t stream) {
  const int blocks = (s.T + TPW - 1) / TPW;
  hipLaunchKernelGGL((router_kernel<NE, TPW, VEC>), dim3(blocks), dim3(kRouterThreads), 0,
                     stream, x, wg, s.T, s.D, s.n, s.K, idx, gate, logits);
  return hipGetLastError();
}

template <int NT>
void launch_ring_t(const Shape& s, const RingSplit& r, const uint16_t* x, const uint16_t* wg,
                   float* part, hipStream_t stream) {
  const dim3 grid(unsigned(r.tiles) * r.S), block(kRingWaves * 64);
  if (r.rg == 1)
    hipLaunchKernelGGL((router_ring_kernel<NT, 1>), grid, block, 0, stream, x, wg, s.T, s.D, s.n,
                       r.S, r.kc, part);
  else
    hipLaunchKernelGGL((router_ring_kernel<NT, 2>), grid, block, 0, stream, x, wg, s.T, s.D, s.n,
                       r.S, r.kc, part);
}

void launch_ring(const Shape& s, const RingSplit& r, const uint16_t* x, const uint16_t* wg,
                 float* part, hipStream_t stream) {
  const int nt = (s.n + 31) / 32 * 2;  // 16-expert tiles, rounded up to even
  switch (nt) {
    case 2: launch_ring_t<2>(s, r, x, wg, part, stream); break;
    case 4: launch_ring_t<4>(s, r, x, wg, part, stream); break;
    case 6: launch_ring_t<6>(s, r, x, wg, part, stream); break;
    case 8: launch_ring_t<8>(s, r, x, wg, part, stream); break;
    case 10: launch_ring_t<10>(s, r, x, wg, part, stream); break;
    case 12: launch_ring_t<12>(s, r, x, wg, part, stream); break;
    case 14: launch_ring_t<14>(s, r, x, wg, part, stream); break;
    default: launch_ring_t<16>(s, r, x, wg, part, stream); break;
  }
}

}  // namespace

size_t route_scratch_bytes(const Shape& s) {
  if (s.T == 0 || uses_fused_router(s) || !uses_matrix_router(s)) return 0;
  const int S = s.n % 4 == 0 ? ring_split(s).S : router_split(s).S;
  return size_t(S) * s.T * s.n * sizeof(float);
}

hipError_t launch_route(const Shape& s, const uint16_t* x, const uint16_t* w_gate,
                        int32_t* topk_idx, float* topk_gate, float* logits, float* scratch,
                        hipStream_t stream) {
  if (s.T == 0) return hipSuccess;
  if (uses_fused_router(s))
    return launch_fused(s, x, w_gate, topk_idx, topk_gate, logits, stream);
  if (!uses_matrix_router(s)) {
    // Up to 64 tokens the router is pure latency: one token per workgroup
    // (more workgroups, a shorter chain each) takes it from 6.5 to 5.4 us at
    // 16 tokens.  Larger batches keep 4 tokens per workgroup so that each W_g
    // row loaded serves 4 tokens.
    if (s.n == 8 && s.T <= 64)
      return launch_router_t<8, 1, true>(s, x, w_gate, topk_idx, topk_gate, logits, stream);
    if (s.n == 8) return launch_router_t<8, 4, true>(s, x, w_gate, topk_idx, topk_gate, logits, stream);
    if (s.n == 16) return launch_router_t<16, 2, true>(s, x, w_gate, topk_idx, topk_gate, logits, stream);
    if (s.n <= 8) return launch_router_t<8, 4, false>(s, x, w_gate, topk_idx, topk_gate, logits, stream);
    return launch_router_t<16, 2, false>(s, x, w_gate, topk_idx, topk_gate, logits, stream);
  }
  int S;
  if (s.n % 4 == 0) {
    const RingSplit r = ring_split(s);
    S = r.S;
    launch_ring(s, r, x, w_gate, scratch, stream);
  } else {
    const RouterSplit r = router_split(s);
    S = r.S;
    launch_partial(s, r, x, w_gate, scratch, stream);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch_select(s, S, scratch, topk_idx, topk_gate, logits, stream);
  return hipGetLastError();
}

}  // namespace moe
