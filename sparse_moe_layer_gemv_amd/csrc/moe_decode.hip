// Weight-streaming expert path for small batches (decode).
//
// The pages note that a sparse MoE layer pays extra memory loads and loses
// efficiency at small batch sizes ("Mixtral of Experts", section 3, remark on
// hardware utilisation; the aipaper.jasonlin.tech summary, limitations).  With
// T <= 64 tokens each expert sees only a handful of rows, so the expert
// products are bound by reading the weights: every touched expert's w1, w3
// and w2 must cross HBM once and nothing else matters.  These kernels do
// exactly that read, once, coalesced, with many loads in flight, and use the
// matrix cores only to keep the arithmetic off the critical path.
//
// Work split: a workgroup owns (expert e, 128 output columns, one weight
// matrix); its waves split the contraction axis.  Per 32-wide step a lane
// loads an 8 x 8 bf16 block of the matrix (8 rows x 16 bytes; 16 lanes cover
// 256 contiguous bytes of a row), transposes it in registers, and feeds 8
// v_mfma_f32_16x16x32_bf16 whose A rows are 16 output columns strided by 8
// and whose B columns are up to 16 token rows of the expert.  The waves'
// partial sums are reduced through LDS in a fixed tree order (deterministic).
//
// First product: w1 and w3 are separate workgroups (twice as many workgroups
// keep more loads in flight than one workgroup reading both), each writing its
// fp32 result a = x.w1 or b = x.w3 per token-slot.  Second product: each lane
// forms its h fragment as bf16(silu(a) * b) while loading it (the same single
// rounding as the tiled path), and the 14336-deep contraction is split into
// partial sums written to separate buffers, added in order by the combine.
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {
namespace {

// 16 bytes of a weight row.  Each weight byte is read exactly once per call,
// so the loads are non-temporal: they do not displace cached data, and the
// stream runs faster (first product 327 -> 296 us at decode, 6.35 TB/s).
__device__ __forceinline__ uint4 load_weight(const uint16_t* p) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}

constexpr int kUpWaves = 8;
constexpr int kDownWaves = 16;

// 8 consecutive h values of one token-slot: bf16(silu(a) * b) from the fp32
// first-product results.
__device__ __forceinline__ uint4 h_fragment(const float* a, const float* b) {
  const f32x4 a0 = *reinterpret_cast<const f32x4*>(a), a1 = *reinterpret_cast<const f32x4*>(a + 4);
  const f32x4 b0 = *reinterpret_cast<const f32x4*>(b), b1 = *reinterpret_cast<const f32x4*>(b + 4);
  return make_uint4(pack_bf16x2(silu(a0[0]) * b0[0], silu(a0[1]) * b0[1]),
                    pack_bf16x2(silu(a0[2]) * b0[2], silu(a0[3]) * b0[3]),
                    pack_bf16x2(silu(a1[0]) * b1[0], silu(a1[1]) * b1[1]),
                    pack_bf16x2(silu(a1[2]) * b1[2], silu(a1[3]) * b1[3]));
}

// UP:   x [T][Kdim] bf16 rows gathered through row_slot; w = w1 or w3 (by
//       workgroup); out = ab fp32 [2][P][Ndim] (a at [0], b at [1], row = slot)
// DOWN: ab rows through row_slot -> h; w = w2; out = y fp32 [cap][Ndim] + ks *
//       split_stride (partial ks over contraction rows [ks*klen, +klen))
//
// SCAN: the expert's token-slots are found by scanning the routing itself
// (topk_idx, P = T*K entries, in slot order, so in the order the permute
// would give them), and the second product writes its rows at the slot index
// instead of the permuted row: no permute pass is needed.  Otherwise they come
// from the permuted layout (expert_count, expert_offset, row_slot).
template <bool UP, int RG, int WAVES, bool SCAN>
__global__ __launch_bounds__(WAVES * 64) void decode_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ ab,
    const int32_t* __restrict__ expert_count, const int32_t* __restrict__ expert_offset,
    const int32_t* __restrict__ row_slot, const int32_t* __restrict__ topk_idx,
    const uint16_t* __restrict__ w0, const uint16_t* __restrict__ w1, void* __restrict__ out,
    int Kdim, int Ndim, int topk, int P, int ncb, int nsplit, int klen, ptrdiff_t split_stride) {
  constexpr int NACC = RG * 8;                     // f32x4 accumulators per lane
  constexpr int RED_SLOTS = WAVES / 2;
  __shared__ float red[RED_SLOTS * NACC * 4 * 64];

  // workgroup -> (expert, column block, matrix or contraction split)
  const int per_e = ncb * (UP ? 2 : nsplit);
  const int e = blockIdx.x / per_e;
  const int r = blockIdx.x - e * per_e;
  const int sub = UP ? (r & 1) : (r % nsplit);     // UP: matrix; DOWN: split
  const int cb = UP ? (r >> 1) : (r / nsplit);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // SCAN: the expert's slots; every token holds an expert at most once, so
  // there are at most T <= 64 of them
  __shared__ int s_list[kStreamMaxTokens];
  __shared__ int s_cnt;
  int cnt, rbase = 0;
  if constexpr (SCAN) {
    if (wave == 0) {
      int c = 0;
      for (int base = 0; base < P; base += 64) {
        const int i = base + lane;
        const bool m = i < P && topk_idx[i] == e;
        const uint64_t b = __ballot(m);
        const int pos = c + __popcll(b & ((uint64_t(1) << lane) - 1));
        if (m && pos < kStreamMaxTokens) s_list[pos] = i;
        c += __popcll(b);
      }
      if (lane == 0) s_cnt = min(c, kStreamMaxTokens);
    }
    __syncthreads();
    cnt = s_cnt;
  } else {
    cnt = expert_count[e];
    rbase = expert_offset[e];
  }
  if (cnt == 0) return;
  const int n0 = cb * 128;
  const int kg = lane >> 4;
  const int nbk = lane & 15;
  const bool col_ok = n0 + nbk * 8 < Ndim;
  const int kbeg = UP ? 0 : sub * klen;
  const int kend = UP ? Kdim : min(Kdim, kbeg + klen);

  // activation row pointers (token row j = lane % 16 + 16 g of the expert)
  const uint16_t* xrow[RG];
  const float* arow[RG];
  const float* brow[RG];
  bool aval[RG];
  int slot_of[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    const int j = (lane & 15) + 16 * g;
    aval[g] = j < cnt;
    int slot = 0;
    if (aval[g]) {
      if constexpr (SCAN) {
        slot = s_list[j];
      } else {
        slot = row_slot[rbase + j];
      }
    }
    slot_of[g] = slot;
    const int sl = slot >= 0 ? slot : 0;
    if (UP) {
      xrow[g] = x + size_t(sl / topk) * Kdim;
    } else {
      arow[g] = ab + size_t(sl) * Kdim;
      brow[g] = ab + (size_t(P) + sl) * Kdim;
    }
  }
  const uint16_t* wp =
      (UP && sub ? w1 : w0) + size_t(e) * Kdim * Ndim + n0 + nbk * 8;

  f32x4 acc[RG][8];
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[g][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int steps = (kend - kbeg + 31) / 32;
  const int per = (steps + WAVES - 1) / WAVES;
  const int s0 = wave * per;
  const int s1 = min(steps, s0 + per);
  for (int s = s0; s < s1; ++s) {
    const int kk = kbeg + s * 32 + kg * 8;
    const bool kok = kk < kend;
    uint4 wv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      wv[j] = (kok && col_ok) ? load_weight(wp + size_t(kk + j) * Ndim) : make_uint4(0, 0, 0, 0);
    bf16x8 xv[RG];
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (kok && aval[g]) {
        if (UP)
          v = *reinterpret_cast<const uint4*>(xrow[g] + kk);
        else
          v = h_fragment(arow[g] + kk, brow[g] + kk);
      }
      xv[g] = as_bf16x8(v);
    }
    uint4 op[8];
    transpose8x8_bf16(wv, op);
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int g = 0; g < RG; ++g)
        acc[g][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(op[c]), xv[g], acc[g][c], 0, 0, 0);
  }

  // Tree reduction over waves: at each level the upper half stores, the lower
  // half adds.  Layout [slot][value][lane] keeps every store/load bank-clean.
#pragma unroll
  for (int half = WAVES / 2; half >= 1; half >>= 1) {
    if (wave >= half && wave < 2 * half) {
      float* dst = red + size_t(wave - half) * NACC * 4 * 64;
      int v = 0;
#pragma unroll
      for (int g = 0; g < RG; ++g)
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
          for (int q = 0; q < 4; ++q, ++v) dst[v * 64 + lane] = acc[g][c][q];
    }
    __syncthreads();
    if (wave < half) {
      const float* src = red + size_t(wave) * NACC * 4 * 64;
      int v = 0;
#pragma unroll
      for (int g = 0; g < RG; ++g)
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
          for (int q = 0; q < 4; ++q, ++v) acc[g][c][q] += src[v * 64 + lane];
    }
    __syncthreads();
  }
  if (wave != 0) return;

  // Lane holds token row (lane & 15) + 16 g and, for register q, the 8
  // consecutive output columns n0 + (4 (lane >> 4) + q) * 8 + c, c = 0..7.
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    if (!aval[g]) continue;
    const int j = (lane & 15) + 16 * g;
    const size_t orow = UP ? size_t(sub) * P + slot_of[g]
                           : (SCAN ? size_t(slot_of[g]) : size_t(rbase + j));
    float* op = static_cast<float*>(out) + (UP ? 0 : sub * split_stride) + orow * Ndim;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int col = n0 + (4 * (lane >> 4) + q) * 8;
      if (col >= Ndim) continue;
      *reinterpret_cast<f32x4*>(op + col) =
          f32x4{acc[g][0][q], acc[g][1][q], acc[g][2][q], acc[g][3][q]};
      *reinterpret_cast<f32x4*>(op + col + 4) =
          f32x4{acc[g][4][q], acc[g][5][q], acc[g][6][q], acc[g][7][q]};
    }
  }
}

template <bool UP, int RG, int WAVES>
void launch_decode_rg(const Shape& s, dim3 grid, const uint16_t* x, const float* ab,
                      const int32_t* cnt, const int32_t* off, const int32_t* row_slot,
                      const int32_t* topk_idx, const uint16_t* w0, const uint16_t* w1, void* out,
                      int Kdim, int Ndim, int P, int ncb, int nsplit, int klen,
                      ptrdiff_t split_stride, hipStream_t stream) {
  auto kern = topk_idx ? decode_kernel<UP, RG, WAVES, true> : decode_kernel<UP, RG, WAVES, false>;
  hipLaunchKernelGGL(kern, grid, dim3(WAVES * 64), 0, stream, x, ab, cnt, off, row_slot, topk_idx,
                     w0, w1, out, Kdim, Ndim, s.K, P, ncb, nsplit, klen, split_stride);
}

template <bool UP, int WAVES>
hipError_t launch_decode_t(const Shape& s, const uint16_t* x, const float* ab, const int32_t* cnt,
                           const int32_t* off, const int32_t* row_slot, const int32_t* topk_idx,
                           const uint16_t* w0, const uint16_t* w1, void* out, int Kdim, int Ndim,
                           int nsplit, ptrdiff_t split_stride, hipStream_t stream) {
  const int ncb = (Ndim + 127) / 128;
  const dim3 grid(s.n * ncb * (UP ? 2 : nsplit));
  const int P = s.T * s.K;
  const int klen = (Kdim + nsplit - 1) / nsplit;
  // more token rows per lane means more accumulators: fewer waves, so the
  // registers fit without spilling
  static_assert(kStreamMaxTokens <= 4 * kDecodeRows, "four row groups per lane at most");
  if (s.T <= kDecodeRows)
    launch_decode_rg<UP, 1, WAVES>(s, grid, x, ab, cnt, off, row_slot, topk_idx, w0, w1, out,
                                   Kdim, Ndim, P, ncb, nsplit, klen, split_stride, stream);
  else if (s.T <= 2 * kDecodeRows)
    launch_decode_rg<UP, 2, WAVES / 2>(s, grid, x, ab, cnt, off, row_slot, topk_idx, w0, w1, out,
                                       Kdim, Ndim, P, ncb, nsplit, klen, split_stride, stream);
  else
    launch_decode_rg<UP, 4, WAVES / 2>(s, grid, x, ab, cnt, off, row_slot, topk_idx, w0, w1, out,
                                       Kdim, Ndim, P, ncb, nsplit, klen, split_stride, stream);
  return hipGetLastError();
}

}  // namespace

size_t decode_scratch_bytes(const Shape& s) {
  return size_t(2) * s.T * s.K * s.H * 4;
}

int decode_down_splits(const Shape& s) {
  // split the contraction when each half still gives every wave whole steps
  return (s.H % 64 == 0 && s.H / 2 >= 32 * kDownWaves) ? 2 : 1;
}

hipError_t launch_decode_up(const Shape& s, const uint16_t* x, const int32_t* expert_count,
                            const int32_t* expert_offset, const int32_t* row_slot,
                            const int32_t* topk_idx, const uint16_t* w1, const uint16_t* w3,
                            float* ab, hipStream_t stream) {
  return launch_decode_t<true, kUpWaves>(s, x, nullptr, expert_count, expert_offset, row_slot,
                                         topk_idx, w1, w3, ab, s.D, s.H, 1, 0, stream);
}

hipError_t launch_decode_down(const Shape& s, const int32_t* expert_count,
                              const int32_t* expert_offset, const int32_t* row_slot,
                              const int32_t* topk_idx, const float* ab, const uint16_t* w2,
                              float* y_rows, int nsplit, ptrdiff_t split_stride,
                              hipStream_t stream) {
  // the most waves (up to kDownWaves) that still give each at least 4 of the
  // 32-deep steps: a short contraction (small experts) over 16 waves would
  // spend its time in the reduction
  const int steps = (s.H + nsplit - 1) / nsplit / 32;
  if (steps >= 4 * kDownWaves)
    return launch_decode_t<false, kDownWaves>(s, nullptr, ab, expert_count, expert_offset,
                                              row_slot, topk_idx, w2, nullptr, y_rows, s.H, s.D,
                                              nsplit, split_stride, stream);
  if (steps >= 4 * 8)
    return launch_decode_t<false, 8>(s, nullptr, ab, expert_count, expert_offset, row_slot,
                                     topk_idx, w2, nullptr, y_rows, s.H, s.D, nsplit,
                                     split_stride, stream);
  return launch_decode_t<false, 4>(s, nullptr, ab, expert_count, expert_offset, row_slot,
                                   topk_idx, w2, nullptr, y_rows, s.H, s.D, nsplit, split_stride,
                                   stream);
}

}  // namespace moe
