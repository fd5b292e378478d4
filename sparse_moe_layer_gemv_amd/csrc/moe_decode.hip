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
// Work split: a workgroup owns (expert e, NB blocks of 128 output columns,
// one weight matrix, one contraction range); its waves form NB groups, group g
// taking block g, and a group's waves split the range.  With NB = 2 a
// workgroup reads 512 contiguous bytes of every weight row at once (two waves
// side by side), which streams faster than 256 in a load-only probe with
// non-temporal loads (7.0 against 6.65 TB/s).  NB and the contraction splits
// are chosen per shape (up_blocks, decode_up_splits, down_blocks,
// decode_down_splits).  Per 32-wide step a lane
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
#include <algorithm>

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
// first-product results, which come as `nparts` contraction partials
// `part_stride` floats apart and are added in order.
__device__ __forceinline__ uint4 h_fragment(const float* a, const float* b, int nparts,
                                            size_t part_stride) {
  f32x4 a0 = *reinterpret_cast<const f32x4*>(a), a1 = *reinterpret_cast<const f32x4*>(a + 4);
  f32x4 b0 = *reinterpret_cast<const f32x4*>(b), b1 = *reinterpret_cast<const f32x4*>(b + 4);
  for (int u = 1; u < nparts; ++u) {
    const float* au = a + u * part_stride;
    const float* bu = b + u * part_stride;
    a0 += *reinterpret_cast<const f32x4*>(au);
    a1 += *reinterpret_cast<const f32x4*>(au + 4);
    b0 += *reinterpret_cast<const f32x4*>(bu);
    b1 += *reinterpret_cast<const f32x4*>(bu + 4);
  }
  return make_uint4(pack_bf16x2(silu(a0[0]) * b0[0], silu(a0[1]) * b0[1]),
                    pack_bf16x2(silu(a0[2]) * b0[2], silu(a0[3]) * b0[3]),
                    pack_bf16x2(silu(a1[0]) * b1[0], silu(a1[1]) * b1[1]),
                    pack_bf16x2(silu(a1[2]) * b1[2], silu(a1[3]) * b1[3]));
}

// UP:   x [T][Kdim] bf16 rows gathered through row_slot; w = w1 or w3 (by
//       workgroup); out = ab fp32 [nsplit][2][P][Ndim] (contraction partial
//       ks; a at [ks][0], b at [ks][1], row = slot)
// DOWN: ab rows (ab_parts partials) through row_slot -> h; w = w2; partial ks
//       of y fp32 [cap][Ndim] at out (ks = 0) or y_part + (ks-1) * split_stride
// Both: partial ks covers contraction rows [ks*klen, +klen).
//
// SCAN: the expert's token-slots are found by scanning the routing itself
// (topk_idx, P = T*K entries, in slot order, so in the order the permute
// would give them), and the second product writes its rows at the slot index
// instead of the permuted row: no permute pass is needed.  Otherwise they come
// from the permuted layout (expert_count, expert_offset, row_slot).
template <bool UP, int RG, int WAVES, int NB, bool SCAN>
__global__ __launch_bounds__(WAVES * 64) void decode_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ ab,
    const int32_t* __restrict__ expert_count, const int32_t* __restrict__ expert_offset,
    const int32_t* __restrict__ row_slot, const int32_t* __restrict__ topk_idx,
    const uint16_t* __restrict__ w0, const uint16_t* __restrict__ w1, void* __restrict__ out,
    float* __restrict__ y_part, int Kdim, int Ndim, int topk, int P, int ncb, int nsplit,
    int klen, size_t split_stride, int ab_parts) {
  constexpr int NACC = RG * 8;                     // f32x4 accumulators per lane
  constexpr int WPG = WAVES / NB;                  // waves per column-block group
  static_assert(WAVES % NB == 0 && (WPG & (WPG - 1)) == 0, "groups of a power of two");
  __shared__ float red[(WAVES / 2) * NACC * 4 * 64];

  // workgroup -> (expert, matrix (UP), column-block group, contraction
  // split), split fastest.  Matrix-major inside an expert (all of w1's
  // column blocks, then w3's) streams faster than alternating w1 and w3
  // between neighbouring workgroups.
  const int groups = (ncb + NB - 1) / NB;
  const int per_mat = groups * nsplit;
  const int per_e = per_mat * (UP ? 2 : 1);
  const int e = blockIdx.x / per_e;
  const int r = blockIdx.x - e * per_e;
  const int ks = r % nsplit;
  const int mat = UP ? r / per_mat : 0;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int grp = wave / WPG, wl = wave - grp * WPG;
  const int cb = ((r - mat * per_mat) / nsplit) * NB + grp;
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
  // Pass blockIdx.y covers the expert's token rows [16 RG y, 16 RG (y + 1)).
  // RG is chosen from T, and an expert holds at most T rows when every token
  // names it at most once (always so under moe_forward, whose router picks K
  // distinct experts, and the only case SCAN serves); a caller's layout for
  // moe_grouped_ffn may name an expert twice for one token, and its rows
  // beyond the first pass are then taken by the further passes of the grid,
  // whose workgroups otherwise exit here.
  const int jb = blockIdx.y * 16 * RG;
  if (cnt <= jb) return;
  const int n0 = cb * 128;
  const int kg = lane >> 4;
  const int nbk = lane & 15;
  const bool col_ok = cb < ncb && n0 + nbk * 8 < Ndim;
  const int kbeg = ks * klen;
  const int kend = min(Kdim, kbeg + klen);
  const size_t ab_stride = size_t(2) * P * Kdim;   // DOWN: floats between ab partials

  // activation row pointers (token row j = jb + lane % 16 + 16 g of the expert)
  const uint16_t* xrow[RG];
  const float* arow[RG];
  const float* brow[RG];
  bool aval[RG];
  int slot_of[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    const int j = jb + (lane & 15) + 16 * g;
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
      (UP && mat ? w1 : w0) + size_t(e) * Kdim * Ndim + (cb < ncb ? n0 : 0) + nbk * 8;

  f32x4 acc[RG][8];
#pragma unroll
  for (int g = 0; g < RG; ++g)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[g][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int steps = (kend - kbeg + 31) / 32;
  const int per = (steps + WPG - 1) / WPG;
  const int s0 = wl * per;
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
          v = h_fragment(arow[g] + kk, brow[g] + kk, ab_parts, ab_stride);
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

  // Tree reduction over each group's waves: at each level the upper half
  // stores, the lower half adds.  Group g uses slots [g WPG/2, (g+1) WPG/2).
  // Layout [slot][value][lane] keeps every store/load bank-clean.
#pragma unroll
  for (int half = WPG / 2; half >= 1; half >>= 1) {
    if (wl >= half && wl < 2 * half) {
      float* dst = red + size_t(grp * (WPG / 2) + wl - half) * NACC * 4 * 64;
      int v = 0;
#pragma unroll
      for (int g = 0; g < RG; ++g)
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
          for (int q = 0; q < 4; ++q, ++v) dst[v * 64 + lane] = acc[g][c][q];
    }
    __syncthreads();
    if (wl < half) {
      const float* src = red + size_t(grp * (WPG / 2) + wl) * NACC * 4 * 64;
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
  if (wl != 0 || cb >= ncb) return;

  // Lane holds token row jb + (lane & 15) + 16 g and, for register q, the 8
  // consecutive output columns n0 + (4 (lane >> 4) + q) * 8 + c, c = 0..7.
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    if (!aval[g]) continue;
    const int j = jb + (lane & 15) + 16 * g;
    const size_t orow = UP ? size_t(ks * 2 + mat) * P + slot_of[g]
                           : (SCAN ? size_t(slot_of[g]) : size_t(rbase + j));
    float* plane = UP || ks == 0 ? static_cast<float*>(out) : y_part + (ks - 1) * split_stride;
    float* op = plane + orow * Ndim;
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

template <bool UP, int RG, int WAVES, int NB>
void launch_decode_rg(const Shape& s, dim3 grid, const uint16_t* x, const float* ab,
                      const int32_t* cnt, const int32_t* off, const int32_t* row_slot,
                      const int32_t* topk_idx, const uint16_t* w0, const uint16_t* w1, void* out,
                      float* y_part, int Kdim, int Ndim, int P, int ncb, int nsplit, int klen,
                      size_t split_stride, int ab_parts, hipStream_t stream) {
  auto kern = topk_idx ? decode_kernel<UP, RG, WAVES, NB, true>
                       : decode_kernel<UP, RG, WAVES, NB, false>;
  hipLaunchKernelGGL(kern, grid, dim3(WAVES * 64), 0, stream, x, ab, cnt, off, row_slot, topk_idx,
                     w0, w1, out, y_part, Kdim, Ndim, s.K, P, ncb, nsplit, klen, split_stride,
                     ab_parts);
}

// Column blocks per workgroup and contraction splits, by measurement (layer
// time at Mixtral decode weights; first product + second product where given):
//  - wide experts (H = 14336, 112 column blocks per matrix) once every expert
//    is likely touched (T*K >= 4n): four blocks per workgroup (448
//    workgroups, all resident at once, where 896 ran in 1.75 rounds) on the
//    half-wave kernel, no split.  Against two blocks: 16 tokens 435 against
//    457 us, 24: 444 against 481, 32: 451 against 484, 48 (forced streaming
//    before): 477 against 561;
//  - wide experts with fewer tokens: two blocks per workgroup (512 bytes of
//    each weight row at once).  At 8 tokens (about 7 of 8 experts touched)
//    four blocks were slower, 345 against 331 us.  Two blocks against one at
//    16 tokens: 293 + 149 us against 295 + 154; splitting the first product
//    in two there (the second then adds two partials of a and b): 294-297 +
//    157.  When few experts can be touched the contraction is split further
//    (decode_up_splits, decode_down_splits);
//  - narrow experts (H = 768, 6 blocks): one block and the first product's
//    contraction split in two (more workgroups): 175 + 97 us, against 183 + 96
//    unsplit and 201 + 92 with two blocks unsplit.
int up_blocks(const Shape& s) {
  if ((s.H + 127) / 128 < 32) return 1;
  return int64_t(s.T) * s.K >= 4 * int64_t(s.n) ? 4 : 2;
}

template <bool UP, int WAVES, int NB>
hipError_t launch_decode_nb(const Shape& s, const uint16_t* x, const float* ab,
                            const int32_t* cnt, const int32_t* off, const int32_t* row_slot,
                            const int32_t* topk_idx, const uint16_t* w0, const uint16_t* w1,
                            void* out, float* y_part, int Kdim, int Ndim, int nsplit,
                            size_t split_stride, int ab_parts, hipStream_t stream) {
  const int ncb = (Ndim + 127) / 128;
  const int groups = (ncb + NB - 1) / NB;
  const int P = s.T * s.K;
  // row passes: one when the experts' slots come from the routing (SCAN: K
  // distinct experts per token, at most T rows each); enough for P = T*K
  // rows on one expert when they come from a caller's permuted layout
  const int rows_per_pass = kDecodeRows * (s.T <= kDecodeRows ? 1 : s.T <= 2 * kDecodeRows ? 2 : 4);
  const int passes = topk_idx ? 1 : (P + rows_per_pass - 1) / rows_per_pass;
  const dim3 grid(s.n * groups * (UP ? 2 : 1) * nsplit, passes);
  const int klen = (Kdim + nsplit - 1) / nsplit;
  // more token rows per lane means more accumulators: fewer waves, so the
  // registers fit without spilling
  static_assert(kStreamMaxTokens <= 4 * kDecodeRows, "four row groups per lane at most");
  // four column blocks per workgroup run on the half-wave shape at any T:
  // each wave then walks the whole contraction of its block, with no
  // reduction across waves (16 tokens: 435 against 450 us per layer)
  if (s.T <= kDecodeRows && NB != 4)
    launch_decode_rg<UP, 1, WAVES, NB>(s, grid, x, ab, cnt, off, row_slot, topk_idx, w0, w1, out,
                                       y_part, Kdim, Ndim, P, ncb, nsplit, klen, split_stride,
                                       ab_parts, stream);
  else if (s.T <= 2 * kDecodeRows)
    launch_decode_rg<UP, 2, WAVES / 2, NB>(s, grid, x, ab, cnt, off, row_slot, topk_idx, w0, w1,
                                           out, y_part, Kdim, Ndim, P, ncb, nsplit, klen,
                                           split_stride, ab_parts, stream);
  else
    launch_decode_rg<UP, 4, WAVES / 2, NB>(s, grid, x, ab, cnt, off, row_slot, topk_idx, w0, w1,
                                           out, y_part, Kdim, Ndim, P, ncb, nsplit, klen,
                                           split_stride, ab_parts, stream);
  return hipGetLastError();
}

template <bool UP, int WAVES>
hipError_t launch_decode_t(const Shape& s, const uint16_t* x, const float* ab, const int32_t* cnt,
                           const int32_t* off, const int32_t* row_slot, const int32_t* topk_idx,
                           const uint16_t* w0, const uint16_t* w1, void* out, float* y_part,
                           int Kdim, int Ndim, int nsplit, size_t split_stride, int ab_parts,
                           int nb, hipStream_t stream) {
  if constexpr (UP && WAVES >= 8) {
    if (nb == 4)
      return launch_decode_nb<UP, WAVES, 4>(s, x, ab, cnt, off, row_slot, topk_idx, w0, w1, out,
                                            y_part, Kdim, Ndim, nsplit, split_stride, ab_parts,
                                            stream);
  }
  if (nb == 2)
    return launch_decode_nb<UP, WAVES, 2>(s, x, ab, cnt, off, row_slot, topk_idx, w0, w1, out,
                                          y_part, Kdim, Ndim, nsplit, split_stride, ab_parts,
                                          stream);
  return launch_decode_nb<UP, WAVES, 1>(s, x, ab, cnt, off, row_slot, topk_idx, w0, w1, out,
                                        y_part, Kdim, Ndim, nsplit, split_stride, ab_parts,
                                        stream);
}

// Workgroups that have work when at most min(n, T*K) experts are touched.
constexpr int kWantActive = 512;
int touched_max(const Shape& s) { return std::min(s.n, s.T * s.K); }

// Contraction splits of the first product: narrow experts split in two; wide
// ones split while too few experts are touched to give the chip kWantActive
// workgroups, as long as each wave keeps at least 4 of the 32-deep steps.
int decode_up_splits(const Shape& s) {
  if (up_blocks(s) == 4) return 1;
  if (up_blocks(s) == 1) return s.D % 64 == 0 && s.D / 2 >= 32 * 4 * kUpWaves ? 2 : 1;
  const int per = ((s.H + 127) / 128 + 1) / 2 * 2;  // workgroups per expert and split
  int n = 1;
  while (n < 4 && touched_max(s) * per * n < kWantActive && s.D % (64 * 2 * n) == 0 &&
         s.D / (2 * n) >= 32 * 4 * (kUpWaves / 2))
    n *= 2;
  return n;
}

// Two column blocks per workgroup in the second product for wide outputs.
int down_blocks(const Shape& s) {
  return (up_blocks(s) >= 2 || decode_up_splits(s) == 1) && (s.D + 127) / 128 >= 2 ? 2 : 1;
}

}  // namespace

size_t decode_scratch_bytes(const Shape& s) {
  return size_t(decode_up_splits(s)) * 2 * s.T * s.K * s.H * 4;
}

int decode_down_splits(const Shape& s) {
  // Split the contraction while each part still gives every wave of a group at
  // least 4 of the 32-deep steps; with two column blocks per workgroup, twice
  // as many parts keep the workgroup count.  When few experts are touched,
  // split further (up to 8) until kWantActive workgroups have work.
  const int nb = down_blocks(s);
  const int wpg = nb == 2 ? kDownWaves / 2 : kDownWaves;
  const int groups = ((s.D + 127) / 128 + nb - 1) / nb;
  int n = 1;
  const int want = nb == 2 ? 4 : 2;
  while (n < want && s.H % (64 * n) == 0 && s.H / (2 * n) >= 32 * 4 * wpg) n *= 2;
  while (n < 8 && touched_max(s) * groups * n < kWantActive && s.H % (64 * 2 * n) == 0 &&
         s.H / (2 * n) >= 32 * 4 * wpg / 2)
    n *= 2;
  return n;
}

hipError_t launch_decode_up(const Shape& s, const uint16_t* x, const int32_t* expert_count,
                            const int32_t* expert_offset, const int32_t* row_slot,
                            const int32_t* topk_idx, const uint16_t* w1, const uint16_t* w3,
                            float* ab, hipStream_t stream) {
  return launch_decode_t<true, kUpWaves>(s, x, nullptr, expert_count, expert_offset, row_slot,
                                         topk_idx, w1, w3, ab, nullptr, s.D, s.H,
                                         decode_up_splits(s), 0, 1, up_blocks(s), stream);
}

hipError_t launch_decode_down(const Shape& s, const int32_t* expert_count,
                              const int32_t* expert_offset, const int32_t* row_slot,
                              const int32_t* topk_idx, const float* ab, const uint16_t* w2,
                              float* y_rows, float* y_part, int nsplit, size_t part_stride,
                              hipStream_t stream) {
  // the most waves (up to kDownWaves) that still give each at least 4 of the
  // 32-deep steps: a short contraction (small experts) over 16 waves would
  // spend its time in the reduction
  const int ab_parts = decode_up_splits(s);
  const int steps = (s.H + nsplit - 1) / nsplit / 32;
  const int nb = down_blocks(s);
  if (steps >= 4 * kDownWaves / nb)
    return launch_decode_t<false, kDownWaves>(s, nullptr, ab, expert_count, expert_offset,
                                              row_slot, topk_idx, w2, nullptr, y_rows, y_part,
                                              s.H, s.D, nsplit, part_stride, ab_parts, nb, stream);
  if (steps >= 4 * 8 / nb)
    return launch_decode_t<false, 8>(s, nullptr, ab, expert_count, expert_offset, row_slot,
                                     topk_idx, w2, nullptr, y_rows, y_part, s.H, s.D, nsplit,
                                     part_stride, ab_parts, nb, stream);
  return launch_decode_t<false, 4>(s, nullptr, ab, expert_count, expert_offset, row_slot,
                                   topk_idx, w2, nullptr, y_rows, y_part, s.H, s.D, nsplit,
                                   part_stride, ab_parts, nb, stream);
}

}  // namespace moe
