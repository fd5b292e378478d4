// Weight-streaming expert path for small batches (decode).
//
// The pages note that a sparse MoE layer pays extra memory loads and loses
// efficiency at small batch sizes ("Mixtral of Experts", section 3, remark on
// hardware utilisation; the aipaper.jasonlin.tech summary, limitations).  With
// up to ~100 tokens each expert sees a few dozen rows at most, so the expert
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
// First product: w1 and w3 are separate workgroups (a workgroup reading both
// would read half as many contiguous bytes of each matrix row), each writing
// its fp32 result a = x.w1 or b = x.w3 per token-slot and contraction
// partial.  A small pass adds the partials and forms h = bf16(silu(a) * b)
// per token-slot, the same single rounding as the tiled path; the second
// product reads h as the first reads x, and its contraction is split into
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

// h = bf16(silu(a) * b) for every token-slot, from the first product's fp32
// results ab [nparts][2][P][H] (contraction partials added in order): one
// thread per 8 consecutive values of a row.  Rows of slots no expert
// computed hold whatever ab held and are never read.
__global__ __launch_bounds__(256) void decode_h_kernel(const float* __restrict__ ab,
                                                       uint16_t* __restrict__ h, size_t n8,
                                                       int nparts, size_t part_stride,
                                                       size_t b_offset) {
  const size_t i = size_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n8) return;
  const float* a = ab + i * 8;
  const float* b = a + b_offset;
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
  *reinterpret_cast<uint4*>(h + i * 8) =
      make_uint4(pack_bf16x2(silu(a0[0]) * b0[0], silu(a0[1]) * b0[1]),
                 pack_bf16x2(silu(a0[2]) * b0[2], silu(a0[3]) * b0[3]),
                 pack_bf16x2(silu(a1[0]) * b1[0], silu(a1[1]) * b1[1]),
                 pack_bf16x2(silu(a1[2]) * b1[2], silu(a1[3]) * b1[3]));
}

// UP:   x [T][Kdim] bf16 rows gathered through row_slot; w = w0 (w1) or w1
//       (w3) by workgroup; out = ab fp32 [nsplit][2][P][Ndim] (contraction
//       partial ks; a at [ks][0], b at [ks][1], row = slot)
// DOWN: x = h bf16 [P][Kdim] (row = slot); w0 = w2; partial ks of y fp32
//       [cap][Ndim] at out (ks = 0) or y_part + (ks-1) * split_stride
// Both: partial ks covers contraction rows [ks*klen, +klen).
//
// SCAN: the expert's token-slots are found by scanning the routing itself
// (topk_idx, P = T*K entries, in slot order, so in the order the permute
// would give them), and the second product writes its rows at the slot index
// instead of the permuted row: no permute pass is needed.  Otherwise they come
// from the permuted layout (expert_count, expert_offset, row_slot).
template <bool UP, int RG, int WAVES, int NB, bool SCAN>
__global__ __launch_bounds__(WAVES * 64) void decode_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ expert_count,
    const int32_t* __restrict__ expert_offset, const int32_t* __restrict__ row_slot,
    const int32_t* __restrict__ topk_idx, const uint16_t* __restrict__ w0,
    const uint16_t* __restrict__ w1, float* __restrict__ out, float* __restrict__ y_part,
    int Kdim, int Ndim, int topk, int P, int ncb, int nsplit, int klen, size_t split_stride) {
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
  // there are at most T <= kStreamMaxTokens of them
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
  // The grid has passes enough for the most rows one expert can hold: T when
  // every token names it at most once (always so under moe_forward, whose
  // router picks K distinct experts, and the only case SCAN serves), T*K for
  // a caller's layout given to moe_grouped_ffn, which may name an expert
  // twice for one token.  Workgroups of passes past an expert's rows exit
  // here; a pass that has rows streams the expert's weights again.
  const int jb = blockIdx.y * 16 * RG;
  if (cnt <= jb) return;
  const int n0 = cb * 128;
  const int kg = lane >> 4;
  const int nbk = lane & 15;
  const bool col_ok = cb < ncb && n0 + nbk * 8 < Ndim;
  const int kbeg = ks * klen;
  const int kend = min(Kdim, kbeg + klen);

  // activation row pointers (token row j = jb + lane % 16 + 16 g of the expert)
  const uint16_t* xrow[RG];
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
    xrow[g] = x + size_t(UP ? sl / topk : sl) * Kdim;
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
      if (kok && aval[g]) v = *reinterpret_cast<const uint4*>(xrow[g] + kk);
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
    float* plane = UP || ks == 0 ? out : y_part + (ks - 1) * split_stride;
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
void launch_decode_rg(const Shape& s, dim3 grid, const uint16_t* x, const int32_t* cnt,
                      const int32_t* off, const int32_t* row_slot, const int32_t* topk_idx,
                      const uint16_t* w0, const uint16_t* w1, float* out, float* y_part, int Kdim,
                      int Ndim, int P, int ncb, int nsplit, int klen, size_t split_stride,
                      hipStream_t stream) {
  auto kern = topk_idx ? decode_kernel<UP, RG, WAVES, NB, true>
                       : decode_kernel<UP, RG, WAVES, NB, false>;
  hipLaunchKernelGGL(kern, grid, dim3(WAVES * 64), 0, stream, x, cnt, off, row_slot, topk_idx, w0,
                     w1, out, y_part, Kdim, Ndim, s.K, P, ncb, nsplit, klen, split_stride);
}

// Column blocks per workgroup and contraction splits, by measurement (layer
// time at Mixtral decode weights; first product + second product where given):
//  - wide experts (H = 14336, 112 column blocks per matrix) once most experts
//    are likely touched (T*K >= 2.5 n): four blocks per workgroup (448
//    workgroups, all resident at once, where 896 ran in 1.75 rounds) on the
//    half-wave kernel, no split.  Against two blocks: 10 tokens 376 against
//    413 us, 12: 378 against 413, 14: 428 against 446, 16: 435 against 457,
//    24: 444 against 481, 32: 451 against 484, 48 (forced streaming before):
//    477 against 561;
//  - wide experts with fewer tokens: two blocks per workgroup (512 bytes of
//    each weight row at once).  At 8 tokens (5 to 7 of 8 experts touched)
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
  return 2 * int64_t(s.T) * s.K >= 5 * int64_t(s.n) ? 4 : 2;
}

template <bool UP, int WAVES, int NB>
hipError_t launch_decode_nb(const Shape& s, const uint16_t* x, const int32_t* cnt,
                            const int32_t* off, const int32_t* row_slot, const int32_t* topk_idx,
                            const uint16_t* w0, const uint16_t* w1, float* out, float* y_part,
                            int Kdim, int Ndim, int nsplit, size_t split_stride,
                            hipStream_t stream) {
  const int ncb = (Ndim + 127) / 128;
  const int groups = (ncb + NB - 1) / NB;
  const int P = s.T * s.K;
  // Row groups of 16 token rows per lane (RG): one up to 16 tokens, two up to
  // 64, four beyond.  Four hold 64 rows in one pass, but their 128
  // accumulators leave a SIMD room for fewer waves: at 48 and 64 tokens two
  // row groups with a second pass (whose workgroups find no rows past the
  // first 32 unless an expert holds more) were faster, 449.7 against 455.0
  // and 460.1 against 465.1 us per layer.  Beyond 64 tokens an expert's rows
  // pass 32 too often, and a second pass streams its weights again.  Four column blocks per workgroup run on
  // the half-wave shape at any T: each wave then walks the whole contraction
  // of its block, with no reduction across waves (16 tokens: 435 against
  // 450 us per layer).
  const int rg = s.T <= kDecodeRows && NB != 4 ? 1 : s.T <= 4 * kDecodeRows ? 2 : 4;
  // row passes: enough for the most rows one expert can hold, T when the
  // slots come from the routing (SCAN: K distinct experts per token), P = T*K
  // when they come from a caller's permuted layout
  const int rows = topk_idx ? s.T : P;
  const int passes = (rows + kDecodeRows * rg - 1) / (kDecodeRows * rg);
  const dim3 grid(s.n * groups * (UP ? 2 : 1) * nsplit, passes);
  const int klen = (Kdim + nsplit - 1) / nsplit;
  if (rg == 1)
    launch_decode_rg<UP, 1, WAVES, NB>(s, grid, x, cnt, off, row_slot, topk_idx, w0, w1, out,
                                       y_part, Kdim, Ndim, P, ncb, nsplit, klen, split_stride,
                                       stream);
  else if (rg == 2)
    launch_decode_rg<UP, 2, WAVES / 2, NB>(s, grid, x, cnt, off, row_slot, topk_idx, w0, w1, out,
                                           y_part, Kdim, Ndim, P, ncb, nsplit, klen, split_stride,
                                           stream);
  else
    launch_decode_rg<UP, 4, WAVES / 2, NB>(s, grid, x, cnt, off, row_slot, topk_idx, w0, w1, out,
                                           y_part, Kdim, Ndim, P, ncb, nsplit, klen, split_stride,
                                           stream);
  return hipGetLastError();
}

template <bool UP, int WAVES>
hipError_t launch_decode_t(const Shape& s, const uint16_t* x, const int32_t* cnt,
                           const int32_t* off, const int32_t* row_slot, const int32_t* topk_idx,
                           const uint16_t* w0, const uint16_t* w1, float* out, float* y_part,
                           int Kdim, int Ndim, int nsplit, size_t split_stride, int nb,
                           hipStream_t stream) {
  if constexpr (UP && WAVES >= 8) {
    if (nb == 4)
      return launch_decode_nb<UP, WAVES, 4>(s, x, cnt, off, row_slot, topk_idx, w0, w1, out,
                                            y_part, Kdim, Ndim, nsplit, split_stride, stream);
  }
  if (nb == 2)
    return launch_decode_nb<UP, WAVES, 2>(s, x, cnt, off, row_slot, topk_idx, w0, w1, out, y_part,
                                          Kdim, Ndim, nsplit, split_stride, stream);
  return launch_decode_nb<UP, WAVES, 1>(s, x, cnt, off, row_slot, topk_idx, w0, w1, out, y_part,
                                        Kdim, Ndim, nsplit, split_stride, stream);
}

// Workgroups that have work when at most min(n, T*K) experts are touched.
constexpr int kWantActive = 512;
int touched_max(const Shape& s) { return std::min(s.n, s.T * s.K); }

// Contraction splits of the first product: narrow experts split in two; wide
// ones split while too few experts are touched to give the chip enough busy
// workgroups, as long as each wave keeps at least 4 of the 32-deep steps.
// The target is kWantActive, doubled for wide experts from T*K >= 2n (with
// two column blocks): at 8 tokens (5 of 8 experts touched in the benchmark
// routing) the first product went from 203 to 188 us.  The same doubling for
// the second product saved 9 us at 8 tokens but cost 9 at 10-14, and for
// smaller T it cost both products (T = 2: 194 -> 208, T = 4: 236 -> 242).
int decode_up_splits(const Shape& s) {
  if (up_blocks(s) == 4) return 1;
  if (up_blocks(s) == 1) return s.D % 64 == 0 && s.D / 2 >= 32 * 4 * kUpWaves ? 2 : 1;
  const int per = ((s.H + 127) / 128 + 1) / 2 * 2;  // workgroups per expert and split
  const int want = int64_t(s.T) * s.K >= 2 * int64_t(s.n) ? 2 * kWantActive : kWantActive;
  int n = 1;
  while (n < 4 && touched_max(s) * per * n < want && s.D % (64 * 2 * n) == 0 &&
         s.D / (2 * n) >= 32 * 4 * (kUpWaves / 2))
    n *= 2;
  return n;
}

// Two column blocks per workgroup in the second product for wide outputs.
int down_blocks(const Shape& s) {
  return (up_blocks(s) >= 2 || decode_up_splits(s) == 1) && (s.D + 127) / 128 >= 2 ? 2 : 1;
}

// fp32 a and b ([S][2][P][H]) then bf16 h ([P][H]), each 256-byte aligned
size_t ab_bytes(const Shape& s) {
  const size_t P = size_t(s.T) * s.K;
  return (size_t(decode_up_splits(s)) * 2 * P * s.H * 4 + 255) / 256 * 256;
}

}  // namespace

size_t decode_scratch_bytes(const Shape& s) {
  return ab_bytes(s) + size_t(s.T) * s.K * s.H * 2;
}

int decode_down_splits(const Shape& s) {
  // Split the contraction while each part still gives every wave of a group at
  // least 4 of the 32-deep steps; with two column blocks per workgroup, twice
  // as many parts keep the workgroup count.  When few experts are touched,
  // split further (up to 8) until kWantActive workgroups have work.  From
  // T*K >= 2n on (most experts touched) two parts and half that target do:
  // the 512 workgroups of 16 waves then take one round instead of two, and
  // the combine adds fewer partials (Mixtral decode weights, layer time: 8
  // tokens 310 -> 299 us, 32: 438 -> 434, 64: 459 -> 450, 12 and 16 the same;
  // below 2n it cost 4 tokens 16 us, so smaller batches keep the first rule).
  const int nb = down_blocks(s);
  const int wpg = nb == 2 ? kDownWaves / 2 : kDownWaves;
  const int groups = ((s.D + 127) / 128 + nb - 1) / nb;
  const bool most = int64_t(s.T) * s.K >= 2 * int64_t(s.n);
  int n = 1;
  const int want = nb == 2 && !most ? 4 : 2;
  while (n < want && s.H % (64 * n) == 0 && s.H / (2 * n) >= 32 * 4 * wpg) n *= 2;
  const int active = most ? kWantActive / 2 : kWantActive;
  while (n < 8 && touched_max(s) * groups * n < active && s.H % (64 * 2 * n) == 0 &&
         s.H / (2 * n) >= 32 * 4 * wpg / 2)
    n *= 2;
  return n;
}

hipError_t launch_decode_up(const Shape& s, const uint16_t* x, const int32_t* expert_count,
                            const int32_t* expert_offset, const int32_t* row_slot,
                            const int32_t* topk_idx, const uint16_t* w1, const uint16_t* w3,
                            void* scratch, hipStream_t stream) {
  return launch_decode_t<true, kUpWaves>(s, x, expert_count, expert_offset, row_slot, topk_idx,
                                         w1, w3, static_cast<float*>(scratch), nullptr, s.D, s.H,
                                         decode_up_splits(s), 0, up_blocks(s), stream);
}

hipError_t launch_decode_down(const Shape& s, const int32_t* expert_count,
                              const int32_t* expert_offset, const int32_t* row_slot,
                              const int32_t* topk_idx, void* scratch, const uint16_t* w2,
                              float* y_rows, float* y_part, int nsplit, size_t part_stride,
                              hipStream_t stream) {
  // h from the first product's a and b, then the product with w2
  const float* ab = static_cast<const float*>(scratch);
  uint16_t* h = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(scratch) + ab_bytes(s));
  const size_t P = size_t(s.T) * s.K;
  const size_t n8 = P * s.H / 8;
  hipLaunchKernelGGL(decode_h_kernel, dim3(unsigned((n8 + 255) / 256)), dim3(256), 0, stream, ab, h,
                     n8, decode_up_splits(s), 2 * P * s.H, P * s.H);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // the most waves (up to kDownWaves) that still give each at least 4 of the
  // 32-deep steps: a short contraction (small experts) over 16 waves would
  // spend its time in the reduction
  const int steps = (s.H + nsplit - 1) / nsplit / 32;
  const int nb = down_blocks(s);
  if (steps >= 4 * kDownWaves / nb)
    return launch_decode_t<false, kDownWaves>(s, h, expert_count, expert_offset, row_slot,
                                              topk_idx, w2, nullptr, y_rows, y_part, s.H, s.D,
                                              nsplit, part_stride, nb, stream);
  if (steps >= 4 * 8 / nb)
    return launch_decode_t<false, 8>(s, h, expert_count, expert_offset, row_slot, topk_idx, w2,
                                     nullptr, y_rows, y_part, s.H, s.D, nsplit, part_stride, nb,
                                     stream);
  return launch_decode_t<false, 4>(s, h, expert_count, expert_offset, row_slot, topk_idx, w2,
                                   nullptr, y_rows, y_part, s.H, s.D, nsplit, part_stride, nb,
                                   stream);
}

}  // namespace moe
