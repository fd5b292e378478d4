// Weight-streaming expert path for small batches (decode).
//
// The pages note that a sparse MoE layer pays extra memory loads and loses
// efficiency at small batch sizes ("Mixtral of Experts", section 3, remark on
// hardware utilisation; the aipaper.jasonlin.tech summary, limitations).  With
// T <= 32 tokens each expert sees only a handful of rows, so the expert
// products are bound by reading the weights: every touched expert's w1, w3
// and w2 must cross HBM once and nothing else matters.  These kernels do
// exactly that read, once, coalesced, with enough loads in flight to keep HBM
// busy, and use the matrix cores only to keep the arithmetic off the critical
// path.
//
// Work split: a workgroup owns (expert e, 128 output columns); its waves split
// the contraction axis.  Per 32-wide step a lane loads an 8 x 8 bf16 block of
// each weight matrix (8 rows x 16 bytes; 16 lanes cover 256 contiguous bytes
// of a row), transposes it in registers, and feeds 8 v_mfma_f32_16x16x32_bf16
// whose A rows are 16 hidden units strided by 8 columns and whose B columns
// are up to 16 token rows of the expert.  The waves' partial sums are reduced
// through LDS in a fixed tree order (deterministic), and wave 0 applies the
// epilogue: silu(a)*b -> bf16 h for the up products, fp32 y for the down ones.
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int kUpWaves = 8;
constexpr int kDownWaves = 16;

__device__ __forceinline__ void transpose8x8_d(const uint4 (&in)[8], uint4 (&out)[8]) {
  uint32_t w[8][4];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    w[j][0] = in[j].x; w[j][1] = in[j].y; w[j][2] = in[j].z; w[j][3] = in[j].w;
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    uint32_t o[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t lo = w[2 * p][c >> 1];
      const uint32_t hi = w[2 * p + 1][c >> 1];
      o[p] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
    }
    out[c] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// UP:   act = x [T][Kdim], rows gathered through row_slot; wa = w1, wb = w3;
//       out = h bf16 [cap][Ndim]
// DOWN: act = h [cap][Kdim], rows are the expert's permuted rows; wa = w2;
//       out = y fp32 [cap][Ndim]
template <bool UP, int RG, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void decode_kernel(
    const uint16_t* __restrict__ act, const int32_t* __restrict__ expert_count,
    const int32_t* __restrict__ expert_offset, const int32_t* __restrict__ row_slot,
    const uint16_t* __restrict__ wa, const uint16_t* __restrict__ wb, void* __restrict__ out,
    int Kdim, int Ndim, int topk, int ncb) {
  constexpr int NMAT = UP ? 2 : 1;
  constexpr int NACC = NMAT * RG * 8;             // f32x4 accumulators per lane
  constexpr int RED_SLOTS = WAVES / 2;
  __shared__ float red[RED_SLOTS * NACC * 4 * 64];

  const int e = blockIdx.x / ncb;
  const int cb = blockIdx.x - e * ncb;
  const int cnt = expert_count[e];
  if (cnt == 0) return;
  const int rbase = expert_offset[e];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n0 = cb * 128;
  const int kg = lane >> 4;
  const int nbk = lane & 15;
  const bool col_ok = n0 + nbk * 8 < Ndim;

  const uint16_t* arow[RG];
  bool aval[RG];
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    const int j = (lane & 15) + 16 * g;
    aval[g] = j < cnt;
    if (UP) {
      const int slot = aval[g] ? row_slot[rbase + j] : 0;
      arow[g] = act + size_t(slot >= 0 ? slot / topk : 0) * Kdim;
    } else {
      arow[g] = act + size_t(rbase + (aval[g] ? j : 0)) * Kdim;
    }
  }
  const size_t wstride = size_t(Kdim) * Ndim;
  const uint16_t* wp[NMAT];
  wp[0] = wa + size_t(e) * wstride + n0 + nbk * 8;
  if (UP) wp[NMAT - 1] = wb + size_t(e) * wstride + n0 + nbk * 8;

  f32x4 acc[NMAT][RG][8];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int g = 0; g < RG; ++g)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[m][g][c] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int steps = (Kdim + 31) / 32;
  const int per = (steps + WAVES - 1) / WAVES;
  const int s0 = wave * per;
  const int s1 = min(steps, s0 + per);
  for (int s = s0; s < s1; ++s) {
    const int kk = s * 32 + kg * 8;
    const bool kok = kk < Kdim;
    uint4 wv[NMAT][8];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        wv[m][j] = (kok && col_ok) ? *reinterpret_cast<const uint4*>(wp[m] + size_t(kk + j) * Ndim)
                                   : make_uint4(0, 0, 0, 0);
    bf16x8 xv[RG];
#pragma unroll
    for (int g = 0; g < RG; ++g)
      xv[g] = as_bf16x8((kok && aval[g]) ? *reinterpret_cast<const uint4*>(arow[g] + kk)
                                         : make_uint4(0, 0, 0, 0));
#pragma unroll
    for (int m = 0; m < NMAT; ++m) {
      uint4 op[8];
      transpose8x8_d(wv[m], op);
#pragma unroll
      for (int c = 0; c < 8; ++c)
#pragma unroll
        for (int g = 0; g < RG; ++g)
          acc[m][g][c] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(op[c]), xv[g], acc[m][g][c], 0, 0, 0);
    }
  }

  // Tree reduction over waves: at each level the upper half stores, the lower
  // half adds.  Layout [slot][value][lane] keeps every store/load bank-clean.
#pragma unroll
  for (int half = WAVES / 2; half >= 1; half >>= 1) {
    if (wave >= half && wave < 2 * half) {
      float* dst = red + size_t(wave - half) * NACC * 4 * 64;
      int v = 0;
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int g = 0; g < RG; ++g)
#pragma unroll
          for (int c = 0; c < 8; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r, ++v) dst[v * 64 + lane] = acc[m][g][c][r];
    }
    __syncthreads();
    if (wave < half) {
      const float* src = red + size_t(wave) * NACC * 4 * 64;
      int v = 0;
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int g = 0; g < RG; ++g)
#pragma unroll
          for (int c = 0; c < 8; ++c)
#pragma unroll
            for (int r = 0; r < 4; ++r, ++v) acc[m][g][c][r] += src[v * 64 + lane];
    }
    __syncthreads();
  }
  if (wave != 0 || !col_ok) return;

  // Lane holds token row (lane & 15) + 16 g and, for register r, the 8
  // consecutive output columns n0 + (4 (lane >> 4) + r) * 8 + c, c = 0..7.
#pragma unroll
  for (int g = 0; g < RG; ++g) {
    if (!aval[g]) continue;
    const size_t row = size_t(rbase + (lane & 15) + 16 * g);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int col = n0 + (4 * (lane >> 4) + r) * 8;
      if (col >= Ndim) continue;
      if constexpr (UP) {
        uint32_t pk[4];
#pragma unroll
        for (int c = 0; c < 8; c += 2)
          pk[c / 2] = pack_bf16x2(silu(acc[0][g][c][r]) * acc[1][g][c][r],
                                  silu(acc[0][g][c + 1][r]) * acc[1][g][c + 1][r]);
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + row * Ndim + col) =
            make_uint4(pk[0], pk[1], pk[2], pk[3]);
      } else {
        float* yp = static_cast<float*>(out) + row * Ndim + col;
        *reinterpret_cast<f32x4*>(yp) =
            f32x4{acc[0][g][0][r], acc[0][g][1][r], acc[0][g][2][r], acc[0][g][3][r]};
        *reinterpret_cast<f32x4*>(yp + 4) =
            f32x4{acc[0][g][4][r], acc[0][g][5][r], acc[0][g][6][r], acc[0][g][7][r]};
      }
    }
  }
}

template <bool UP, int WAVES>
hipError_t launch_decode_t(const Shape& s, const uint16_t* act, const int32_t* cnt,
                           const int32_t* off, const int32_t* row_slot, const uint16_t* wa,
                           const uint16_t* wb, void* out, int Kdim, int Ndim,
                           hipStream_t stream) {
  const int ncb = (Ndim + 127) / 128;
  const int grid = s.n * ncb;
  if (s.T <= kDecodeRows)
    hipLaunchKernelGGL((decode_kernel<UP, 1, WAVES>), dim3(grid), dim3(WAVES * 64), 0, stream,
                       act, cnt, off, row_slot, wa, wb, out, Kdim, Ndim, s.K, ncb);
  else
    hipLaunchKernelGGL((decode_kernel<UP, 2, WAVES>), dim3(grid), dim3(WAVES * 64), 0, stream,
                       act, cnt, off, row_slot, wa, wb, out, Kdim, Ndim, s.K, ncb);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_up(const Shape& s, const uint16_t* x, const int32_t* expert_count,
                            const int32_t* expert_offset, const int32_t* row_slot,
                            const uint16_t* w1, const uint16_t* w3, uint16_t* h,
                            hipStream_t stream) {
  return launch_decode_t<true, kUpWaves>(s, x, expert_count, expert_offset, row_slot, w1, w3, h,
                                         s.D, s.H, stream);
}

hipError_t launch_decode_down(const Shape& s, const int32_t* expert_count,
                              const int32_t* expert_offset, const uint16_t* h,
                              const uint16_t* w2, float* y_rows, hipStream_t stream) {
  return launch_decode_t<false, kDownWaves>(s, h, expert_count, expert_offset, nullptr, w2,
                                            nullptr, y_rows, s.H, s.D, stream);
}

}  // namespace moe
