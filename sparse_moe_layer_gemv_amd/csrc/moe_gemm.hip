// Grouped expert GEMMs on the CDNA4 matrix cores (bf16 in, fp32 accumulate).
//
// "Mixtral of Experts", section 2.1: each expert is a SwiGLU feed-forward
// block and every token is routed to K = 2 of them; Megablocks is cited there
// for casting the expert FFNs as large matrix products over unequal token
// groups.  Here the groups are the expert segments built by the permute step
// (padded to 256 rows), and two kernels evaluate
//     up:   h[r]  = silu(x_t . w1_e) * (x_t . w3_e)     (bf16 out, fp32 math)
//     down: y[r]  = h[r] . w2_e                          (fp32 out)
// for every permuted row r of expert e (token t = row_slot[r] / K).
//
// Tiling (both kernels): a 256-thread workgroup (4 wavefronts, one per SIMD)
// owns a 256-row x 256-column output tile and walks the contraction axis in
// 64-wide steps through a double-buffered LDS stage (2 x 64 KiB).  Each wave
// owns a 128 x 128 sub-tile held as 4 x 4 accumulators of
// v_mfma_f32_32x32x16_bf16 (256 fp32 per lane).  In the up kernel the 256
// columns are 128 columns of w1 and the same 128 columns of w3, so each wave
// holds a and b for identical (row, column) pairs and applies silu(a)*b in
// registers before a single bf16 rounding.
//
// Layouts: weights are row-major with the output axis contiguous ([D][H],
// [H][D]), but the matrix-core operand wants 8 consecutive contraction
// elements per lane.  Each thread therefore loads an 8 x 8 block (8 rows of
// 16 bytes, coalesced along the output axis), transposes it in registers with
// byte permutes, and stores 8 contraction-contiguous 16-byte chunks into LDS.
// LDS rows are 128 bytes (64 bf16 of the contraction axis) with the 16-byte
// chunk index XOR-swizzled so both the transposed stores and the operand
// reads spread over all banks.
//
// The weight operand is fed to the matrix core as the "A" (row) side and the
// activations as "B", so each lane's accumulator holds 4 consecutive output
// columns of one token row: h is stored as 8-byte and y as 16-byte vectors.
//
// Workgroup order: the hardware hands workgroup ids to the 8 XCDs round-robin,
// and each XCD has its own L2.  The block id is remapped so every XCD works on
// a contiguous range of tiles, and tiles are rastered in groups of 4 row-tiles
// so the ~32 workgroups resident on one XCD share 4 activation panels and 8
// weight panels in its L2.
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int BM = 256;          // rows (token-slots) per tile
constexpr int BK = 64;           // contraction step
constexpr int BNC = 256;         // output columns per tile held in LDS
constexpr int NTHR = 256;
constexpr int A_BYTES = BM * BK * 2;    // 32 KiB
constexpr int B_BYTES = BNC * BK * 2;   // 32 KiB
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
constexpr int GROUP_M = 4;

static_assert(BM == kTileM, "segment granule must equal the row tile");

// LDS byte offset of 16-byte chunk c (0..7) of activation row m.
__device__ __forceinline__ uint32_t a_off(int m, int c) {
  return uint32_t(m) * 128u + (uint32_t((c ^ (m & 7))) << 4);
}
// LDS byte offset of 16-byte chunk c of weight column n (contraction-contiguous).
__device__ __forceinline__ uint32_t b_off(int n, int c) {
  return uint32_t(n) * 128u + (uint32_t(c ^ (n & 7) ^ ((n >> 3) & 7)) << 4);
}

__device__ __forceinline__ void lds_store16(uint8_t* smem, uint32_t off, uint4 v) {
  *reinterpret_cast<uint4*>(smem + off) = v;
}
__device__ __forceinline__ bf16x8 lds_load16(const uint8_t* smem, uint32_t off) {
  return as_bf16x8(*reinterpret_cast<const uint4*>(smem + off));
}

// Transpose an 8x8 block of bf16: in[j] holds row j (8 columns), out[c] gets
// column c (8 rows).  One byte-permute per output word.
__device__ __forceinline__ void transpose8x8(const uint4 (&in)[8], uint4 (&out)[8]) {
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

// XCD-aware tile mapping.  Workgroup L runs on XCD L % 8.  Valid workgroups
// (L < total) are renumbered so XCD x gets a contiguous range, then the range
// is rastered in groups of GROUP_M row-tiles with the row index fastest.
__device__ __forceinline__ bool map_tile(int L, int mt_count, int nt_count, int& mt, int& nt) {
  const int total = mt_count * nt_count;
  if (L >= total) return false;
  const int xcd = L & 7;
  const int local = L >> 3;
  const int q = total >> 3, rem = total & 7;
  const int v = xcd * q + min(xcd, rem) + local;
  const int group = GROUP_M * nt_count;
  const int g = v / group;
  const int r = v - g * group;
  const int rows_in_group = min(GROUP_M, mt_count - g * GROUP_M);
  mt = g * GROUP_M + r % rows_in_group;
  nt = r / rows_in_group;
  return true;
}

// Expert owning permuted row `row0` (segments are tile-aligned).
__device__ __forceinline__ int expert_of_row(const int32_t* __restrict__ offset, int n, int row0) {
  int e = 0;
  while (e + 1 < n && offset[e + 1] <= row0) ++e;
  return e;
}

// One 64-wide contraction step of the wave's 128x128 sub-tile.
//   smem_a: activation stage, smem_b: weight stage
//   a_row0: first activation row of this wave, b_col0[j]: first weight column of fragment j
__device__ __forceinline__ void mma_stage(const uint8_t* smem_a, const uint8_t* smem_b, int lane,
                                          int a_row0, const int (&b_col)[4], f32x16 (&acc)[4][4]) {
  const int l32 = lane & 31;
  const int hi = lane >> 5;
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) {
    const int c = kk * 2 + hi;
    bf16x8 xf[4], wf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) xf[i] = lds_load16(smem_a, a_off(a_row0 + i * 32 + l32, c));
#pragma unroll
    for (int j = 0; j < 4; ++j) wf[j] = lds_load16(smem_b, b_off(b_col[j] + l32, c));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[j], xf[i], acc[i][j], 0, 0, 0);
  }
}

// ---------------------------------------------------------------------------
// up: h = silu(x w1) * (x w3)
// ---------------------------------------------------------------------------
template <bool EVEN>
__global__ __launch_bounds__(NTHR, 1) void grouped_up_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ expert_offset,
    const int32_t* __restrict__ row_slot, const uint16_t* __restrict__ w1,
    const uint16_t* __restrict__ w3, uint16_t* __restrict__ h, int D, int H, int n, int K) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE_BYTES];

  const int mt_count = expert_offset[n] / BM;
  const int nt_count = (H + 127) / 128;
  int mt, nt;
  if (!map_tile(blockIdx.x, mt_count, nt_count, mt, nt)) return;
  const int row0 = mt * BM;
  const int e = expert_of_row(expert_offset, n, row0);
  const int n0 = nt * 128;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // activation loads: chunk ac of rows ar + 32 i
  const int ac = tid & 7;
  const int ar = tid >> 3;
  const uint16_t* xrow[8];
  bool xvalid[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int slot = row_slot[row0 + ar + 32 * i];
    xvalid[i] = slot >= 0;
    const int tok = xvalid[i] ? slot / K : 0;
    xrow[i] = x + size_t(tok) * D + ac * 8;
  }
  // weight loads: matrix wmat, chunk row-block kc (8 rows), column block nb (8 cols)
  const int wmat = wave >> 1;
  const int kc = ((wave & 1) << 2) | (lane >> 4);
  const int nb = lane & 15;
  const uint16_t* wbase = (wmat ? w3 : w1) + size_t(e) * D * H + size_t(kc * 8) * H + n0 + nb * 8;
  const bool wcol_ok = EVEN || (n0 + nb * 8 < H);

  uint4 ra[8], rb[8];
  auto load_stage = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool ok = xvalid[i] && (EVEN || k0 + ac * 8 < D);
      ra[i] = ok ? *reinterpret_cast<const uint4*>(xrow[i] + k0) : make_uint4(0, 0, 0, 0);
    }
    const bool kok = EVEN || (k0 + kc * 8 < D);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      rb[j] = (wcol_ok && kok) ? *reinterpret_cast<const uint4*>(wbase + size_t(k0 + j) * H)
                               : make_uint4(0, 0, 0, 0);
  };
  auto store_stage = [&](uint8_t* st) {
#pragma unroll
    for (int i = 0; i < 8; ++i) lds_store16(st, a_off(ar + 32 * i, ac), ra[i]);
    uint4 tb[8];
    transpose8x8(rb, tb);
    uint8_t* sb = st + A_BYTES;
#pragma unroll
    for (int c = 0; c < 8; ++c) lds_store16(sb, b_off(wmat * 128 + nb * 8 + c, kc), tb[c]);
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int wm = wave >> 1, wn = wave & 1;
  const int a_row0 = wm * 128;
  const int b_col[4] = {wn * 64, wn * 64 + 32, 128 + wn * 64, 128 + wn * 64 + 32};

  const int ksteps = (D + BK - 1) / BK;
  load_stage(0);
  store_stage(smem);
  __syncthreads();
  for (int ks = 0; ks < ksteps; ++ks) {
    uint8_t* cur = smem + (ks & 1) * STAGE_BYTES;
    uint8_t* nxt = smem + ((ks + 1) & 1) * STAGE_BYTES;
    const bool more = ks + 1 < ksteps;
    if (more) load_stage((ks + 1) * BK);
    mma_stage(cur, cur + A_BYTES, lane, a_row0, b_col, acc);
    if (more) store_stage(nxt);
    __syncthreads();
  }

  // epilogue: lane holds token row (a_row0 + 32 i + lane%32) and, per
  // register quad q, 4 consecutive columns starting at 8 q + 4 (lane/32)
  const int l32 = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = row0 + a_row0 + i * 32 + l32;
    uint16_t* hrow = h + size_t(m) * H;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = n0 + wn * 64 + jj * 32 + q * 8 + hi * 4;
        if (!EVEN && col >= H) continue;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float a = acc[i][jj][q * 4 + r];
          const float b = acc[i][jj + 2][q * 4 + r];
          v[r] = silu(a) * b;
        }
        uint2 pk;
        pk.x = pack_bf16x2(v[0], v[1]);
        pk.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2*>(hrow + col) = pk;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// down: y = h w2
// ---------------------------------------------------------------------------
template <bool EVEN>
__global__ __launch_bounds__(NTHR, 1) void grouped_down_kernel(
    const int32_t* __restrict__ expert_offset, const uint16_t* __restrict__ h,
    const uint16_t* __restrict__ w2, float* __restrict__ y, int D, int H, int n) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * STAGE_BYTES];

  const int mt_count = expert_offset[n] / BM;
  const int nt_count = (D + BNC - 1) / BNC;
  int mt, nt;
  if (!map_tile(blockIdx.x, mt_count, nt_count, mt, nt)) return;
  const int row0 = mt * BM;
  const int e = expert_of_row(expert_offset, n, row0);
  const int n0 = nt * BNC;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  const int ac = tid & 7;
  const int ar = tid >> 3;
  const uint16_t* hrow = h + size_t(row0 + ar) * H + ac * 8;
  const size_t hstride32 = size_t(32) * H;

  const int kc = tid >> 5;   // 0..7
  const int nb = tid & 31;   // 0..31
  const uint16_t* wbase = w2 + size_t(e) * H * D + size_t(kc * 8) * D + n0 + nb * 8;
  const bool wcol_ok = EVEN || (n0 + nb * 8 < D);

  uint4 ra[8], rb[8];
  auto load_stage = [&](int k0) {
    const bool aok = EVEN || (k0 + ac * 8 < H);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      ra[i] = aok ? *reinterpret_cast<const uint4*>(hrow + i * hstride32 + k0) : make_uint4(0, 0, 0, 0);
    const bool kok = EVEN || (k0 + kc * 8 < H);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      rb[j] = (wcol_ok && kok) ? *reinterpret_cast<const uint4*>(wbase + size_t(k0 + j) * D)
                               : make_uint4(0, 0, 0, 0);
  };
  auto store_stage = [&](uint8_t* st) {
#pragma unroll
    for (int i = 0; i < 8; ++i) lds_store16(st, a_off(ar + 32 * i, ac), ra[i]);
    uint4 tb[8];
    transpose8x8(rb, tb);
    uint8_t* sb = st + A_BYTES;
#pragma unroll
    for (int c = 0; c < 8; ++c) lds_store16(sb, b_off(nb * 8 + c, kc), tb[c]);
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int wm = wave >> 1, wn = wave & 1;
  const int a_row0 = wm * 128;
  const int b_col[4] = {wn * 128, wn * 128 + 32, wn * 128 + 64, wn * 128 + 96};

  const int ksteps = (H + BK - 1) / BK;
  load_stage(0);
  store_stage(smem);
  __syncthreads();
  for (int ks = 0; ks < ksteps; ++ks) {
    uint8_t* cur = smem + (ks & 1) * STAGE_BYTES;
    uint8_t* nxt = smem + ((ks + 1) & 1) * STAGE_BYTES;
    const bool more = ks + 1 < ksteps;
    if (more) load_stage((ks + 1) * BK);
    mma_stage(cur, cur + A_BYTES, lane, a_row0, b_col, acc);
    if (more) store_stage(nxt);
    __syncthreads();
  }

  const int l32 = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = row0 + a_row0 + i * 32 + l32;
    float* yrow = y + size_t(m) * D;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = n0 + b_col[j] + q * 8 + hi * 4;
        if (!EVEN && col >= D) continue;
        f32x4 v = {acc[i][j][q * 4 + 0], acc[i][j][q * 4 + 1], acc[i][j][q * 4 + 2],
                   acc[i][j][q * 4 + 3]};
        *reinterpret_cast<f32x4*>(yrow + col) = v;
      }
    }
  }
}

}  // namespace

hipError_t launch_grouped_up(const Shape& s, const uint16_t* x, const int32_t* expert_offset,
                             const int32_t* row_slot, const uint16_t* w1, const uint16_t* w3,
                             uint16_t* h, hipStream_t stream) {
  const int mt_max = int(s.cap / BM);
  const int nt = (s.H + 127) / 128;
  const int grid = mt_max * nt;
  if (grid == 0) return hipSuccess;
  const bool even = (s.H % 128 == 0) && (s.D % BK == 0);
  if (even)
    hipLaunchKernelGGL(grouped_up_kernel<true>, dim3(grid), dim3(NTHR), 0, stream, x,
                       expert_offset, row_slot, w1, w3, h, s.D, s.H, s.n, s.K);
  else
    hipLaunchKernelGGL(grouped_up_kernel<false>, dim3(grid), dim3(NTHR), 0, stream, x,
                       expert_offset, row_slot, w1, w3, h, s.D, s.H, s.n, s.K);
  return hipGetLastError();
}

hipError_t launch_grouped_down(const Shape& s, const int32_t* expert_offset, const uint16_t* h,
                               const uint16_t* w2, float* y_rows, hipStream_t stream) {
  const int mt_max = int(s.cap / BM);
  const int nt = (s.D + BNC - 1) / BNC;
  const int grid = mt_max * nt;
  if (grid == 0) return hipSuccess;
  const bool even = (s.D % BNC == 0) && (s.H % BK == 0);
  if (even)
    hipLaunchKernelGGL(grouped_down_kernel<true>, dim3(grid), dim3(NTHR), 0, stream,
                       expert_offset, h, w2, y_rows, s.D, s.H, s.n);
  else
    hipLaunchKernelGGL(grouped_down_kernel<false>, dim3(grid), dim3(NTHR), 0, stream,
                       expert_offset, h, w2, y_rows, s.D, s.H, s.n);
  return hipGetLastError();
}

}  // namespace moe
