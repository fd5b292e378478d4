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
// 64-wide steps through two LDS stages of 64 KiB.  Each wave owns a 128 x 128
// sub-tile held as 4 x 4 accumulators of v_mfma_f32_32x32x16_bf16 (256 fp32
// per lane, in the accumulation registers).  In the up kernel the 256 columns
// are 128 columns of w1 and the same 128 columns of w3, so each wave holds a
// and b for identical (row, column) pairs and applies silu(a)*b in registers
// before a single bf16 rounding.
//
// Data path: both operands go from HBM straight into LDS with buffer loads in
// LDS-DMA mode (no staging registers, no LDS store instructions).  A DMA
// instruction writes 64 lanes x 16 bytes contiguously, so the LDS layout is
// chosen through the global address each lane fetches:
//  - activations (contraction-contiguous rows) land as 128-byte rows with the
//    16-byte chunk index XOR-swizzled by the row, and are read back as
//    128-bit fragments;
//  - weights are row-major with the OUTPUT axis contiguous ([D][H], [H][D]);
//    they land untransposed as 256-byte rows (64 contraction rows x 128
//    columns per sub-tile, chunks swizzled by the row), and the matrix-core
//    operand (8 consecutive contraction elements per lane) is formed by the
//    gfx950 transposing LDS read ds_read_b64_tr_b16: each 16-lane group reads
//    a 4 x 16 block and every lane receives 4 contraction elements of one
//    column.
// Rows of padding get an out-of-range buffer offset, which the hardware
// returns as zeros.  The weight fragments are the matrix core's "A" (row)
// side and the activations "B", so each lane's accumulator holds 4
// consecutive output columns of one token row: h is stored as 8-byte and y as
// 16-byte vectors.
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

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int BM = 256;          // rows (token-slots) per tile
constexpr int BK = 64;           // contraction step
constexpr int SUBN = 128;        // columns per weight sub-tile
constexpr int NTHR = 256;
constexpr int A_BYTES = BM * BK * 2;        // 32 KiB
constexpr int B_SUB_BYTES = BK * SUBN * 2;  // 16 KiB
constexpr int GROUP_M = 4;
constexpr uint32_t kOOB = 0x80000000u;      // buffer offset beyond any resource (< 2^31 bytes): reads as 0
constexpr int kRsrcWord3 = 0x00020000;      // raw buffer, 32-bit data (gfx9 family)

static_assert(BM == kTileM, "segment granule must equal the row tile");

// Two LDS stages as distinct objects, so the compiler can tell the DMA into
// one stage from the reads of the other.
__shared__ __attribute__((aligned(1024))) uint8_t g_a0[A_BYTES];
__shared__ __attribute__((aligned(1024))) uint8_t g_a1[A_BYTES];
__shared__ __attribute__((aligned(1024))) uint8_t g_b0[2 * B_SUB_BYTES];
__shared__ __attribute__((aligned(1024))) uint8_t g_b1[2 * B_SUB_BYTES];

__device__ __forceinline__ lds_u8* lds(uint8_t* p) { return (lds_u8*)(p); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), kRsrcWord3);
}

// 16 bytes per lane from buffer offset voff + soff into LDS at dst + 16 * lane.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, lds_u8* dst, uint32_t voff,
                                      uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16,
                                           voff, soff, 0, 0);
}

__device__ __forceinline__ bf16x8 lds_read128(const uint8_t* base, uint32_t off) {
  return as_bf16x8(*reinterpret_cast<const uint4*>(base + off));
}

// Weight fragment: two transposing 64-bit reads, 4 contraction rows apart.
__device__ __forceinline__ bf16x8 lds_read_wfrag(uint8_t* base, uint32_t off) {
  v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(lds(base) + off));
  v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(lds(base) + off + 4 * SUBN * 2));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  v8i16 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
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

// Per-lane state of one tile: DMA offsets and LDS read offsets.
struct TileCtx {
  __amdgpu_buffer_rsrc_t ra;      // activation rows
  __amdgpu_buffer_rsrc_t rb;      // this wave's weight sub-tile
  uint32_t a_voff[8];             // per DMA instruction (row), lane part
  uint32_t b_voff;                // lane part of the weight DMA offset
  uint32_t b_row_bytes;           // bytes per weight row (N * 2)
  int a_dst, b_dst;               // wave's LDS destination offsets within a stage
  uint32_t x_rd[4];               // activation fragment read offsets, per kk
  uint32_t w_rd[4];               // weight fragment read offsets, per fragment j
};

template <bool EVEN>
__device__ __forceinline__ void issue_stage(const TileCtx& c, uint8_t* sa, uint8_t* sb, int k0) {
#pragma unroll
  for (int i = 0; i < 8; ++i) dma16(c.ra, lds(sa) + c.a_dst + i * 8 * 128, c.a_voff[i], k0 * 2);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t rows = uint32_t(k0 + i * 4) * c.b_row_bytes;
    if (EVEN)
      dma16(c.rb, lds(sb) + c.b_dst + i * 4 * SUBN * 2, c.b_voff, rows);
    else
      dma16(c.rb, lds(sb) + c.b_dst + i * 4 * SUBN * 2, c.b_voff + rows, 0);
  }
}

__device__ __forceinline__ void read_frags(const TileCtx& c, uint8_t* sa, uint8_t* sb, int kk,
                                           bf16x8 (&xf)[4], bf16x8 (&wf)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) wf[j] = lds_read_wfrag(sb, c.w_rd[j] + kk * 16 * SUBN * 2);
#pragma unroll
  for (int i = 0; i < 4; ++i) xf[i] = lds_read128(sa, c.x_rd[kk] + i * 32 * 128);
}

__device__ __forceinline__ void mma16(const bf16x8 (&xf)[4], const bf16x8 (&wf)[4],
                                      f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[j], xf[i], acc[i][j], 0, 0, 0);
}

// One 64-deep stage: fragments of step kk+1 are read while the 16 products of
// step kk run; scheduling barriers keep the two register sets from merging.
__device__ __forceinline__ void compute_stage(const TileCtx& c, uint8_t* sa, uint8_t* sb,
                                              f32x16 (&acc)[4][4]) {
  bf16x8 x0[4], w0[4], x1[4], w1[4];
  read_frags(c, sa, sb, 0, x0, w0);
  __builtin_amdgcn_sched_barrier(0);
  read_frags(c, sa, sb, 1, x1, w1);
  mma16(x0, w0, acc);
  __builtin_amdgcn_sched_barrier(0);
  read_frags(c, sa, sb, 2, x0, w0);
  mma16(x1, w1, acc);
  __builtin_amdgcn_sched_barrier(0);
  read_frags(c, sa, sb, 3, x1, w1);
  mma16(x0, w0, acc);
  __builtin_amdgcn_sched_barrier(0);
  mma16(x1, w1, acc);
  __builtin_amdgcn_sched_barrier(0);
}

// Main loop over the contraction axis with two static LDS stages: the DMA of
// step k+1 runs while step k is multiplied out of the other stage.
template <bool EVEN>
__device__ __forceinline__ void run_tile(const TileCtx& c, int ksteps, f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  issue_stage<EVEN>(c, g_a0, g_b0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int ks = 0;
  for (; ks + 2 <= ksteps; ks += 2) {
    issue_stage<EVEN>(c, g_a1, g_b1, (ks + 1) * BK);
    compute_stage(c, g_a0, g_b0, acc);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (ks + 2 < ksteps) issue_stage<EVEN>(c, g_a0, g_b0, (ks + 2) * BK);
    compute_stage(c, g_a1, g_b1, acc);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (ks < ksteps) compute_stage(c, g_a0, g_b0, acc);  // odd number of steps
}

// Lane-dependent LDS offsets shared by both kernels.
//   sub[j], cb[j]: weight sub-tile and first column (within it) of fragment j
__device__ __forceinline__ void setup_reads(TileCtx& c, int lane, int wm, const int (&sub)[4],
                                            const int (&cb)[4]) {
  const int l32 = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int m = wm * 128 + l32;
    c.x_rd[kk] = uint32_t(m * 128 + (((2 * kk + hi) ^ (m & 7)) << 4));
  }
  const int g = lane >> 4, j16 = lane & 15;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int kr = 8 * (g >> 1) + (j16 >> 2);                    // contraction row in the step
    const int chunk = ((cb[j] >> 3) ^ ((j16 >> 2) << 2)) + 2 * (g & 1) + ((j16 & 3) >> 1);
    c.w_rd[j] = uint32_t(sub[j] * B_SUB_BYTES + kr * SUBN * 2 + chunk * 16 + (j16 & 1) * 8);
  }
}

// Lane part of the weight DMA: wave `wave` fills rows (wave&1)*32 .. +32 of
// sub-tile wave>>1; lane l covers row +l/16, physical chunk l%16.
__device__ __forceinline__ void setup_b_dma(TileCtx& c, int lane, int wave, int col0, int n_cols) {
  const int kr = (wave & 1) * 32 + (lane >> 4);
  const int lc = (lane & 15) ^ ((lane >> 4) << 2);
  c.b_row_bytes = uint32_t(n_cols) * 2;
  c.b_voff = uint32_t(kr) * c.b_row_bytes + uint32_t(col0 + lc * 8) * 2;
  c.b_dst = (wave >> 1) * B_SUB_BYTES + (wave & 1) * 32 * SUBN * 2;
}

// ---------------------------------------------------------------------------
// up: h = silu(x w1) * (x w3)
// ---------------------------------------------------------------------------
template <bool EVEN>
__global__ __launch_bounds__(NTHR, 1) void grouped_up_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ expert_offset,
    const int32_t* __restrict__ row_slot, const uint16_t* __restrict__ w1,
    const uint16_t* __restrict__ w3, uint16_t* __restrict__ h, int T, int D, int H, int n, int K) {
  const int mt_count = expert_offset[n] / BM;
  const int nt_count = (H + SUBN - 1) / SUBN;
  int mt, nt;
  if (!map_tile(blockIdx.x, mt_count, nt_count, mt, nt)) return;
  const int row0 = mt * BM;
  const int e = expert_of_row(expert_offset, n, row0);
  const int n0 = nt * SUBN;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  TileCtx c;
  c.ra = make_rsrc(x, uint32_t(T) * D * 2);
  const size_t wsz = size_t(D) * H;
  c.rb = make_rsrc(((wave >> 1) ? w3 : w1) + size_t(e) * wsz, uint32_t(wsz * 2));
  // activation DMA: instruction i covers rows wave*64 + i*8 .. +8; lane l
  // fetches row +l/8, logical chunk (l%8) ^ (row%8)
  const int lc = (lane & 7) ^ ((lane >> 3) & 7);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int slot = row_slot[row0 + wave * 64 + i * 8 + (lane >> 3)];
    const uint32_t tok = uint32_t(max(slot, 0)) / uint32_t(K);
    c.a_voff[i] = slot >= 0 ? tok * uint32_t(D) * 2 + lc * 16 : kOOB;
  }
  c.a_dst = wave * 64 * 128;
  setup_b_dma(c, lane, wave, n0, H);
  const int wm = wave >> 1, wn = wave & 1;
  const int sub[4] = {0, 0, 1, 1};
  const int cb[4] = {wn * 64, wn * 64 + 32, wn * 64, wn * 64 + 32};
  setup_reads(c, lane, wm, sub, cb);

  f32x16 acc[4][4];
  run_tile<EVEN>(c, (D + BK - 1) / BK, acc);

  // lane holds token row (wm*128 + 32 i + lane%32) and, per register quad q,
  // 4 consecutive columns starting at 8 q + 4 (lane/32)
  const int l32 = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = row0 + wm * 128 + i * 32 + l32;
    uint16_t* hrow = h + size_t(m) * H;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = n0 + wn * 64 + jj * 32 + q * 8 + hi * 4;
        if (!EVEN && col >= H) continue;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = silu(acc[i][jj][q * 4 + r]) * acc[i][jj + 2][q * 4 + r];
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
  const int mt_count = expert_offset[n] / BM;
  const int nt_count = (D + 2 * SUBN - 1) / (2 * SUBN);
  int mt, nt;
  if (!map_tile(blockIdx.x, mt_count, nt_count, mt, nt)) return;
  const int row0 = mt * BM;
  const int e = expert_of_row(expert_offset, n, row0);
  const int n0 = nt * 2 * SUBN;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  TileCtx c;
  c.ra = make_rsrc(h + size_t(row0) * H, uint32_t(BM) * H * 2);
  const size_t wsz = size_t(H) * D;
  c.rb = make_rsrc(w2 + size_t(e) * wsz, uint32_t(wsz * 2));
  const int lc = (lane & 7) ^ ((lane >> 3) & 7);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int m = wave * 64 + i * 8 + (lane >> 3);
    c.a_voff[i] = uint32_t(m) * uint32_t(H) * 2 + lc * 16;
  }
  c.a_dst = wave * 64 * 128;
  setup_b_dma(c, lane, wave, n0 + (wave >> 1) * SUBN, D);
  const int wm = wave >> 1, wn = wave & 1;
  const int sub[4] = {wn, wn, wn, wn};
  const int cb[4] = {0, 32, 64, 96};
  setup_reads(c, lane, wm, sub, cb);

  f32x16 acc[4][4];
  run_tile<EVEN>(c, (H + BK - 1) / BK, acc);

  const int l32 = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = row0 + wm * 128 + i * 32 + l32;
    float* yrow = y + size_t(m) * D;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = n0 + wn * SUBN + j * 32 + q * 8 + hi * 4;
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
  const int nt = (s.H + SUBN - 1) / SUBN;
  const int grid = mt_max * nt;
  if (grid == 0) return hipSuccess;
  const bool even = (s.H % SUBN == 0) && (s.D % BK == 0);
  if (even)
    hipLaunchKernelGGL(grouped_up_kernel<true>, dim3(grid), dim3(NTHR), 0, stream, x,
                       expert_offset, row_slot, w1, w3, h, s.T, s.D, s.H, s.n, s.K);
  else
    hipLaunchKernelGGL(grouped_up_kernel<false>, dim3(grid), dim3(NTHR), 0, stream, x,
                       expert_offset, row_slot, w1, w3, h, s.T, s.D, s.H, s.n, s.K);
  return hipGetLastError();
}

hipError_t launch_grouped_down(const Shape& s, const int32_t* expert_offset, const uint16_t* h,
                               const uint16_t* w2, float* y_rows, hipStream_t stream) {
  const int mt_max = int(s.cap / BM);
  const int nt = (s.D + 2 * SUBN - 1) / (2 * SUBN);
  const int grid = mt_max * nt;
  if (grid == 0) return hipSuccess;
  const bool even = (s.D % (2 * SUBN) == 0) && (s.H % BK == 0);
  if (even)
    hipLaunchKernelGGL(grouped_down_kernel<true>, dim3(grid), dim3(NTHR), 0, stream,
                       expert_offset, h, w2, y_rows, s.D, s.H, s.n);
  else
    hipLaunchKernelGGL(grouped_down_kernel<false>, dim3(grid), dim3(NTHR), 0, stream,
                       expert_offset, h, w2, y_rows, s.D, s.H, s.n);
  return hipGetLastError();
}

}  // namespace moe
