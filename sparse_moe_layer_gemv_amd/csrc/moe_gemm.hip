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
// a contiguous range of tiles ordered expert by expert, with an expert's
// row-tiles consecutive, so the workgroups resident on one XCD share each
// weight panel and a few activation panels in its L2.
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {
namespace {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int BM = 256;          // rows (token-slots) per tile
constexpr int BK = 32;           // contraction depth of one pipeline step
constexpr int SUBN = 128;        // columns per weight sub-tile
constexpr int NTHR = 256;
// Activations are staged 2 steps (64 contraction elements, 128-byte rows) at a
// time so every DMA request is a full 128-byte line; weights one step at a
// time (their rows are already 256 bytes).
constexpr int A_BYTES = BM * 2 * BK * 2;    // 32 KiB: 256 rows of 128 bytes
constexpr int B_SUB_BYTES = BK * SUBN * 2;  // 8 KiB: 32 rows of 256 bytes
constexpr int B_BYTES = 2 * B_SUB_BYTES;    // 16 KiB: two sub-tiles
constexpr int NB = 4;                       // weight stages: DMA 3 steps ahead
constexpr int NA = 2;                       // activation stages (2 steps each)
constexpr int A_DMA = 8;                    // activation DMA instructions per wave per A stage
constexpr int B_DMA = 4;                    // weight DMA instructions per wave per step
constexpr uint32_t kOOB = 0x80000000u;      // buffer offset beyond any resource (< 2^31 bytes): reads as 0
constexpr int kRsrcWord3 = 0x00020000;      // raw buffer, 32-bit data (gfx9 family)

static_assert(BM == kTileM, "segment granule must equal the row tile");

// LDS stages as distinct objects, so the compiler can tell the DMA into one
// stage from the reads of another (128 KiB in total).
__shared__ __attribute__((aligned(1024))) uint8_t g_a0[A_BYTES];
__shared__ __attribute__((aligned(1024))) uint8_t g_a1[A_BYTES];
__shared__ __attribute__((aligned(1024))) uint8_t g_b0[B_BYTES];
__shared__ __attribute__((aligned(1024))) uint8_t g_b1[B_BYTES];
__shared__ __attribute__((aligned(1024))) uint8_t g_b2[B_BYTES];
__shared__ __attribute__((aligned(1024))) uint8_t g_b3[B_BYTES];

template <int S>
__device__ __forceinline__ uint8_t* a_stage() {
  static_assert(S >= 0 && S < NA, "stage index");
  if constexpr (S == 0) return g_a0;
  else return g_a1;
}
template <int S>
__device__ __forceinline__ uint8_t* b_stage() {
  static_assert(S >= 0 && S < NB, "stage index");
  if constexpr (S == 0) return g_b0;
  else if constexpr (S == 1) return g_b1;
  else if constexpr (S == 2) return g_b2;
  else return g_b3;
}

// s_waitcnt with the vector-memory counter limited to n and LDS operations
// drained (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4));
}

// Workgroup barrier without the memory fence of __syncthreads(): the fence
// would wait for every outstanding DMA, including the ones meant to stay in
// flight across the barrier.  Completion of the DMA that must be visible is
// waited for explicitly (wait_vmcnt) before this.
__device__ __forceinline__ void stage_barrier() { asm volatile("s_barrier" ::: "memory"); }

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
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds(base) + off));
  v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds(base) + off + 4 * SUBN * 2));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  v8i16 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// XCD-aware, expert-grouped tile mapping.  The hardware hands workgroup ids to
// the 8 XCDs round-robin (workgroup L runs on XCD L % 8) and each XCD has its
// own L2.  Valid workgroups (L < total tiles) are renumbered so that XCD x
// gets a contiguous range v of a linear tile order, and that order walks the
// experts one after the other; within an expert, column-tile by column-tile,
// with all of the expert's row-tiles consecutive.  So the workgroups resident
// on one XCD at a time work on one expert and share each weight panel (read
// once into that L2) and a few activation panels.
//   offset: segment starts (tile-aligned), n experts, nu: column units per row
//   tile.  Returns false for workgroups beyond the valid tiles.
__device__ __forceinline__ bool map_tile(int L, const int32_t* __restrict__ offset, int n,
                                         int nu, int& mt, int& unit) {
  const int mt_count = offset[n] / BM;
  const int total = mt_count * nu;
  if (L >= total) return false;
  const int xcd = L & 7;
  const int local = L >> 3;
  const int q = total >> 3, rem = total & 7;
  int v = xcd * q + min(xcd, rem) + local;
  // expert of linear tile v
  int e = 0, m0 = 0;
  for (; e < n; ++e) {
    const int me = (offset[e + 1] - offset[e]) / BM;
    if (v < me * nu) {
      mt = m0 + v % me;
      unit = v / me;
      return true;
    }
    v -= me * nu;
    m0 += me;
  }
  return false;  // not reached: v < total
}

// Expert owning permuted row `row0` (segments are tile-aligned).
__device__ __forceinline__ int expert_of_row(const int32_t* __restrict__ offset, int n, int row0) {
  int e = 0;
  while (e + 1 < n && offset[e + 1] <= row0) ++e;
  return e;
}

// Per-lane state of one tile: DMA offsets and LDS read offsets.
//
// LDS layouts:
//   activation stage: row m (128 bytes = 64 contraction elements), 16-byte
//     chunk c at m*128 + ((c ^ ((m >> 1) & 7)) << 4), so the 16 rows read by
//     one 16-lane group of a 128-bit fragment read hit 16 different bank groups;
//   weight stage: sub-tile s, contraction row k (256 bytes = 128 columns),
//     chunk c at s*B_SUB_BYTES + k*256 + ((c ^ ((k & 3) << 2)) << 4), so the
//     4 rows x 32 bytes of one transposing read hit distinct banks.
struct TileCtx {
  __amdgpu_buffer_rsrc_t ra;      // activation rows
  __amdgpu_buffer_rsrc_t rb;      // this wave's weight sub-tile
  uint32_t a_voff[A_DMA];         // per activation DMA instruction, lane part
  uint32_t b_voff;                // lane part of the weight DMA offset
  uint32_t b_row_bytes;           // bytes per weight row (N * 2)
  int a_dst, b_dst;               // wave's LDS destination offsets within a stage
  uint32_t x_rd[4];               // activation fragment read offsets, per 16-deep slice
  uint32_t w_rd[4];               // weight fragment read offsets, per fragment j
  int kbase;                      // first contraction element of this tile's range
};

// DMA of the activation rows for contraction elements [k0, k0 + 64);
// instructions [I0, I1) of the wave's A_DMA (the rows come in two halves).
template <int I0 = 0, int I1 = A_DMA>
__device__ __forceinline__ void issue_a(const TileCtx& c, uint8_t* st, int k0) {
#pragma unroll
  for (int i = I0; i < I1; ++i)
    dma16(c.ra, lds(st) + c.a_dst + i * 8 * 128, c.a_voff[i], uint32_t(c.kbase + k0) * 2);
}

// DMA of both weight sub-tiles for contraction rows [k0, k0 + 32).
template <bool EVEN>
__device__ __forceinline__ void issue_b(const TileCtx& c, uint8_t* st, int k0) {
#pragma unroll
  for (int i = 0; i < B_DMA; ++i) {
    const uint32_t rows = uint32_t(c.kbase + k0 + i * 4) * c.b_row_bytes;
    if (EVEN)
      dma16(c.rb, lds(st) + c.b_dst + i * 4 * SUBN * 2, c.b_voff, rows);
    else
      dma16(c.rb, lds(st) + c.b_dst + i * 4 * SUBN * 2, c.b_voff + rows, 0);
  }
}

// Matrix-core operands of one 16-deep slice: 4 activation fragments (rows) and
// 4 weight fragments (columns).
struct Frags {
  bf16x8 x[4], w[4];
};

// Fragments of 16-deep slice q (0..3) of activation stage sa and slice kk
// (0..1) of weight stage sb.
__device__ __forceinline__ void read_frags(const TileCtx& c, uint8_t* sa, uint8_t* sb, int q,
                                           int kk, Frags& f) {
#pragma unroll
  for (int j = 0; j < 4; ++j) f.w[j] = lds_read_wfrag(sb, c.w_rd[j] + kk * 16 * SUBN * 2);
#pragma unroll
  for (int i = 0; i < 4; ++i) f.x[i] = lds_read128(sa, c.x_rd[q] + i * 32 * 128);
}

__device__ __forceinline__ void mma16(const Frags& f, f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.w[j], f.x[i], acc[i][j], 0, 0, 0);
}

// One 32-deep step s out of activation stage SA (half H) and weight stage SB.
// On entry f0 holds the fragments of the step's first 16-slice; on exit (when
// not LAST) those of the next step's first slice.  The barrier sits between
// the two 16-slices:
//   1. (ISSUE_B) start the DMA of the weights of step s+3, read the second
//      slice's fragments, run the first slice's 16 products;
//   2. wait for this wave's LDS reads and for the loads of step s+1 (WAITN
//      loads may stay in flight), then barrier: every wave is done reading
//      this step's stages and step s+1 has landed everywhere;
//   3. (ISSUE_A) start the DMA of half of the activation rows of the stage
//      after next, read the next step's first-slice fragments, run the
//      second slice's 16 products.
// The DMA and LDS reads of each half are interleaved one by one with its
// products, so no step starts with an exposed LDS read and the wave never
// blocks on a burst of DMA issue.

// Scheduling groups: spread NV vector-memory (DMA) and ND LDS-read
// instructions evenly between the 16 matrix products of the current region,
// so neither a burst of DMA issue (which stalls the wave once the address
// queue is full) nor a burst of LDS reads holds back the matrix core.
template <int I, int NV, int ND>
__device__ __forceinline__ void interleave_from() {
  if constexpr (I < 16) {
    constexpr int kMfma = 0x008, kVmemRead = 0x020, kDsRead = 0x100;
    constexpr int dv = (NV + 15) / 16, dd = (ND + 15) / 16;
    constexpr int nv = (NV - I * dv) < dv ? (NV - I * dv) : dv;
    constexpr int nd = (ND - I * dd) < dd ? (ND - I * dd) : dd;
    __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
    if constexpr (nv > 0) __builtin_amdgcn_sched_group_barrier(kVmemRead, nv, 0);
    if constexpr (nd > 0) __builtin_amdgcn_sched_group_barrier(kDsRead, nd, 0);
    interleave_from<I + 1, NV, ND>();
  }
}
template <int NV, int ND>
__device__ __forceinline__ void interleave16() {
  interleave_from<0, NV, ND>();
}

template <bool EVEN, bool ISSUE_B, bool ISSUE_A, int WAITN, bool LAST, int SA, int H, int SB>
__device__ __forceinline__ void pipeline_step(const TileCtx& c, int s, Frags& f0,
                                              f32x16 (&acc)[4][4]) {
  constexpr int kFragReads = 12;  // 8 transposing + 4 128-bit reads per slice
  constexpr int kHalfA = A_DMA / 2;
  Frags f1;
  // first half: weights of step s+3 into the stage step s-1 used
  if (ISSUE_B) issue_b<EVEN>(c, b_stage<(SB + 3) % NB>(), (s + 3) * BK);
  read_frags(c, a_stage<SA>(), b_stage<SB>(), 2 * H + 1, 1, f1);
  mma16(f0, acc);
  interleave16<ISSUE_B ? B_DMA : 0, kFragReads>();
  __builtin_amdgcn_sched_barrier(0);
  if (!LAST) {
    wait_vmcnt<WAITN>();
    stage_barrier();
    // second half: half of the activation rows of the stage after next
    if (ISSUE_A) {
      if (H == 1)   // odd step 2t+1: first half of stage t+2, into this step's stage
        issue_a<0, kHalfA>(c, a_stage<SA>(), (s + 3) * BK);
      else          // even step 2t+2: second half of stage t+2, into the other stage
        issue_a<kHalfA, A_DMA>(c, a_stage<(SA + 1) % NA>(), (s + 2) * BK);
    }
    constexpr int SA_N = (H == 1) ? (SA + 1) % NA : SA;
    read_frags(c, a_stage<SA_N>(), b_stage<(SB + 1) % NB>(), 2 * (1 - H), 0, f0);
  }
  mma16(f1, acc);
  if (!LAST) interleave16<ISSUE_A ? kHalfA : 0, kFragReads>();
  __builtin_amdgcn_sched_barrier(0);
}

// Main loop over the contraction axis in 32-deep steps.  Step s reads weight
// stage s%4 and half s%2 of activation stage (s/2)%2.  Loads issued per wave,
// in order, four per half-step: in the first half of step s the weights of
// step s+3 (into the stage step s-1 used); in the second half of odd step
// 2t+1 the first half of activation stage t+2 (steps 2t+4, 2t+5, into the
// stage steps 2t, 2t+1 used) and in the second half of even step 2t+2 its
// second half.  Before the barrier of step s the data of step s+1 must have
// landed (vmcnt counts loads in issue order):
//   even s: weights s+1 -> in flight after it: 4 activation rows, weights
//           s+2, 4 activation rows, weights s+3 = 4 * 4 loads;
//   odd s:  the activation stage of step s+1, completed in the second half
//           of step s-1 -> in flight after it: weights s+3.
// The steady-state loop issues without branches: a branch around a DMA would
// hide from the compiler which stage is in flight and force a full wait
// before every LDS read.
template <bool EVEN>
__device__ __forceinline__ void run_tile_even(const TileCtx& c, int ksteps, f32x16 (&acc)[4][4]) {
  // ksteps is a multiple of 4, at least 8.  Prologue: the loads that steps
  // -3..-1 would have issued.
  constexpr int kHalfA = A_DMA / 2;
  issue_b<EVEN>(c, b_stage<0>(), 0);
  issue_a<0, kHalfA>(c, a_stage<0>(), 0);
  issue_b<EVEN>(c, b_stage<1>(), BK);
  issue_a<kHalfA, A_DMA>(c, a_stage<0>(), 0);
  issue_b<EVEN>(c, b_stage<2>(), 2 * BK);
  issue_a<0, kHalfA>(c, a_stage<1>(), 2 * BK);
  wait_vmcnt<B_DMA + kHalfA>();
  stage_barrier();
  Frags f0;
  read_frags(c, a_stage<0>(), b_stage<0>(), 0, 0, f0);
  constexpr int W_EVEN = 2 * B_DMA + 2 * kHalfA, W_ODD = B_DMA;
  int s = 0;
  for (; s + 8 <= ksteps; s += 4) {
    pipeline_step<EVEN, true, true, W_EVEN, false, 0, 0, 0>(c, s + 0, f0, acc);
    pipeline_step<EVEN, true, true, W_ODD, false, 0, 1, 1>(c, s + 1, f0, acc);
    pipeline_step<EVEN, true, true, W_EVEN, false, 1, 0, 2>(c, s + 2, f0, acc);
    pipeline_step<EVEN, true, true, W_ODD, false, 1, 1, 3>(c, s + 3, f0, acc);
  }
  // last 4 steps: only the weights of the final step and the second half of
  // the final activation stage remain to be fetched
  pipeline_step<EVEN, true, true, W_EVEN, false, 0, 0, 0>(c, s + 0, f0, acc);
  pipeline_step<EVEN, false, false, 0, false, 0, 1, 1>(c, s + 1, f0, acc);
  pipeline_step<EVEN, false, false, 0, false, 1, 0, 2>(c, s + 2, f0, acc);
  pipeline_step<EVEN, false, false, 0, true, 1, 1, 3>(c, s + 3, f0, acc);
}

// Any number of steps: the same stages with run-time guards and full waits.
template <bool EVEN, int SA, int H, int SB>
__device__ __forceinline__ void guarded_step(const TileCtx& c, int s, int ksteps,
                                             f32x16 (&acc)[4][4]) {
  if (s >= ksteps) return;
  Frags f0, f1;
  read_frags(c, a_stage<SA>(), b_stage<SB>(), 2 * H, 0, f0);
  read_frags(c, a_stage<SA>(), b_stage<SB>(), 2 * H + 1, 1, f1);
  mma16(f0, acc);
  mma16(f1, acc);
  wait_vmcnt<0>();
  stage_barrier();
  if (s + 4 < ksteps) issue_b<EVEN>(c, b_stage<SB>(), (s + 4) * BK);
  if (H == 1 && s + 3 < ksteps) issue_a(c, a_stage<SA>(), (s + 3) * BK);
}

template <bool EVEN>
__device__ __forceinline__ void run_tile_guarded(const TileCtx& c, int ksteps, f32x16 (&acc)[4][4]) {
  issue_b<EVEN>(c, b_stage<0>(), 0);
  if (1 < ksteps) issue_b<EVEN>(c, b_stage<1>(), BK);
  issue_a(c, a_stage<0>(), 0);
  if (2 < ksteps) issue_b<EVEN>(c, b_stage<2>(), 2 * BK);
  if (3 < ksteps) issue_b<EVEN>(c, b_stage<3>(), 3 * BK);
  if (2 < ksteps) issue_a(c, a_stage<1>(), 2 * BK);
  wait_vmcnt<0>();
  stage_barrier();
  for (int s = 0; s < ksteps; s += 4) {
    guarded_step<EVEN, 0, 0, 0>(c, s + 0, ksteps, acc);
    guarded_step<EVEN, 0, 1, 1>(c, s + 1, ksteps, acc);
    guarded_step<EVEN, 1, 0, 2>(c, s + 2, ksteps, acc);
    guarded_step<EVEN, 1, 1, 3>(c, s + 3, ksteps, acc);
  }
}

template <bool EVEN, bool GUARD>
__device__ __forceinline__ void run_tile(const TileCtx& c, int ksteps, f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  if (GUARD)
    run_tile_guarded<EVEN>(c, ksteps, acc);
  else
    run_tile_even<EVEN>(c, ksteps, acc);
}

// Lane-dependent LDS read offsets shared by both kernels.
//   sub[j], cb[j]: weight sub-tile and first column (within it) of fragment j
__device__ __forceinline__ void setup_reads(TileCtx& c, int lane, int wm, const int (&sub)[4],
                                            const int (&cb)[4]) {
  const int l32 = lane & 31, hi = lane >> 5;
  const int m = wm * 128 + l32;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    c.x_rd[q] = uint32_t(m * 128 + (((2 * q + hi) ^ ((m >> 1) & 7)) << 4));
  const int g = lane >> 4, j16 = lane & 15;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int kr = 8 * (g >> 1) + (j16 >> 2);                    // contraction row in the step
    const int chunk = ((cb[j] >> 3) ^ ((j16 >> 2) << 2)) + 2 * (g & 1) + ((j16 & 3) >> 1);
    c.w_rd[j] = uint32_t(sub[j] * B_SUB_BYTES + kr * SUBN * 2 + chunk * 16 + (j16 & 1) * 8);
  }
}

// Activation DMA: instruction i of wave w covers rows w*64 + i*8 .. +8; lane
// l fetches row +l/8, logical chunk (l%8) ^ ((row >> 1) & 7).
__device__ __forceinline__ int a_dma_row(int wave, int i, int lane) { return wave * 64 + i * 8 + (lane >> 3); }
__device__ __forceinline__ int a_dma_chunk(int i, int lane) { return (lane & 7) ^ ((i * 4 + (lane >> 4)) & 7); }

// Weight DMA: wave w fills rows (w&1)*16 .. +16 of sub-tile w>>1; instruction
// i covers 4 rows, lane l row +l/16 and physical chunk l%16.
__device__ __forceinline__ void setup_b_dma(TileCtx& c, int lane, int wave, int col0, int n_cols) {
  const int kr = (wave & 1) * 16 + (lane >> 4);
  const int lc = (lane & 15) ^ ((lane >> 4) << 2);
  c.b_row_bytes = uint32_t(n_cols) * 2;
  c.b_voff = uint32_t(kr) * c.b_row_bytes + uint32_t(col0 + lc * 8) * 2;
  c.b_dst = (wave >> 1) * B_SUB_BYTES + (wave & 1) * 16 * SUBN * 2;
}

// ---------------------------------------------------------------------------
// up: h = silu(x w1) * (x w3)
// ---------------------------------------------------------------------------
template <bool EVEN, bool KPOW2>
__global__ __launch_bounds__(NTHR, 1) void grouped_up_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ expert_offset,
    const int32_t* __restrict__ row_slot, const uint16_t* __restrict__ w1,
    const uint16_t* __restrict__ w3, uint16_t* __restrict__ h, int T, int D, int H, int n, int K,
    int k_shift) {
  const int nt_count = (H + SUBN - 1) / SUBN;
  int mt, nt;
  if (!map_tile(blockIdx.x, expert_offset, n, nt_count, mt, nt)) return;
  const int row0 = mt * BM;
  const int e = expert_of_row(expert_offset, n, row0);
  const int n0 = nt * SUBN;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  TileCtx c;
  c.kbase = 0;
  c.ra = make_rsrc(x, uint32_t(T) * D * 2);
  const size_t wsz = size_t(D) * H;
  c.rb = make_rsrc(((wave >> 1) ? w3 : w1) + size_t(e) * wsz, uint32_t(wsz * 2));
  // activation DMA: instruction i covers rows wave*64 + i*8 .. +8; lane l
  // fetches row +l/8, logical chunk (l%8) ^ (row%8)
  // all row_slot loads first, then the token arithmetic (a branch around a
  // division would serialise the loads)
  int slot[A_DMA];
#pragma unroll
  for (int i = 0; i < A_DMA; ++i) slot[i] = row_slot[row0 + a_dma_row(wave, i, lane)];
#pragma unroll
  for (int i = 0; i < A_DMA; ++i) {
    const uint32_t u = uint32_t(max(slot[i], 0));
    const uint32_t tok = KPOW2 ? (u >> k_shift) : u / uint32_t(K);
    const uint32_t off = tok * uint32_t(D) * 2 + a_dma_chunk(i, lane) * 16;
    c.a_voff[i] = slot[i] >= 0 ? off : kOOB;
  }
  c.a_dst = wave * 64 * 128;
  setup_b_dma(c, lane, wave, n0, H);
  const int wm = wave >> 1, wn = wave & 1;
  const int sub[4] = {0, 0, 1, 1};
  const int cb[4] = {wn * 64, wn * 64 + 32, wn * 64, wn * 64 + 32};
  setup_reads(c, lane, wm, sub, cb);

  f32x16 acc[4][4];
  run_tile<EVEN, !EVEN>(c, (D + BK - 1) / BK, acc);

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
// The contraction (H) can be split into `nsplit` ranges of `klen` elements;
// split ks writes its partial product to y + ks * split_stride, and the
// partials are added (in split order) by the consumer.  This evens out the
// last round of workgroups when the tile count is not a multiple of the CUs.
template <bool EVEN>
__global__ __launch_bounds__(NTHR, 1) void grouped_down_kernel(
    const int32_t* __restrict__ expert_offset, const uint16_t* __restrict__ h,
    const uint16_t* __restrict__ w2, float* __restrict__ y, int D, int H, int n, int nsplit,
    int klen, ptrdiff_t split_stride) {
  const int nt_count = (D + 2 * SUBN - 1) / (2 * SUBN);
  int mt, unit;
  if (!map_tile(blockIdx.x, expert_offset, n, nt_count * nsplit, mt, unit)) return;
  const int nt = unit / nsplit;
  const int ks = unit - nt * nsplit;
  const int row0 = mt * BM;
  const int e = expert_of_row(expert_offset, n, row0);
  const int n0 = nt * 2 * SUBN;
  y += ks * split_stride;  // may point into another allocation (the workspace)

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  TileCtx c;
  c.kbase = ks * klen;
  c.ra = make_rsrc(h + size_t(row0) * H, uint32_t(BM) * H * 2);
  const size_t wsz = size_t(H) * D;
  c.rb = make_rsrc(w2 + size_t(e) * wsz, uint32_t(wsz * 2));
#pragma unroll
  for (int i = 0; i < A_DMA; ++i)
    c.a_voff[i] = uint32_t(a_dma_row(wave, i, lane)) * uint32_t(H) * 2 + a_dma_chunk(i, lane) * 16;
  c.a_dst = wave * 64 * 128;
  setup_b_dma(c, lane, wave, n0 + (wave >> 1) * SUBN, D);
  const int wm = wave >> 1, wn = wave & 1;
  const int sub[4] = {wn, wn, wn, wn};
  const int cb[4] = {0, 32, 64, 96};
  setup_reads(c, lane, wm, sub, cb);

  f32x16 acc[4][4];
  run_tile<EVEN, !EVEN>(c, (min(klen, H - c.kbase) + BK - 1) / BK, acc);

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
  const bool even = (s.H % SUBN == 0) && (s.D % (4 * BK) == 0) && s.D >= 8 * BK;
  // slot -> token is a shift when K is a power of two
  const bool pow2 = (s.K & (s.K - 1)) == 0;
  const int k_shift = pow2 ? __builtin_ctz(unsigned(s.K)) : 0;
  auto kern = even ? (pow2 ? grouped_up_kernel<true, true> : grouped_up_kernel<true, false>)
                   : (pow2 ? grouped_up_kernel<false, true> : grouped_up_kernel<false, false>);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NTHR), 0, stream, x, expert_offset, row_slot, w1, w3,
                     h, s.T, s.D, s.H, s.n, s.K, k_shift);
  return hipGetLastError();
}

int grouped_down_splits(const Shape& s) {
  const int klen = s.H / 2;
  return (s.H % (2 * 4 * BK) == 0 && klen >= 8 * BK && s.D % (2 * SUBN) == 0) ? 2 : 1;
}

hipError_t launch_grouped_down(const Shape& s, const int32_t* expert_offset, const uint16_t* h,
                               const uint16_t* w2, float* y_rows, int nsplit, ptrdiff_t split_stride,
                               hipStream_t stream) {
  const int mt_max = int(s.cap / BM);
  const int nt = (s.D + 2 * SUBN - 1) / (2 * SUBN);
  const int grid = mt_max * nt * nsplit;
  if (grid == 0) return hipSuccess;
  const int klen = s.H / nsplit;
  const bool even = (s.D % (2 * SUBN) == 0) && (klen % (4 * BK) == 0) && klen >= 8 * BK &&
                    klen * nsplit == s.H;
  if (even)
    hipLaunchKernelGGL(grouped_down_kernel<true>, dim3(grid), dim3(NTHR), 0, stream,
                       expert_offset, h, w2, y_rows, s.D, s.H, s.n, nsplit, klen, split_stride);
  else
    hipLaunchKernelGGL(grouped_down_kernel<false>, dim3(grid), dim3(NTHR), 0, stream,
                       expert_offset, h, w2, y_rows, s.D, s.H, s.n, 1, s.H, split_stride);
  return hipGetLastError();
}

}  // namespace moe
