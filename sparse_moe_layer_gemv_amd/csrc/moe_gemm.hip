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
// Tiling (both kernels): a workgroup of 8 wavefronts owns a 256-row x
// 256-column output tile.  Waves 0-3 (group 0) own rows 0-127 and waves 4-7
// (group 1) rows 128-255; inside a group wave w owns 64 columns, held as 4 x 2
// accumulators of v_mfma_f32_32x32x16_bf16 (128 fp32 per lane).  In the up
// kernel the 256 columns are 128 columns of w1 and the same 128 columns of
// w3, so each wave holds a and b for identical (row, column) pairs and
// applies silu(a)*b in registers before a single bf16 rounding.
//
// Data path: both operands go from HBM straight into LDS with buffer loads in
// LDS-DMA mode (no staging registers, no LDS store instructions).  A DMA
// instruction writes 64 lanes x 16 bytes contiguously, so the LDS layout is
// chosen through the global address each lane fetches:
//  - activations (contraction-contiguous rows) land in blocks of 64
//    contraction elements as 128-byte rows (full cache lines) with the
//    16-byte chunk index XOR-swizzled by the row, and are read back as
//    128-bit fragments;
//  - weights are row-major with the OUTPUT axis contiguous ([D][H], [H][D]);
//    they land untransposed in stages of 32 contraction rows of 256 bytes
//    (128 columns per sub-tile, chunks swizzled by the row), and the
//    matrix-core operand (8 consecutive contraction elements per lane) is
//    formed by the gfx950 transposing LDS read ds_read_b64_tr_b16: each
//    16-lane group reads a 4 x 16 block and every lane receives 4 contraction
//    elements of one column.
// Rows of padding get an out-of-range buffer offset, which the hardware
// returns as zeros.  The weight fragments are the matrix core's "A" (row)
// side and the activations "B", so each lane's accumulator holds 4
// consecutive output columns of one token row: h is stored as 8-byte and y as
// 16-byte vectors.
//
// Schedule: a wave can issue one 1 KiB vector-memory instruction only every
// ~120 cycles and blocks meanwhile, so a wave that both feeds the matrix core
// and issues its own loads leaves the matrix core idle.  The two groups
// therefore alternate (one wave of each group shares a SIMD): in phase 2s
// group 0 runs the 16 products of 32-deep step s while group 1 reads its
// fragments of step s and issues its share of the loads 3-4 steps ahead; in
// phase 2s+1 the roles swap.  A barrier closes every phase, and the
// multiplying wave runs at raised priority.  LDS: 3 activation blocks of 32
// KiB and 4 weight stages of 16 KiB (160 KiB).
//
// Workgroup order: the hardware hands workgroup ids to the 8 XCDs round-robin,
// and each XCD has its own L2.  The block id is remapped so every XCD works on
// a contiguous range of tiles ordered expert by expert, with an expert's
// row-tiles consecutive, so the workgroups resident on one XCD share each
// weight panel and a few activation panels in its L2.
#include <algorithm>
#include <atomic>

#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace moe {
namespace {

constexpr int BM = 256;                       // rows (token-slots) per tile
constexpr int BK = 32;                        // contraction depth of one step
constexpr int SUBN = 128;                     // columns per weight sub-tile
constexpr int NWAVES = 8;
constexpr int NTHR = NWAVES * 64;
constexpr int FM = 4;                         // 32-row fragments per wave (128 rows)
constexpr int FN = 2;                         // 32-column fragments per wave (64 columns)
constexpr int A_ROW = 2 * BK * 2;             // 128 bytes: one activation row of a block (2 steps)
constexpr int A_BYTES = BM * A_ROW;           // 32 KiB per activation block
constexpr int B_SUB_BYTES = BK * SUBN * 2;    // 8 KiB: 32 rows of 256 bytes
constexpr int B_BYTES = 2 * B_SUB_BYTES;      // 16 KiB per weight stage
constexpr int NA = 3;                         // activation blocks (steps 2u, 2u+1 in block u % 3)
constexpr int NB = 4;                         // weight stages (step s in stage s % 4)
constexpr int A_DMA = A_BYTES / 1024 / NWAVES;  // 4 activation DMA instructions per wave per block
constexpr int B_DMA = B_BYTES / 1024 / NWAVES;  // 2 weight DMA instructions per wave per stage

static_assert(BM == kTileM, "segment granule must equal the row tile");
static_assert(A_DMA == 4 && B_DMA == 2, "DMA split assumes 4 + 2 instructions per wave");

// Row-tile classes.  A tile of class FMW has FMW 32-row fragments per wave and
// covers 64 FMW rows: 256 (FMW = 4, the full tile), 128 (2) or 64 (1); group g
// owns rows [32 FMW g, 32 FMW (g + 1)).  An expert with at most 128 slots (a
// small batch, or a lightly routed expert) is one tile of 128 or 64 rows: it
// multiplies 128 or 64 rows, not 256, and moves a half or a quarter of the
// activation bytes; its weight bytes and the pipeline are those of a full
// tile.  Larger experts keep full tiles, their last one padded: a tail tile
// run apart from its expert's full tiles (a launch of its own) fetched the
// expert's weight panels from HBM a second time instead of sharing them in L2
// with the full tiles, and made the skewed workload 8% slower.  The class is
// chosen per tile inside one persistent launch, in the tile order below.  The
// activation block of a class holds 64 FMW rows of 128 bytes, loaded by
// AW(FMW) waves, each AR(FMW) rows as AD(FMW) DMA instructions of 8 rows
// (1 KiB); with FMW = 1 only group 0 loads activations.
template <int FMW> constexpr int a_waves() { return FMW == 1 ? NWAVES / 2 : NWAVES; }
template <int FMW> constexpr int a_rows_per_wave() { return 64 * FMW / a_waves<FMW>(); }
// activation DMA instructions per block for a wave of group G
template <int FMW, int G> constexpr int a_dma() {
  return (FMW == 1 && G == 1) ? 0 : a_rows_per_wave<FMW>() / 8;
}
// loads one memory phase issues per wave of group G (weights + half an
// activation block)
template <int FMW, int G> constexpr int phase_loads() { return B_DMA + a_dma<FMW, G>() / 2; }
static_assert(a_dma<4, 0>() == A_DMA && a_dma<4, 1>() == A_DMA, "full tiles: 4 per wave");
static_assert(a_dma<2, 0>() == 2 && a_dma<2, 1>() == 2 && a_dma<1, 0>() == 2, "half, quarter tiles");
// runtime forms for a tile's class
__device__ __forceinline__ int a_rows_per_wave_rt(int fmw) { return fmw == 4 ? 32 : 16; }

// Class of the tiles of an expert with c slots (EVEN shapes; the ragged path
// runs full tiles only).
template <bool EVEN>
__device__ __forceinline__ int tile_fmw(int c) {
  if (!EVEN) return FM;
  return c <= 64 ? 1 : (c <= 128 ? 2 : 4);
}

// LDS blocks/stages as distinct objects, so the compiler can tell the DMA into
// one from the reads of another (160 KiB in total).
__shared__ __attribute__((aligned(1024))) uint8_t g_a0[A_BYTES];
__shared__ __attribute__((aligned(1024))) uint8_t g_a1[A_BYTES];
__shared__ __attribute__((aligned(1024))) uint8_t g_a2[A_BYTES];
__shared__ __attribute__((aligned(1024))) uint8_t g_b0[B_BYTES];
__shared__ __attribute__((aligned(1024))) uint8_t g_b1[B_BYTES];
__shared__ __attribute__((aligned(1024))) uint8_t g_b2[B_BYTES];
__shared__ __attribute__((aligned(1024))) uint8_t g_b3[B_BYTES];

template <int S>
__device__ __forceinline__ uint8_t* a_block() {
  static_assert(S >= 0 && S < NA, "block index");
  if constexpr (S == 0) return g_a0;
  else if constexpr (S == 1) return g_a1;
  else return g_a2;
}
template <int S>
__device__ __forceinline__ uint8_t* b_stage() {
  static_assert(S >= 0 && S < NB, "stage index");
  if constexpr (S == 0) return g_b0;
  else if constexpr (S == 1) return g_b1;
  else if constexpr (S == 2) return g_b2;
  else return g_b3;
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
// experts one after the other; within an expert, row block by row block, and
// within a block column-tile by column-tile with the block's row-tiles
// consecutive.  So the workgroups resident on one XCD at a time work on one
// expert and share each weight panel (read once into that L2) and a few
// activation panels.  An expert with fewer than 2 kRowBlock row tiles is one
// block; a larger one is cut into blocks of kRowBlock to 2 kRowBlock - 1 row
// tiles.  One XCD runs 32 tiles at a time, and with all of a large expert's
// row tiles side by side (32 of them for one expert of 8192 rows) its whole
// activation panel was fetched again for every column tile; with blocks, each
// weight panel is fetched once per block instead.
//   offset: segment starts (tile-aligned), n experts, nu: column units per row
//   tile.  Returns false for workgroups beyond the valid tiles.
// Expert e's tiles are v in [nu*offset[e]/BM, nu*offset[e+1]/BM), so the
// expert is the last e whose segment starts at or before v: a binary search
// over the monotone offsets (empty experts share their start with the next
// one, and the last of equal starts is the non-empty segment).  mt is the
// tile's row tile within its expert.
constexpr int kRowBlock = 8;  // row tiles per block of the tile order

__device__ __forceinline__ void decode_tile(int v, const int32_t* __restrict__ offset, int n,
                                            int nu, int& mt, int& unit, int& expert) {
  int lo = 0, hi = n - 1;  // invariant: the answer lies in [lo, hi]
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((offset[mid] / BM) * nu <= v) lo = mid; else hi = mid - 1;
  }
  const int m0 = offset[lo] / BM;
  const int me = offset[lo + 1] / BM - m0;
  const int vl = v - m0 * nu;
  if (me < 2 * kRowBlock) {  // one block
    mt = vl % me;
    unit = vl / me;
    expert = lo;
    return;
  }
  // nb = me / kRowBlock blocks of q or q + 1 row tiles, the first r of them
  // the larger; block b covers tiles [nu*start, nu*(start + size)) of the
  // expert, so vl / nu locates it
  const int nb = me / kRowBlock;
  const int q = me / nb, r = me - q * nb;
  const int rp = vl / nu;
  const int b = rp < r * (q + 1) ? rp / (q + 1) : r + (rp - r * (q + 1)) / q;
  const int start = b * q + min(b, r);
  const int size = q + (b < r ? 1 : 0);
  const int w = vl - nu * start;
  mt = start + w % size;
  unit = w / size;
  expert = lo;
}

__device__ __forceinline__ bool map_tile(int L, const int32_t* __restrict__ offset, int n,
                                         int nu, int& mt, int& unit, int& expert) {
  const int mt_count = offset[n] / BM;
  const int total = mt_count * nu;
  if (L >= total) return false;
  const int xcd = L & 7;
  const int local = L >> 3;
  const int q = total >> 3, rem = total & 7;
  decode_tile(xcd * q + min(xcd, rem) + local, offset, n, nu, mt, unit, expert);
  return true;
}

// Last-round split of the first product.  With few rows per expert a tile is
// bound by the weight bytes one compute unit can pull, so when the last round
// of tiles is at most half full (and at most kSplitMaxRounds full rounds come
// before it) its tiles run as two halves of the contraction each, on twice as
// many workgroups: every workgroup of that round streams half a panel.  A
// half writes its fp32 a and b to `part`, and up_split_fixup_kernel adds the
// two halves in order and forms h.  Tile t = R G + i of that round (R full
// rounds of G workgroups) is units R G + 2 i and R G + 2 i + 1.
constexpr int kSplitMaxRounds = 4;
constexpr size_t kSplitUnitFloats = size_t(BM) * 2 * SUBN;  // a and b of one tile

struct SplitPlan {
  int R, tail;
  bool on;
};
__device__ __forceinline__ SplitPlan split_plan(int total, int G, bool enabled) {
  SplitPlan p;
  p.R = total / G;
  p.tail = total - p.R * G;
  p.on = enabled && p.tail > 0 && 2 * p.tail <= G && p.R <= kSplitMaxRounds;
  return p;
}

// Per-lane state of one tile: DMA offsets and LDS read offsets.
//
// LDS layouts:
//   activation block: row m (128 bytes = 64 contraction elements), 16-byte
//     chunk c at m*128 + ((c ^ ((m >> 1) & 7)) << 4), so the 16 rows read by
//     one 16-lane group of a 128-bit fragment read hit 16 different bank
//     groups;
//   weight stage: sub-tile s, contraction row k (256 bytes = 128 columns),
//     chunk c at s*B_SUB_BYTES + k*256 + ((c ^ ((k & 3) << 2)) << 4), so the
//     4 rows x 32 bytes of one transposing read hit distinct banks.
struct TileCtx {
  __amdgpu_buffer_rsrc_t ra;      // activation rows
  __amdgpu_buffer_rsrc_t rb;      // this wave's weight sub-tile
  uint32_t a_voff[A_DMA];         // per activation DMA instruction, lane part
  uint32_t b_voff;                // lane part of the weight DMA offset
  uint32_t b_row_bytes;           // bytes per weight row (N * 2)
  int a_dst, b_dst;               // wave's LDS destination offsets within a block / stage
  uint32_t x_rd[4];               // activation fragment read offsets, per 16-deep slice of a block
  uint32_t w_rd[FN];              // weight fragment read offsets, per fragment j
  int kbase;                      // first contraction element of this tile's range
  int klast_b;                    // offset (from kbase) of the last 32-deep step
  int klast_a;                    // offset of the last 64-deep activation block
};

// DMA of activation instructions [I0, I1) of this wave for the block starting
// at contraction offset k0 (64 elements), and of this wave's 2 weight
// instructions for the step at k0 (32 rows).  With EVEN shapes every access is
// inside the operands and the contraction offset rides in the scalar offset;
// otherwise it goes into the range-checked vector offset, so weight rows past
// the contraction end read as zero (and activation columns past it meet those
// zero rows).
// past: the step lies beyond the contraction's end (a surplus load of the
// last steps, issued only to keep the number of loads in flight the same on
// every step): its offset is out of range, so the hardware returns zeros
// without a memory access, into a stage no wave reads.
template <bool EVEN, bool WNT, int I0, int I1>
__device__ __forceinline__ void issue_a(const TileCtx& c, uint8_t* blk, int k0, bool past = false) {
  const uint32_t kb = uint32_t(c.kbase + k0) * 2;
#pragma unroll
  for (int i = I0; i < I1; ++i) {
    const uint32_t voff = past ? kOOB : c.a_voff[i];
    if (EVEN)
      dma16(c.ra, lds(blk) + c.a_dst + i * 1024, voff, kb);
    else
      dma16(c.ra, lds(blk) + c.a_dst + i * 1024, voff + kb, 0);
  }
}
template <bool EVEN, bool WNT>
__device__ __forceinline__ void issue_b(const TileCtx& c, uint8_t* st, int k0, bool past = false) {
  const uint32_t voff = past ? kOOB : c.b_voff;
#pragma unroll
  for (int i = 0; i < B_DMA; ++i) {
    const uint32_t rows = uint32_t(c.kbase + k0 + i * 4) * c.b_row_bytes;
    if (EVEN)
      dma16<WNT>(c.rb, lds(st) + c.b_dst + i * 1024, voff, rows);
    else
      dma16<WNT>(c.rb, lds(st) + c.b_dst + i * 1024, voff + rows, 0);
  }
}

// Matrix-core operands of one 16-deep slice: FMW activation fragments (rows)
// and 2 weight fragments (columns).
template <int FMW>
struct Frags {
  bf16x8 x[FMW], w[FN];
};

// Slice q (0..3) of an activation block and slice kk (0..1) of a weight stage.
template <int FMW>
__device__ __forceinline__ void read_frags(const TileCtx& c, uint8_t* blk, uint8_t* st, int q,
                                           int kk, Frags<FMW>& f) {
#pragma unroll
  for (int j = 0; j < FN; ++j) f.w[j] = lds_read_wfrag(st, c.w_rd[j] + kk * 16 * SUBN * 2);
#pragma unroll
  for (int i = 0; i < FMW; ++i) f.x[i] = lds_read128(blk, c.x_rd[q] + i * 32 * A_ROW);
}

template <int FMW>
__device__ __forceinline__ void mma(const Frags<FMW>& f, f32x16 (&acc)[FM][FN]) {
#pragma unroll
  for (int i = 0; i < FMW; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.w[j], f.x[i], acc[i][j], 0, 0, 0);
}

// Compute phase: the 8 FMW products of one step, both slices' fragments read
// before (in the memory phase), so the matrix core runs them back to back.
template <int FMW>
__device__ __forceinline__ void compute_phase(const Frags<FMW>& f0, const Frags<FMW>& f1,
                                              f32x16 (&acc)[FM][FN]) {
  __builtin_amdgcn_s_setprio(1);
  mma(f0, acc);
  mma(f1, acc);
  __builtin_amdgcn_sched_barrier(0);
}

// Memory phase for step s (S = s % 12), wave group G:
//  - read both slices of step R (s for group 1, s + 1 for group 0) into f0, f1;
//  - issue the weights of step s + 3 and half of this wave's share of the
//    activation block of steps s + 4, s + 5 (even s) or s + 3, s + 4 (odd s).
// The reads are placed ahead of the DMA issue (which blocks the wave) so they
// complete meanwhile.  Loads of steps past the end are still issued, so the
// count of loads in flight is the same on every step (phase_loads<FMW, G>),
// but with an out-of-range offset: they read no memory and land (as zeros)
// in stages nobody reads.  Clamped to the last step instead, they fetched it
// again (from HBM where weights are loaded non-temporally): fine_prefill
// 0.947-0.950 -> 0.932-0.940 ms per step, prefill unchanged.
template <bool EVEN, bool WNT, int FMW, int G, int S, int R>
__device__ __forceinline__ void memory_phase(const TileCtx& c, int s, Frags<FMW>& f0,
                                             Frags<FMW>& f1) {
  constexpr int RB = R % NB, RA = (R / 2) % NA, RH = R & 1;
  constexpr int SB = (S + 3) % NB;            // stage of step s + 3
  constexpr int SA = (S / 2 + 2) % NA;        // block of steps 2(u+2), 2(u+2)+1, u = s / 2
  constexpr int AD = a_dma<FMW, G>(), HALF = AD / 2;
  __builtin_amdgcn_s_setprio(0);
  read_frags<FMW>(c, a_block<RA>(), b_stage<RB>(), 2 * RH, 0, f0);
  read_frags<FMW>(c, a_block<RA>(), b_stage<RB>(), 2 * RH + 1, 1, f1);
  __builtin_amdgcn_sched_barrier(0);
  issue_b<EVEN, WNT>(c, b_stage<SB>(), min((s + 3) * BK, c.klast_b), (s + 3) * BK > c.klast_b);
  if constexpr ((S & 1) == 0)
    issue_a<EVEN, WNT, 0, HALF>(c, a_block<SA>(), min((s + 4) * BK, c.klast_a),
                                (s + 4) * BK > c.klast_a);
  else
    issue_a<EVEN, WNT, HALF, AD>(c, a_block<SA>(), min((s + 3) * BK, c.klast_a),
                                 (s + 3) * BK > c.klast_a);
  __builtin_amdgcn_sched_barrier(0);
}

// One contraction step s (S = s % 12) for wave group G, in two phases.
//   group 0: compute(s) | wait | barrier | memory(read s+1) | barrier
//   group 1: memory(read s) | wait | barrier | compute(s) | barrier
// The wait at the end of the first phase makes this wave's loads of step s+1
// complete.  Every memory phase of a wave issues L = phase_loads<FMW, G>
// loads (4 in a full tile), counted in issue order, and the last ones step
// s+1 needs were issued in memory phase s-2, so group 0 (last memory phase
// s-1) may leave L in flight and group 1 (last memory phase s) 2 L.  After
// the barrier, step s+1 is visible to every wave.
template <bool EVEN, bool WNT, int FMW, int G, int S>
__device__ __forceinline__ void step(const TileCtx& c, int s, Frags<FMW>& f0, Frags<FMW>& f1,
                                     f32x16 (&acc)[FM][FN]) {
  constexpr int L = phase_loads<FMW, G>();
  if constexpr (G == 0) {
    compute_phase(f0, f1, acc);
    wait_vmcnt<L>();
    stage_barrier();
    memory_phase<EVEN, WNT, FMW, G, S, S + 1>(c, s, f0, f1);
    stage_barrier();
  } else {
    memory_phase<EVEN, WNT, FMW, G, S, S>(c, s, f0, f1);
    wait_vmcnt<2 * L>();
    stage_barrier();
    compute_phase(f0, f1, acc);
    stage_barrier();
  }
}

template <bool EVEN, bool WNT, int FMW, int G, int I>
__device__ __forceinline__ void tail_step(const TileCtx& c, int s0, int r, Frags<FMW>& f0,
                                          Frags<FMW>& f1, f32x16 (&acc)[FM][FN]) {
  if (r > I) step<EVEN, WNT, FMW, G, I>(c, s0 + I, f0, f1, acc);
}

// Phase of the ring schedule: step s of a tile runs as phase (s + SH) % 12,
// which fixes its weight stage (phase % 4) and activation block
// ((phase / 2) % 3).  With ksteps % 12 == 8 (the Mixtral contractions: 128
// steps, and 224 per half of the second product) the shift SH = 4 runs the
// first 8 steps as phases 4..11 in straight-line code, and the rest as whole
// 12-step rounds of the loop, so no step sits in the guarded tail (where the
// compiler waits for every load in flight before each step's reads).
constexpr int kShiftSteps = 4;
__device__ __forceinline__ bool phase_shifted(int ksteps) { return ksteps % 12 == 8; }

// Prologue of the ping-pong: every wave issues its share of the weights of
// steps 0..2 and of the activation blocks of steps 0..3 (phases SH ..
// SH + 3); memory phase s then issues step s + 3 onwards.  The LDS must be
// free (every wave past its last reads).
template <bool EVEN, bool WNT, int FMW, int G, int SH = 0>
__device__ __forceinline__ void pp_prologue(const TileCtx& c) {
  constexpr int AD = a_dma<FMW, G>();
  issue_b<EVEN, WNT>(c, b_stage<SH % NB>(), 0);
  issue_a<EVEN, WNT, 0, AD>(c, a_block<(SH / 2) % NA>(), 0);
  issue_b<EVEN, WNT>(c, b_stage<(SH + 1) % NB>(), BK);
  issue_b<EVEN, WNT>(c, b_stage<(SH + 2) % NB>(), 2 * BK);
  issue_a<EVEN, WNT, 0, AD>(c, a_block<(SH / 2 + 1) % NA>(), min(2 * BK, c.klast_a));
}

// Main loop over the contraction (ksteps even, >= 4 steps of 32), after
// pp_prologue.  A wave's loads (plain and direct-to-LDS) complete in issue
// order; LOADS_AFTER more loads were issued after the prologue's.  Stores may
// also be pending; they only make the count stricter, so the wait below holds
// whatever their order relative to the loads.
template <bool EVEN, bool WNT, int FMW, int G, int LOADS_AFTER, int SH = 0>
__device__ __forceinline__ void run_tile_pp_main(const TileCtx& c, int ksteps,
                                                 f32x16 (&acc)[FM][FN]) {
  static_assert(SH == 0 || SH == kShiftSteps, "two schedules");
  // weight step 0 and this wave's share of activation block 0 (the
  // prologue's first 2 + AD loads) landed
  wait_vmcnt<2 * B_DMA + a_dma<FMW, G>() + LOADS_AFTER>();
  stage_barrier();
  Frags<FMW> f0, f1;
  if (G == 0) {
    read_frags<FMW>(c, a_block<(SH / 2) % NA>(), b_stage<SH % NB>(), 0, 0, f0);
    read_frags<FMW>(c, a_block<(SH / 2) % NA>(), b_stage<SH % NB>(), 1, 1, f1);
  }
  int s = 0;
  if constexpr (SH == kShiftSteps) {  // steps 0..7 as phases 4..11 (ksteps % 12 == 8)
    step<EVEN, WNT, FMW, G, 4>(c, 0, f0, f1, acc);
    step<EVEN, WNT, FMW, G, 5>(c, 1, f0, f1, acc);
    step<EVEN, WNT, FMW, G, 6>(c, 2, f0, f1, acc);
    step<EVEN, WNT, FMW, G, 7>(c, 3, f0, f1, acc);
    step<EVEN, WNT, FMW, G, 8>(c, 4, f0, f1, acc);
    step<EVEN, WNT, FMW, G, 9>(c, 5, f0, f1, acc);
    step<EVEN, WNT, FMW, G, 10>(c, 6, f0, f1, acc);
    step<EVEN, WNT, FMW, G, 11>(c, 7, f0, f1, acc);
    s = 8;
  }
  for (; s + 12 <= ksteps; s += 12) {
    step<EVEN, WNT, FMW, G, 0>(c, s + 0, f0, f1, acc);
    step<EVEN, WNT, FMW, G, 1>(c, s + 1, f0, f1, acc);
    step<EVEN, WNT, FMW, G, 2>(c, s + 2, f0, f1, acc);
    step<EVEN, WNT, FMW, G, 3>(c, s + 3, f0, f1, acc);
    step<EVEN, WNT, FMW, G, 4>(c, s + 4, f0, f1, acc);
    step<EVEN, WNT, FMW, G, 5>(c, s + 5, f0, f1, acc);
    step<EVEN, WNT, FMW, G, 6>(c, s + 6, f0, f1, acc);
    step<EVEN, WNT, FMW, G, 7>(c, s + 7, f0, f1, acc);
    step<EVEN, WNT, FMW, G, 8>(c, s + 8, f0, f1, acc);
    step<EVEN, WNT, FMW, G, 9>(c, s + 9, f0, f1, acc);
    step<EVEN, WNT, FMW, G, 10>(c, s + 10, f0, f1, acc);
    step<EVEN, WNT, FMW, G, 11>(c, s + 11, f0, f1, acc);
  }
  // 0..11 remaining steps (none with the shifted schedule); s is a multiple
  // of 12, so their stage and block indices are those of steps 0..10
  if constexpr (SH == 0) {
    const int r = ksteps - s;
    tail_step<EVEN, WNT, FMW, G, 0>(c, s, r, f0, f1, acc);
    tail_step<EVEN, WNT, FMW, G, 1>(c, s, r, f0, f1, acc);
    tail_step<EVEN, WNT, FMW, G, 2>(c, s, r, f0, f1, acc);
    tail_step<EVEN, WNT, FMW, G, 3>(c, s, r, f0, f1, acc);
    tail_step<EVEN, WNT, FMW, G, 4>(c, s, r, f0, f1, acc);
    tail_step<EVEN, WNT, FMW, G, 5>(c, s, r, f0, f1, acc);
    tail_step<EVEN, WNT, FMW, G, 6>(c, s, r, f0, f1, acc);
    tail_step<EVEN, WNT, FMW, G, 7>(c, s, r, f0, f1, acc);
    tail_step<EVEN, WNT, FMW, G, 8>(c, s, r, f0, f1, acc);
    tail_step<EVEN, WNT, FMW, G, 9>(c, s, r, f0, f1, acc);
    tail_step<EVEN, WNT, FMW, G, 10>(c, s, r, f0, f1, acc);
  }
  // the surplus loads must land before the workgroup's LDS is released
  wait_vmcnt<0>();
}

template <bool EVEN, bool WNT, int FMW, int G>
__device__ __forceinline__ void run_tile_pp(const TileCtx& c, int ksteps,
                                            f32x16 (&acc)[FM][FN]) {
  if (phase_shifted(ksteps)) {
    pp_prologue<EVEN, WNT, FMW, G, kShiftSteps>(c);
    run_tile_pp_main<EVEN, WNT, FMW, G, 0, kShiftSteps>(c, ksteps, acc);
  } else {
    pp_prologue<EVEN, WNT, FMW, G>(c);
    run_tile_pp_main<EVEN, WNT, FMW, G, 0>(c, ksteps, acc);
  }
}

// Any number of steps (ragged shapes, full tiles only): one activation block
// and one weight stage per step pair, every wave loads and computes in the
// same phase, full waits.
template <bool EVEN, bool WNT>
__device__ __forceinline__ void run_tile_simple(const TileCtx& c, int ksteps, f32x16 (&acc)[FM][FN]) {
  for (int s = 0; s < ksteps; s += 2) {
    issue_a<EVEN, WNT, 0, A_DMA>(c, a_block<0>(), s * BK);
    issue_b<EVEN, WNT>(c, b_stage<0>(), s * BK);
    if (s + 1 < ksteps) issue_b<EVEN, WNT>(c, b_stage<1>(), (s + 1) * BK);
    wait_vmcnt<0>();
    stage_barrier();
    Frags<FM> f0, f1;
    read_frags<FM>(c, a_block<0>(), b_stage<0>(), 0, 0, f0);
    read_frags<FM>(c, a_block<0>(), b_stage<0>(), 1, 1, f1);
    mma(f0, acc);
    mma(f1, acc);
    if (s + 1 < ksteps) {
      read_frags<FM>(c, a_block<0>(), b_stage<1>(), 2, 0, f0);
      read_frags<FM>(c, a_block<0>(), b_stage<1>(), 3, 1, f1);
      mma(f0, acc);
      mma(f1, acc);
    }
    wait_vmcnt<0>();
    stage_barrier();
  }
}

template <bool EVEN, bool WNT, int FMW>
__device__ __forceinline__ void run_tile(const TileCtx& c, int ksteps, int group,
                                         f32x16 (&acc)[FM][FN]) {
#pragma unroll
  for (int i = 0; i < FMW; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};
  // the ragged path and the smaller row classes never meet: the launchers use
  // the classes only for EVEN shapes, which have at least the 4 steps (2
  // activation blocks) the ping-pong needs
  static_assert(EVEN || FMW == FM, "ragged shapes use full tiles");
  if constexpr (FMW == FM) {
    if (!EVEN || ksteps < 4) {
      run_tile_simple<EVEN, WNT>(c, ksteps, acc);
      return;
    }
  }
  if constexpr (EVEN) {
    if (group == 0)
      run_tile_pp<EVEN, WNT, FMW, 0>(c, ksteps, acc);
    else
      run_tile_pp<EVEN, WNT, FMW, 1>(c, ksteps, acc);
  }
}

// Lane-dependent LDS read offsets shared by both kernels.
//   fmw: the tile's class; wm: group (rows 32 fmw wm .. +32 fmw of the tile);
//   sub[j], cb[j]: weight sub-tile and first column (within it) of fragment j
__device__ __forceinline__ void setup_reads(TileCtx& c, int lane, int fmw, int wm,
                                            const int (&sub)[FN], const int (&cb)[FN]) {
  const int l32 = lane & 31, hi = lane >> 5;
  const int m = wm * 32 * fmw + l32;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    c.x_rd[q] = uint32_t(m * A_ROW + (((2 * q + hi) ^ ((m >> 1) & 7)) << 4));
  const int g = lane >> 4, j16 = lane & 15;
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int kr = 8 * (g >> 1) + (j16 >> 2);                    // contraction row in the slice
    const int chunk = ((cb[j] >> 3) ^ ((j16 >> 2) << 2)) + 2 * (g & 1) + ((j16 & 3) >> 1);
    c.w_rd[j] = uint32_t(sub[j] * B_SUB_BYTES + kr * SUBN * 2 + chunk * 16 + (j16 & 1) * 8);
  }
}

// Activation DMA: instruction i of wave w covers rows w*AR + i*8 .. +8 (AR =
// a_rows_per_wave: 32 in a full tile, 16 in the smaller classes); lane l
// fetches row +l/8 into physical chunk l%8, i.e. logical chunk
// (l%8) ^ ((row >> 1) & 7) = (l%8) ^ ((4 i + l/16) & 7), since AR/2 * w is a
// multiple of 8.
__device__ __forceinline__ int a_dma_row(int fmw, int wave, int i, int lane) {
  static_assert((a_rows_per_wave<4>() / 2) % 8 == 0 && (a_rows_per_wave<2>() / 2) % 8 == 0 &&
                    (a_rows_per_wave<1>() / 2) % 8 == 0,
                "swizzle independent of the wave");
  return wave * a_rows_per_wave_rt(fmw) + i * 8 + (lane >> 3);
}
__device__ __forceinline__ int a_dma_chunk(int i, int lane) { return (lane & 7) ^ ((i * 4 + (lane >> 4)) & 7); }

// Weight DMA: waves 0-3 fill sub-tile 0, waves 4-7 sub-tile 1; wave w fills
// rows (w%4)*8 .. +8 of its sub-tile; instruction i covers 4 rows, lane l
// row +l/16 and physical chunk l%16.
__device__ __forceinline__ int b_sub_of_wave(int wave) { return wave >> 2; }
__device__ __forceinline__ void setup_b_dma(TileCtx& c, int lane, int wave, int col0, int n_cols) {
  const int kr = (wave & 3) * 8 + (lane >> 4);
  const int lc = (lane & 15) ^ ((lane >> 4) << 2);
  c.b_row_bytes = uint32_t(n_cols) * 2;
  c.b_voff = uint32_t(kr) * c.b_row_bytes + uint32_t(col0 + lc * 8) * 2;
  c.b_dst = b_sub_of_wave(wave) * B_SUB_BYTES + (wave & 3) * 8 * SUBN * 2;
}

__device__ __forceinline__ void set_klast(TileCtx& c, int ksteps) {
  c.klast_b = (ksteps - 1) * BK;
  c.klast_a = ((ksteps - 1) & ~1) * BK;
}

// The first wait of a tile's main loop allows 4 + AD + LOADS_AFTER loads in
// flight (see run_tile_pp_main); the per-tile class makes the count a runtime
// value here, dispatched to the immediate each case needs.
template <bool EVEN, bool WNT, int G, int LOADS_AFTER>
__device__ __forceinline__ void run_class(const TileCtx& c, int fmw, int ksteps,
                                          f32x16 (&acc)[FM][FN]) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16{};
  const bool sh = phase_shifted(ksteps);  // as prologue_class chose for this tile
  if (fmw == 4) {
    if (sh) run_tile_pp_main<EVEN, WNT, 4, G, LOADS_AFTER, kShiftSteps>(c, ksteps, acc);
    else run_tile_pp_main<EVEN, WNT, 4, G, LOADS_AFTER>(c, ksteps, acc);
  } else if (fmw == 2) {
    if (sh) run_tile_pp_main<EVEN, WNT, 2, G, LOADS_AFTER, kShiftSteps>(c, ksteps, acc);
    else run_tile_pp_main<EVEN, WNT, 2, G, LOADS_AFTER>(c, ksteps, acc);
  } else {
    if (sh) run_tile_pp_main<EVEN, WNT, 1, G, LOADS_AFTER, kShiftSteps>(c, ksteps, acc);
    else run_tile_pp_main<EVEN, WNT, 1, G, LOADS_AFTER>(c, ksteps, acc);
  }
}

// ksteps: the tile's contraction steps, which choose its schedule (the main
// loop must be run with the same ksteps).
template <bool EVEN, bool WNT, int G>
__device__ __forceinline__ void prologue_class(const TileCtx& c, int fmw, int ksteps) {
  const bool sh = phase_shifted(ksteps);
  if (fmw == 4) {
    if (sh) pp_prologue<EVEN, WNT, 4, G, kShiftSteps>(c);
    else pp_prologue<EVEN, WNT, 4, G>(c);
  } else if (fmw == 2) {
    if (sh) pp_prologue<EVEN, WNT, 2, G, kShiftSteps>(c);
    else pp_prologue<EVEN, WNT, 2, G>(c);
  } else {
    if (sh) pp_prologue<EVEN, WNT, 1, G, kShiftSteps>(c);
    else pp_prologue<EVEN, WNT, 1, G>(c);
  }
}

// ---------------------------------------------------------------------------
// up: h = silu(x w1) * (x w3)
// ---------------------------------------------------------------------------
// The persistent loop of one wave of group G.
template <bool EVEN, bool WNT, bool KPOW2, int G>
__device__ __forceinline__ void up_tiles(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ expert_count,
    const int32_t* __restrict__ expert_offset, const int32_t* __restrict__ row_slot,
    const uint16_t* __restrict__ w1, const uint16_t* __restrict__ w3, uint16_t* __restrict__ h,
    float* __restrict__ part, int T, int D, int H, int n, int K, int k_shift) {
  const int nt_count = (H + SUBN - 1) / SUBN;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // wave (wm = G, wn): rows 32 fmw wm .. +32 fmw, columns wn*32 .. +32 of
  // both w1 (fragment 0) and w3 (fragment 1)
  const int wm = G, wn = wave & 3;
  const int sub[FN] = {0, 1};
  const int cb[FN] = {wn * 32, wn * 32};
  const int ksteps = (D + BK - 1) / BK;
  const size_t wsz = size_t(D) * H;

  // Row slots of a tile's activation rows: A_DMA per wave for every class
  // (the rows of the instructions a smaller class does not issue are other
  // rows of the expert's segment, in range and unused), so that the main
  // loop's first wait counts the same loads whatever the next tile's class.
  auto load_slots = [&](int (&sl)[A_DMA], int row0, int fmw) {
#pragma unroll
    for (int i = 0; i < A_DMA; ++i) sl[i] = row_slot[row0 + a_dma_row(fmw, wave, i, lane)];
  };

  // kp: -1 for a whole tile, else the contraction half it covers
  auto make_ctx = [&](int nt_, int e_, int fmw, const int (&sl)[A_DMA], int kp) {
    TileCtx c;
    c.kbase = kp < 0 ? 0 : kp * (ksteps / 2) * BK;
    c.ra = make_rsrc(x, uint32_t(T) * D * 2);
    c.rb = make_rsrc((b_sub_of_wave(wave) ? w3 : w1) + size_t(e_) * wsz, uint32_t(wsz * 2));
#pragma unroll
    for (int i = 0; i < A_DMA; ++i) {
      const uint32_t u = uint32_t(max(sl[i], 0));
      const uint32_t tok = KPOW2 ? (u >> k_shift) : u / uint32_t(K);
      const uint32_t off = tok * uint32_t(D) * 2 + a_dma_chunk(i, lane) * 16;
      c.a_voff[i] = sl[i] >= 0 ? off : kOOB;
    }
    c.a_dst = wave * a_rows_per_wave_rt(fmw) * A_ROW;
    setup_b_dma(c, lane, wave, nt_ * SUBN, H);
    setup_reads(c, lane, fmw, wm, sub, cb);
    set_klast(c, kp < 0 ? ksteps : ksteps / 2);
    return c;
  };

  // Epilogue: lane holds token row (32 FMW wm + 32 i + lane%32) and, per
  // register quad q, 4 consecutive columns starting at 8 q + 4 (lane/32).
  // Lanes l and l+32 hold the two halves of the same 8 columns; they swap one
  // half so that the lower lane writes quads 0 and 2 and the upper lane quads
  // 1 and 3, each as one 16-byte store.
  auto store_rows = [&](const f32x16 (&acc)[FM][FN], int i, int m, int n0) {
    const int hi = lane >> 5;
    uint16_t* hrow = h + size_t(m) * H;
    uint2 pk[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = silu(acc[i][0][q * 4 + r]) * acc[i][1][q * 4 + r];
      pk[q].x = pack_bf16x2(v[0], v[1]);
      pk[q].y = pack_bf16x2(v[2], v[3]);
    }
#pragma unroll
    for (int qq = 0; qq < 4; qq += 2) {
      const uint2 send = hi ? pk[qq] : pk[qq + 1];
      const uint2 mine = hi ? pk[qq + 1] : pk[qq];
      const uint32_t rx = __shfl_xor(send.x, 32, 64), ry = __shfl_xor(send.y, 32, 64);
      const int col = n0 + wn * 32 + (qq + hi) * 8;
      if (!EVEN && col >= H) continue;  // H is a multiple of 8: all 8 columns or none
      *reinterpret_cast<uint4*>(hrow + col) =
          hi ? make_uint4(rx, ry, mine.x, mine.y) : make_uint4(mine.x, mine.y, rx, ry);
    }
  };
  auto store_h = [&](const f32x16 (&acc)[FM][FN], int row0, int n0, int fmw) {
    const int l32 = lane & 31;
#pragma unroll
    for (int i = 0; i < FM; ++i)
      if (i < fmw) store_rows(acc, i, row0 + wm * 32 * fmw + i * 32 + l32, n0);
  };
  // A contraction half: fp32 a (columns 0..127) and b (128..255) of the
  // tile's rows, row-major, into unit u's slot of `part`.
  auto store_part = [&](const f32x16 (&acc)[FM][FN], int u, int fmw) {
    const int l32 = lane & 31, hi = lane >> 5;
    float* base = part + size_t(u) * kSplitUnitFloats;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (i >= fmw) continue;
      float* prow = base + size_t(wm * 32 * fmw + i * 32 + l32) * 2 * SUBN;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = wn * 32 + q * 8 + hi * 4;
        *reinterpret_cast<f32x4*>(prow + col) =
            f32x4{acc[i][0][q * 4], acc[i][0][q * 4 + 1], acc[i][0][q * 4 + 2], acc[i][0][q * 4 + 3]};
        *reinterpret_cast<f32x4*>(prow + SUBN + col) =
            f32x4{acc[i][1][q * 4], acc[i][1][q * 4 + 1], acc[i][1][q * 4 + 2], acc[i][1][q * 4 + 3]};
      }
    }
  };

  // Persistent: one workgroup per compute unit walks tiles L, L + G, ... (G a
  // multiple of 8, so L stays on its XCD and the XCD's tile order is
  // unchanged), without a workgroup launch between tiles.  The next tile's
  // mapping and row slots are read while this tile runs, and (EVEN shapes)
  // its prologue loads are issued before this tile's stores, so their latency
  // hides behind the epilogue.  Per tile the wave issues, in this order: the
  // row slots of the tile after next (A_DMA loads, always, so the first wait
  // of the main loop can count them), the main loop, then the next tile's
  // prologue and this tile's stores.
  // Work units: tiles, and with the last-round split (EVEN shapes, `part`
  // given) that round's tiles as two contraction halves each.
  const int total = (expert_offset[n] / BM) * nt_count;
  const SplitPlan sp = split_plan(total, gridDim.x, EVEN && part != nullptr);
  const int split0 = sp.R * int(gridDim.x);  // first unit of the split round
  const int units = sp.on ? split0 + 2 * sp.tail : total;
  auto map_unit = [&](int L_, int& mt_, int& nt_, int& e_, int& kp_) -> bool {
    if (L_ >= units) return false;
    kp_ = -1;
    int lt = L_;
    if (sp.on && L_ >= split0) {
      kp_ = (L_ - split0) & 1;
      lt = split0 + ((L_ - split0) >> 1);
    }
    return map_tile(lt, expert_offset, n, nt_count, mt_, nt_, e_);
  };

  int L = blockIdx.x;
  int mt, nt, e, kp;
  if (!map_unit(L, mt, nt, e, kp)) return;
  int fmw = tile_fmw<EVEN>(expert_count[e]);
  int row0 = expert_offset[e] + mt * BM;
  int slot[A_DMA];
  load_slots(slot, row0, fmw);
  TileCtx c = make_ctx(nt, e, fmw, slot, kp);
  if constexpr (EVEN) prologue_class<true, WNT, G>(c, fmw, kp < 0 ? ksteps : ksteps / 2);
  for (;;) {
    int mt2 = 0, nt2 = 0, e2 = 0, kp2 = -1;
    const bool more = map_unit(L + gridDim.x, mt2, nt2, e2, kp2);
    // a valid tile when there is no next one
    const int fmw2 = more ? tile_fmw<EVEN>(expert_count[e2]) : fmw;
    const int row0_next = more ? expert_offset[e2] + mt2 * BM : row0;
    asm volatile("" ::: "memory");
    load_slots(slot, row0_next, fmw2);
    asm volatile("" ::: "memory");

    f32x16 acc[FM][FN];
    if constexpr (EVEN) {
      run_class<true, WNT, G, A_DMA>(c, fmw, kp < 0 ? ksteps : ksteps / 2, acc);
    } else {
      run_tile<EVEN, WNT, FM>(c, ksteps, G, acc);
    }
    stage_barrier();  // every wave is past this tile's LDS use
    const int n0 = nt * SUBN;
    if (more) {
      c = make_ctx(nt2, e2, fmw2, slot, kp2);
      asm volatile("" ::: "memory");
      if constexpr (EVEN) prologue_class<true, WNT, G>(c, fmw2, kp2 < 0 ? ksteps : ksteps / 2);
      asm volatile("" ::: "memory");
    }
    if (kp < 0)
      store_h(acc, row0, n0, fmw);
    else
      store_part(acc, L - split0, fmw);
    if (!more) return;
    L += gridDim.x;
    row0 = row0_next;
    nt = nt2;
    fmw = fmw2;
    kp = kp2;
  }
}

// h for the tiles of a split last round: a = a0 + a1 and b = b0 + b1 from the
// two halves (in that order), h = bf16(silu(a) * b), for the tile's 64 FMW
// rows.  Workgroup i takes tile R G + i of that round; the plan is recomputed
// from the same offsets and grid size the first product used, and nothing
// runs when it did not split.
__global__ __launch_bounds__(256) void up_split_fixup_kernel(
    const int32_t* __restrict__ expert_count, const int32_t* __restrict__ expert_offset,
    const float* __restrict__ part, uint16_t* __restrict__ h, int H, int n, int G) {
  const int nt_count = H / SUBN;
  const SplitPlan sp = split_plan((expert_offset[n] / BM) * nt_count, G, true);
  const int i = blockIdx.x;
  if (!sp.on || i >= sp.tail) return;
  int mt, nt, e;
  if (!map_tile(sp.R * G + i, expert_offset, n, nt_count, mt, nt, e)) return;
  const int rows = 64 * tile_fmw<true>(expert_count[e]);
  const size_t row0 = size_t(expert_offset[e]) + size_t(mt) * BM;
  const int n0 = nt * SUBN;
  const float* p0 = part + size_t(2 * i) * kSplitUnitFloats;
  const float* p1 = p0 + kSplitUnitFloats;
  for (int q = threadIdx.x; q < rows * (SUBN / 8); q += 256) {
    const int r = q / (SUBN / 8), c8 = (q % (SUBN / 8)) * 8;
    const float* a0 = p0 + size_t(r) * 2 * SUBN + c8;
    const float* a1 = p1 + size_t(r) * 2 * SUBN + c8;
    float v[8];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const f32x4 x0 = *reinterpret_cast<const f32x4*>(a0 + 4 * half);
      const f32x4 x1 = *reinterpret_cast<const f32x4*>(a1 + 4 * half);
      const f32x4 y0 = *reinterpret_cast<const f32x4*>(a0 + SUBN + 4 * half);
      const f32x4 y1 = *reinterpret_cast<const f32x4*>(a1 + SUBN + 4 * half);
#pragma unroll
      for (int j = 0; j < 4; ++j) v[4 * half + j] = silu(x0[j] + x1[j]) * (y0[j] + y1[j]);
    }
    *reinterpret_cast<uint4*>(h + (row0 + r) * H + n0 + c8) =
        make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                   pack_bf16x2(v[6], v[7]));
  }
}

template <bool EVEN, bool WNT, bool KPOW2>
__global__ __launch_bounds__(NTHR, 1) void grouped_up_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ expert_count,
    const int32_t* __restrict__ expert_offset, const int32_t* __restrict__ row_slot,
    const uint16_t* __restrict__ w1, const uint16_t* __restrict__ w3, uint16_t* __restrict__ h,
    float* __restrict__ part, int T, int D, int H, int n, int K, int k_shift) {
  // the wave's group is fixed for the whole launch: waves 0-3 own the first
  // half of every tile's rows, waves 4-7 the rest
  if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) < 4)
    up_tiles<EVEN, WNT, KPOW2, 0>(x, expert_count, expert_offset, row_slot, w1, w3, h, part, T,
                                  D, H, n, K, k_shift);
  else
    up_tiles<EVEN, WNT, KPOW2, 1>(x, expert_count, expert_offset, row_slot, w1, w3, h, part, T,
                                  D, H, n, K, k_shift);
}

// ---------------------------------------------------------------------------
// down: y = h w2
// ---------------------------------------------------------------------------
// One tile of class FMW for wave group G: 64 FMW rows from row0 of expert e,
// 256 output columns from n0, over the contraction range [kbase, kbase + 32 *
// ksteps), stored to y for the rows that hold slots (rows past the expert's
// slots are padding: nothing reads them, so they are not written).
template <bool EVEN, bool WNT, int FMW, int G>
__device__ __forceinline__ void down_tile(const int32_t* __restrict__ expert_count,
                                          const int32_t* __restrict__ expert_offset,
                                          const uint16_t* __restrict__ h,
                                          const uint16_t* __restrict__ w2, float* y,
                                          int D, int H, int row0, int n0, int e, int kbase,
                                          int ksteps) {
  constexpr int AD = a_dma<FMW, G>();
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  TileCtx c;
  c.kbase = kbase;
  c.ra = make_rsrc(h + size_t(row0) * H, uint32_t(64 * FMW) * H * 2);
  const size_t wsz = size_t(H) * D;
  c.rb = make_rsrc(w2 + size_t(e) * wsz, uint32_t(wsz * 2));
#pragma unroll
  for (int i = 0; i < AD; ++i)
    c.a_voff[i] = uint32_t(a_dma_row(FMW, wave, i, lane)) * uint32_t(H) * 2 +
                  a_dma_chunk(i, lane) * 16;
  c.a_dst = wave * a_rows_per_wave<FMW>() * A_ROW;
  setup_b_dma(c, lane, wave, n0 + b_sub_of_wave(wave) * SUBN, D);
  // wave (wm = G, wn): rows 32 FMW wm .. +32 FMW, columns wn*64 .. +64 of the
  // 256-column tile (sub-tile wn/2)
  const int wm = G, wn = wave & 3;
  const int sub[FN] = {wn >> 1, wn >> 1};
  const int cb[FN] = {(wn & 1) * 64, (wn & 1) * 64 + 32};
  setup_reads(c, lane, FMW, wm, sub, cb);

  f32x16 acc[FM][FN];
  set_klast(c, ksteps);
  run_tile<EVEN, WNT, FMW>(c, ksteps, wm, acc);

  const int rend = expert_offset[e] + expert_count[e];
  const int l32 = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int i = 0; i < FMW; ++i) {
    const int m = row0 + wm * 32 * FMW + i * 32 + l32;
    if (m >= rend) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = n0 + wn * 64 + j * 32 + q * 8 + hi * 4;
        if (!EVEN && col >= D) continue;
        f32x4 v = {acc[i][j][q * 4 + 0], acc[i][j][q * 4 + 1], acc[i][j][q * 4 + 2],
                   acc[i][j][q * 4 + 3]};
        *reinterpret_cast<f32x4*>(y + size_t(m) * D + col) = v;
      }
    }
  }
}

// The contraction (H) can be split into `nsplit` (1 or 2) ranges of `klen`
// elements; range 0 writes its partial product to y and range 1 to y_part
// (which may lie in another allocation), and the consumer adds the two.
template <bool EVEN, bool WNT, int G>
__device__ __forceinline__ void down_tiles(
    const int32_t* __restrict__ expert_count, const int32_t* __restrict__ expert_offset,
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ w2, float* __restrict__ y,
    int D, int H, int n, int nsplit, int klen, float* __restrict__ y_part) {
  const int nt_count = (D + 2 * SUBN - 1) / (2 * SUBN);
  // persistent, as the first product: tiles L, L + G, ... of this XCD, the
  // next tile's mapping read while the current one runs
  int L = blockIdx.x;
  int mt, unit, e;
  if (!map_tile(L, expert_offset, n, nt_count * nsplit, mt, unit, e)) return;
  for (;;) {
    int mt2 = 0, unit2 = 0, e2 = 0;
    const bool more = map_tile(L + gridDim.x, expert_offset, n, nt_count * nsplit, mt2, unit2, e2);
    // Units run contraction range by contraction range: the workgroups that
    // one XCD runs together (several units x all row-tiles of an expert) then
    // work on the same h columns for different output columns and share each
    // h slice in L2.  With column-tile-major units they straddled both ranges,
    // and the h re-fetches doubled.
    const int ks = unit / nt_count;
    const int nt = unit - ks * nt_count;
    const int kbase = ks * klen;
    const int ksteps = (min(klen, H - kbase) + BK - 1) / BK;
    const int row0 = expert_offset[e] + mt * BM;
    float* out = ks == 0 ? y : y_part;
    const int fmw = tile_fmw<EVEN>(expert_count[e]);
    if (fmw == 4 || !EVEN)
      down_tile<EVEN, WNT, FM, G>(expert_count, expert_offset, h, w2, out, D, H, row0,
                                  nt * 2 * SUBN, e, kbase, ksteps);
    else if constexpr (EVEN) {
      if (fmw == 2)
        down_tile<EVEN, WNT, 2, G>(expert_count, expert_offset, h, w2, out, D, H, row0,
                                   nt * 2 * SUBN, e, kbase, ksteps);
      else
        down_tile<EVEN, WNT, 1, G>(expert_count, expert_offset, h, w2, out, D, H, row0,
                                   nt * 2 * SUBN, e, kbase, ksteps);
    }
    stage_barrier();  // every wave is past this tile's LDS use before the next tile's loads
    if (!more) return;
    L += gridDim.x;
    mt = mt2;
    unit = unit2;
    e = e2;
  }
}

template <bool EVEN, bool WNT>
__global__ __launch_bounds__(NTHR, 1) void grouped_down_kernel(
    const int32_t* __restrict__ expert_count, const int32_t* __restrict__ expert_offset,
    const uint16_t* __restrict__ h, const uint16_t* __restrict__ w2, float* __restrict__ y,
    int D, int H, int n, int nsplit, int klen, float* __restrict__ y_part) {
  if (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6) < 4)
    down_tiles<EVEN, WNT, 0>(expert_count, expert_offset, h, w2, y, D, H, n, nsplit, klen, y_part);
  else
    down_tiles<EVEN, WNT, 1>(expert_count, expert_offset, h, w2, y, D, H, n, nsplit, klen, y_part);
}


// One workgroup per compute unit (a multiple of 8, so that tile L + G stays
// on the XCD of tile L); read once per device (devices 0..63; any further
// device is queried on every call).  Host threads may race here; they all
// store the same value.
int persistent_workgroups() {
  constexpr int kCachedDevices = 64;
  static std::atomic<int> cached[kCachedDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  const bool cacheable = dev < kCachedDevices;
  int g = cacheable ? cached[dev].load(std::memory_order_relaxed) : 0;
  if (g == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 8)
      cus = 256;
    g = cus / 8 * 8;
    if (cacheable) cached[dev].store(g, std::memory_order_relaxed);
  }
  return g;
}

// Weight panels: a panel serves every row tile of its expert, and the
// workgroups of one XCD run an expert's row tiles together, so with several
// row tiles per expert it is read once into L2 and shared.  With about one
// row tile per expert (many small experts: ~205 rows each at 160 experts,
// top-8) nothing shares it, and it is loaded non-temporally, so it does not
// displace the activations that are shared.  Measured: fine_prefill
// 0.970 -> 0.931 ms per step; at Mixtral prefill (~4.5 row tiles per expert)
// the non-temporal form was 4% slower.
bool weights_streamed(const Shape& s) {
  return int64_t(s.T) * s.K <= int64_t(s.n) * BM;
}

}  // namespace

// The last-round split (see SplitPlan) is for shapes of at most 128 slots per
// expert on average, where a tile is bound by its weight bytes, and whose
// contraction halves keep the ping-pong's even step count of at least 4.
namespace {
constexpr int kSplitMaxUnits = 256;  // scratch slots: one per workgroup of the round
bool split_eligible(const Shape& s) {
  const int ksteps = s.D / BK;
  return s.H % SUBN == 0 && s.D % (2 * BK) == 0 && ksteps % 4 == 0 && ksteps >= 8 &&
         int64_t(s.T) * s.K <= int64_t(128) * s.n;
}
}  // namespace

size_t grouped_up_scratch_bytes(const Shape& s) {
  return split_eligible(s) ? size_t(kSplitMaxUnits) * kSplitUnitFloats * sizeof(float) : 0;
}

hipError_t launch_grouped_up(const Shape& s, const uint16_t* x, const int32_t* expert_count,
                             const int32_t* expert_offset, const int32_t* row_slot,
                             const uint16_t* w1, const uint16_t* w3, uint16_t* h, void* scratch,
                             size_t scratch_bytes, hipStream_t stream) {
  const int mt_max = int(s.cap / BM);
  const int nt = (s.H + SUBN - 1) / SUBN;
  if (mt_max * nt == 0) return hipSuccess;
  const int grid = std::min(mt_max * nt, persistent_workgroups());
  const bool even = (s.H % SUBN == 0) && (s.D % (2 * BK) == 0) && s.D >= 4 * BK;
  // the last-round split when the scratch holds a slot per workgroup
  const size_t part_need = size_t(grid) * kSplitUnitFloats * sizeof(float);
  float* part = split_eligible(s) && scratch && scratch_bytes >= part_need
                    ? static_cast<float*>(scratch)
                    : nullptr;
  // slot -> token is a shift when K is a power of two
  const bool pow2 = (s.K & (s.K - 1)) == 0;
  const int k_shift = pow2 ? __builtin_ctz(unsigned(s.K)) : 0;
  const bool wnt = weights_streamed(s);
  auto kern = even ? (wnt ? (pow2 ? grouped_up_kernel<true, true, true>
                                  : grouped_up_kernel<true, true, false>)
                          : (pow2 ? grouped_up_kernel<true, false, true>
                                  : grouped_up_kernel<true, false, false>))
                   : (wnt ? (pow2 ? grouped_up_kernel<false, true, true>
                                  : grouped_up_kernel<false, true, false>)
                          : (pow2 ? grouped_up_kernel<false, false, true>
                                  : grouped_up_kernel<false, false, false>));
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NTHR), 0, stream, x, expert_count, expert_offset,
                     row_slot, w1, w3, h, part, s.T, s.D, s.H, s.n, s.K, k_shift);
  if (part) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // at most half a round of tiles is split
    hipLaunchKernelGGL(up_split_fixup_kernel, dim3(grid / 2 > 0 ? grid / 2 : 1), dim3(256), 0,
                       stream, expert_count, expert_offset, part, h, s.H, s.n, grid);
  }
  return hipGetLastError();
}

// Splitting the second product's contraction in two doubles its tiles (for
// few, large experts there are otherwise too few to fill the chip) but also
// doubles the fp32 rows written here and read back by the combine.  So split
// only when the expected tile count is low: rows ~ T*K plus half a padding
// tile per expert, over the D / 128 column tiles.
int grouped_down_splits(const Shape& s) {
  const int klen = s.H / 2;
  if (!(s.H % (4 * BK) == 0 && klen >= 8 * BK && s.D % (2 * SUBN) == 0)) return 1;
  const int64_t est_rows = int64_t(s.T) * s.K + int64_t(s.n) * BM / 2;
  const int64_t est_tiles = (est_rows / BM) * (s.D / SUBN);
  return est_tiles < 4096 ? 2 : 1;
}

hipError_t launch_grouped_down(const Shape& s, const int32_t* expert_count,
                               const int32_t* expert_offset, const uint16_t* h,
                               const uint16_t* w2, float* y_rows, int nsplit, float* y_part,
                               hipStream_t stream) {
  if (nsplit < 1 || nsplit > 2 || (nsplit == 2 && !y_part)) return hipErrorInvalidValue;
  const int mt_max = int(s.cap / BM);
  const int nt = (s.D + 2 * SUBN - 1) / (2 * SUBN);
  if (mt_max * nt * nsplit == 0) return hipSuccess;
  const int grid = std::min(mt_max * nt * nsplit, persistent_workgroups());
  const int klen = s.H / nsplit;
  const bool even = (s.D % (2 * SUBN) == 0) && (klen % (2 * BK) == 0) && klen >= 4 * BK &&
                    klen * nsplit == s.H;
  const bool wnt = weights_streamed(s);
  if (even) {
    auto kern = wnt ? grouped_down_kernel<true, true> : grouped_down_kernel<true, false>;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(NTHR), 0, stream, expert_count, expert_offset, h,
                       w2, y_rows, s.D, s.H, s.n, nsplit, klen, y_part);
  } else {
    // the ragged kernel runs the whole contraction: only one partial
    // (grouped_down_splits never splits such shapes)
    if (nsplit != 1) return hipErrorInvalidValue;
    auto kern = wnt ? grouped_down_kernel<false, true> : grouped_down_kernel<false, false>;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(NTHR), 0, stream, expert_count, expert_offset, h,
                       w2, y_rows, s.D, s.H, s.n, 1, s.H, y_part);
  }
  return hipGetLastError();
}

}  // namespace moe
