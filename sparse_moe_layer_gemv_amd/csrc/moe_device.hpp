// Device-side helpers shared by the libmoe kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// silu(z) = z * sigmoid(z) = z / (1 + e^-z); e^-z overflowing to +inf gives -0.
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// Transpose of an 8 x 8 block of bf16: in[j] holds row j (8 values, 16
// bytes); out[c] gets column c, that is element c of every row, row j at
// position j.  This turns 8 rows of a row-major [contraction][column] matrix
// into the 8-deep contraction fragments a matrix-core operand takes per lane.
__device__ __forceinline__ void transpose8x8_bf16(const uint4 (&in)[8], uint4 (&out)[8]) {
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

// ---------------------------------------------------------------------------
// Buffer resources and direct-to-LDS loads
// ---------------------------------------------------------------------------
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr uint32_t kOOB = 0x80000000u;  // buffer offset beyond any resource (< 2^31 bytes): reads as 0
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data (gfx9 family)

// s_waitcnt with the vector-memory counter limited to n and LDS operations
// drained (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4));
}

// s_waitcnt for this wave's LDS operations only (lgkmcnt 0; vmcnt and expcnt
// left at their maxima).  A barrier does not wait for issued LDS reads, so a
// stage must be drained this way before a barrier that lets other waves
// overwrite it.
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

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
// The range check applies to voff: an offset that must read as zero goes there.
// NT: non-temporal cache policy (data read once, not to be kept in the caches).
template <bool NT = false>
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, lds_u8* dst, uint32_t voff,
                                      uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16,
                                           voff, soff, 0, NT ? 2 : 0);
}

// Butterfly sum over the 64 lanes of a wavefront; every lane gets the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

}  // namespace moe
