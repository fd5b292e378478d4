// cu_issue_probe: a measurement program, not part of libmoe.
//
// Per-compute-unit issue costs that bound the ping-pong of the grouped expert
// products, measured with s_memtime inside one workgroup per compute unit
// (256 workgroups), every wave looping 2000 times over one instruction
// pattern:
//   mfma_dma  v_mfma_f32_32x32x16_bf16 with and without 1 KiB LDS-DMA loads
//             (buffer_load_dwordx4 ... lds, 16 bytes per lane) in the same
//             wave's stream: what a DMA costs the wave's products
//   lds_read  ds_read_b128 and the transposing ds_read_b64_tr_b16 from
//             conflict-free addresses, alone and with LDS-DMA writes beside
//             them: LDS read bytes per clock per compute unit
// Waves: 4 (one per SIMD) or 8 (two per SIMD, the products' occupancy).  DMA
// sources lie in a 1 MiB buffer (L2-resident), destinations in the wave's
// own LDS; every access is in range.  Prints one JSON line per case, with
// the cycles per loop iteration of the slowest wave.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#define CHECK(x)                                                                        \
  do {                                                                                  \
    hipError_t e_ = (x);                                                                \
    if (e_ != hipSuccess) {                                                             \
      fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
      exit(1);                                                                          \
    }                                                                                   \
  } while (0)

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

constexpr int kIters = 2000;
constexpr int kSrcBytes = 1 << 20;
constexpr int kWaveLds = 20 * 1024;  // 16 KiB read region + 4 KiB DMA region per wave

// vmcnt <= N, expcnt and lgkmcnt left at their maxima (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ void dma(__amdgpu_buffer_rsrc_t r, uint8_t* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lds_u8*)dst,
                                           16, voff, 0, 0, 0);
}

#define PIN __builtin_amdgcn_sched_barrier(0)

// Patterns per iteration (M = 4 products):
//   0: M M            1: M M D          2: M D M
//   3: D M M          4: D D            5: M D M D
template <int P, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void mfma_dma(const uint8_t* src, float* out,
                                                       unsigned long long* cyc) {
  __shared__ __attribute__((aligned(1024))) uint8_t sm[WAVES * 4096];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src), 0, kSrcBytes, 0x00020000);
  bf16x8 a, b;
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(0.01f * (lane + e));
    b[e] = static_cast<__bf16>(0.02f * (lane - e));
  }
  f32x16 acc[8];
  for (int i = 0; i < 8; ++i) acc[i] = f32x16{};
  uint8_t* base = sm + wave * 4096;
  const uint32_t voff = uint32_t(((blockIdx.x * WAVES + wave) * 1024 + lane * 16) % kSrcBytes);
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
#pragma unroll 1
  for (int it = 0; it < kIters; ++it) {
    uint8_t* d0 = base + (it & 3) * 1024;
    uint8_t* d1 = base + ((it + 2) & 3) * 1024;
    const uint32_t v0 = (voff + it * 65536u) % kSrcBytes;
    const uint32_t v1 = (voff + it * 65536u + 32768u) % kSrcBytes;
    PIN;
    if constexpr (P == 3) dma(r, d0, v0);
    if constexpr (P == 4) { dma(r, d0, v0); dma(r, d1, v1); }
    PIN;
    if constexpr (P != 4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
      PIN;
      if constexpr (P == 2 || P == 5) dma(r, d0, v0);
      PIN;
#pragma unroll
      for (int i = 4; i < 8; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
      PIN;
      if constexpr (P == 1) dma(r, d0, v0);
      if constexpr (P == 5) dma(r, d1, v1);
      PIN;
    }
    wait_vm<4>();  // at most 4 DMAs of this wave in flight
  }
  wait_vm<0>();
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  float s = 0.f;
  for (int i = 0; i < 8; ++i)
    for (int e = 0; e < 16; ++e) s += acc[i][e];
  __syncthreads();
  s += static_cast<float>(sm[(threadIdx.x * 37) % (WAVES * 4096)]);
  out[blockIdx.x * WAVES * 64 + threadIdx.x] = s;
  if (lane == 0) cyc[blockIdx.x * WAVES + wave] = t1 - t0;
}

// Patterns per iteration: 0: 8 x ds_read_b128 (8 KiB per wave);
// 1: 8 x ds_read_b64_tr_b16 (4 KiB); 2: pattern 0 plus one 1 KiB LDS-DMA.
template <int P, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void lds_read(const uint8_t* src, uint32_t* out,
                                                       unsigned long long* cyc) {
  __shared__ __attribute__((aligned(1024))) uint8_t sm[WAVES * kWaveLds];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < WAVES * kWaveLds / 4; i += WAVES * 64)
    reinterpret_cast<uint32_t*>(sm)[i] = i * 2654435761u;
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(src), 0, kSrcBytes, 0x00020000);
  uint8_t* wbase = sm + wave * kWaveLds;
  const uint32_t voff = uint32_t(((blockIdx.x * WAVES + wave) * 1024 + lane * 16) % kSrcBytes);
  __syncthreads();
  uint4 accv = make_uint4(0, 0, 0, 0);
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
#pragma unroll 1
  for (int it = 0; it < kIters; ++it) {
    if constexpr (P == 0 || P == 2) {
      uint4 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        v[i] = *reinterpret_cast<const uint4*>(wbase + ((i + it) & 15) * 1024 + lane * 16);
      if constexpr (P == 2) dma(r, wbase + 16384 + (it & 3) * 1024, (voff + it * 65536u) % kSrcBytes);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        accv.x ^= v[i].x; accv.y ^= v[i].y; accv.z ^= v[i].z; accv.w ^= v[i].w;
      }
      if constexpr (P == 2) wait_vm<4>();
    } else {
      v4i16 v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i)
        v[i] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16*)(lds_u8*)(wbase + ((i + it) & 15) * 1024 + lane * 8));
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        accv.x ^= uint32_t(uint16_t(v[i][0])) | (uint32_t(uint16_t(v[i][1])) << 16);
        accv.y ^= uint32_t(uint16_t(v[i][2])) | (uint32_t(uint16_t(v[i][3])) << 16);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0x7 << 4);  // vmcnt 0, lgkmcnt 0
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  out[blockIdx.x * WAVES * 64 + threadIdx.x] = accv.x ^ accv.y ^ accv.z ^ accv.w;
  if (lane == 0) cyc[blockIdx.x * WAVES + wave] = t1 - t0;
}

constexpr int kBlocks = 256;

double slowest_cycles_per_iter(const unsigned long long* d_cyc, int waves) {
  std::vector<unsigned long long> h(kBlocks * waves);
  CHECK(hipMemcpy(h.data(), d_cyc, h.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost));
  unsigned long long mx = 0;
  for (auto v : h) mx = v > mx ? v : mx;
  return double(mx) / kIters;
}

const char* kMfmaDmaNames[] = {"8 mfma", "8 mfma, dma", "4 mfma, dma, 4 mfma", "dma, 8 mfma",
                               "2 dma", "4 mfma, dma, 4 mfma, dma"};

template <int P, int WAVES>
void run_mfma_dma(const uint8_t* src, float* out, unsigned long long* cyc) {
  for (int rep = 0; rep < 2; ++rep) mfma_dma<P, WAVES><<<kBlocks, WAVES * 64>>>(src, out, cyc);
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  printf("{\"probe\": \"mfma_dma\", \"pattern\": \"%s\", \"waves\": %d, \"cycles_per_iter\": %.1f}\n",
         kMfmaDmaNames[P], WAVES, slowest_cycles_per_iter(cyc, WAVES));
}

const char* kLdsNames[] = {"8 ds_read_b128", "8 ds_read_b64_tr_b16", "8 ds_read_b128, dma"};

template <int P, int WAVES>
void run_lds(const uint8_t* src, uint32_t* out, unsigned long long* cyc) {
  for (int rep = 0; rep < 2; ++rep) lds_read<P, WAVES><<<kBlocks, WAVES * 64>>>(src, out, cyc);
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  const double c = slowest_cycles_per_iter(cyc, WAVES);
  const double bytes = (P == 1 ? 4096.0 : 8192.0) * WAVES;
  printf("{\"probe\": \"lds_read\", \"pattern\": \"%s\", \"waves\": %d, \"cycles_per_iter\": %.1f, "
         "\"read_bytes_per_clk_cu\": %.1f}\n", kLdsNames[P], WAVES, c, bytes / c);
}

}  // namespace

int main() {
  uint8_t* src;
  float* outf;
  uint32_t* outu;
  unsigned long long* cyc;
  CHECK(hipMalloc(&src, kSrcBytes));
  CHECK(hipMemset(src, 1, kSrcBytes));
  CHECK(hipMalloc(&outf, kBlocks * 8 * 64 * sizeof(float)));
  CHECK(hipMalloc(&outu, kBlocks * 8 * 64 * sizeof(uint32_t)));
  CHECK(hipMalloc(&cyc, kBlocks * 8 * sizeof(unsigned long long)));
  run_mfma_dma<0, 4>(src, outf, cyc); run_mfma_dma<1, 4>(src, outf, cyc);
  run_mfma_dma<2, 4>(src, outf, cyc); run_mfma_dma<3, 4>(src, outf, cyc);
  run_mfma_dma<4, 4>(src, outf, cyc); run_mfma_dma<5, 4>(src, outf, cyc);
  run_mfma_dma<0, 8>(src, outf, cyc); run_mfma_dma<1, 8>(src, outf, cyc);
  run_mfma_dma<2, 8>(src, outf, cyc); run_mfma_dma<4, 8>(src, outf, cyc);
  run_mfma_dma<5, 8>(src, outf, cyc);
  run_lds<0, 4>(src, outu, cyc); run_lds<1, 4>(src, outu, cyc); run_lds<2, 4>(src, outu, cyc);
  run_lds<0, 8>(src, outu, cyc); run_lds<1, 8>(src, outu, cyc); run_lds<2, 8>(src, outu, cyc);
  CHECK(hipFree(src));
  CHECK(hipFree(outf));
  CHECK(hipFree(outu));
  CHECK(hipFree(cyc));
  return 0;
}
