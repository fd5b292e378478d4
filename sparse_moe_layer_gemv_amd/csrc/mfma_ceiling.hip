// mfma_ceiling: a measurement program, not part of libmoe.
//
// Sustained rate of v_mfma_f32_32x32x16_bf16 over the whole chip with the
// operands held in registers: no memory traffic inside the timed loop.  One
// workgroup of 8 waves per compute unit (2 per SIMD) and 8 accumulator tiles
// of 32x32 per wave, the occupancy and accumulator count of the grouped
// expert products.  The operands rotate over 4 register sets of random bf16
// values in [-1, 1), so the multipliers see changing data every instruction;
// with `zero` set they are all zero.  Under the board's power limit the
// clock, and so the rate, depends on that data: this gives the ceiling that
// a bf16 product on random data can reach on this chip, next to the
// 2.5 PFLOP/s dense peak at the 2.4 GHz top clock.
//
//   mfma_ceiling [blocks=256] [iters=1500] [launches=100] [zero=0]
//
// Prints one JSON line: FLOP/s over `launches` back-to-back launches (after 5
// untimed), and the clock that rate implies if every compute unit issued an
// MFMA every cycle (4096 bf16 FLOP per CU per clock, 256 CUs).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define CHECK(x)                                                                        \
  do {                                                                                  \
    hipError_t e_ = (x);                                                                \
    if (e_ != hipSuccess) {                                                             \
      fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
      exit(1);                                                                          \
    }                                                                                   \
  } while (0)

namespace {

constexpr int kThreads = 512;      // 8 waves
constexpr int kSeedWords = 65536;  // operand pool, indexed modulo its size

__global__ __launch_bounds__(kThreads) void mfma_burn(const uint16_t* __restrict__ pool,
                                                      float* __restrict__ out, int iters) {
  const int gtid = blockIdx.x * kThreads + threadIdx.x;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[s][e] = __builtin_bit_cast(__bf16, pool[(gtid * 64 + s * 16 + e) & (kSeedWords - 1)]);
      b[s][e] = __builtin_bit_cast(__bf16, pool[(gtid * 64 + s * 16 + 8 + e) & (kSeedWords - 1)]);
    }
  f32x16 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x16{};
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(s + (i >> 2)) & 3], b[(s + i) & 3],
                                                         acc[i], 0, 0, 0);
  // one store per lane keeps the products live
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) r += acc[i][e];
  out[gtid] = r;
}

}  // namespace

int main(int argc, char** argv) {
  const int blocks = argc > 1 ? atoi(argv[1]) : 256;
  const int iters = argc > 2 ? atoi(argv[2]) : 1500;
  const int launches = argc > 3 ? atoi(argv[3]) : 100;
  const int zero = argc > 4 ? atoi(argv[4]) : 0;
  if (blocks < 1 || blocks > 4096 || iters < 1 || iters > 100000 || launches < 1 ||
      launches > 10000) {
    fprintf(stderr, "usage: mfma_ceiling [blocks 1..4096] [iters 1..100000] [launches 1..10000] [zero 0|1]\n");
    return 2;
  }
  // random bf16 in [-1, 1): random sign, exponent 2^-15 .. 2^-1, random mantissa
  std::vector<uint16_t> pool(kSeedWords);
  uint32_t st = 12345u;
  for (auto& v : pool) {
    st = st * 1664525u + 1013904223u;
    const uint32_t sign = st >> 31, ex = 0x70u + ((st >> 24) & 0x0eu), man = (st >> 8) & 0x7fu;
    v = zero ? 0 : static_cast<uint16_t>((sign << 15) | (ex << 7) | man);
  }
  uint16_t* d_pool;
  float* d_out;
  CHECK(hipMalloc(&d_pool, kSeedWords * sizeof(uint16_t)));
  CHECK(hipMalloc(&d_out, static_cast<size_t>(blocks) * kThreads * sizeof(float)));
  CHECK(hipMemcpy(d_pool, pool.data(), kSeedWords * sizeof(uint16_t), hipMemcpyHostToDevice));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  for (int w = 0; w < 5; ++w) mfma_burn<<<blocks, kThreads>>>(d_pool, d_out, iters);
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  CHECK(hipEventRecord(e0));
  for (int l = 0; l < launches; ++l) mfma_burn<<<blocks, kThreads>>>(d_pool, d_out, iters);
  CHECK(hipEventRecord(e1));
  CHECK(hipEventSynchronize(e1));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  // per wave and iteration: 32 MFMAs of 32x32x16, 2*32*32*16 FLOP each
  const double flop = static_cast<double>(launches) * blocks * 8 * iters * 32 * 32768.0;
  const double tflops = flop / (ms * 1e-3) / 1e12;
  const double ghz = tflops * 1e12 / (4096.0 * 256) / 1e9;
  printf("{\"kernel\": \"mfma_burn\", \"operands\": \"%s\", \"blocks\": %d, \"iters\": %d, "
         "\"launches\": %d, \"ms_per_launch\": %.4f, \"tflops\": %.1f, \"frac_of_2500\": %.4f, "
         "\"implied_ghz\": %.3f}\n",
         zero ? "zero" : "random", blocks, iters, launches, ms / launches, tflops, tflops / 2500.0, ghz);
  std::vector<float> o(static_cast<size_t>(blocks) * kThreads);
  CHECK(hipMemcpy(o.data(), d_out, o.size() * sizeof(float), hipMemcpyDeviceToHost));
  double sum = 0;
  for (float v : o) sum += v;
  fprintf(stderr, "checksum %g\n", sum);
  CHECK(hipFree(d_pool));
  CHECK(hipFree(d_out));
  return 0;
}
