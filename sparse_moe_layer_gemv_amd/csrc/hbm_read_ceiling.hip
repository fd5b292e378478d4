// hbm_read_ceiling: a measurement program, not part of libmoe.
//
// Sustained HBM read bandwidth of the whole chip: every workgroup streams a
// contiguous share of a buffer far larger than the 256 MB last-level cache
// (MALL) with 16-byte loads per lane and folds what it reads into one value
// per thread, so nothing but the reads reaches memory.  This is the ceiling a
// weight-streaming kernel can approach; the published 8 TB/s is the interface
// rate.
//
//   hbm_read_ceiling [gib=4] [blocks=2048] [threads=512] [unroll=8] [nt=1] [launches=20]
//
// nt=1 loads with the non-temporal hint (as the weight streams do), nt=0
// with the default policy.  Prints one JSON line with the bytes read per
// second over `launches` back-to-back passes (after 3 untimed).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>

#define CHECK(x)                                                                        \
  do {                                                                                  \
    hipError_t e_ = (x);                                                                \
    if (e_ != hipSuccess) {                                                             \
      fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_), __FILE__, __LINE__); \
      exit(1);                                                                          \
    }                                                                                   \
  } while (0)

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Workgroup b reads the 16-byte words [b*per_block, (b+1)*per_block), each
// pass of the block covering blockDim.x * U consecutive words.  per_block is a
// multiple of blockDim.x * U (checked on the host), so every load is in range.
template <int U, bool NT>
__global__ void read_stream(const u32x4* __restrict__ src, size_t per_block, uint32_t* __restrict__ out) {
  const u32x4* p = src + blockIdx.x * per_block + threadIdx.x;
  const size_t passes = per_block / (static_cast<size_t>(blockDim.x) * U);
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t i = 0; i < passes; ++i) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = NT ? __builtin_nontemporal_load(p + u * blockDim.x) : p[u * blockDim.x];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
    p += static_cast<size_t>(blockDim.x) * U;
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

template <int U>
void launch(bool nt, int blocks, int threads, const u32x4* src, size_t per_block, uint32_t* out) {
  if (nt)
    read_stream<U, true><<<blocks, threads>>>(src, per_block, out);
  else
    read_stream<U, false><<<blocks, threads>>>(src, per_block, out);
}

void launch_any(int unroll, bool nt, int blocks, int threads, const u32x4* src, size_t per_block,
                uint32_t* out) {
  switch (unroll) {
    case 1: launch<1>(nt, blocks, threads, src, per_block, out); break;
    case 2: launch<2>(nt, blocks, threads, src, per_block, out); break;
    case 4: launch<4>(nt, blocks, threads, src, per_block, out); break;
    default: launch<8>(nt, blocks, threads, src, per_block, out); break;
  }
}

}  // namespace

int main(int argc, char** argv) {
  const int gib = argc > 1 ? atoi(argv[1]) : 4;
  const int blocks = argc > 2 ? atoi(argv[2]) : 2048;
  const int threads = argc > 3 ? atoi(argv[3]) : 512;
  const int unroll = argc > 4 ? atoi(argv[4]) : 8;
  const int nt = argc > 5 ? atoi(argv[5]) : 1;
  const int launches = argc > 6 ? atoi(argv[6]) : 20;
  if (gib < 1 || gib > 64 || blocks < 1 || blocks > 65536 || (threads != 256 && threads != 512 &&
      threads != 1024) || (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8) ||
      launches < 1 || launches > 1000) {
    fprintf(stderr, "usage: hbm_read_ceiling [gib 1..64] [blocks] [threads 256|512|1024] [unroll 1|2|4|8] [nt 0|1] [launches]\n");
    return 2;
  }
  const size_t words = (static_cast<size_t>(gib) << 30) / 16;
  const size_t chunk = static_cast<size_t>(threads) * unroll;
  const size_t per_block = words / blocks / chunk * chunk;  // whole passes only
  if (per_block == 0) {
    fprintf(stderr, "buffer too small for %d blocks\n", blocks);
    return 2;
  }
  const size_t bytes_read = per_block * blocks * 16;
  u32x4* src;
  uint32_t* out;
  CHECK(hipMalloc(&src, words * 16));
  CHECK(hipMalloc(&out, static_cast<size_t>(blocks) * threads * sizeof(uint32_t)));
  CHECK(hipMemset(src, 0x5a, words * 16));
  CHECK(hipDeviceSynchronize());
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  for (int w = 0; w < 3; ++w) launch_any(unroll, nt != 0, blocks, threads, src, per_block, out);
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  CHECK(hipEventRecord(e0));
  for (int l = 0; l < launches; ++l) launch_any(unroll, nt != 0, blocks, threads, src, per_block, out);
  CHECK(hipEventRecord(e1));
  CHECK(hipEventSynchronize(e1));
  float ms = 0.f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  const double gbs = static_cast<double>(bytes_read) * launches / (ms * 1e-3) / 1e9;
  printf("{\"kernel\": \"read_stream\", \"bytes_per_pass\": %zu, \"blocks\": %d, \"threads\": %d, "
         "\"unroll\": %d, \"nontemporal\": %d, \"launches\": %d, \"us_per_pass\": %.1f, "
         "\"gbs\": %.0f, \"frac_of_8000\": %.4f}\n",
         bytes_read, blocks, threads, unroll, nt, launches, ms * 1e3 / launches, gbs, gbs / 8000.0);
  CHECK(hipFree(src));
  CHECK(hipFree(out));
  return 0;
}
