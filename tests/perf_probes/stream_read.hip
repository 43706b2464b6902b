// Practical read rate of the decode workloads' K/V bytes from cold caches:
// a plain streaming read (16-byte non-temporal loads, grid-stride, one
// float written per thread so the loads are kept) of the bytes one decode
// call reads. c5 MQA (B = 16, N_kv = 8192, one kv head, d = 128, bf16)
// reads 64 MiB of K and V; c5 GQA (eight kv heads) 512 MiB. Before each
// timed launch a 1 GiB fill evicts the caches, as the decode benchmark
// does; only the read is between the events. Several grid sizes are timed
// (256 threads per workgroup), and the best is the ceiling a single
// streaming kernel reaches on that many bytes.
//
// Build: hipcc -O3 --offload-arch=gfx950
//        -Xclang -target-feature -Xclang -packed-fp32-ops stream_read.hip
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>

#define CHECK(x)                                                            \
  do {                                                                      \
    hipError_t e_ = (x);                                                    \
    if (e_ != hipSuccess) {                                                 \
      printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      exit(1);                                                              \
    }                                                                       \
  } while (0)

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void stream_read(const u32x4* __restrict__ src, size_t n,
                                                   float* __restrict__ out) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  unsigned int acc = 0;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = (float)acc;
}

__global__ __launch_bounds__(256) void fill(unsigned int* p, size_t n, unsigned int v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

int main() {
  const size_t sizes[2] = {(size_t)64 << 20, (size_t)512 << 20};
  const int grids[5] = {256, 512, 1024, 2048, 4096};
  const size_t flush_bytes = (size_t)1 << 30;
  u32x4* src;
  unsigned int* flush;
  float* out;
  CHECK(hipMalloc(&src, sizes[1]));
  CHECK(hipMalloc(&flush, flush_bytes));
  CHECK(hipMalloc(&out, (size_t)4096 * 256 * sizeof(float)));
  hipLaunchKernelGGL(fill, dim3(4096), dim3(256), 0, 0, (unsigned int*)src, sizes[1] / 4, 7u);
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  for (size_t bytes : sizes) {
    for (int g : grids) {
      const int reps = 20;
      float total = 0.0f;
      for (int r = -2; r < reps; ++r) {
        hipLaunchKernelGGL(fill, dim3(4096), dim3(256), 0, 0, flush, flush_bytes / 4, (unsigned)r);
        CHECK(hipEventRecord(e0));
        hipLaunchKernelGGL(stream_read, dim3(g), dim3(256), 0, 0, src, bytes / 16, out);
        CHECK(hipEventRecord(e1));
        CHECK(hipEventSynchronize(e1));
        float ms = 0.0f;
        CHECK(hipEventElapsedTime(&ms, e0, e1));
        if (r >= 0) total += ms;
      }
      CHECK(hipGetLastError());
      const double us = total / reps * 1e3;
      printf("%4zu MiB, %4d workgroups: %.2f us, %.2f TB/s (cold)\n", bytes >> 20, g, us,
             bytes / (us * 1e-6) / 1e12);
      fflush(stdout);
    }
  }
  CHECK(hipFree(src));
  CHECK(hipFree(flush));
  CHECK(hipFree(out));
  return 0;
}
