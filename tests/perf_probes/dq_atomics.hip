// Cost of accumulating dQ with float32 atomics, the alternative to the
// query-stationary dQ kernel that recomputes S and dP ([KB] "FlashAttention：
// 为什么少搬数据，反而算得更快" §05: whether recomputing beats re-reading
// depends on the hardware and the workload).
//
// A key-stationary backward that also formed dQ would, for every (key block,
// query tile) pair under the causal mask, add a BQ x D float32 tile into a
// dQ accumulator with atomics. This program issues exactly that stream of
// atomic adds (hardware global_atomic_add_f32, no return value), with no
// arithmetic, for the causal bf16 workloads B = 1, H = 32, d = 128, N = 4096
// and 8192, with key blocks of 128 and 256 rows and 64-row query tiles. Its
// time is a lower bound on that path's atomic traffic alone, to be set
// against the whole dQ kernel. The same tiles written with plain stores
// show the part that is not the atomic read-modify-write.
//
// Build: hipcc -O3 --offload-arch=gfx950 -munsafe-fp-atomics
//        -Xclang -target-feature -Xclang -packed-fp32-ops dq_atomics.hip
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>

constexpr int H = 32, D = 128, BQ = 64, THREADS = 256;

#define CHECK(x)                                                       \
  do {                                                                 \
    hipError_t e_ = (x);                                               \
    if (e_ != hipSuccess) {                                            \
      printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      exit(1);                                                         \
    }                                                                  \
  } while (0)

// One workgroup per (head, key block), walking the query tiles that see the
// block (causal: tiles from the block's first key on), like a key-stationary
// backward. Each tile is BQ * D = 8192 floats, 32 per thread, each wave
// instruction covering 1 KiB of consecutive addresses.
template <bool ATOMIC>
__global__ __launch_bounds__(THREADS) void tile_adds(float* acc, int N, int BK) {
  const int nkb = N / BK;
  const int kb = blockIdx.x % nkb;
  const int h = blockIdx.x / nkb;
  const float v = 1e-3f * (threadIdx.x + 1);
  for (int qt = (kb * BK) / BQ; qt < N / BQ; ++qt) {
    float* tile = acc + ((size_t)h * N + (size_t)qt * BQ) * D;
#pragma unroll
    for (int i = 0; i < BQ * D / THREADS; ++i) {
      const int idx = i * THREADS + threadIdx.x;
      if constexpr (ATOMIC)
        __hip_atomic_fetch_add(tile + idx, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        tile[idx] = v + qt;
    }
  }
}

int main() {
  const int Ns[2] = {4096, 8192}, BKs[2] = {128, 256};
  float* acc;
  CHECK(hipMalloc(&acc, (size_t)H * 8192 * D * sizeof(float)));
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  for (int N : Ns) {
    for (int BK : BKs) {
      CHECK(hipMemset(acc, 0, (size_t)H * N * D * sizeof(float)));
      const int grid = H * (N / BK);
      long long tiles = 0;
      for (int kb = 0; kb < N / BK; ++kb) tiles += N / BQ - (kb * BK) / BQ;
      tiles *= H;
      const double bytes = (double)tiles * BQ * D * sizeof(float);
      for (int atomic = 1; atomic >= 0; --atomic) {
        auto launch = [&] {
          if (atomic)
            hipLaunchKernelGGL(tile_adds<true>, dim3(grid), dim3(THREADS), 0, 0, acc, N, BK);
          else
            hipLaunchKernelGGL(tile_adds<false>, dim3(grid), dim3(THREADS), 0, 0, acc, N, BK);
        };
        for (int w = 0; w < 3; ++w) launch();
        CHECK(hipEventRecord(e0));
        const int reps = 5;
        for (int r = 0; r < reps; ++r) launch();
        CHECK(hipEventRecord(e1));
        CHECK(hipEventSynchronize(e1));
        CHECK(hipGetLastError());
        float ms = 0.0f;
        CHECK(hipEventElapsedTime(&ms, e0, e1));
        ms /= reps;
        printf("N=%d key block %d: %s %.1f us per launch, %lld tiles, %.3f GiB, %.2f TB/s\n", N, BK,
               atomic ? "atomic adds " : "plain stores", ms * 1e3, tiles, bytes / (1 << 30),
               bytes / (ms * 1e-3) / 1e12);
        fflush(stdout);
      }
    }
  }
  CHECK(hipFree(acc));
  return 0;
}
