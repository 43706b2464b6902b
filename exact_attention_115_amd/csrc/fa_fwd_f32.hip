// Float32 forward: exact attention with true float32 arithmetic throughout.
//
// Same structure as the 16-bit path ([BLOG] "AI infra. 一层全看懂(五)Flash
// Attention" §五: outer loop over query tiles, inner loop over key/value
// tiles held on chip), but every product is a float32 FMA on the vector ALUs:
// the float32 workloads are small, and this keeps their error at float32
// rounding (the 16-bit matrix cores would round the operands).
//
// One wavefront per workgroup. Each query row is owned by D / 64 lanes, each
// holding 64 of its dims: the scaled query, the output row, and (redundantly)
// the row's online-softmax state (m, l, U) of [KB]
// "FlashAttention：为什么少搬数据，反而算得更快" §04. A score is the sum of the
// lanes' partial dot products (one exchange between the two half-waves at
// d = 128), so every lane keeps 2 x 64 + 32 floats and nothing spills.
// Key/value tiles of 32 rows are staged in LDS and read by all lanes of a
// half-wave at the same address (an LDS broadcast).
#include <math.h>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr int kKeys = 32;  // keys per LDS tile
constexpr int kDims = 64;  // dims per lane

template <int D>
__global__ __launch_bounds__(64) void fwd_f32_kernel(const float* __restrict__ Q,
                                                     const float* __restrict__ K,
                                                     const float* __restrict__ V,
                                                     float* __restrict__ O, float* __restrict__ LSE,
                                                     int Hq, int G, int Nq, int Nkv, float scale,
                                                     int causal) {
  constexpr int LPR = D / kDims;   // lanes per row
  constexpr int kRows = 64 / LPR;  // query rows per workgroup
  __shared__ float Ks[kKeys][D];
  __shared__ float Vs[kKeys][D];

  const int lane = threadIdx.x;
  const int part = lane / kRows;   // which 64 dims of the row
  const int c0 = part * kDims;
  const int ntiles = (Nq + kRows - 1) / kRows;
  const int tile = blockIdx.x % ntiles;
  const int bh = blockIdx.x / ntiles;
  const int hq = bh % Hq;
  const int b = bh / Hq;
  const int hkv = hq / G;
  const int Hkv = Hq / G;
  const int row = tile * kRows + lane % kRows;
  const int offset = Nkv - Nq;  // causal: key j visible to row i iff j <= i + offset

  const size_t qbase = ((size_t)(b * Hq + hq) * Nq) * D;
  const size_t kbase = ((size_t)(b * Hkv + hkv) * Nkv) * D;

  float q[kDims];
  float u[kDims];
#pragma unroll
  for (int c = 0; c < kDims; ++c) {
    q[c] = row < Nq ? Q[qbase + (size_t)row * D + c0 + c] * scale : 0.0f;
    u[c] = 0.0f;
  }
  float m = -INFINITY;
  float l = 0.0f;

  // Keys this workgroup may need: up to the last key its last row can see.
  const int last_row = min(Nq, (tile + 1) * kRows) - 1;
  int key_end = Nkv;
  if (causal) key_end = min(Nkv, max(0, last_row + offset + 1));

  for (int k0 = 0; k0 < key_end; k0 += kKeys) {
    __syncthreads();
    for (int idx = lane; idx < kKeys * D; idx += 64) {
      const int j = idx / D, c = idx % D;
      const int key = k0 + j;
      const bool in = key < Nkv;
      Ks[j][c] = in ? K[kbase + (size_t)key * D + c] : 0.0f;
      Vs[j][c] = in ? V[kbase + (size_t)key * D + c] : 0.0f;
    }
    __syncthreads();

    float s[kKeys];
    float mt = -INFINITY;
#pragma unroll 4
    for (int j = 0; j < kKeys; ++j) {
      const int key = k0 + j;
      float acc = 0.0f;
#pragma unroll
      for (int c = 0; c < kDims; ++c) acc = fmaf(q[c], Ks[j][c0 + c], acc);
      if constexpr (LPR == 2) acc += __shfl_xor(acc, 32, 64);  // the other half's dims
      const bool vis = key < Nkv && (!causal || key <= row + offset);
      s[j] = vis ? acc : -INFINITY;
      mt = fmaxf(mt, s[j]);
    }
    const float m_new = fmaxf(m, mt);
    if (m_new == -INFINITY) continue;  // nothing visible yet: state unchanged
    const float a = (m == -INFINITY) ? 0.0f : expf(m - m_new);
    l *= a;
#pragma unroll
    for (int c = 0; c < kDims; ++c) u[c] *= a;
#pragma unroll 4
    for (int j = 0; j < kKeys; ++j) {
      const float p = expf(s[j] - m_new);
      l += p;
#pragma unroll
      for (int c = 0; c < kDims; ++c) u[c] = fmaf(p, Vs[j][c0 + c], u[c]);
    }
    m = m_new;
  }

  if (row >= Nq) return;
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
  for (int c = 0; c < kDims; ++c) O[qbase + (size_t)row * D + c0 + c] = u[c] * inv;
  if (part == 0) LSE[(size_t)(b * Hq + hq) * Nq + row] = l > 0.0f ? m + logf(l) : -INFINITY;
}

}  // namespace

hipError_t launch_fwd_f32(const Problem& p, const FwdPtrs& t, hipStream_t stream) {
  const int rows = 64 / (p.d / kDims);  // query rows per workgroup
  dim3 grid(((p.Nq + rows - 1) / rows) * p.Hq * p.B);
  dim3 block(64);
  const float* q = static_cast<const float*>(t.q);
  const float* k = static_cast<const float*>(t.k);
  const float* v = static_cast<const float*>(t.v);
  float* o = static_cast<float*>(t.o);
  if (p.d == 64)
    hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, block, 0, stream, q, k, v, o, t.lse, p.Hq, p.G,
                       p.Nq, p.Nkv, p.scale, p.causal);
  else
    hipLaunchKernelGGL(fwd_f32_kernel<128>, grid, block, 0, stream, q, k, v, o, t.lse, p.Hq, p.G,
                       p.Nq, p.Nkv, p.scale, p.causal);
  return hipGetLastError();
}

}  // namespace fa
