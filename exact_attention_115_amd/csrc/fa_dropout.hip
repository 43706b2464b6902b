// The dropout keep mask as bytes (fa_dropout_mask): the attention kernels
// draw the same decisions tile by tile and never store them; this kernel
// writes them out so a caller can inspect or test them.
#include "fa_internal.h"
#include "fa_philox.h"

namespace fa {
namespace {

// One thread per (head, query row, 32-key group).
__global__ __launch_bounds__(256) void dropout_mask_kernel(uint8_t* __restrict__ keep, int Nq,
                                                           int Nkv, int groups, long long total,
                                                           DropParams dp) {
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total) return;
  const int g = (int)(t % groups);
  const long long rest = t / groups;
  const int row = (int)(rest % Nq);
  const long long bh = rest / Nq;
  const uint32_t bits = keep_bits((uint32_t)g, (uint32_t)row, (uint32_t)bh, dp);
  uint8_t* out = keep + ((size_t)bh * Nq + row) * (size_t)Nkv + (size_t)g * 32;
  const int n = min(32, Nkv - g * 32);
  for (int i = 0; i < n; ++i) out[i] = (uint8_t)((bits >> i) & 1u);
}

}  // namespace

hipError_t launch_dropout_mask(uint8_t* keep, int B, int Hq, int Nq, int Nkv, const DropParams& dp,
                               hipStream_t stream) {
  const int groups = (Nkv + 31) / 32;
  const long long total = (long long)B * Hq * Nq * groups;
  const long long blocks = (total + 255) / 256;
  hipLaunchKernelGGL(dropout_mask_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, keep, Nq,
                     Nkv, groups, total, dp);
  return hipGetLastError();
}

}  // namespace fa
