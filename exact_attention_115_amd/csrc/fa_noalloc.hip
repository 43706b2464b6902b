// fa_bwd_noalloc: the backward with the workspace taken from a static device
// array instead of the caller, for callers that cannot allocate device
// memory (HIP graph capture, allocation-free serving loops).
//
// The array `scratch` is a file-scope __device__ variable: every GPU the
// library runs on holds its own copy, at its own address. In host code its
// name only stands for the symbol; the device address of the current GPU's
// copy comes from hipGetSymbolAddress, looked up once per device on that
// device's first call (with the device current) and cached. Kernels receive
// that address, exactly as they receive a caller's workspace in fa_bwd.
#include <mutex>

#include "fa_internal.h"

namespace fa {
namespace {

constexpr size_t kScratchBytes = FA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_lock;
void* g_addr[kMaxDevices];  // device address of `scratch` per device, once looked up

int scratch_workspace(size_t bytes, void** ws) {
  if (bytes > kScratchBytes) return FA_ERR_SCRATCH;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_HIP;
  std::lock_guard<std::mutex> guard(g_lock);
  if (!g_addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FA_ERR_HIP;
    g_addr[dev] = p;
  }
  *ws = g_addr[dev];
  return FA_OK;
}

}  // namespace
}  // namespace fa

extern "C" int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dO, void* dq, void* dk, void* dv,
                              int B, int Hq, int Hkv, int Nq, int Nkv, int d, float scale,
                              int causal, fa_dtype dt, hipStream_t stream) {
  return fa::bwd_with_library_workspace(q, k, v, o, lse, dO, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, d,
                                        scale, causal, dt, stream, fa::scratch_workspace);
}
