// Device-side helpers shared by the gfx950 kernels: 16-bit element traits,
// the 32x32x16 matrix-core (MFMA) wrapper, and small lane utilities.
//
// Matrix-core operand layout used throughout (v_mfma_f32_32x32x16_{bf16,f16},
// one 64-lane wave, C[32x32] += A[32x16] * B[16x32]); with lane = 32*h + c:
//   A: lane holds A[row c][k = 8h .. 8h+7]
//   B: lane holds B[k = 8h .. 8h+7][col c]
//   C: lane holds C[row 8*(r/4) + 4h + r%4][col c] in accumulator r = 0..15
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Stage barriers of the debug build (compiled with -DFA_STAGE_BARRIERS).
// FA_STAGE_WAIT waits for every memory operation the wave has in flight;
// FA_STAGE_SYNC does that and then a workgroup barrier. The pipelined
// kernels place FA_STAGE_SYNC between a step's copy issue and its compute
// (and in every round that only copies, so all waves meet it equally
// often); the decode kernel, whose waves pipeline independently, places
// FA_STAGE_WAIT after each copy issue. Both change only when data arrives,
// never what is computed, so the debug build must give bit-identical
// results: a difference exposes a buffer read before its copy landed, or
// overwritten while it was still being read. In the normal build both are
// empty.
#ifdef FA_STAGE_BARRIERS
#define FA_STAGE_WAIT()                \
  do {                                 \
    asm volatile("" ::: "memory");     \
    __builtin_amdgcn_s_waitcnt(0);     \
  } while (0)
#define FA_STAGE_SYNC() \
  do {                  \
    FA_STAGE_WAIT();    \
    __syncthreads();    \
  } while (0)
#else
#define FA_STAGE_WAIT() ((void)0)
#define FA_STAGE_SYNC() ((void)0)
#endif

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

struct BF16 {
  using vec8 = bf16x8;
  using vec2 = bf16x2;
  __device__ static inline f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline uint16_t from_float(float x) {
    __bf16 h = static_cast<__bf16>(x);
    return __builtin_bit_cast(uint16_t, h);
  }
  __device__ static inline float to_float(uint16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x) << 16);
  }
};

struct F16 {
  using vec8 = f16x8;
  using vec2 = f16x2;
  __device__ static inline f32x16 mfma(vec8 a, vec8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  __device__ static inline uint16_t from_float(float x) {
    _Float16 h = static_cast<_Float16>(x);
    return __builtin_bit_cast(uint16_t, h);
  }
  __device__ static inline float to_float(uint16_t x) {
    return static_cast<float>(__builtin_bit_cast(_Float16, x));
  }
};

// Pack two floats into one 32-bit word of two 16-bit elements (lo first),
// rounding to nearest even: one v_cvt_pk_{bf16,f16}_f32 on gfx950.
template <typename T>
__device__ inline uint32_t pack2(float lo, float hi) {
  f32x2 x;
  x[0] = lo;
  x[1] = hi;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, typename T::vec2));
}

// Eight floats -> one 8-element 16-bit matrix-core operand.
template <typename T>
__device__ inline typename T::vec8 pack8(const float* x) {
  u32x4 w;
  w[0] = pack2<T>(x[0], x[1]);
  w[1] = pack2<T>(x[2], x[3]);
  w[2] = pack2<T>(x[4], x[5]);
  w[3] = pack2<T>(x[6], x[7]);
  return __builtin_bit_cast(typename T::vec8, w);
}

template <typename T>
__device__ inline typename T::vec8 as_vec8(u32x4 w) {
  return __builtin_bit_cast(typename T::vec8, w);
}

__device__ inline f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}

// 16-byte global load / store (global_load_dwordx4 / global_store_dwordx4).
__device__ inline u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ inline void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ inline u32x4 zero_u32x4() {
  u32x4 z;
  z[0] = z[1] = z[2] = z[3] = 0u;
  return z;
}

// Value of lane (lane ^ 32): exchange between the two halves of the wave.
__device__ inline float swap_halves(float x) { return __shfl_xor(x, 32, 64); }

// The matrix-core row of the score tile that accumulator r of half h holds,
// once the A-operand rows were loaded in the order row_perm() gives: keys
// 8h .. 8h+7 for r = 0..7 and 16+8h .. 16+8h+7 for r = 8..15, so each lane's
// first eight accumulators are eight consecutive keys (see row_perm).
__device__ inline int acc_key(int h, int r) { return (r < 8) ? (8 * h + r) : (16 + 8 * h + (r - 8)); }

// Row order in which a lane loads its A-operand row: swapping bits 2 and 3 of
// the row index makes the C accumulators r = 0..7 of half h hold rows
// 8h..8h+7 (and r = 8..15 rows 16+8h..16+8h+7), i.e. contiguous runs of
// eight, which is exactly the B-operand k-layout of the next product.
__device__ inline int row_perm(int i) {
  return (i & ~0xC) | ((i & 0x4) << 1) | ((i & 0x8) >> 1);
}

}  // namespace fa
