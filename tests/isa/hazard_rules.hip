// Matrix-core hazard probes for gfx950 (compiled to assembly by
// tests/test_isa_hazards.py, never run): each kernel puts one producer right
// before one consumer, written with the builtins, so the compiler's own
// hazard recognizer places the wait states the pair needs. The test reads
// those counts back and checks that the rules applied to the inline-assembly
// products (tests/isa_hazards.py RULES) are at least as strict.
#include <hip/hip_runtime.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

#define MFMA(a, b, c) \
  __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0)
#define FENCE __builtin_amdgcn_sched_barrier(0)

__device__ inline void store(float* o, f32x16 c) {
  for (int i = 0; i < 16; ++i) o[i * 64 + threadIdx.x] = c[i];
}

// valu_to_srcab: a vector-ALU write of the A operand, then the product.
__global__ void probe_valu_to_srca(float* o, const unsigned* in) {
  u32x4 a = *(const u32x4*)(in + 4 * threadIdx.x), b = *(const u32x4*)(in + 256 + 4 * threadIdx.x);
  f32x16 c = {};
  FENCE;
  a[3] ^= 0x1234u;
  FENCE;
  store(o, MFMA(a, b, c));
}

// valu_to_srcab: the same for the B operand.
__global__ void probe_valu_to_srcb(float* o, const unsigned* in) {
  u32x4 a = *(const u32x4*)(in + 4 * threadIdx.x), b = *(const u32x4*)(in + 256 + 4 * threadIdx.x);
  f32x16 c = {};
  FENCE;
  b[3] ^= 0x1234u;
  FENCE;
  store(o, MFMA(a, b, c));
}

// valu_to_srcc: a vector-ALU write of the accumulator input.
__global__ void probe_valu_to_srcc(float* o, const unsigned* in) {
  u32x4 a = *(const u32x4*)(in + 4 * threadIdx.x);
  f32x16 c;
  for (int i = 0; i < 16; ++i) c[i] = __builtin_bit_cast(float, in[512 + i * 64 + threadIdx.x]);
  FENCE;
  for (int i = 0; i < 16; ++i) c[i] *= 3.0f;
  FENCE;
  store(o, MFMA(a, a, c));
}

// xdl_to_read: a product's result read by the vector ALU.
__global__ void probe_xdl_to_read(float* o, const unsigned* in) {
  u32x4 a = *(const u32x4*)(in + 4 * threadIdx.x);
  f32x16 c = {};
  c = MFMA(a, a, c);
  FENCE;
  o[threadIdx.x] = c[0] * 2.0f;
}

// xdl_to_read: a product's result read as the next product's A operand.
__global__ void probe_xdl_to_srca(float* o, const unsigned* in) {
  u32x4 a = *(const u32x4*)(in + 4 * threadIdx.x);
  f32x16 c = {};
  c = MFMA(a, a, c);
  FENCE;
  u32x4 x = {__builtin_bit_cast(unsigned, c[0]), __builtin_bit_cast(unsigned, c[1]),
             __builtin_bit_cast(unsigned, c[2]), __builtin_bit_cast(unsigned, c[3])};
  f32x16 d = {};
  store(o, MFMA(x, a, d));
}

// A chain of accumulations into the same registers (needs no wait state).
__global__ void probe_chain(float* o, const unsigned* in) {
  u32x4 a = *(const u32x4*)(in + 4 * threadIdx.x);
  f32x16 c = {};
  c = MFMA(a, a, c);
  FENCE;
  store(o, MFMA(a, a, c));
}
