// Dropout keep bits from the counter-based generator Philox4x64-10
// (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2,
// 3", SC 2011). Dropout acts on the attention probabilities, a step page
// [KB] "FlashAttention：为什么少搬数据，反而算得更快" §04 lists among those the tiled
// computation must still handle; as with P itself ([KB] §05) the mask is
// rebuilt where it is needed and never stored.
//
// Element (b, h, i, j) -- query head h, query row i, key j -- takes byte
// t = j mod 32 of the 256-bit block philox(counter, key) with
// counter = (j / 32, i, b * Hq + h, offset) and key = (seed, 0); byte t is
// bits 8 (t mod 8) .. +7 of output word t / 8. The element is kept iff that
// byte is >= theta. keep_bits() returns the 32 decisions of one key group as
// a word (bit t: key 32 * group + t).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct DropParams {
  uint64_t seed;
  uint64_t offset;
  uint32_t theta;  // keep iff byte >= theta (0 keeps everything)
  float rscale;    // 256 / (256 - theta)
};

// The 128-bit product a * b: returns its low 64 bits and stores the high
// 64 bits in *hi. Both halves come from the same four 32 x 32 -> 64 partial
// products (a = a1 2^32 + a0, b = b1 2^32 + b0), each a multiply-add of two
// 32-bit values into a 64-bit one that cannot overflow.
__host__ __device__ __forceinline__ uint64_t mulhilo64(uint64_t a, uint64_t b, uint64_t* hi) {
  const uint64_t a0 = (uint32_t)a, a1 = a >> 32, b0 = (uint32_t)b, b1 = b >> 32;
  const uint64_t p00 = a0 * b0;
  const uint64_t p01 = a0 * b1 + (p00 >> 32);
  const uint64_t p10 = a1 * b0 + (uint32_t)p01;
  *hi = a1 * b1 + (p01 >> 32) + (p10 >> 32);
  return (p10 << 32) | (uint32_t)p00;
}

// The four output words of Philox4x64-10 for counter c and key (k0, k1).
__host__ __device__ __forceinline__ void philox4x64_10(uint64_t c[4], uint64_t k0, uint64_t k1) {
  constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    uint64_t hi0, hi1;
    const uint64_t lo0 = mulhilo64(M0, c[0], &hi0), lo1 = mulhilo64(M1, c[2], &hi1);
    const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
    k0 += W0;
    k1 += W1;
  }
}

// Bit b of the result (b = 0..3) is 1 iff byte b of x is >= the byte y8
// (y4 = y8 replicated in all four bytes). Per byte: with the top bits set
// aside, (x | 0x80) - (y & 0x7f) keeps its top bit iff the low seven bits of
// x are >= those of y, and no borrow crosses bytes; the top bits of x and y
// then decide (x wins if only x has it, ties fall to the low bits).
__host__ __device__ __forceinline__ uint32_t bytes_ge4(uint32_t x, uint32_t y4) {
  constexpr uint32_t H = 0x80808080u;
  const uint32_t z = (x | H) - (y4 & ~H);
  const uint32_t ge = ((x & ~y4) | (~(x ^ y4) & z)) & H;
  // Gather the four top bits (positions 7, 15, 23, 31) into bits 0..3.
  return ((ge >> 7) * 0x00204081u) >> 21 & 0xFu;
}

// The keep decisions of keys 32 * group .. 32 * group + 31 of query row `row`
// of head bh (= b * Hq + h).
__host__ __device__ __forceinline__ uint32_t keep_bits(uint32_t group, uint32_t row, uint32_t bh,
                                                       const DropParams& dp) {
  uint64_t c[4] = {group, row, bh, dp.offset};
  philox4x64_10(c, dp.seed, 0);
  const uint32_t y4 = dp.theta * 0x01010101u;
  uint32_t bits = 0;
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    const uint32_t x = (uint32_t)(c[w >> 1] >> (32 * (w & 1)));
    bits |= bytes_ge4(x, y4) << (4 * w);
  }
  return bits;
}

// x if bit b of the keep word kw is set, else +0.
__device__ __forceinline__ float keep_f(float x, uint32_t kw, int b) {
  return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, x) &
                                       (uint32_t)((int32_t)(kw << (31 - b)) >> 31));
}

// Keep word of the 64-key tile j for a lane of the transposed-score layout
// (lane (h, c) holds query row `row`; its accumulator r of key block kb is
// key 64 j + 32 kb + 8 h + r for r < 8 and 64 j + 32 kb + 16 + 8 h + r - 8
// otherwise): bit 16 kb + r is that key's decision. Half h draws key group
// 2 j + h and the two halves swap the bytes the other needs; all 64 lanes
// must take part.
__device__ __forceinline__ uint32_t row_keep_word(int j, uint32_t row, uint32_t bh, int h,
                                                  const DropParams& dp) {
  const uint32_t own = keep_bits((uint32_t)(2 * j + h), row, bh, dp);
  const uint32_t other = (uint32_t)__shfl_xor((int)own, 32, 64);
  const uint32_t g0 = h ? other : own, g1 = h ? own : other;
  const int sh = 8 * h;
  return ((g0 >> sh) & 0xFFu) | (((g0 >> (16 + sh)) & 0xFFu) << 8) |
         (((g1 >> sh) & 0xFFu) << 16) | (((g1 >> (16 + sh)) & 0xFFu) << 24);
}

}  // namespace fa
