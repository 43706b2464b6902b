// FP8 (E4M3) forward on the gfx950 matrix cores (fa_fwd_fp8).
//
// Page [KB] "FlashAttention：为什么少搬数据，反而算得更快" §07 notes that the Hopper
// generation adds an FP8 path to the same algorithm. Here q, k and v arrive as
// OCP E4M3 codes with one float32 descale factor per tensor, and the method
// is the forward of fa_fwd.hip ([BLOG] §五 outer loop over query tiles, inner
// loop over key/value tiles, the online softmax of [KB] §04): per key tile
// S^T = K Q^T on v_mfma_f32_32x32x64_f8f6f4 (both operands E4M3, float32
// results; the product's own sum of 64 terms is coarser than a float32
// running sum: on random E4M3 operands its error reached 2^-12.9 of the sum
// of the terms' magnitudes), the row state (m, l, U) in float32, P = exp2(S * c - m)
// rounded to E4M3 for U += V^T P^T on the same product, and at the end
// O = descale_v * U / l in bf16 and LSE = m + ln l.
//
// gfx950 mapping (as the 16-bit forward, with 8-bit operands):
// * one query row per lane (S^T = K Q^T), so the softmax row work is
//   lane-local; Q^T is held in registers as two 32-byte B operands;
// * a 32x32x64 product's two operands pair byte t of lane (h, c) with byte t
//   of lane (h, c') along the contraction: for QK^T lane (h, c) supplies
//   dims 64 kc + 32 h .. + 31 of its key (A) or query (B) row; for PV the
//   32 bytes of lane half h are the keys {8h .. 8h+7, 16+8h .., 32+8h ..,
//   48+8h ..} of the tile in that order, which is exactly where the
//   accumulators of S^T put this lane's scores (K rows fed in row_perm
//   order), so P goes from the score registers to the B operand directly;
// * K and V tiles (64 keys x 128 bytes) reach LDS by direct global -> LDS
//   copies in a layout of 8-row blocks: byte (row, col) at
//   1024 (row / 8) + 128 ((col / 16) xor ((row / 8) & 1)) + 16 (row % 8)
//   + col % 16. A K operand read (16 bytes for 16 lanes of 16 rows) and a
//   transposed V read (ds_read_b64_tr_b8: 16 lanes gather 8 rows x 16 bytes,
//   128 contiguous bytes) then touch every LDS bank once, and each copy
//   instruction moves one contiguous kilobyte (8 rows) of global memory;
// * the running maximum is raised only when a tile's row sum would pass
//   kSumLimit8 = 256 (as in the 16-bit forward), which keeps every P value
//   below E4M3's largest finite value, 448.
#include <math.h>

#include "fa_device.h"
#include "fa_internal.h"
#include "fa_tile.h"

namespace fa {
namespace {

constexpr float LN2 = 0.69314718055994530942f;
constexpr float LOG2E = 1.44269504088896340736f;
constexpr float kSumLimit8 = 256.0f;
constexpr int D8 = 128;         // head dim = bytes per row
constexpr int TB8 = BC * D8;    // bytes per K or V tile

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

struct Fp8Args {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  uint16_t* o;
  float* lse;
  int B, Hq, Hkv, G, Nq, Nkv, n_qtiles;
  float scale_log2;  // scale * log2(e) * descale_q * descale_k
  float descale_v;
};

__device__ __forceinline__ f32x16 mfma8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Direct copies of one tile: block r8 (rows 8 r8 .. 8 r8 + 7) is one
// instruction; lane L lands at LDS byte 1024 r8 + 16 L, which the layout
// assigns to row 8 r8 + L % 8, 16-byte chunk (L / 8) xor (r8 & 1).
template <int NW>
__device__ __forceinline__ void dma8(uint8_t* tile, const uint8_t* head, uint32_t head_bytes,
                                     int key0, int wave, int lane) {
  constexpr int PW = 8 / NW;  // blocks per wave
  const uint32_t start = (uint32_t)key0 * D8;
  const uint32_t left = head_bytes - __builtin_amdgcn_readfirstlane(min(head_bytes, start));
  const __amdgpu_buffer_rsrc_t r = make_rsrc(head + start, left);
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const int r8 = wave * PW + i;
    const uint32_t src = (uint32_t)((8 * r8 + (lane & 7)) * D8 + 16 * ((lane >> 3) ^ (r8 & 1)));
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)(tile + r8 * 1024), 16, src, 0, 0, 0);
  }
}

// Two floats rounded to E4M3 (nearest even) into bytes 2 hi, 2 hi + 1 of w.
__device__ __forceinline__ int pk8(float a, float b, int w, bool hi) {
  return hi ? __builtin_amdgcn_cvt_pk_fp8_f32(a, b, w, true)
            : __builtin_amdgcn_cvt_pk_fp8_f32(a, b, w, false);
}

__device__ __forceinline__ i32x2 tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(p));
}

// K operand (A of S^T = K Q^T) for product i (key block kb = i % 2, dim chunk
// kc = i / 2): two 16-byte reads at the lane's bases ka0, ka1.
__device__ __forceinline__ i32x8 kfrag8(const uint8_t* kt, uint32_t ka0, uint32_t ka1, int i) {
  const uint8_t* p = kt + (i & 1) * 4096 + (i >> 1) * 512;
  const u32x4 lo = *reinterpret_cast<const u32x4*>(p + ka0);
  const u32x4 hi = *reinterpret_cast<const u32x4*>(p + ka1);
  i32x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// V^T operand (A of O^T += V^T P^T) for dim block od: four transposed reads,
// run q giving keys 16 q + 8 h .. + 7 of dim 32 od + c.
__device__ __forceinline__ i32x8 vfrag8(const uint8_t* vt, uint32_t vb, int od) {
  i32x8 r;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const i32x2 x = tr8(vt + vb + q * 2048 + od * 256);
    r[2 * q] = x[0];
    r[2 * q + 1] = x[1];
  }
  return r;
}

// P = exp2(S c - m) of the 16 pairs of this lane's scores rounded to E4M3:
// byte 2e, 2e + 1 of pk (pair e: accumulators 2 (e % 8), +1 of block e / 8).
// Returns the lane's sum of the unrounded values.
__device__ __forceinline__ float exp_tile8(const f32x16* s, float sl2, float m, i32x8& pk) {
  float psum = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float p0 = __builtin_amdgcn_exp2f(fmaf(s[e >> 3][2 * (e & 7)], sl2, -m));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(s[e >> 3][2 * (e & 7) + 1], sl2, -m));
    pk[e >> 1] = pk8(p0, p1, pk[e >> 1], (e & 1) != 0);
    psum += p0 + p1;
  }
  return psum;
}

// One pipeline step: scores of tile i + 2 (4 products), U += V^T P^T of tile
// i (4 products, P in pc) and the exponentials of tile i + 1 (two pairs per
// product), one interleaved stream; operands read two products ahead.
__device__ __forceinline__ float fused8(const uint8_t* kt, uint32_t ka0, uint32_t ka1,
                                        const i32x8* qf, f32x16* sn, const uint8_t* vt,
                                        uint32_t vb, const i32x8& pc, f32x16* oacc,
                                        const f32x16* se, float sl2, float m, i32x8& pn) {
  sn[0] = zero16();
  sn[1] = zero16();
  i32x8 kf[4], vf[4];
  kf[0] = kfrag8(kt, ka0, ka1, 0);
  kf[1] = kfrag8(kt, ka0, ka1, 1);
  vf[0] = vfrag8(vt, vb, 0);
  vf[1] = vfrag8(vt, vb, 1);
  float psum = 0.0f;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int i = t >> 1;
    if ((t & 1) == 0) {
      if (i + 2 < 4) kf[i + 2] = kfrag8(kt, ka0, ka1, i + 2);
      sn[i & 1] = mfma8(kf[i], qf[i >> 1], sn[i & 1]);
    } else {
      if (i + 2 < 4) vf[i + 2] = vfrag8(vt, vb, i + 2);
      oacc[i] = mfma8(vf[i], pc, oacc[i]);
    }
#pragma unroll
    for (int e = 2 * t; e < 2 * t + 2; ++e) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(se[e >> 3][2 * (e & 7)], sl2, -m));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(se[e >> 3][2 * (e & 7) + 1], sl2, -m));
      pn[e >> 1] = pk8(p0, p1, pn[e >> 1], (e & 1) != 0);
      psum += p0 + p1;
    }
    asm volatile("" : "+v"(psum));
    __builtin_amdgcn_sched_barrier(0);
  }
  return psum;
}

template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// NW waves of 32 query rows per workgroup, as the 16-bit forward: 8 (256
// rows, one workgroup per CU) when the grid fills the GPU, else 4.
template <bool CAUSAL, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void fwd_fp8_kernel(Fp8Args a) {
  constexpr int BR = 32 * NW;
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf0[TB8];
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf1[TB8];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf0[TB8];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf1[TB8];
  auto kslot = [&](int x) __attribute__((always_inline)) -> uint8_t* { return x ? kbuf1 : kbuf0; };
  auto vslot = [&](int x) __attribute__((always_inline)) -> uint8_t* { return x ? vbuf1 : vbuf0; };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int h = lane >> 5;
  const int c = lane & 31;

  const TileId id = tile_of(blockIdx.x, a.B, a.Hq, a.Hkv, a.G, a.n_qtiles);
  const int qt = id.qt, b = id.b, hq = id.hq;
  const int hkv = hq / a.G;
  const int Nq = a.Nq, Nkv = a.Nkv;
  const int offset = Nkv - Nq;
  const size_t bh = (size_t)b * a.Hq + hq;
  const int q0 = qt * BR + wave * 32;
  const int qrow = q0 + c;

  const int kv_tiles = (Nkv + BC - 1) / BC;
  int n_tiles = kv_tiles;
  if (CAUSAL) {
    const int last_key = min(Nq, (qt + 1) * BR) - 1 + offset;
    n_tiles = last_key < 0 ? 0 : min(kv_tiles, last_key / BC + 1);
  }
  const int wave_last_key = CAUSAL ? min(Nq - 1, q0 + 31) + offset : Nkv - 1;
  const int n_w = (q0 >= Nq || wave_last_key < 0) ? 0 : min(n_tiles, wave_last_key / BC + 1);

  const size_t kv_off = ((size_t)b * a.Hkv + hkv) * Nkv * D8;
  const uint32_t kv_bytes = (uint32_t)min(Nkv, n_tiles * BC) * D8;
  const uint8_t* const khead = a.k + kv_off;
  const uint8_t* const vhead = a.v + kv_off;
  auto load_k = [&](int j, uint8_t* dst) __attribute__((always_inline)) {
    dma8<NW>(dst, khead, kv_bytes, j * BC, wave, lane);
  };
  auto load_v = [&](int j, uint8_t* dst) __attribute__((always_inline)) {
    dma8<NW>(dst, vhead, kv_bytes, j * BC, wave, lane);
  };

  // Operand read bases. K: row row_perm(c) of key block 0, the two 16-byte
  // chunks 2h, 2h + 1 of dim chunk 0 (swizzled by the row block's parity).
  const int krow = row_perm(c);
  const int kp = (krow >> 3) & 1;
  const uint32_t kbase = (uint32_t)((krow >> 3) * 1024 + (krow & 7) * 16);
  const uint32_t ka0 = kbase + (uint32_t)((2 * h + kp) * 128);
  const uint32_t ka1 = kbase + (uint32_t)((2 * h + (1 - kp)) * 128);
  // V: block 2q + h, chunk (2 od + c / 16) xor h, byte 8 (c % 16).
  const uint32_t vb = (uint32_t)(h * 1024 + (((c >> 4) ^ h) * 128) + 8 * (c & 15));

  // Q^T as two B operands: dims 64 kc + 32 h .. + 31 of this lane's row.
  i32x8 qf[2];
  const uint8_t* qp = a.q + (bh * Nq + qrow) * D8;
#pragma unroll
  for (int kc = 0; kc < 2; ++kc) {
    const u32x4 lo = qrow < Nq ? ld16(qp + kc * 64 + h * 32) : zero_u32x4();
    const u32x4 hi = qrow < Nq ? ld16(qp + kc * 64 + h * 32 + 16) : zero_u32x4();
    qf[kc][0] = lo[0]; qf[kc][1] = lo[1]; qf[kc][2] = lo[2]; qf[kc][3] = lo[3];
    qf[kc][4] = hi[0]; qf[kc][5] = hi[1]; qf[kc][6] = hi[2]; qf[kc][7] = hi[3];
  }

  f32x16 oacc[4];
#pragma unroll
  for (int od = 0; od < 4; ++od) oacc[od] = zero16();
  float m_run = -INFINITY;
  float l_run = 0.0f;
  const float sl2 = a.scale_log2;

  auto mask_tile = [&](int j, f32x16* s) __attribute__((always_inline)) {
    const int key0 = j * BC;
    const bool need_mask = (key0 + BC > Nkv) || (CAUSAL && key0 + BC - 1 > q0 + offset);
    if (need_mask) {
      const int lim = CAUSAL ? min(Nkv - 1, qrow + offset) : Nkv - 1;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (key0 + kb * 32 + acc_key(h, r) > lim) s[kb][r] = -INFINITY;
    }
  };
  auto fix_max = [&](const f32x16* s, i32x8& p, float psum) __attribute__((always_inline)) {
    if (__builtin_expect(__any(!(psum <= kSumLimit8)), 0)) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = fmaxf(mx, swap_halves(mx)) * sl2;
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int od = 0; od < 4; ++od)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[od][r] *= alpha;
      m_run = m_new;
      psum = exp_tile8(s, sl2, (m_new == -INFINITY) ? 0.0f : m_new, p);
    }
    return psum;
  };

  f32x16 sa[2], sb[2];
  i32x8 pa, pb;
#pragma unroll
  for (int i = 0; i < 8; ++i) pa[i] = pb[i] = 0;

  // Prologue: K tiles 0, 1 and V tile 0; scores and P of tile 0, scores of
  // tile 1; then K tile 2 into the buffer of K tile 0.
  load_k(0, kbuf0);
  load_k(1, kbuf1);
  load_v(0, vbuf0);
  __syncthreads();
  if (n_w > 0) {
    sa[0] = zero16();
    sa[1] = zero16();
#pragma unroll
    for (int i = 0; i < 4; ++i) sa[i & 1] = mfma8(kfrag8(kbuf0, ka0, ka1, i), qf[i >> 1], sa[i & 1]);
    mask_tile(0, sa);
    l_run += fix_max(sa, pa, exp_tile8(sa, sl2, m_run, pa));
    sb[0] = zero16();
    sb[1] = zero16();
#pragma unroll
    for (int i = 0; i < 4; ++i) sb[i & 1] = mfma8(kfrag8(kbuf1, ka0, ka1, i), qf[i >> 1], sb[i & 1]);
  }
  __syncthreads();
  load_k(2, kbuf0);
  __syncthreads();

  auto step = [&](int i, f32x16* se, const i32x8& pc, f32x16* sn, i32x8& pn, const uint8_t* kt,
                  const uint8_t* vt) __attribute__((always_inline)) {
    const bool live = i + 1 < n_w;
    if (live) mask_tile(i + 1, se);
    const float psum = fused8(kt, ka0, ka1, qf, sn, vt, vb, pc, oacc, se, sl2, m_run, pn);
    if (live) l_run += fix_max(se, pn, psum);
  };

  for (int i0 = 0; i0 < n_w; i0 += 2) {
    static_for<2>([&](auto rc) __attribute__((always_inline)) {
      constexpr int r = decltype(rc)::value;
      const int i = i0 + r;
      if (i < n_w) {
        load_k(i + 3, kslot(r ^ 1));
        load_v(i + 1, vslot(r ^ 1));
        FA_STAGE_SYNC();
        if constexpr (r == 0)
          step(i, sb, pa, sa, pb, kslot(0), vslot(0));
        else
          step(i, sa, pb, sb, pa, kslot(1), vslot(1));
        __syncthreads();
      }
    });
  }
  for (int i = n_w; i < n_tiles; ++i) {
    load_k(i + 3, kslot((i + 1) & 1));
    load_v(i + 1, vslot((i + 1) & 1));
    FA_STAGE_SYNC();
    __syncthreads();
  }

  // O = descale_v * U / l (bf16), LSE = m + ln l.
  const float l = l_run + swap_halves(l_run);
  if (qrow < Nq) {
    const float inv = l > 0.0f ? a.descale_v / l : 0.0f;
    uint16_t* orow = a.o + (bh * Nq + qrow) * D8;
#pragma unroll
    for (int od = 0; od < 4; ++od)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 out;
        out[0] = pack2<BF16>(oacc[od][4 * g + 0] * inv, oacc[od][4 * g + 1] * inv);
        out[1] = pack2<BF16>(oacc[od][4 * g + 2] * inv, oacc[od][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + od * 32 + g * 8 + h * 4) = out;
      }
    if (h == 0) a.lse[bh * Nq + qrow] = l > 0.0f ? (m_run + __log2f(l)) * LN2 : -INFINITY;
  }
}

template <int NW>
hipError_t launch_nw(const Problem& p, const Fp8Ptrs& t, hipStream_t stream) {
  constexpr int BR = 32 * NW;
  Fp8Args a;
  a.q = static_cast<const uint8_t*>(t.q);
  a.k = static_cast<const uint8_t*>(t.k);
  a.v = static_cast<const uint8_t*>(t.v);
  a.o = static_cast<uint16_t*>(t.o);
  a.lse = t.lse;
  a.B = p.B;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.G = p.G;
  a.Nq = p.Nq;
  a.Nkv = p.Nkv;
  a.n_qtiles = (p.Nq + BR - 1) / BR;
  a.scale_log2 = p.scale * LOG2E * t.descale_q * t.descale_k;
  a.descale_v = t.descale_v;
  dim3 grid(a.n_qtiles * p.B * p.Hq);
  if (p.causal)
    hipLaunchKernelGGL((fwd_fp8_kernel<true, NW>), grid, dim3(64 * NW), 0, stream, a);
  else
    hipLaunchKernelGGL((fwd_fp8_kernel<false, NW>), grid, dim3(64 * NW), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const Problem& p, const Fp8Ptrs& t, hipStream_t stream) {
  const long long big_tiles = (long long)p.B * p.Hq * ((p.Nq + 255) / 256);
  return (big_tiles >= 256 && p.Nq >= 4096) ? launch_nw<8>(p, t, stream)
                                            : launch_nw<4>(p, t, stream);
}

}  // namespace fa
