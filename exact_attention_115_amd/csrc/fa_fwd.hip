// 16-bit (bf16 / fp16) forward on the gfx950 matrix cores.
//
// Method ([BLOG] "AI infra. 一层全看懂(五)Flash Attention" §五; [KB]
// "FlashAttention：为什么少搬数据，反而算得更快" §03-§04): one workgroup per
// tile of 256 or 128 query rows (the outer loop); it walks the key/value tiles of 64
// rows its rows may see (the inner loop). Each score tile S = Q K^T is
// produced on chip, scaled, masked and folded at once into per-row online
// softmax state -- m (running maximum), l (running sum of exp(s - m)) and the
// un-normalised output U, with the held part rescaled by exp(m_old - m_new)
// ([KB] §04) -- then discarded. Only O and the row LSE = m + ln l leave the
// chip, so no N x N matrix is ever written to memory.
//
// gfx950 mapping:
// * 8 or 4 waves per workgroup (two waves per SIMD either way: one 8-wave
//   workgroup or two 4-wave ones per CU), 32 query rows per wave. The score
//   tile is computed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16: the
//   query index is the matrix-core column, so every lane owns ONE query row
//   (half of its keys in each half-wave) and the row max / row sum need only
//   lane-local work plus one exchange between the two half-waves.
// * K rows are fed to the matrix core in the order row_perm() gives, which
//   leaves each lane's accumulators holding runs of 8 consecutive keys: they
//   are, unchanged, the B operand (P^T) of O^T += V^T P^T, so P never leaves
//   registers.
// * O^T = V^T P^T keeps the output accumulator lane = query as well, so the
//   per-row rescale is lane-local. V stays row-major in LDS; its transpose is
//   taken by the gfx950 transposed LDS read (see fa_tile.h).
// * K and V tiles are double-buffered in LDS. Each wave runs a three-stage
//   software pipeline: in step i it multiplies P of tile i by V tile i,
//   exponentiates the scores of tile i + 1 and computes the scores of tile
//   i + 2, as one interleaved instruction stream, while the global loads of
//   K tile i + 3 and V tile i + 1 are in flight; one barrier per tile.
// * Exponentials use exp2 with log2(e) folded into the scale; the LSE is
//   converted back to natural-log units at the end.
// * Few vector-ALU operations per score (the matrix cores outrun them): P is
//   rounded to 16 bits once per tile (one packed conversion per two scores),
//   while the row sum l adds the unrounded float32 values, so the LSE keeps
//   float32 accuracy. The running maximum is not recomputed for every tile:
//   the tile's exponentials are first taken against the maximum held so
//   far, and only when their sum in some row exceeds kSumLimit (or the row
//   had no maximum yet) is the tile's true maximum found, U and l rescaled
//   by exp(m_old - m_new) and the exponentials redone. Every U and l stay
//   relative to the same m, so O = U / l and LSE = m + ln l are unchanged,
//   and P stays below kSumLimit.
#include <math.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"
#include "fa_tile.h"

namespace fa {
namespace {

constexpr float LN2 = 0.69314718055994530942f;
constexpr float LOG2E = 1.44269504088896340736f;
// Largest per-lane sum of a tile's exponentials accepted without moving the
// running maximum (bounds every P value; fits bf16 and fp16).
constexpr float kSumLimit = 1024.0f;

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int B, Hq, Hkv, G, Nq, Nkv, n_qtiles;
  float scale_log2;
  DropParams drop;  // used only by the dropout instantiations
};


// S^T = K Q^T for the 64 keys of the K tile at ks (DMA layout; kb0, kb1:
// this lane's k_read_base for even and odd kc): two 32-key blocks,
// accumulator r of block kb holds key kb * 32 + acc_key(h, r) of this lane's
// query row.
template <typename T, int D>
__device__ __forceinline__ void qk_tile(const uint8_t* ks, uint32_t kb0, uint32_t kb1,
                               const typename T::vec8* qf, f32x16* s) {
  constexpr int RB = DmaTile<D>::RB;
  constexpr int KC = D / 16;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    s[kb] = zero16();
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const uint8_t* p = ks + ((kc & 1) ? kb1 : kb0) + kb * 32 * RB + (kc >> 1) * 1024;
      s[kb] = T::mfma(as_vec8<T>(*reinterpret_cast<const u32x4*>(p)), qf[kc], s[kb]);
    }
  }
}

// P = exp2(S * scale_log2 - m) rounded to 16 bits, pk[4 ch + t] holding the
// keys 16 ch + 8 h + 2t, +1 of this lane's row (the B operand of chunk ch of
// O^T += V^T P^T); returns this lane's sum of the unrounded values. With
// dropout, values whose bit of kw (bit 2i, 2i + 1 for pair i) is clear enter
// P as zero but still count in the sum.
template <typename T, bool DROP = false>
__device__ __forceinline__ float exp_tile(const f32x16* s, float sl2, float m, uint32_t* pk,
                                          uint32_t kw = ~0u) {
  float psum = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float p0 = __builtin_amdgcn_exp2f(fmaf(s[i >> 3][2 * (i & 7)], sl2, -m));
    const float p1 = __builtin_amdgcn_exp2f(fmaf(s[i >> 3][2 * (i & 7) + 1], sl2, -m));
    if constexpr (DROP)
      pk[i] = pack2<T>(keep_f(p0, kw, 2 * i), keep_f(p1, kw, 2 * i + 1));
    else
      pk[i] = pack2<T>(p0, p1);
    psum += p0 + p1;
  }
  return psum;
}

// One step of the software pipeline, as a single interleaved instruction
// stream (the three parts are independent of each other):
//   * scores of tile i + 2:   sn = K Q^T         (kt: that K tile, D/8 products)
//   * output of tile i:       U += V^T P^T        (vt: V tile i, pc: P of tile i,
//                                                  D/8 products)
//   * exponentials of tile i + 1: pn = 16-bit exp2(se * scale_log2 - m)
// Matrix-core products alternate between the two products; every product's
// LDS operands are read two products ahead; each product is followed by its
// share of the exponentials; scheduling fences keep that order. Returns this
// lane's sum of the (unrounded) exponentials. With dropout, kw is the keep
// word of tile i + 1 (see exp_tile).
template <typename T, int D, bool DROP = false>
__device__ __forceinline__ float fused_tile(const uint8_t* kt, uint32_t kr0, uint32_t kr1,
                                   const typename T::vec8* qf, f32x16* sn, const uint8_t* vt,
                                   uint32_t vr, const uint32_t* pc, f32x16* oacc,
                                   const f32x16* se, float sl2, float m, uint32_t* pn,
                                   uint32_t kw = ~0u) {
  using V8 = typename T::vec8;
  constexpr int RB = DmaTile<D>::RB;
  constexpr int OD = D / 32;
  constexpr int NQ = D / 8;   // score products: kb = q % 2, kc = q / 2
  constexpr int NP = 4 * OD;  // output products: ch = p / OD, od = p % OD
  static_assert(NQ == NP, "alternating products");
  constexpr int NM = NQ + NP;
  auto kfrag = [&](int q) {
    const int kb = q & 1, kc = q >> 1;
    return *reinterpret_cast<const u32x4*>(kt + ((kc & 1) ? kr1 : kr0) + kb * 32 * RB +
                                           (kc >> 1) * 1024);
  };
  auto vfrag = [&](int p) { return load_vt_dma<T, D>(vt, vr, p / OD, p % OD); };
  sn[0] = zero16();
  sn[1] = zero16();
  u32x4 kf[NQ];
  V8 vf[NP];
  kf[0] = kfrag(0);
  kf[1] = kfrag(1);
  vf[0] = vfrag(0);
  vf[1] = vfrag(1);
  float psum = 0.0f, e0 = 0.0f, e1 = 0.0f;
#pragma unroll
  for (int t = 0; t < NM; ++t) {
    const int i = t >> 1;
    if ((t & 1) == 0) {
      if (i + 2 < NQ) kf[i + 2] = kfrag(i + 2);
      sn[i & 1] = T::mfma(as_vec8<T>(kf[i]), qf[i >> 1], sn[i & 1]);
    } else {
      if (i + 2 < NP) vf[i + 2] = vfrag(i + 2);
      const int ch = i / OD, od = i % OD;
      u32x4 w;
      w[0] = pc[4 * ch + 0];
      w[1] = pc[4 * ch + 1];
      w[2] = pc[4 * ch + 2];
      w[3] = pc[4 * ch + 3];
      oacc[od] = T::mfma(vf[i], as_vec8<T>(w), oacc[od]);
    }
    if constexpr (NM == 32) {  // half a pair of exponentials per product
      const int e = t >> 1;
      if ((t & 1) == 0) {
        e0 = __builtin_amdgcn_exp2f(fmaf(se[e >> 3][2 * (e & 7)], sl2, -m));
        e1 = __builtin_amdgcn_exp2f(fmaf(se[e >> 3][2 * (e & 7) + 1], sl2, -m));
      } else {
        if constexpr (DROP)
          pn[e] = pack2<T>(keep_f(e0, kw, 2 * e), keep_f(e1, kw, 2 * e + 1));
        else
          pn[e] = pack2<T>(e0, e1);
        psum += e0 + e1;
      }
    } else {  // one pair per product
      const int e = t;
      const float p0 = __builtin_amdgcn_exp2f(fmaf(se[e >> 3][2 * (e & 7)], sl2, -m));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(se[e >> 3][2 * (e & 7) + 1], sl2, -m));
      if constexpr (DROP)
        pn[e] = pack2<T>(keep_f(p0, kw, 2 * e), keep_f(p1, kw, 2 * e + 1));
      else
        pn[e] = pack2<T>(p0, p1);
      psum += p0 + p1;
    }
    // Keep the running sum in step (otherwise its adds drift to the end).
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

// NW waves of 32 query rows per workgroup: 8 (256 rows, one workgroup per
// CU, every staged K/V tile shared by 8 waves) when there are enough query
// tiles to fill the GPU, else 4 (128 rows, two workgroups per CU).
//
// Key/value tiles go through two LDS buffers each, loaded directly from
// global memory. Step i of the software pipeline reads K tile i + 2 and V
// tile i while the loads of K tile i + 3 and V tile i + 1 are in flight.
//
// DROP: dropout on P (keep words from keep_bits, one generator call per lane
// per tile; the two half-waves exchange the halves of their key groups), O
// scaled by 1 / (1 - p) at the end.
template <typename T, int D, bool CAUSAL, int NW, bool DROP>
__global__ __launch_bounds__(64 * NW, 8 / NW) void fwd_mfma_kernel(FwdArgs a) {
  constexpr int BR = 32 * NW;       // query rows per workgroup
  using V8 = typename T::vec8;
  using DT = DmaTile<D, NW>;
  constexpr int KC = D / 16;  // k-chunks of the QK^T contraction
  constexpr int OD = D / 32;  // 32-wide output column blocks
  constexpr int TB = DT::BYTES;

  // One array per buffer: with the step loop unrolled by two every access
  // names its buffer statically, so the compiler can see that a step's
  // operand reads never touch the buffers the in-flight loads are filling
  // and does not make the reads wait for those loads.
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf0[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf1[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf0[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf1[TB];
  auto kslot = [&](int x) __attribute__((always_inline)) -> uint8_t* { return x ? kbuf1 : kbuf0; };
  auto vslot = [&](int x) __attribute__((always_inline)) -> uint8_t* { return x ? vbuf1 : vbuf0; };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int h = lane >> 5;
  const int c = lane & 31;

  const TileId id = tile_of(blockIdx.x, a.B, a.Hq, a.Hkv, a.G, a.n_qtiles);
  const int qt = id.qt;
  const int b = id.b;
  const int hq = id.hq;
  const int hkv = hq / a.G;
  const int Nq = a.Nq, Nkv = a.Nkv;
  const int offset = Nkv - Nq;
  const size_t bh = (size_t)b * a.Hq + hq;

  const int q0 = qt * BR + wave * 32;  // first query row of this wave
  const int qrow = q0 + c;             // the row this lane owns

  // Key tiles this workgroup stages, and the ones this wave computes (the
  // wave's rows may stop seeing keys earlier under the causal mask).
  const int kv_tiles = (Nkv + BC - 1) / BC;
  int n_tiles = kv_tiles;
  if (CAUSAL) {
    const int last_key = min(Nq, (qt + 1) * BR) - 1 + offset;
    n_tiles = last_key < 0 ? 0 : min(kv_tiles, last_key / BC + 1);
  }
  const int wave_last_key = CAUSAL ? min(Nq - 1, q0 + 31) + offset : Nkv - 1;
  const int n_w = (q0 >= Nq || wave_last_key < 0) ? 0 : min(n_tiles, wave_last_key / BC + 1);

  const uint16_t* qptr = a.q + bh * Nq * D;
  const size_t kv_off = ((size_t)b * a.Hkv + hkv) * Nkv * D;
  // Bytes of K / V the workgroup may read: loads of later tiles fill zeros
  // without touching memory, so the pipeline may always issue its loads.
  const uint32_t kv_bytes = (uint32_t)min(Nkv, n_tiles * BC) * D * 2u;
  const uint16_t* const khead = a.k + kv_off;
  const uint16_t* const vhead = a.v + kv_off;
  const uint32_t k_src = k_dma_src<D, NW>(wave, lane);
  const uint32_t v_src = v_dma_src<D, NW>(wave, lane);
  const uint32_t kr0 = k_read_base<D>(h, c, 0);
  const uint32_t kr1 = k_read_base<D>(h, c, 1);
  const uint32_t vr = v_read_base<D>(h, c);
  constexpr int KS = DT::K_STEP, VS = DT::V_STEP;
  auto load_k = [&](int j, uint8_t* dst) __attribute__((always_inline)) {
    dma_tile<D, NW, KS>(dst, khead, kv_bytes, j * BC, wave, k_src);
  };
  auto load_v = [&](int j, uint8_t* dst) __attribute__((always_inline)) {
    dma_tile<D, NW, VS>(dst, vhead, kv_bytes, j * BC, wave, v_src);
  };

  // Q^T as the B operand: lane holds Q[qrow][16 kc + 8h .. +7].
  V8 qf[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
    qf[kc] = as_vec8<T>(qrow < Nq ? ld16(qptr + (size_t)qrow * D + kc * 16 + h * 8) : zero_u32x4());

  f32x16 oacc[OD];
#pragma unroll
  for (int od = 0; od < OD; ++od) oacc[od] = zero16();
  float m_run = -INFINITY;  // running max of scaled scores, log2 units
  float l_run = 0.0f;       // this half-wave's share of the running sum
  const float sl2 = a.scale_log2;

  // Mask keys past the end and, when causal, keys after the row's limit, in
  // the scores s of tile j.
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
  // When the exponentials p of scores s (taken against m_run) summed to more
  // than kSumLimit in some row: move the maximum to the true running maximum,
  // rescale what U and l hold, and redo p. Returns the new sum.
  auto fix_max = [&](const f32x16* s, uint32_t* p, float psum, uint32_t kw)
                     __attribute__((always_inline)) {
    if (__builtin_expect(__any(!(psum <= kSumLimit)), 0)) {
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
      for (int od = 0; od < OD; ++od)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[od][r] *= alpha;
      m_run = m_new;
      psum = exp_tile<T, DROP>(s, sl2, (m_new == -INFINITY) ? 0.0f : m_new, p, kw);
    }
    return psum;
  };

  // Dropout keep word of tile j for this lane (bit 16 kb + r: key
  // 64 j + 32 kb + acc_key(h, r)).
  auto keep_word = [&](int j) __attribute__((always_inline)) -> uint32_t {
    if constexpr (!DROP)
      return ~0u;
    else
      return row_keep_word(j, (uint32_t)qrow, (uint32_t)bh, h, a.drop);
  };

  // Pipeline state entering step i: scores of tile i + 1 and the 16-bit P of
  // tile i (already counted in l). Step i computes the scores of tile i + 2,
  // U += P_i V_i and P of tile i + 1. The two score arrays and the two P
  // arrays swap roles every step.
  f32x16 sa[2], sb[2];
  uint32_t pa[16], pb[16];

  // Prologue: K tiles 0 and 1 and V tile 0; scores and P of tile 0, scores
  // of tile 1; then K tile 2 into the buffer of K tile 0.
  load_k(0, kbuf0);
  load_k(1, kbuf1);
  load_v(0, vbuf0);
  __syncthreads();
  if (n_w > 0) {
    qk_tile<T, D>(kbuf0, kr0, kr1, qf, sa);
    mask_tile(0, sa);
    const uint32_t kw0 = keep_word(0);
    l_run += fix_max(sa, pa, exp_tile<T, DROP>(sa, sl2, m_run, pa, kw0), kw0);
    qk_tile<T, D>(kbuf1, kr0, kr1, qf, sb);
  }
  __syncthreads();
  load_k(2, kbuf0);
  __syncthreads();  // K tile 2 is read by step 0

  // Step i: loads of K tile i + 3 into buffer (i + 1) % 2 (last read for
  // the scores computed in step i - 1) and V tile i + 1 into buffer
  // (i + 1) % 2 (V tile i - 1, read in step i - 1); every wave passed the
  // barrier ending step i - 1, so neither buffer is still being read.
  auto step = [&](int i, f32x16* se, const uint32_t* pc, f32x16* sn, uint32_t* pn,
                  const uint8_t* kt, const uint8_t* vt) __attribute__((always_inline)) {
    const bool live = i + 1 < n_w;  // is there a tile i + 1 for this wave?
    uint32_t kw = ~0u;
    if (live) {
      mask_tile(i + 1, se);
      kw = keep_word(i + 1);
    }
    float psum = fused_tile<T, D, DROP>(kt, kr0, kr1, qf, sn, vt, vr, pc, oacc, se, sl2, m_run, pn, kw);
    if (live) l_run += fix_max(se, pn, psum, kw);
  };

  // Every wave runs n_tiles (loads, barrier) rounds and computes the first
  // n_w of them; the barrier also waits for the wave's own loads.
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

  // Epilogue: O = U / l, LSE = m + ln l (natural log).
  const float l = l_run + swap_halves(l_run);
  if (qrow < Nq) {
    const float inv = l > 0.0f ? (DROP ? a.drop.rscale : 1.0f) / l : 0.0f;
    uint16_t* orow = a.o + (bh * Nq + qrow) * D;
#pragma unroll
    for (int od = 0; od < OD; ++od)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 out;
        out[0] = pack2<T>(oacc[od][4 * g + 0] * inv, oacc[od][4 * g + 1] * inv);
        out[1] = pack2<T>(oacc[od][4 * g + 2] * inv, oacc[od][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + od * 32 + g * 8 + h * 4) = out;
      }
    if (h == 0) a.lse[bh * Nq + qrow] = l > 0.0f ? (m_run + __log2f(l)) * LN2 : -INFINITY;
  }
}

template <typename T, int D, int NW, bool DROP>
hipError_t launch_nw(const Problem& p, const FwdPtrs& t, hipStream_t stream, const DropParams* dp) {
  constexpr int BR = 32 * NW;
  FwdArgs a;
  a.q = static_cast<const uint16_t*>(t.q);
  a.k = static_cast<const uint16_t*>(t.k);
  a.v = static_cast<const uint16_t*>(t.v);
  a.o = static_cast<uint16_t*>(t.o);
  a.lse = t.lse;
  a.B = p.B;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.G = p.G;
  a.Nq = p.Nq;
  a.Nkv = p.Nkv;
  a.n_qtiles = (p.Nq + BR - 1) / BR;
  a.scale_log2 = p.scale * LOG2E;
  a.drop = dp ? *dp : DropParams{0, 0, 0, 1.0f};
  dim3 grid(a.n_qtiles * p.B * p.Hq);
  if (p.causal)
    hipLaunchKernelGGL((fwd_mfma_kernel<T, D, true, NW, DROP>), grid, dim3(64 * NW), 0, stream, a);
  else
    hipLaunchKernelGGL((fwd_mfma_kernel<T, D, false, NW, DROP>), grid, dim3(64 * NW), 0, stream, a);
  return hipGetLastError();
}

// 256-row workgroups when they alone fill the 256 CUs and the key range is
// long (N_q >= 4096), else 128-row ones: on shorter sequences two workgroups
// per CU overlap one's start-up with the other's main loop, which outweighs
// sharing each K/V tile among 8 waves instead of 4.
template <typename T, int D, bool DROP>
hipError_t launch_drop(const Problem& p, const FwdPtrs& t, hipStream_t stream, const DropParams* dp) {
  const long long big_tiles = (long long)p.B * p.Hq * ((p.Nq + 255) / 256);
  return (big_tiles >= 256 && p.Nq >= 4096) ? launch_nw<T, D, 8, DROP>(p, t, stream, dp)
                                            : launch_nw<T, D, 4, DROP>(p, t, stream, dp);
}

template <typename T, int D>
hipError_t launch_typed(const Problem& p, const FwdPtrs& t, hipStream_t stream, const DropParams* dp) {
  return dp ? launch_drop<T, D, true>(p, t, stream, dp) : launch_drop<T, D, false>(p, t, stream, dp);
}

}  // namespace

hipError_t launch_fwd_mfma(const Problem& p, const FwdPtrs& t, hipStream_t stream,
                           const DropParams* dp) {
  if (p.dt == FA_BF16) {
    return p.d == 64 ? launch_typed<BF16, 64>(p, t, stream, dp)
                     : launch_typed<BF16, 128>(p, t, stream, dp);
  }
  return p.d == 64 ? launch_typed<F16, 64>(p, t, stream, dp) : launch_typed<F16, 128>(p, t, stream, dp);
}

}  // namespace fa
