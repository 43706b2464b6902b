// Backward pass (bf16 / fp16) on the gfx950 matrix cores.
//
// Method ([KB] "FlashAttention：为什么少搬数据，反而算得更快" §05; [NEWS]
// "FlashAttention技术原理详解"): the forward kept only O and the row statistic
// LSE, so each probability tile is rebuilt on chip, P = exp(scale Q K^T - LSE),
// used for the gradients, and dropped; no N x N matrix is read or written.
// Gradients of sum(dO * O) (the textbook chain rule; the pages print no
// formula):
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D_i = sum_c dO_ic O_ic,
//   dQ = scale dS K,  dK = scale dS^T Q.
// (D_i equals sum_j P_ij dP_ij because O = P V.)
//
// Three stages on one stream:
//   0  dQ:    one workgroup per query tile recomputes P and dS over the key
//             tiles and keeps dQ in registers (fa_bwd_dq.hip); it also
//             stores -D_i and -LSE_i / scale for every query row (float32,
//             in the workspace): the starting values of stage 1's dP and S
//             accumulators.
//   1  dK/dV: one workgroup per 128-key block of one (b, kv head). K and V of
//             the block stay in registers; the workgroup loops over the query
//             heads of the group (GQA/MQA: dK, dV summed in registers, no
//             atomics) and over the 64-row query tiles that can see the block
//             (causal: only tiles at or below the diagonal). Q / dO tiles go
//             through a ring of four LDS slots, loaded two tiles ahead of
//             their use. Per tile:
//               S = Q K^T and dP = dO V^T  (lane = key, 16 query rows / lane)
//               P, dS in registers
//               dV^T += dO^T P,  dK^T += Q^T dS   (accumulated in registers;
//               the transposed operands come from transposed LDS reads)
//             and finally writes dK (times scale) and dV. When there are too
//             few key blocks to fill the GPU (e.g. MQA), the query heads of a
//             group are split over several workgroups, which write float32
//             partial dK, dV to the workspace instead.
//   2  with a split head group only: dK = scale * sum of partials, dV = sum.
#include <math.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"
#include "fa_tile.h"

namespace fa {
namespace {

constexpr float LOG2E = 1.44269504088896340736f;
constexpr int NTB = 256;  // threads per workgroup
constexpr int BKV = 128;  // keys per workgroup (32 per wave)
constexpr int BQ = 64;    // query rows per inner tile

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dO;
  uint16_t* dk;
  uint16_t* dv;
  const float* lneg;   // -LSE / scale per query row (-inf: row saw no key)
  const float* nd;     // -D per query row (-D / r with dropout)
  float* dk_part;
  float* dv_part;
  int Hq, Hkv, G, Nq, Nkv, n_kblocks, n_bk, gsplit;
  float scale, scale_log2;
  DropParams drop;  // used only by the dropout instantiations
};

// ---------------------------------------------------------------- stage 1
// Accumulator start values from a tile's per-row terms x (64 floats in LDS):
// accumulator r of block qb holds query row qb * 32 + acc_key(h, r), two
// runs of eight consecutive rows per block.
__device__ __forceinline__ void init_rows(const float* x, int h, f32x16* acc) {
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int run = 0; run < 2; ++run)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(x + qb * 32 + run * 16 + 8 * h + 4 * half);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[qb][run * 8 + half * 4 + j] = v[j];
      }
}

// Matrix-core products of the dK/dV kernel, issued from inline assembly so
// that each accumulator stays in the register file its users need: the
// scores and dP (read by the vector ALU) in vector registers with the
// stationary K, V operand in accumulation registers (mfma_rows), dK and dV
// (read once, at the end) in accumulation registers (mfma_acc).
//
// The compiler places no wait states around inline assembly, and the
// hardware does not interlock these hazards of a 32x32x16 product (the wait
// states are those the compiler's hazard recognizer inserts for the same
// pairs written with builtins; tests/isa/hazard_rules.hip):
//   * vector-ALU write of an A / B operand or of the accumulator input, then
//     the product: 2. The A operands come from LDS (ordered by s_waitcnt);
//     the B operands of mfma_acc (P, dS) are packed in the step before the
//     one that uses them; the S / dP accumulators start from LDS loads
//     (init_rows) and dK / dV from zeros written once, before the loop. The
//     last tile's products (dkdv_tail), whose P / dS registers the compiler
//     selects with v_cndmask right before them, use mfma_acc_guarded, which
//     waits 2 states first.
//   * the product's result read by any other instruction (or overwritten by
//     the vector ALU): 12. Scores and dP are read only after xdl_wait()
//     (24); dK and dV only after the final xdl_wait().
//   * the result read as the next product's accumulator input, into the
//     same registers (the chains of S, dP, dK, dV): none.
// tests/test_isa_hazards.py compiles this file and checks every dK/dV
// instantiation's assembly against these rules, following the control flow,
// so that a change of instruction order or register allocation that breaks
// one of them fails on the CPU.
template <typename T>
__device__ __forceinline__ void mfma_rows(f32x16& c, typename T::vec8 a, typename T::vec8& b) {
  // b is tied in and out so that it is used in place, not copied per product.
  if constexpr (std::is_same_v<T, BF16>)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %2, %1, %0" : "+v"(c), "+a"(b) : "v"(a));
  else
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %2, %1, %0" : "+v"(c), "+a"(b) : "v"(a));
}
template <typename T>
__device__ __forceinline__ void mfma_acc(f32x16& c, typename T::vec8 a, typename T::vec8 b) {
  if constexpr (std::is_same_v<T, BF16>)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
// mfma_acc with two wait states before the product, for call sites where
// the compiler may write an operand register with a vector-ALU instruction
// just before (it selects the tail's P / dS registers with v_cndmask).
template <typename T>
__device__ __forceinline__ void mfma_acc_guarded(f32x16& c, typename T::vec8 a, typename T::vec8 b) {
  if constexpr (std::is_same_v<T, BF16>)
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
  else
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
// 24 wait states: more than a 32x32x16 product needs before another
// instruction may read its result.
__device__ __forceinline__ void xdl_wait() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// One step of the dK/dV pipeline for query tile i, as a single interleaved
// instruction stream of three independent parts:
//   * scores and dP of tile i + 1: sn = Q' K^T, dpn = dO' V^T (rows of the
//     next Q / dO tiles read from LDS; K, V stationary B operands)
//   * dV^T += dO^T P and dK^T += Q^T dS of tile i - 1 (PREV; transposed LDS
//     reads of that tile's Q / dO, its P and dS already rounded in pp, dsp)
//   * P = exp2(scale_log2 S') and dS = P dP' of tile i, rounded to 16 bits
//     into pc, dsc, where S' = S - LSE / scale and dP' = dP - D: the
//     accumulators of tile i + 1 start from its rows' -LSE / scale and -D
//     (ln, dn: those rows in LDS)
// Matrix-core products alternate between row and transposed products; LDS
// operands are read two products of their kind ahead; scheduling fences keep
// the order. Element pair e of a lane is keys' query rows 32 (e / 8) +
// acc_key(h, 2 (e % 8)), +1 (consecutive), and pc[4 ch + t] / dsc[4 ch + t]
// hold query rows 16 ch + 8 h + 2t, +1: the B operands of chunk ch.
//
// DROP (dropout, keep word kw: bit 2e, 2e + 1 for pair e): P enters dV as
// P o Z, and dS / r = P (Z ? dP' : -D / r) with the dP accumulators started
// from -D / r (dnc: tile i's -D / r rows); the factor r is applied to dK and
// dV at the end.
template <typename T, int D, bool PREV, bool DROP = false>
__device__ __forceinline__ void dkdv_step(
    const uint8_t* qn, const uint8_t* gn, const uint8_t* qp, const uint8_t* gp, uint32_t kr0,
    uint32_t kr1, uint32_t kt0, uint32_t kt1, typename T::vec8* kf, typename T::vec8* vf,
    f32x16* sn, f32x16* dpn, f32x16* dk, f32x16* dv, const uint32_t* pp, const uint32_t* dsp,
    const f32x16* s, const f32x16* dpc, const float* ln, const float* dn, int h, float sl2,
    uint32_t* pc, uint32_t* dsc, uint32_t kw = ~0u, const float* dnc = nullptr) {
  using V8 = typename T::vec8;
  constexpr int RB = DmaTile<D>::RB;
  constexpr int KC = D / 16;
  constexpr int OD = D / 32;
  constexpr int NR = 4 * KC;  // row products: x = r % 2 (S / dP), qb = (r / 2) % 2, kc = r / 4
  constexpr int NT = 8 * OD;  // transposed products: y = t % 2 (dV / dK), ch = (t / 2) / OD, od = (t / 2) % OD
  constexpr int NM = NR + NT;
  static_assert(64 % NM == 0, "whole parts per product");
  auto rfrag = [&](int r) {
    const int x = r & 1, qb = (r >> 1) & 1, kc = r >> 2;
    return *reinterpret_cast<const u32x4*>((x ? gn : qn) + ((kc & 1) ? kr1 : kr0) + qb * 32 * RB +
                                           (kc >> 1) * 1024);
  };
  auto tfrag = [&](int t) {
    const int y = t & 1, ch = (t >> 1) / OD, od = (t >> 1) % OD;
    return load_kt_dma<T, D>(y ? qp : gp, kt0, kt1, ch, od);
  };
  // With PREV the step opens with LEAD transposed products, which need no
  // row terms: their operands are read first, then the row terms of tile
  // i + 1 (16 reads) and the first row operands, so the first products do
  // not wait for the row-term reads (LDS returns in order).
  constexpr int LEAD = PREV ? 4 : 0;
  u32x4 rf[NR];
  V8 tf[NT];
  if constexpr (PREV) {
    tf[0] = tfrag(0);
    tf[1] = tfrag(1);
  }
  __builtin_amdgcn_sched_barrier(0);
  init_rows(ln, h, sn);
  init_rows(dn, h, dpn);
  rf[0] = rfrag(0);
  rf[1] = rfrag(1);
  __builtin_amdgcn_sched_barrier(0);
  float e0 = 0.0f, e1 = 0.0f;
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    // Product of slot m: without PREV, row product m / 2 on even slots;
    // with PREV, transposed products 0 .. LEAD - 1, then row j and
    // transposed j + LEAD alternating, then the last LEAD row products.
    bool is_row;
    int i;
    if constexpr (!PREV) {
      is_row = (m & 1) == 0;
      i = m >> 1;
    } else if (m < LEAD) {
      is_row = false;
      i = m;
    } else if (m < LEAD + 2 * (NT - LEAD)) {
      is_row = ((m - LEAD) & 1) == 0;
      i = ((m - LEAD) >> 1) + (is_row ? 0 : LEAD);
    } else {
      is_row = true;
      i = m - NT;
    }
    if (is_row) {
      if (i + 2 < NR) rf[i + 2] = rfrag(i + 2);
      const int x = i & 1, qb = (i >> 1) & 1, kc = i >> 2;
      if (x)
        mfma_rows<T>(dpn[qb], as_vec8<T>(rf[i]), vf[kc]);
      else
        mfma_rows<T>(sn[qb], as_vec8<T>(rf[i]), kf[kc]);
    } else if constexpr (PREV) {
      if (i + 2 < NT) tf[i + 2] = tfrag(i + 2);
      const int y = i & 1, ch = (i >> 1) / OD, od = (i >> 1) % OD;
      const uint32_t* w4 = (y ? dsp : pp) + 4 * ch;
      u32x4 w;
      w[0] = w4[0];
      w[1] = w4[1];
      w[2] = w4[2];
      w[3] = w4[3];
      if (y)
        mfma_acc<T>(dk[od], tf[i], as_vec8<T>(w));
      else
        mfma_acc<T>(dv[od], tf[i], as_vec8<T>(w));
    }
    // Tile i's P and dS: the 16 pairs in four parts each (fma + exp, the
    // rounding of P, the dS factors, the rounding of dS), spread evenly
    // over the NM products.
    constexpr int PARTS = 64 / NM;  // parts per product: 1 (d = 128) or 2 (d = 64)
#pragma unroll
    for (int u = 0; u < PARTS; ++u) {
      const int pidx = m * PARTS + u;
      const int e = pidx >> 2, part = pidx & 3;
      const int kb = e >> 3, r = 2 * (e & 7);
      if (part == 0) {
        e0 = __builtin_amdgcn_exp2f(s[kb][r] * sl2);
        e1 = __builtin_amdgcn_exp2f(s[kb][r + 1] * sl2);
      } else if (part == 1) {
        if constexpr (DROP)
          pc[e] = pack2<T>(keep_f(e0, kw, 2 * e), keep_f(e1, kw, 2 * e + 1));
        else
          pc[e] = pack2<T>(e0, e1);
      } else if (part == 2) {
        if constexpr (DROP) {
          const f32x2 nv = *reinterpret_cast<const f32x2*>(dnc + kb * 32 + acc_key(h, r));
          e0 = e0 * (((kw >> (2 * e)) & 1u) ? dpc[kb][r] : nv[0]);
          e1 = e1 * (((kw >> (2 * e + 1)) & 1u) ? dpc[kb][r + 1] : nv[1]);
        } else {
          e0 = e0 * dpc[kb][r];
          e1 = e1 * dpc[kb][r + 1];
        }
      } else {
        dsc[e] = pack2<T>(e0, e1);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// dV^T += dO^T P and dK^T += Q^T dS of one tile (the pipeline's last).
template <typename T, int D>
__device__ __forceinline__ void dkdv_tail(const uint8_t* qp, const uint8_t* gp, uint32_t kt0,
                                          uint32_t kt1, f32x16* dk, f32x16* dv, const uint32_t* pp,
                                          const uint32_t* dsp) {
  using V8 = typename T::vec8;
  constexpr int OD = D / 32;
#pragma unroll
  for (int ch = 0; ch < 4; ++ch) {
    u32x4 wp, ws;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      wp[t] = pp[4 * ch + t];
      ws[t] = dsp[4 * ch + t];
    }
#pragma unroll
    for (int od = 0; od < OD; ++od) {
      mfma_acc_guarded<T>(dv[od], load_kt_dma<T, D>(gp, kt0, kt1, ch, od), as_vec8<T>(wp));
      mfma_acc_guarded<T>(dk[od], load_kt_dma<T, D>(qp, kt0, kt1, ch, od), as_vec8<T>(ws));
    }
  }
}

// Rows of a Q-like tile: S[query][key] (accumulator r of block qb holds
// query qb * 32 + acc_key(h, r), lane column = this wave's key c) from the
// K-layout tile xs and the stationary B operand xf.
template <typename T, int D>
__device__ __forceinline__ void tile_rows(const uint8_t* xs, uint32_t kb0, uint32_t kb1,
                                          typename T::vec8* xf, const float* x0, int h,
                                          f32x16* s) {
  constexpr int RB = DmaTile<D>::RB;
  constexpr int KC = D / 16;
  init_rows(x0, h, s);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      const uint8_t* p = xs + ((kc & 1) ? kb1 : kb0) + qb * 32 * RB + (kc >> 1) * 1024;
      mfma_rows<T>(s[qb], as_vec8<T>(*reinterpret_cast<const u32x4*>(p)), xf[kc]);
    }
  }
}

template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

// One workgroup of 4 waves per 128-key block (32 keys per wave) of one
// (b, kv head) and one share of the head group. Q / dO tiles of BQ = 64 rows
// (and their -LSE / scale, -D rows) go through a ring of 4 LDS slots filled by direct
// global -> LDS loads two tiles ahead; step i reads tile i + 1 (rows), tile
// i + 1 (row terms) and tile i - 1 (transposed). One wave per SIMD: the stationary
// K, V, the dK, dV accumulators and two tiles of scores and P need more than
// the 256 registers two waves per SIMD would leave.
//
// DROP: dropout. Each tile's keep bits are drawn once per lane (lane l: query
// row l of the tile, the wave's 32 keys) and turned through LDS into the
// lane = key layout.
template <typename T, int D, bool CAUSAL, bool DROP>
__global__ __launch_bounds__(NTB, 1) void bwd_dkdv_kernel(BwdArgs a) {
  using V8 = typename T::vec8;
  using DT = DmaTile<D, 4>;
  constexpr int KC = D / 16;
  constexpr int OD = D / 32;
  constexpr int TB = DT::BYTES;
  static_assert(BQ == BC, "query tiles use the key-tile layout");

  __shared__ __attribute__((aligned(1024))) uint8_t qs0[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t qs1[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t qs2[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t qs3[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t gs0[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t gs1[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t gs2[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t gs3[TB];
  __shared__ __attribute__((aligned(256))) float ls0[BQ], ls1[BQ], ls2[BQ], ls3[BQ];
  __shared__ __attribute__((aligned(256))) float ds0[BQ], ds1[BQ], ds2[BQ], ds3[BQ];
  __shared__ __attribute__((aligned(256))) uint32_t kwbuf[DROP ? 4 * BQ : 4];
  auto qslot = [&](int x) __attribute__((always_inline)) -> uint8_t* {
    return x == 0 ? qs0 : x == 1 ? qs1 : x == 2 ? qs2 : qs3;
  };
  auto gslot = [&](int x) __attribute__((always_inline)) -> uint8_t* {
    return x == 0 ? gs0 : x == 1 ? gs1 : x == 2 ? gs2 : gs3;
  };
  auto lslot = [&](int x) __attribute__((always_inline)) -> float* {
    return x == 0 ? ls0 : x == 1 ? ls1 : x == 2 ? ls2 : ls3;
  };
  auto dslot = [&](int x) __attribute__((always_inline)) -> float* {
    return x == 0 ? ds0 : x == 1 ? ds1 : x == 2 ? ds2 : ds3;
  };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int h = lane >> 5;
  const int c = lane & 31;

  // Key blocks in ascending order: under the causal mask the first blocks
  // are seen by the most query tiles, so the heaviest work starts first.
  const int gsi = blockIdx.x % a.gsplit;  // which share of the head group
  const int rest = blockIdx.x / a.gsplit;
  const int kt = rest / a.n_bk;
  const int bk = rest % a.n_bk;
  const int b = bk / a.Hkv;
  const int hkv = bk % a.Hkv;
  const int Nq = a.Nq, Nkv = a.Nkv;
  const int offset = Nkv - Nq;
  const int kblk0 = kt * BKV;
  const int kw0 = kblk0 + wave * 32;  // first key of this wave
  const int my_key = kw0 + c;         // the key this lane's column holds

  // Stationary K and V as B operands: lane holds row my_key, dims 16kc + 8h.
  const uint16_t* kbase = a.k + (size_t)bk * Nkv * D;
  const uint16_t* vbase = a.v + (size_t)bk * Nkv * D;
  V8 kf[KC], vf[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    const bool in = my_key < Nkv;
    kf[kc] = as_vec8<T>(in ? ld16(kbase + (size_t)my_key * D + kc * 16 + h * 8) : zero_u32x4());
    vf[kc] = as_vec8<T>(in ? ld16(vbase + (size_t)my_key * D + kc * 16 + h * 8) : zero_u32x4());
  }
  f32x16 dk[OD], dv[OD];
#pragma unroll
  for (int od = 0; od < OD; ++od) {
    dk[od] = zero16();
    dv[od] = zero16();
  }

  // Query tiles that can see some key of this block, for each of this
  // workgroup's query heads, flattened into one sequence.
  const int n_qt = (Nq + BQ - 1) / BQ;
  int qt_begin = 0;
  if (CAUSAL) {
    const int first_q = kblk0 - offset;  // first query that sees key kblk0
    qt_begin = first_q <= 0 ? 0 : min(n_qt, first_q / BQ);
  }
  const int per_head = n_qt - qt_begin;
  const int heads = a.G / a.gsplit;
  const int total = per_head * heads;
  const int hq0 = hkv * a.G + gsi * heads;

  const uint32_t src = k_dma_src<D, 4>(wave, lane);
  const uint32_t kr0 = k_read_base<D>(h, c, 0);
  const uint32_t kr1 = k_read_base<D>(h, c, 1);
  const uint32_t kt0 = kt_read_base<D>(h, c, 0);
  const uint32_t kt1 = kt_read_base<D>(h, c, 1);
  // Tile t (query head, first row) into slot x: Q and dO rows (reads past
  // N_q fill zeros, which add nothing to dK, dV), -LSE / scale and -D rows.
  // Each copy's buffer resource starts at the tile's own first row (64-bit
  // address arithmetic) and spans only the tile's rows, so the 32-bit range
  // of the resource never depends on the length of the query sequence.
  auto load_tile = [&](int t, int x) __attribute__((always_inline)) {
    if (t >= total) return;
    const int hq = hq0 + t / per_head;
    const int qi0 = (qt_begin + t % per_head) * BQ;  // < Nq
    const size_t r0 = ((size_t)b * a.Hq + hq) * Nq + qi0;
    const uint32_t rows_left = (uint32_t)min(Nq - qi0, BQ);
    const uint32_t tile_bytes = rows_left * (uint32_t)DT::RB;
    dma_tile<D, 4, DT::K_STEP>(qslot(x), a.q + r0 * D, tile_bytes, 0, wave, src);
    dma_tile<D, 4, DT::K_STEP>(gslot(x), a.dO + r0 * D, tile_bytes, 0, wave, src);
    if (wave < 2) {
      const float* rows = (wave == 0 ? a.lneg : a.nd) + r0;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          make_rsrc(rows, rows_left * 4u),
          (__attribute__((address_space(3))) void*)(wave == 0 ? lslot(x) : dslot(x)), 4,
          (uint32_t)lane * 4u, 0, 0, 0);
    }
  };
  // Mask tile t's scores s where a key is past the end or, when causal,
  // after the query's limit.
  auto mask_tile = [&](int t, f32x16* s) __attribute__((always_inline)) {
    const int qi0 = (qt_begin + t % per_head) * BQ;
    const bool need_mask = (kw0 + 32 > Nkv) || (CAUSAL && kw0 + 31 > qi0 + offset);
    if (need_mask) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          bool vis = my_key < Nkv;
          if (CAUSAL) vis = vis && (my_key <= qi0 + qb * 32 + acc_key(h, r) + offset);
          s[qb][r] = vis ? s[qb][r] : -INFINITY;
        }
    }
  };

  // Dropout keep word of tile t for this lane (bit 16 qb + r: query row
  // qb * 32 + acc_key(h, r) of the tile, key my_key). Lane l draws row l's
  // decisions for the wave's 32 keys; the words go through this wave's LDS
  // block, and each lane picks its key's bit from its 32 rows.
  auto keep_word = [&](int t) __attribute__((always_inline)) -> uint32_t {
    if constexpr (!DROP) {
      return ~0u;
    } else {
      const int hq = hq0 + t / per_head;
      const int qi0 = (qt_begin + t % per_head) * BQ;
      const uint32_t w = keep_bits((uint32_t)(kw0 >> 5), (uint32_t)(qi0 + lane),
                                   (uint32_t)(b * a.Hq + hq), a.drop);
      uint32_t* buf = kwbuf + wave * BQ;
      buf[lane] = w;
      __builtin_amdgcn_wave_barrier();
      uint32_t kw = 0;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int run = 0; run < 2; ++run)
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(buf + qb * 32 + run * 16 + 8 * h + 4 * half);
#pragma unroll
            for (int j = 0; j < 4; ++j) kw |= ((x[j] >> c) & 1u) << (16 * qb + 8 * run + 4 * half + j);
          }
      __builtin_amdgcn_wave_barrier();
      return kw;
    }
  };

  // Pipeline state entering step i: scores and dP of tile i, P and dS of tile
  // i - 1. Tile t's scores live in sa/da and its P, dS in pa/za when t is
  // even, in sb/db and pb/zb when t is odd.
  f32x16 sa[2], da[2], sb[2], db[2];
  uint32_t pa[16], za[16], pb[16], zb[16];
  const float sl2 = a.scale_log2;

  // Prologue: tiles 0 and 1; scores of tile 0; step 0 (no tile -1).
  load_tile(0, 0);
  load_tile(1, 1);
  __syncthreads();
  if (total > 0) {
    tile_rows<T, D>(qs0, kr0, kr1, kf, ls0, h, sa);
    tile_rows<T, D>(gs0, kr0, kr1, vf, ds0, h, da);
    load_tile(2, 2);
    FA_STAGE_SYNC();
    const uint32_t kwt = keep_word(0);
    xdl_wait();
    mask_tile(0, sa);
    dkdv_step<T, D, false, DROP>(qs1, gs1, qs3, gs3, kr0, kr1, kt0, kt1, kf, vf, sb, db, dk, dv, pb,
                                 zb, sa, da, ls1, ds1, h, sl2, pa, za, kwt, ds0);
  }
  __syncthreads();

  // Step i: tile i + 2 loads into slot (i + 2) % 4, whose tile i - 2 was
  // last read in step i - 1 (every wave passed the barrier that ended it);
  // the step reads slots (i + 1) % 4 (rows and row terms) and
  // (i - 1) % 4 (transposed). With i = 1 + 4 n + r every slot and array is
  // named statically.
  for (int i0 = 1; i0 < total; i0 += 4) {
    static_for<4>([&](auto rc) __attribute__((always_inline)) {
      constexpr int r = decltype(rc)::value;
      constexpr bool even = (r & 1) == 1;  // is tile i = i0 + r even?
      const int i = i0 + r;
      if (i < total) {
        load_tile(i + 2, (r + 3) & 3);
        FA_STAGE_SYNC();
        f32x16* s = even ? sa : sb;
        f32x16* dpc = even ? da : db;
        const uint32_t kwt = keep_word(i);
        xdl_wait();  // the scores and dP of tile i were written last step
        mask_tile(i, s);
        dkdv_step<T, D, true, DROP>(qslot((r + 2) & 3), gslot((r + 2) & 3), qslot(r & 3),
                                    gslot(r & 3), kr0, kr1, kt0, kt1, kf, vf, even ? sb : sa,
                                    even ? db : da, dk, dv, even ? pb : pa, even ? zb : za, s, dpc,
                                    lslot((r + 2) & 3), dslot((r + 2) & 3), h, sl2, even ? pa : pb,
                                    even ? za : zb, kwt, dslot((r + 1) & 3));
        __syncthreads();
      }
    });
  }
  // The last tile's dV, dK.
  if (total > 0) {
    const int x = (total - 1) & 3;
    const bool odd = (total - 1) & 1;
    dkdv_tail<T, D>(qslot(x), gslot(x), kt0, kt1, dk, dv, odd ? pb : pa, odd ? zb : za);
  }
  xdl_wait();

  // ---- dK = scale * (sum dS^T Q) and dV (lane = key, 16 dims per tile); a
  // split head group writes float32 partial sums that stage 2 adds up. With
  // dropout both carry the keep factor r.
  if constexpr (DROP) {
#pragma unroll
    for (int od = 0; od < OD; ++od)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        dk[od][i] *= a.drop.rscale;
        dv[od][i] *= a.drop.rscale;
      }
  }
  if (my_key < Nkv) {
    const size_t row = (size_t)bk * Nkv + my_key;
    if (a.gsplit == 1) {
      uint16_t* dkrow = a.dk + row * D;
      uint16_t* dvrow = a.dv + row * D;
#pragma unroll
      for (int od = 0; od < OD; ++od)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          u32x2 ok, ov;
          ok[0] = pack2<T>(dk[od][4 * g4 + 0] * a.scale, dk[od][4 * g4 + 1] * a.scale);
          ok[1] = pack2<T>(dk[od][4 * g4 + 2] * a.scale, dk[od][4 * g4 + 3] * a.scale);
          ov[0] = pack2<T>(dv[od][4 * g4 + 0], dv[od][4 * g4 + 1]);
          ov[1] = pack2<T>(dv[od][4 * g4 + 2], dv[od][4 * g4 + 3]);
          const int d0 = od * 32 + g4 * 8 + h * 4;
          *reinterpret_cast<u32x2*>(dkrow + d0) = ok;
          *reinterpret_cast<u32x2*>(dvrow + d0) = ov;
        }
    } else {
      const size_t plane = (size_t)a.n_bk * Nkv * D;
      float* pk = a.dk_part + gsi * plane + row * D;
      float* pv = a.dv_part + gsi * plane + row * D;
#pragma unroll
      for (int od = 0; od < OD; ++od)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          f32x4 xk, xv;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            xk[i] = dk[od][4 * g4 + i];
            xv[i] = dv[od][4 * g4 + i];
          }
          const int d0 = od * 32 + g4 * 8 + h * 4;
          *reinterpret_cast<f32x4*>(pk + d0) = xk;
          *reinterpret_cast<f32x4*>(pv + d0) = xv;
        }
    }
  }
}

// ---------------------------------------------------------------- stage 2
// dK = scale * sum of the partial sums, dV = sum, when the head group of a
// key block was split across workgroups (fixed order: deterministic).
template <typename T>
__global__ __launch_bounds__(NTB) void bwd_kv_reduce_kernel(const float* __restrict__ pk,
                                                            const float* __restrict__ pv,
                                                            uint16_t* __restrict__ dk,
                                                            uint16_t* __restrict__ dv, size_t n4,
                                                            int parts, float scale) {
  const size_t i = (size_t)blockIdx.x * NTB + threadIdx.x;
  if (i >= n4) return;
  f32x4 sk = *reinterpret_cast<const f32x4*>(pk + i * 4);
  f32x4 sv = *reinterpret_cast<const f32x4*>(pv + i * 4);
  for (int g = 1; g < parts; ++g) {
    const f32x4 xk = *reinterpret_cast<const f32x4*>(pk + (size_t)g * n4 * 4 + i * 4);
    const f32x4 xv = *reinterpret_cast<const f32x4*>(pv + (size_t)g * n4 * 4 + i * 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sk[j] += xk[j];
      sv[j] += xv[j];
    }
  }
  u32x2 ok, ov;
  ok[0] = pack2<T>(sk[0] * scale, sk[1] * scale);
  ok[1] = pack2<T>(sk[2] * scale, sk[3] * scale);
  ov[0] = pack2<T>(sv[0], sv[1]);
  ov[1] = pack2<T>(sv[2], sv[3]);
  *reinterpret_cast<u32x2*>(dk + i * 4) = ok;
  *reinterpret_cast<u32x2*>(dv + i * 4) = ov;
}

BwdArgs make_args(const Problem& p, const BwdPtrs& t) {
  BwdArgs a;
  a.q = static_cast<const uint16_t*>(t.q);
  a.k = static_cast<const uint16_t*>(t.k);
  a.v = static_cast<const uint16_t*>(t.v);
  a.dO = static_cast<const uint16_t*>(t.dO);
  a.dk = static_cast<uint16_t*>(t.dk);
  a.dv = static_cast<uint16_t*>(t.dv);
  a.lneg = t.lneg;
  a.nd = t.nd;
  a.dk_part = t.dk_part;
  a.dv_part = t.dv_part;
  a.gsplit = bwd_group_split(p);
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.G = p.G;
  a.Nq = p.Nq;
  a.Nkv = p.Nkv;
  a.n_kblocks = (p.Nkv + BKV - 1) / BKV;
  a.n_bk = p.B * p.Hkv;
  a.scale = p.scale;
  a.scale_log2 = p.scale * LOG2E;
  a.drop = t.drop ? *t.drop : DropParams{0, 0, 0, 1.0f};
  return a;
}

template <typename T, int D>
hipError_t main_typed(const Problem& p, const BwdPtrs& t, hipStream_t stream) {
  const BwdArgs a = make_args(p, t);
  if (a.n_kblocks == 0 || a.n_bk == 0) return hipSuccess;
  dim3 grid((unsigned)(a.n_kblocks * a.n_bk * a.gsplit));
  if (t.drop) {
    if (p.causal)
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, true, true>), grid, dim3(NTB), 0, stream, a);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, false, true>), grid, dim3(NTB), 0, stream, a);
  } else {
    if (p.causal)
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, true, false>), grid, dim3(NTB), 0, stream, a);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, false, false>), grid, dim3(NTB), 0, stream, a);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t reduce_typed(const Problem& p, const BwdPtrs& t, hipStream_t stream) {
  const int parts = bwd_group_split(p);
  const size_t n4 = (size_t)p.B * p.Hkv * p.Nkv * p.d / 4;
  if (parts > 1 && n4 > 0) {
    dim3 grid((unsigned)((n4 + NTB - 1) / NTB));
    hipLaunchKernelGGL((bwd_kv_reduce_kernel<T>), grid, dim3(NTB), 0, stream, t.dk_part,
                       t.dv_part, static_cast<uint16_t*>(t.dk), static_cast<uint16_t*>(t.dv), n4,
                       parts, p.scale);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_bwd_main(const Problem& p, const BwdPtrs& t, hipStream_t stream) {
  if (p.dt == FA_BF16) return p.d == 64 ? main_typed<BF16, 64>(p, t, stream) : main_typed<BF16, 128>(p, t, stream);
  return p.d == 64 ? main_typed<F16, 64>(p, t, stream) : main_typed<F16, 128>(p, t, stream);
}

hipError_t launch_bwd_reduce(const Problem& p, const BwdPtrs& t, hipStream_t stream) {
  return p.dt == FA_BF16 ? reduce_typed<BF16>(p, t, stream) : reduce_typed<F16>(p, t, stream);
}

}  // namespace fa
