// Backward, dQ (bf16 / fp16) on the gfx950 matrix cores.
//
// Method ([KB] "FlashAttention：为什么少搬数据，反而算得更快" §05: the forward
// kept only O and the row statistic LSE, so each probability tile is rebuilt
// on chip from it): for a tile of query rows, stream the key/value tiles the
// rows may see (as in the forward, [BLOG] §五 outer loop over query tiles,
// inner loop over key/value tiles) and per tile recompute
//   S = scale Q K^T,  P = exp(S - LSE),  dP = dO V^T,  dS = P (dP - D),
// then add
//   dQ += scale dS K.
// dQ stays in registers for the whole key range and is written once, in the
// input dtype: no atomics, no float32 accumulator in memory.
//
// This is the first backward stage: each lane also forms its row's
// D_i = sum_c dO_ic O_ic from the O and dO values it loads (its half of the
// row's dims, plus the other half-wave's), and stores the row terms -D_i and
// -LSE_i / scale that the key-block stage (fa_bwd.hip) starts its
// accumulators from.
//
// gfx950 mapping (as the forward kernel): one query row per lane; S^T = K Q^T
// and dP^T = V dO^T on v_mfma_f32_32x32x16 with Q and dO held as B operands
// in registers and K, V rows read from LDS; the rows' LSE and D are lane
// constants; dS^T is rounded to 16 bits in registers and is directly the B
// operand of dQ^T += K^T dS^T, whose A operand comes from transposed LDS
// reads of the same K tile. K and V tiles are double-buffered in LDS and
// filled by direct global -> LDS loads one tile ahead.
#include <math.h>

#include "fa_device.h"
#include "fa_internal.h"
#include "fa_tile.h"

namespace fa {
namespace {

constexpr float LOG2E = 1.44269504088896340736f;

struct DqArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dO;
  const uint16_t* o;
  const float* lse;
  float* nd;    // out: -D per query row (-D / r with dropout)
  float* lneg;  // out: -LSE / scale per query row (-inf: row saw no key)
  uint16_t* dq;
  int B, Hq, Hkv, G, Nq, Nkv, n_qtiles;
  float scale, scale_log2, inv_scale, inv_r;
  DropParams drop;  // used only by the dropout instantiations
};

// NW waves of 32 query rows per workgroup (8 when the grid fills the GPU,
// else 4), as in the forward.
//
// DROP: dropout with keep factor r; the row term is -D / r (also stored in
// nd), so dS / r = P ((Z ? dP : 0) - D / r), and dQ carries r at the end.
// The keep words are drawn as in the forward.
template <typename T, int D, bool CAUSAL, int NW, bool DROP>
__global__ __launch_bounds__(64 * NW, 8 / NW) void bwd_dq_kernel(DqArgs a) {
  constexpr int BR = 32 * NW;
  using V8 = typename T::vec8;
  using DT = DmaTile<D, NW>;
  constexpr int KC = D / 16;
  constexpr int OD = D / 32;
  constexpr int TB = DT::BYTES;

  // K and V tiles, both in the K layout (rows read for the products with Q
  // and dO, K also read transposed for dQ); one array per buffer so every
  // access names its buffer statically (the step loop is unrolled by two).
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf0[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf1[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf0[TB];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf1[TB];

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
  const bool has_row = qrow < Nq;

  const int kv_tiles = (Nkv + BC - 1) / BC;
  int n_tiles = kv_tiles;
  if (CAUSAL) {
    const int last_key = min(Nq, (qt + 1) * BR) - 1 + offset;
    n_tiles = last_key < 0 ? 0 : min(kv_tiles, last_key / BC + 1);
  }
  const int wave_last_key = CAUSAL ? min(Nq - 1, q0 + 31) + offset : Nkv - 1;
  const int n_w = (q0 >= Nq || wave_last_key < 0) ? 0 : min(n_tiles, wave_last_key / BC + 1);

  const size_t kv_off = ((size_t)b * a.Hkv + hkv) * Nkv * D;
  const uint32_t kv_bytes = (uint32_t)min(Nkv, n_tiles * BC) * D * 2u;
  const uint16_t* const khead = a.k + kv_off;
  const uint16_t* const vhead = a.v + kv_off;
  const uint32_t src = k_dma_src<D, NW>(wave, lane);
  const uint32_t kr0 = k_read_base<D>(h, c, 0);
  const uint32_t kr1 = k_read_base<D>(h, c, 1);
  const uint32_t kt0 = kt_read_base<D>(h, c, 0);
  const uint32_t kt1 = kt_read_base<D>(h, c, 1);
  auto load_kv = [&](int j, uint8_t* kd, uint8_t* vd) __attribute__((always_inline)) {
    dma_tile<D, NW, DT::K_STEP>(kd, khead, kv_bytes, j * BC, wave, src);
    dma_tile<D, NW, DT::K_STEP>(vd, vhead, kv_bytes, j * BC, wave, src);
  };

  // Q and dO of this lane's row as B operands (dims 16 kc + 8 h .. + 7), its
  // LSE (log2 units; +inf for a row that saw no key, so P = 0) and the row
  // term -D, D summed over this lane's dims and then the other half-wave's.
  // A lane past the last row loads row N_q - 1 instead: the loads then need
  // no branch and issue back to back. Such a lane's results stay in its own
  // registers (every value below is per row) and are never stored.
  const size_t row_off = bh * Nq + min(qrow, Nq - 1);
  const uint16_t* qp = a.q + row_off * D;
  const uint16_t* gp = a.dO + row_off * D;
  const uint16_t* op = a.o + row_off * D;
  const float lse_row = a.lse[row_off];
  V8 qf[KC], gf[KC];
  u32x4 gb[KC], ob[KC];  // dO and O of the same dims, for D
#pragma unroll
  for (int kc = 0; kc < KC; ++kc) {
    gb[kc] = ld16(gp + kc * 16 + h * 8);
    ob[kc] = ld16(op + kc * 16 + h * 8);
    qf[kc] = as_vec8<T>(ld16(qp + kc * 16 + h * 8));
    gf[kc] = as_vec8<T>(gb[kc]);
  }
  __builtin_amdgcn_sched_barrier(0);  // all row loads issue before the first copy
  // Set once the first K/V tile's copy is in flight (see below).
  float lse2 = INFINITY, ndrow = 0.0f;
  const float sl2 = a.scale_log2;

  f32x16 acc[OD];
#pragma unroll
  for (int od = 0; od < OD; ++od) acc[od] = zero16();

  // One key tile, as one instruction stream of 48 products with the vector
  // work spread over the last 32 (scheduling fences keep the order):
  //   S = K Q^T (16 products), then the mask on tiles that need it;
  //   dP = V dO^T (16): each followed by the exponentials of one pair of
  //     scores, P = exp2(S scale_log2 - LSE) kept in float32 in place of S;
  //   dQ^T += K^T dS^T (16, four per 16-key chunk ch): dS = P (dP - D)
  //     of the pairs of chunk ch, rounded to 16 bits, is formed while the
  //     products of chunk ch - 1 run (chunk 0's during the last dP products).
  // LDS operands are read two products ahead.
  auto compute = [&](int j, const uint8_t* kt, const uint8_t* vt) __attribute__((always_inline)) {
    constexpr int RB = DT::RB;
    uint32_t kw = ~0u;
    if constexpr (DROP) kw = row_keep_word(j, (uint32_t)qrow, (uint32_t)bh, h, a.drop);
    f32x16 s[2], dp[2];
    auto rfrag = [&](const uint8_t* xs, int q) {
      const int kb = q / KC, kc = q % KC;
      return *reinterpret_cast<const u32x4*>(xs + ((kc & 1) ? kr1 : kr0) + kb * 32 * RB +
                                             (kc >> 1) * 1024);
    };
    constexpr int NR = 2 * KC;  // products per score block pair (S or dP)
    u32x4 rf[NR];
    s[0] = zero16();
    s[1] = zero16();
    rf[0] = rfrag(kt, 0);
    rf[1] = rfrag(kt, 1);
#pragma unroll
    for (int q = 0; q < NR; ++q) {
      if (q + 2 < NR) rf[q + 2] = rfrag(kt, q + 2);
      s[q / KC] = T::mfma(as_vec8<T>(rf[q]), qf[q % KC], s[q / KC]);
    }
    const int key0 = j * BC;
    if ((key0 + BC > Nkv) || (CAUSAL && key0 + BC - 1 > q0 + offset)) {
      const int lim = CAUSAL ? min(Nkv - 1, qrow + offset) : Nkv - 1;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (key0 + kb * 32 + acc_key(h, r) > lim) s[kb][r] = -INFINITY;
    }
    // ds[4 ch + t] holds dS of keys 16 ch + 8 h + 2t, +1 (the B operand of
    // chunk ch of dQ^T += K^T dS^T); pair e of the scores is accumulators
    // 2 (e % 8), +1 of block e / 8.
    uint32_t ds[16];
    auto exp_pair = [&](int e) __attribute__((always_inline)) {
      const int kb = e >> 3, r = 2 * (e & 7);
      s[kb][r] = __builtin_amdgcn_exp2f(fmaf(s[kb][r], sl2, -lse2));
      s[kb][r + 1] = __builtin_amdgcn_exp2f(fmaf(s[kb][r + 1], sl2, -lse2));
    };
    auto ds_pair = [&](int e) __attribute__((always_inline)) {
      const int kb = e >> 3, r = 2 * (e & 7);
      if constexpr (DROP)
        ds[e] = pack2<T>(s[kb][r] * (keep_f(dp[kb][r], kw, 2 * e) + ndrow),
                         s[kb][r + 1] * (keep_f(dp[kb][r + 1], kw, 2 * e + 1) + ndrow));
      else
        ds[e] = pack2<T>(s[kb][r] * (dp[kb][r] + ndrow), s[kb][r + 1] * (dp[kb][r + 1] + ndrow));
    };
    dp[0] = zero16();
    dp[1] = zero16();
    rf[0] = rfrag(vt, 0);
    rf[1] = rfrag(vt, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < NR; ++q) {
      if (q + 2 < NR) rf[q + 2] = rfrag(vt, q + 2);
      dp[q / KC] = T::mfma(as_vec8<T>(rf[q]), gf[q % KC], dp[q / KC]);
      // 16 pairs of exponentials over the NR products, then the dS of
      // chunk 0 (block 0's dP is complete once half the products ran).
#pragma unroll
      for (int e = q * 16 / NR; e < (q + 1) * 16 / NR; ++e) exp_pair(e);
      if (q >= NR / 2 + NR / 4) {
#pragma unroll
        for (int e = (q - NR / 2 - NR / 4) * 4 / (NR / 4); e < (q + 1 - NR / 2 - NR / 4) * 4 / (NR / 4);
             ++e)
          ds_pair(e);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    V8 tf[4 * OD];
    tf[0] = load_kt_dma<T, D>(kt, kt0, kt1, 0, 0);
    tf[1] = load_kt_dma<T, D>(kt, kt0, kt1, 0, 1 % OD);
#pragma unroll
    for (int t = 0; t < 4 * OD; ++t) {
      const int ch = t / OD, od = t % OD;
      if (t + 2 < 4 * OD) tf[t + 2] = load_kt_dma<T, D>(kt, kt0, kt1, (t + 2) / OD, (t + 2) % OD);
      u32x4 w;
      w[0] = ds[4 * ch + 0];
      w[1] = ds[4 * ch + 1];
      w[2] = ds[4 * ch + 2];
      w[3] = ds[4 * ch + 3];
      acc[od] = T::mfma(tf[t], as_vec8<T>(w), acc[od]);
      // dS of chunk ch + 1 while chunk ch's products run.
      if (ch + 1 < 4) {
#pragma unroll
        for (int e = 4 * (ch + 1) + od * 4 / OD; e < 4 * (ch + 1) + (od + 1) * 4 / OD; ++e) ds_pair(e);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Tile j is computed from buffers j % 2 while tile j + 1 loads into the
  // others (last read during tile j - 1; every wave passed the barrier that
  // ended it). Every wave runs n_tiles rounds and computes the first n_w.
  load_kv(0, kbuf0, vbuf0);
  __builtin_amdgcn_sched_barrier(0);
  // The row terms, while the first tile's copy is in flight.
  {
    float dsum = 0.0f;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dsum = fmaf(T::to_float(ob[kc][i] & 0xffffu), T::to_float(gb[kc][i] & 0xffffu), dsum);
        dsum = fmaf(T::to_float(ob[kc][i] >> 16), T::to_float(gb[kc][i] >> 16), dsum);
      }
    ndrow = -(dsum + swap_halves(dsum)) * a.inv_r;
    if (has_row) {
      if (lse_row != -INFINITY) lse2 = lse_row * LOG2E;
      if (h == 0) {
        a.nd[row_off] = ndrow;
        a.lneg[row_off] = lse_row == -INFINITY ? -INFINITY : -lse_row * a.inv_scale;
      }
    }
  }
  __syncthreads();
  for (int j = 0; j < n_tiles; j += 2) {
    load_kv(j + 1, kbuf1, vbuf1);
    FA_STAGE_SYNC();
    if (j < n_w) compute(j, kbuf0, vbuf0);
    __syncthreads();
    if (j + 1 < n_tiles) {
      load_kv(j + 2, kbuf0, vbuf0);
      FA_STAGE_SYNC();
      if (j + 1 < n_w) compute(j + 1, kbuf1, vbuf1);
      __syncthreads();
    }
  }

  // dQ = scale * sum over key tiles of dS K (lane = query row, accumulator
  // rows = dims).
  if (has_row) {
    uint16_t* row = a.dq + (bh * Nq + qrow) * D;
    const float sc = DROP ? a.scale * a.drop.rscale : a.scale;
#pragma unroll
    for (int od = 0; od < OD; ++od)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 out;
        out[0] = pack2<T>(acc[od][4 * g + 0] * sc, acc[od][4 * g + 1] * sc);
        out[1] = pack2<T>(acc[od][4 * g + 2] * sc, acc[od][4 * g + 3] * sc);
        *reinterpret_cast<u32x2*>(row + od * 32 + g * 8 + h * 4) = out;
      }
  }
}

template <typename T, int D, int NW, bool DROP>
hipError_t launch_nw(const Problem& p, const BwdPtrs& t, hipStream_t stream) {
  DqArgs a;
  a.q = static_cast<const uint16_t*>(t.q);
  a.k = static_cast<const uint16_t*>(t.k);
  a.v = static_cast<const uint16_t*>(t.v);
  a.dO = static_cast<const uint16_t*>(t.dO);
  a.o = static_cast<const uint16_t*>(t.o);
  a.lse = t.lse;
  a.nd = t.nd;
  a.lneg = t.lneg;
  a.dq = static_cast<uint16_t*>(t.dq);
  a.B = p.B;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.G = p.G;
  a.Nq = p.Nq;
  a.Nkv = p.Nkv;
  a.n_qtiles = (p.Nq + 32 * NW - 1) / (32 * NW);
  a.scale = p.scale;
  a.scale_log2 = p.scale * LOG2E;
  a.inv_scale = 1.0f / p.scale;
  a.inv_r = t.drop ? 1.0f / t.drop->rscale : 1.0f;
  a.drop = t.drop ? *t.drop : DropParams{0, 0, 0, 1.0f};
  dim3 grid((unsigned)(a.n_qtiles * p.B * p.Hq));
  if (p.causal)
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, true, NW, DROP>), grid, dim3(64 * NW), 0, stream, a);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<T, D, false, NW, DROP>), grid, dim3(64 * NW), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_typed(const Problem& p, const BwdPtrs& t, hipStream_t stream) {
  const long long big_tiles = (long long)p.B * p.Hq * ((p.Nq + 255) / 256);
  const bool big = big_tiles >= 256 && p.Nq >= 4096;
  if (t.drop) return big ? launch_nw<T, D, 8, true>(p, t, stream) : launch_nw<T, D, 4, true>(p, t, stream);
  return big ? launch_nw<T, D, 8, false>(p, t, stream) : launch_nw<T, D, 4, false>(p, t, stream);
}

}  // namespace

hipError_t launch_bwd_dq_rows(const Problem& p, const BwdPtrs& t, hipStream_t stream) {
  if ((size_t)p.B * p.Hq * p.Nq == 0) return hipSuccess;
  if (p.dt == FA_BF16)
    return p.d == 64 ? launch_typed<BF16, 64>(p, t, stream) : launch_typed<BF16, 128>(p, t, stream);
  return p.d == 64 ? launch_typed<F16, 64>(p, t, stream) : launch_typed<F16, 128>(p, t, stream);
}

}  // namespace fa
