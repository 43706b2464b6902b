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
//   0  pre:   D_i for every query row (float32, in the workspace).
//   1  dK/dV: one workgroup per 128-key block of one (b, kv head). K and V of
//             the block stay in registers; the workgroup loops over the query
//             heads of the group (GQA/MQA: dK, dV summed in registers, no
//             atomics) and over the 64-row query tiles that can see the block
//             (causal: only tiles at or below the diagonal). Q / dO tiles are
//             double-buffered in LDS, the next one loading while the current
//             one is used. Per tile:
//               S = Q K^T and dP = dO V^T  (lane = key, 16 query rows / lane)
//               P, dS in registers
//               dV^T += dO^T P,  dK^T += Q^T dS   (accumulated in registers;
//               the transposed operands come from transposed LDS reads)
//             and finally writes dK (times scale) and dV. When there are too
//             few key blocks to fill the GPU (e.g. MQA), the query heads of a
//             group are split over several workgroups, which write float32
//             partial dK, dV to the workspace instead.
//   2  dQ:    one workgroup per query tile recomputes P and dS over the key
//             tiles and keeps dQ in registers (fa_bwd_dq.hip); with a split
//             head group, also dK = scale * sum of partials, dV = sum.
#include <math.h>

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
  const uint16_t* o;
  const float* lse;
  const uint16_t* dO;
  uint16_t* dk;
  uint16_t* dv;
  float* delta;
  float* dk_part;
  float* dv_part;
  int Hq, Hkv, G, Nq, Nkv, n_kblocks, n_bk, gsplit;
  float scale, scale_log2;
};

// ---------------------------------------------------------------- stage 0
// D_i = sum_c dO_ic O_ic in float32.
template <typename T, int D>
__global__ __launch_bounds__(NTB) void bwd_pre_kernel(const uint16_t* __restrict__ o,
                                                      const uint16_t* __restrict__ dO,
                                                      float* __restrict__ delta, size_t rows) {
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  constexpr int RPB = NTB / CPR;
  const int t = threadIdx.x;
  const size_t row = (size_t)blockIdx.x * RPB + t / CPR;
  const int ch = t % CPR;
  float acc = 0.0f;
  if (row < rows) {
    const u32x4 a = ld16(o + row * D + ch * 8);
    const u32x4 g = ld16(dO + row * D + ch * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = fmaf(T::to_float(a[i] & 0xffffu), T::to_float(g[i] & 0xffffu), acc);
      acc = fmaf(T::to_float(a[i] >> 16), T::to_float(g[i] >> 16), acc);
    }
  }
#pragma unroll
  for (int m = CPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (row < rows && ch == 0) delta[row] = acc;
}

// ---------------------------------------------------------------- stage 1
template <int D>
struct BwdLds {
  static constexpr int RS = D + 16;    // row stride of Q, dO tiles (32-byte pad)
  static constexpr int TILE = BQ * RS;
  static constexpr int Q_OFF = 0;                  // [2][BQ][RS]
  static constexpr int DO_OFF = Q_OFF + 2 * TILE;  // [2][BQ][RS]
  static constexpr int ELEMS = DO_OFF + 2 * TILE;
};

// Q / dO tile of BQ rows (plus the rows' LSE and D) held in registers between
// the global loads and the LDS write, so the loads of the next tile overlap
// the work on the current one.
template <int D>
struct QTileRegs {
  static constexpr int CH = (BQ * D / 8) / NTB;  // 16-byte chunks per thread, per tensor
  u32x4 q[CH];
  u32x4 g[CH];
  float lse2, delta;
};

template <int D>
__device__ inline void load_q_tile(QTileRegs<D>& r, const uint16_t* __restrict__ qh,
                                   const uint16_t* __restrict__ doh, const float* __restrict__ lse,
                                   const float* __restrict__ delta, int qi0, int Nq, int tid) {
#pragma unroll
  for (int i = 0; i < QTileRegs<D>::CH; ++i) {
    const int id = tid + NTB * i;
    const int row = id / (D / 8), dc = id % (D / 8);
    const bool in = qi0 + row < Nq;
    const size_t off = (size_t)(qi0 + row) * D + dc * 8;
    r.q[i] = in ? ld16(qh + off) : zero_u32x4();
    r.g[i] = in ? ld16(doh + off) : zero_u32x4();
  }
  if (tid < BQ) {
    const int row = qi0 + tid;
    r.lse2 = INFINITY;  // rows past the end, and rows that saw no key: P = 0
    r.delta = 0.0f;
    if (row < Nq) {
      const float l = lse[row];
      if (l != -INFINITY) r.lse2 = l * LOG2E;
      r.delta = delta[row];
    }
  }
}

template <int D>
__device__ inline void store_q_tile(const QTileRegs<D>& r, uint16_t* qs, uint16_t* gs,
                                    float* lse_s, float* del_s, int tid) {
  using L = BwdLds<D>;
#pragma unroll
  for (int i = 0; i < QTileRegs<D>::CH; ++i) {
    const int id = tid + NTB * i;
    const int row = id / (D / 8), dc = id % (D / 8);
    *reinterpret_cast<u32x4*>(qs + row * L::RS + dc * 8) = r.q[i];
    *reinterpret_cast<u32x4*>(gs + row * L::RS + dc * 8) = r.g[i];
  }
  if (tid < BQ) {
    lse_s[tid] = r.lse2;
    del_s[tid] = r.delta;
  }
}

// Two workgroups per CU at d = 64; at d = 128 the stationary K, V and the
// dK, dV accumulators alone take 192 of the 256 registers two waves per SIMD
// would leave, so one.
template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(NTB, D == 64 ? 2 : 1) void bwd_main_kernel(BwdArgs a) {
  using L = BwdLds<D>;
  using V8 = typename T::vec8;
  constexpr int KC = D / 16;
  constexpr int OD = D / 32;

  __shared__ __attribute__((aligned(16))) uint16_t sm[L::ELEMS];
  __shared__ __attribute__((aligned(16))) float lse_s[2][BQ];
  __shared__ __attribute__((aligned(16))) float del_s[2][BQ];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int h = lane >> 5;
  const int c = lane & 31;

  // Key blocks in ascending order: under the causal mask the first blocks
  // are seen by the most query tiles, so the heaviest work starts first.
  const int gsi = blockIdx.x % a.gsplit;   // which share of the head group
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

  const uint16_t* kbase = a.k + (size_t)bk * Nkv * D;
  const uint16_t* vbase = a.v + (size_t)bk * Nkv * D;

  // Stationary K and V as B operands: lane holds row my_key, dims 16kc + 8h.
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
  // workgroup's query heads, flattened into one loop.
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

  QTileRegs<D> regs;
  if (total > 0) {
    const size_t rb = ((size_t)b * a.Hq + hq0) * Nq;
    load_q_tile<D>(regs, a.q + rb * D, a.dO + rb * D, a.lse + rb, a.delta + rb, qt_begin * BQ, Nq, tid);
    store_q_tile<D>(regs, sm + L::Q_OFF, sm + L::DO_OFF, lse_s[0], del_s[0], tid);
  }
  __syncthreads();

  for (int it = 0; it < total; ++it) {
    const int buf = it & 1;
    const int hq = hq0 + it / per_head;
    const int qi0 = (qt_begin + it % per_head) * BQ;
    const size_t rowbase = ((size_t)b * a.Hq + hq) * Nq;
    const bool more = it + 1 < total;
    if (more) {
      const int hq_n = hq0 + (it + 1) / per_head;
      const int qi_n = (qt_begin + (it + 1) % per_head) * BQ;
      const size_t rb = ((size_t)b * a.Hq + hq_n) * Nq;
      load_q_tile<D>(regs, a.q + rb * D, a.dO + rb * D, a.lse + rb, a.delta + rb, qi_n, Nq, tid);
    }
    const uint16_t* qs = sm + L::Q_OFF + buf * L::TILE;
    const uint16_t* gs = sm + L::DO_OFF + buf * L::TILE;
    const float* ls = lse_s[buf];
    const float* ds_ = del_s[buf];

    // ---- S = Q K^T and dP = dO V^T (rows: query, columns: this wave's keys)
    f32x16 s[2], dp[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      s[qb] = zero16();
      dp[qb] = zero16();
      const uint16_t* qrow = qs + (qb * 32 + row_perm(c)) * L::RS + h * 8;
      const uint16_t* grow = gs + (qb * 32 + row_perm(c)) * L::RS + h * 8;
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        s[qb] = T::mfma(as_vec8<T>(*reinterpret_cast<const u32x4*>(qrow + kc * 16)), kf[kc], s[qb]);
        dp[qb] = T::mfma(as_vec8<T>(*reinterpret_cast<const u32x4*>(grow + kc * 16)), vf[kc], dp[qb]);
      }
    }
    // ---- P = exp(scale S - LSE), dS = P (dP - D); masks only where needed.
    const bool need_mask = (kw0 + 32 > Nkv) || (CAUSAL && kw0 + 31 > qi0 + offset);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int lq = qb * 32 + acc_key(h, r);
        float p = __builtin_amdgcn_exp2f(fmaf(s[qb][r], a.scale_log2, -ls[lq]));
        if (need_mask) {
          bool vis = my_key < Nkv;
          if (CAUSAL) vis = vis && (my_key <= qi0 + lq + offset);
          p = vis ? p : 0.0f;
        }
        s[qb][r] = p;
        dp[qb][r] = p * (dp[qb][r] - ds_[lq]);
      }
    // ---- dV^T += dO^T P and dK^T += Q^T dS (contraction over the BQ queries);
    // the transposed operands come from transposed LDS reads.
#pragma unroll
    for (int ch = 0; ch < BQ / 16; ++ch) {
      float pv[8], dv8[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        pv[t] = s[ch >> 1][(ch & 1) * 8 + t];
        dv8[t] = dp[ch >> 1][(ch & 1) * 8 + t];
      }
      const V8 pf = pack8<T>(pv);
      const V8 dsf = pack8<T>(dv8);
#pragma unroll
      for (int od = 0; od < OD; ++od) {
        dv[od] = T::mfma(load_vt_operand<T, L::RS>(gs, h, c, ch * 16, od * 32), pf, dv[od]);
        dk[od] = T::mfma(load_vt_operand<T, L::RS>(qs, h, c, ch * 16, od * 32), dsf, dk[od]);
      }
    }
    if (more)
      store_q_tile<D>(regs, sm + L::Q_OFF + (buf ^ 1) * L::TILE, sm + L::DO_OFF + (buf ^ 1) * L::TILE,
                      lse_s[buf ^ 1], del_s[buf ^ 1], tid);
    __syncthreads();
  }

  // ---- dK = scale * (sum dS^T Q) and dV (lane = key, 16 dims per tile); a
  // split head group writes float32 partial sums that stage 2 adds up.
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
  a.o = static_cast<const uint16_t*>(t.o);
  a.lse = t.lse;
  a.dO = static_cast<const uint16_t*>(t.dO);
  a.dk = static_cast<uint16_t*>(t.dk);
  a.dv = static_cast<uint16_t*>(t.dv);
  a.delta = t.delta;
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
  return a;
}

template <typename T, int D>
hipError_t pre_typed(const Problem& p, const BwdPtrs& t, hipStream_t stream) {
  const size_t rows = (size_t)p.B * p.Hq * p.Nq;
  if (rows == 0) return hipSuccess;
  constexpr int RPB = NTB / (D / 8);
  dim3 grid((unsigned)((rows + RPB - 1) / RPB));
  hipLaunchKernelGGL((bwd_pre_kernel<T, D>), grid, dim3(NTB), 0, stream,
                     static_cast<const uint16_t*>(t.o), static_cast<const uint16_t*>(t.dO), t.delta,
                     rows);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t main_typed(const Problem& p, const BwdPtrs& t, hipStream_t stream) {
  const BwdArgs a = make_args(p, t);
  if (a.n_kblocks == 0 || a.n_bk == 0) return hipSuccess;
  dim3 grid((unsigned)(a.n_kblocks * a.n_bk * a.gsplit));
  if (p.causal)
    hipLaunchKernelGGL((bwd_main_kernel<T, D, true>), grid, dim3(NTB), 0, stream, a);
  else
    hipLaunchKernelGGL((bwd_main_kernel<T, D, false>), grid, dim3(NTB), 0, stream, a);
  return hipGetLastError();
}

template <typename T>
hipError_t dq_typed(const Problem& p, const BwdPtrs& t, hipStream_t stream) {
  const hipError_t e = launch_bwd_dq_rows(p, t, stream);
  if (e != hipSuccess) return e;
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

hipError_t launch_bwd_pre(const Problem& p, const BwdPtrs& t, hipStream_t stream) {
  if (p.dt == FA_BF16) return p.d == 64 ? pre_typed<BF16, 64>(p, t, stream) : pre_typed<BF16, 128>(p, t, stream);
  return p.d == 64 ? pre_typed<F16, 64>(p, t, stream) : pre_typed<F16, 128>(p, t, stream);
}

hipError_t launch_bwd_main(const Problem& p, const BwdPtrs& t, hipStream_t stream) {
  if (p.dt == FA_BF16) return p.d == 64 ? main_typed<BF16, 64>(p, t, stream) : main_typed<BF16, 128>(p, t, stream);
  return p.d == 64 ? main_typed<F16, 64>(p, t, stream) : main_typed<F16, 128>(p, t, stream);
}

hipError_t launch_bwd_dq(const Problem& p, const BwdPtrs& t, hipStream_t stream) {
  return p.dt == FA_BF16 ? dq_typed<BF16>(p, t, stream) : dq_typed<F16>(p, t, stream);
}

}  // namespace fa
