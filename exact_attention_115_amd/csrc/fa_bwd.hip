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
//   0  pre:   D_i for every query row; clear the float32 dQ accumulator.
//   1  main:  one workgroup per 128-key block of one (b, kv head). K and V of
//             the block stay in registers; the workgroup loops over the query
//             heads of the group (GQA/MQA: dK, dV summed in registers, no
//             atomics) and over the 64-row query tiles that can see the block
//             (causal: only tiles at or below the diagonal). Per tile:
//               S = Q K^T and dP = dO V^T  (lane = key, 16 query rows / lane)
//               P, dS in registers
//               dV^T += dO^T P,  dK^T += Q^T dS   (accumulated in registers)
//               dS -> LDS as [query][key]; dQ += dS K for the 128 keys,
//               added to the float32 accumulator with atomics
//             and finally writes dK (times scale) and dV.
//   2  dq:    dq = scale * accumulator, rounded to the input dtype.
#include <math.h>

#include "fa_device.h"
#include "fa_internal.h"

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
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* dq_acc;
  float* delta;
  int Hq, Hkv, G, Nq, Nkv, n_kblocks, n_bk;
  float scale, scale_log2;
};

// ---------------------------------------------------------------- stage 0
// D_i = sum_c dO_ic O_ic in float32; clear the dQ accumulator row.
template <typename T, int D>
__global__ __launch_bounds__(NTB) void bwd_pre_kernel(const uint16_t* __restrict__ o,
                                                      const uint16_t* __restrict__ dO,
                                                      float* __restrict__ delta,
                                                      float* __restrict__ dq_acc, size_t rows) {
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
    f32x4 z;
    z[0] = z[1] = z[2] = z[3] = 0.0f;
    *reinterpret_cast<f32x4*>(dq_acc + row * D + ch * 8) = z;
    *reinterpret_cast<f32x4*>(dq_acc + row * D + ch * 8 + 4) = z;
  }
#pragma unroll
  for (int m = CPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (row < rows && ch == 0) delta[row] = acc;
}

// ---------------------------------------------------------------- stage 1
template <int D>
struct BwdLds {
  static constexpr int QS = D + 8;     // Q, dO row stride   [BQ][D]
  static constexpr int TS = BQ + 8;    // Q^T, dO^T stride   [D][BQ]
  static constexpr int SS = BKV + 8;   // dS [BQ][BKV], K^T [D][BKV] stride
  static constexpr int Q_OFF = 0;
  static constexpr int DO_OFF = Q_OFF + BQ * QS;
  static constexpr int QT_OFF = DO_OFF + BQ * QS;
  static constexpr int DOT_OFF = QT_OFF + D * TS;
  static constexpr int DS_OFF = DOT_OFF + D * TS;
  static constexpr int KT_OFF = DS_OFF + BQ * SS;
  static constexpr int ELEMS = KT_OFF + D * SS;
};

// Write a block of 4 rows x 8 columns (held as 4 x 16 bytes) to LDS both
// row-major and transposed (8 runs of 4 elements).
__device__ inline void put_rows_and_transpose(const u32x4 (&x)[4], uint16_t* rm, int rm_stride,
                                              uint16_t* tr, int tr_stride) {
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) *reinterpret_cast<u32x4*>(rm + rr * rm_stride) = x[rr];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int w = e >> 1, sh = (e & 1) * 16;
    u32x2 out;
    out[0] = ((x[0][w] >> sh) & 0xffffu) | (((x[1][w] >> sh) & 0xffffu) << 16);
    out[1] = ((x[2][w] >> sh) & 0xffffu) | (((x[3][w] >> sh) & 0xffffu) << 16);
    *reinterpret_cast<u32x2*>(tr + e * tr_stride) = out;
  }
}

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(NTB) void bwd_main_kernel(BwdArgs a) {
  using L = BwdLds<D>;
  using V8 = typename T::vec8;
  constexpr int KC = D / 16;
  constexpr int OD = D / 32;
  constexpr int ITEMS = (BQ / 4) * (D / 8);  // 4x8 blocks of a Q / dO tile

  __shared__ __attribute__((aligned(16))) uint16_t sm[L::ELEMS];
  __shared__ __attribute__((aligned(16))) float lse_s[BQ];
  __shared__ __attribute__((aligned(16))) float del_s[BQ];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int h = lane >> 5;
  const int c = lane & 31;

  // Key blocks in ascending order: under the causal mask the first blocks
  // are seen by the most query tiles, so the heaviest work starts first.
  const int kt = blockIdx.x / a.n_bk;
  const int bk = blockIdx.x % a.n_bk;
  const int b = bk / a.Hkv;
  const int hkv = bk % a.Hkv;
  const int Nq = a.Nq, Nkv = a.Nkv;
  const int offset = Nkv - Nq;
  const int kblk0 = kt * BKV;
  const int my_key = kblk0 + wave * 32 + c;  // the key this lane's column holds

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
  // K^T of the block in LDS for dQ = dS K.
  {
    constexpr int KITEMS = (BKV / 4) * (D / 8);
    for (int it = tid; it < KITEMS; it += NTB) {
      const int r4 = it / (D / 8), dc = it % (D / 8);
      u32x4 x[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int key = kblk0 + r4 * 4 + rr;
        x[rr] = key < Nkv ? ld16(kbase + (size_t)key * D + dc * 8) : zero_u32x4();
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1, sh = (e & 1) * 16;
        u32x2 out;
        out[0] = ((x[0][w] >> sh) & 0xffffu) | (((x[1][w] >> sh) & 0xffffu) << 16);
        out[1] = ((x[2][w] >> sh) & 0xffffu) | (((x[3][w] >> sh) & 0xffffu) << 16);
        *reinterpret_cast<u32x2*>(sm + L::KT_OFF + (dc * 8 + e) * L::SS + r4 * 4) = out;
      }
    }
  }

  f32x16 dk[OD], dv[OD];
#pragma unroll
  for (int od = 0; od < OD; ++od) {
    dk[od] = zero16();
    dv[od] = zero16();
  }

  // Query tiles that can see some key of this block.
  const int n_qt = (Nq + BQ - 1) / BQ;
  int qt_begin = 0;
  if (CAUSAL) {
    const int first_q = kblk0 - offset;  // first query that sees key kblk0
    qt_begin = first_q <= 0 ? 0 : first_q / BQ;
  }

  for (int g = 0; g < a.G; ++g) {
    const int hq = hkv * a.G + g;
    const size_t rowbase = ((size_t)b * a.Hq + hq) * Nq;
    const uint16_t* qh = a.q + rowbase * D;
    const uint16_t* doh = a.dO + rowbase * D;
    for (int qt = qt_begin; qt < n_qt; ++qt) {
      const int qi0 = qt * BQ;
      // ---- stage the Q and dO tiles (row-major and transposed), LSE, D.
      if (tid < ITEMS) {
        const int r4 = tid / (D / 8), dc = tid % (D / 8);
        u32x4 xq[4], xd[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int row = qi0 + r4 * 4 + rr;
          const bool in = row < Nq;
          xq[rr] = in ? ld16(qh + (size_t)row * D + dc * 8) : zero_u32x4();
          xd[rr] = in ? ld16(doh + (size_t)row * D + dc * 8) : zero_u32x4();
        }
        put_rows_and_transpose(xq, sm + L::Q_OFF + (r4 * 4) * L::QS + dc * 8, L::QS,
                               sm + L::QT_OFF + (dc * 8) * L::TS + r4 * 4, L::TS);
        put_rows_and_transpose(xd, sm + L::DO_OFF + (r4 * 4) * L::QS + dc * 8, L::QS,
                               sm + L::DOT_OFF + (dc * 8) * L::TS + r4 * 4, L::TS);
      }
      if (tid < BQ) {
        const int row = qi0 + tid;
        float l2 = INFINITY, dl = 0.0f;
        if (row < Nq) {
          const float l = a.lse[rowbase + row];
          // A row that saw no key (LSE = -inf) has P = 0: use +inf.
          l2 = (l == -INFINITY) ? INFINITY : l * LOG2E;
          dl = a.delta[rowbase + row];
        }
        lse_s[tid] = l2;
        del_s[tid] = dl;
      }
      __syncthreads();

      // ---- S = Q K^T and dP = dO V^T (rows: query, columns: this wave's keys)
      f32x16 s[2], dp[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        s[qb] = zero16();
        dp[qb] = zero16();
        const uint16_t* qrow = sm + L::Q_OFF + (qb * 32 + row_perm(c)) * L::QS + h * 8;
        const uint16_t* drow = sm + L::DO_OFF + (qb * 32 + row_perm(c)) * L::QS + h * 8;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          s[qb] = T::mfma(as_vec8<T>(*reinterpret_cast<const u32x4*>(qrow + kc * 16)), kf[kc], s[qb]);
          dp[qb] = T::mfma(as_vec8<T>(*reinterpret_cast<const u32x4*>(drow + kc * 16)), vf[kc], dp[qb]);
        }
      }
      // ---- P = exp(scale S - LSE) (masked -> 0), dS = P (dP - D)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int lq = qb * 32 + acc_key(h, r);
          const int query = qi0 + lq;
          bool vis = my_key < Nkv && query < Nq;
          if (CAUSAL) vis = vis && (my_key <= query + offset);
          const float p = vis ? __builtin_amdgcn_exp2f(fmaf(s[qb][r], a.scale_log2, -lse_s[lq])) : 0.0f;
          s[qb][r] = p;
          dp[qb][r] = p * (dp[qb][r] - del_s[lq]);
        }
      // ---- dV^T += dO^T P and dK^T += Q^T dS (contraction over the 64 queries)
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
          const V8 a1 = as_vec8<T>(*reinterpret_cast<const u32x4*>(
              sm + L::DOT_OFF + (od * 32 + c) * L::TS + ch * 16 + h * 8));
          dv[od] = T::mfma(a1, pf, dv[od]);
          const V8 a2 = as_vec8<T>(*reinterpret_cast<const u32x4*>(
              sm + L::QT_OFF + (od * 32 + c) * L::TS + ch * 16 + h * 8));
          dk[od] = T::mfma(a2, dsf, dk[od]);
        }
      }
      // ---- dS to LDS as [query][key] (16-bit) for the dQ product.
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sm[L::DS_OFF + (qb * 32 + acc_key(h, r)) * L::SS + wave * 32 + c] = T::from_float(dp[qb][r]);
      __syncthreads();

      // ---- dQ[query][d] += sum over the block's 128 keys of dS K.
      // Output tiles (query block qb, dim block od); D = 128: 8 tiles, 2 per
      // wave; D = 64: 4 tiles, 1 per wave. Lane = dim column, so each atomic
      // instruction touches 32 consecutive floats of two rows.
      constexpr int TILES = 2 * OD;
      constexpr int PER_WAVE = TILES / 4;
#pragma unroll
      for (int ti = 0; ti < PER_WAVE; ++ti) {
        const int tile = wave * PER_WAVE + ti;
        const int qb = tile / OD, od = tile % OD;
        f32x16 acc = zero16();
        const uint16_t* dsrow = sm + L::DS_OFF + (qb * 32 + c) * L::SS + h * 8;
        const uint16_t* ktrow = sm + L::KT_OFF + (od * 32 + c) * L::SS + h * 8;
#pragma unroll
        for (int ch = 0; ch < BKV / 16; ++ch) {
          const V8 dsa = as_vec8<T>(*reinterpret_cast<const u32x4*>(dsrow + ch * 16));
          const V8 ktb = as_vec8<T>(*reinterpret_cast<const u32x4*>(ktrow + ch * 16));
          acc = T::mfma(dsa, ktb, acc);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int query = qi0 + qb * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (query < Nq)
            atomicAdd(a.dq_acc + (rowbase + query) * D + od * 32 + c, acc[r]);
        }
      }
    }
  }

  // ---- write dK = scale * (sum dS^T Q), dV (lane = key, 16 dims per tile).
  if (my_key < Nkv) {
    uint16_t* dkrow = a.dk + ((size_t)bk * Nkv + my_key) * D;
    uint16_t* dvrow = a.dv + ((size_t)bk * Nkv + my_key) * D;
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
  }
}

// ---------------------------------------------------------------- stage 2
template <typename T>
__global__ __launch_bounds__(NTB) void bwd_dq_kernel(const float* __restrict__ acc,
                                                     uint16_t* __restrict__ dq, size_t n8,
                                                     float scale) {
  const size_t i = (size_t)blockIdx.x * NTB + threadIdx.x;
  if (i >= n8) return;
  const f32x4 x0 = *reinterpret_cast<const f32x4*>(acc + i * 8);
  const f32x4 x1 = *reinterpret_cast<const f32x4*>(acc + i * 8 + 4);
  u32x4 out;
  out[0] = pack2<T>(x0[0] * scale, x0[1] * scale);
  out[1] = pack2<T>(x0[2] * scale, x0[3] * scale);
  out[2] = pack2<T>(x1[0] * scale, x1[1] * scale);
  out[3] = pack2<T>(x1[2] * scale, x1[3] * scale);
  st16(dq + i * 8, out);
}

BwdArgs make_args(const Problem& p, const BwdPtrs& t) {
  BwdArgs a;
  a.q = static_cast<const uint16_t*>(t.q);
  a.k = static_cast<const uint16_t*>(t.k);
  a.v = static_cast<const uint16_t*>(t.v);
  a.o = static_cast<const uint16_t*>(t.o);
  a.lse = t.lse;
  a.dO = static_cast<const uint16_t*>(t.dO);
  a.dq = static_cast<uint16_t*>(t.dq);
  a.dk = static_cast<uint16_t*>(t.dk);
  a.dv = static_cast<uint16_t*>(t.dv);
  a.dq_acc = t.dq_acc;
  a.delta = t.delta;
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
                     t.dq_acc, rows);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t main_typed(const Problem& p, const BwdPtrs& t, hipStream_t stream) {
  const BwdArgs a = make_args(p, t);
  if (a.n_kblocks == 0 || a.n_bk == 0) return hipSuccess;
  dim3 grid((unsigned)(a.n_kblocks * a.n_bk));
  if (p.causal)
    hipLaunchKernelGGL((bwd_main_kernel<T, D, true>), grid, dim3(NTB), 0, stream, a);
  else
    hipLaunchKernelGGL((bwd_main_kernel<T, D, false>), grid, dim3(NTB), 0, stream, a);
  return hipGetLastError();
}

template <typename T>
hipError_t dq_typed(const Problem& p, const BwdPtrs& t, hipStream_t stream) {
  const size_t n8 = (size_t)p.B * p.Hq * p.Nq * p.d / 8;
  if (n8 == 0) return hipSuccess;
  dim3 grid((unsigned)((n8 + NTB - 1) / NTB));
  hipLaunchKernelGGL((bwd_dq_kernel<T>), grid, dim3(NTB), 0, stream, t.dq_acc,
                     static_cast<uint16_t*>(t.dq), n8, p.scale);
  return hipGetLastError();
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
