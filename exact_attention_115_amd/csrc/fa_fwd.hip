// 16-bit (bf16 / fp16) forward on the gfx950 matrix cores.
//
// Method ([BLOG] "AI infra. 一层全看懂(五)Flash Attention" §五; [KB]
// "FlashAttention：为什么少搬数据，反而算得更快" §03-§04): one workgroup per
// tile of 128 query rows (the outer loop); it walks the key/value tiles of 64
// rows its rows may see (the inner loop). Each score tile S = Q K^T is
// produced on chip, scaled, masked and folded at once into per-row online
// softmax state -- m (running maximum), l (running sum of exp(s - m)) and the
// un-normalised output U, with the held part rescaled by exp(m_old - m_new)
// ([KB] §04) -- then discarded. Only O and the row LSE = m + ln l leave the
// chip, so no N x N matrix is ever written to memory.
//
// gfx950 mapping:
// * 4 waves per workgroup, 32 query rows per wave. The score tile is computed
//   transposed, S^T = K Q^T, on v_mfma_f32_32x32x16: the query index is the
//   matrix-core column, so every lane owns ONE query row (half of its keys in
//   each half-wave) and the row max / row sum need only lane-local work plus
//   one exchange between the two half-waves.
// * K rows are fed to the matrix core in the order row_perm() gives, which
//   leaves each lane's accumulators holding runs of 8 consecutive keys: they
//   are, unchanged, the B operand (P^T) of O^T += V^T P^T, so P never leaves
//   registers.
// * O^T = V^T P^T keeps the output accumulator lane = query as well, so the
//   per-row rescale is lane-local. V stays row-major in LDS; its transpose is
//   taken by the gfx950 transposed LDS read (see fa_tile.h).
// * K and V^T tiles are double-buffered in LDS; the global loads of tile j+1
//   are issued before the matrix-core work of tile j, one barrier per tile.
// * Exponentials use exp2 with log2(e) folded into the scale; the LSE is
//   converted back to natural-log units at the end.
#include <math.h>

#include "fa_device.h"
#include "fa_internal.h"
#include "fa_tile.h"

namespace fa {
namespace {

constexpr int BR = 128;     // query rows per workgroup
constexpr float LN2 = 0.69314718055994530942f;
constexpr float LOG2E = 1.44269504088896340736f;
// Growth of the row maximum (log2 units) tolerated before rescaling.
constexpr float kRescaleSlack = 8.0f;

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int Hq, G, Nq, Nkv, n_qtiles, n_bh;
  float scale_log2;
};

template <typename T, int D, bool CAUSAL>
__global__ __launch_bounds__(NT, 2) void fwd_mfma_kernel(FwdArgs a) {
  using L = KVTileLds<D>;
  using V8 = typename T::vec8;
  constexpr int KC = D / 16;  // k-chunks of the QK^T contraction
  constexpr int OD = D / 32;  // 32-wide output column blocks

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * L::STAGE];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int h = lane >> 5;
  const int c = lane & 31;

  // Heaviest (last) query tiles first so the causal tail is short.
  const int w = blockIdx.x;
  const int qt = a.n_qtiles - 1 - w / a.n_bh;
  const int bh = w % a.n_bh;
  const int b = bh / a.Hq;
  const int hq = bh % a.Hq;
  const int Hkv = a.Hq / a.G;
  const int hkv = hq / a.G;
  const int Nq = a.Nq, Nkv = a.Nkv;
  const int offset = Nkv - Nq;

  const int q0 = qt * BR + wave * 32;  // first query row of this wave
  const int qrow = q0 + c;             // the row this lane owns

  const uint16_t* qptr = a.q + ((size_t)bh * Nq) * D;
  const uint16_t* kbase = a.k + ((size_t)(b * Hkv + hkv) * Nkv) * D;
  const uint16_t* vbase = a.v + ((size_t)(b * Hkv + hkv) * Nkv) * D;

  // Q^T as the B operand: lane holds Q[qrow][16 kc + 8h .. +7].
  V8 qf[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
    qf[kc] = as_vec8<T>(qrow < Nq ? ld16(qptr + (size_t)qrow * D + kc * 16 + h * 8) : zero_u32x4());

  // Key tiles this workgroup needs.
  const int kv_tiles = (Nkv + BC - 1) / BC;
  int n_tiles = kv_tiles;
  if (CAUSAL) {
    const int last_key = min(Nq, (qt + 1) * BR) - 1 + offset;
    n_tiles = last_key < 0 ? 0 : min(kv_tiles, last_key / BC + 1);
  }
  // Last key any row of this wave may see (wave-uniform).
  const int wave_last_row = min(Nq - 1, q0 + 31);
  const int wave_last_key = CAUSAL ? wave_last_row + offset : Nkv - 1;
  const bool wave_has_rows = q0 < Nq;

  f32x16 oacc[OD];
#pragma unroll
  for (int od = 0; od < OD; ++od) oacc[od] = zero16();
  float m_run = -INFINITY;  // running max of scaled scores, log2 units
  float l_run = 0.0f;       // this half-wave's share of the running sum

  KVTileRegs<D> regs;
  if (n_tiles > 0) {
    load_kv_tile<D>(regs, kbase, vbase, 0, Nkv, tid);
    store_kv_tile<D>(regs, smem, smem + L::K_ELEMS, tid);
  }
  __syncthreads();

  int stage = 0;
  for (int j = 0; j < n_tiles; ++j) {
    const bool more = j + 1 < n_tiles;
    if (more) load_kv_tile<D>(regs, kbase, vbase, (j + 1) * BC, Nkv, tid);

    const uint16_t* ks = smem + stage * L::STAGE;
    const uint16_t* vt = ks + L::K_ELEMS;
    const int key0 = j * BC;

    if (wave_has_rows && key0 <= wave_last_key) {
      // S^T for keys key0 + [0, 64): two 32-key blocks.
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = zero16();
        const uint16_t* krow = ks + (kb * 32 + row_perm(c)) * L::RS + h * 8;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          const V8 ka = as_vec8<T>(*reinterpret_cast<const u32x4*>(krow + kc * 16));
          s[kb] = T::mfma(ka, qf[kc], s[kb]);
        }
      }
      // Mask keys past the end and, when causal, keys after the row's limit.
      const bool need_mask = (key0 + BC > Nkv) || (CAUSAL && key0 + BC - 1 > q0 + offset);
      if (need_mask) {
        const int lim = CAUSAL ? min(Nkv - 1, qrow + offset) : Nkv - 1;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (key0 + kb * 32 + acc_key(h, r) > lim) s[kb][r] = -INFINITY;
      }
      // Online softmax update ([KB] §04) in log2 units. The running
      // maximum is only moved (and U, l rescaled) when some row of the wave
      // sees a score more than kRescaleSlack above it; otherwise the stale
      // maximum is kept. Both U and l are always relative to the same m, so
      // O = U / l and LSE = m + log l are unchanged; p stays <= 2^slack.
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = fmaxf(mx, swap_halves(mx)) * a.scale_log2;
      if (__any(mx > m_run + kRescaleSlack)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = (m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int od = 0; od < OD; ++od)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[od][r] *= alpha;
        m_run = m_new;
      }
      const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
      float psum = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][r], a.scale_log2, -m_use));
          s[kb][r] = p;
          psum += p;
        }
      l_run += psum;

      // O^T += V^T P^T over four 16-key chunks.
#pragma unroll
      for (int ch = 0; ch < 4; ++ch) {
        float pv[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) pv[t] = s[ch >> 1][(ch & 1) * 8 + t];
        const V8 pf = pack8<T>(pv);
#pragma unroll
        for (int od = 0; od < OD; ++od) {
          const V8 va = load_vt_operand<T, L::RS>(vt, h, c, ch * 16, od * 32);
          oacc[od] = T::mfma(va, pf, oacc[od]);
        }
      }
    }

    if (more) {
      uint16_t* nks = smem + (stage ^ 1) * L::STAGE;
      store_kv_tile<D>(regs, nks, nks + L::K_ELEMS, tid);
    }
    __syncthreads();
    stage ^= 1;
  }

  // Epilogue: O = U / l, LSE = m + ln l (natural log).
  const float l = l_run + swap_halves(l_run);
  if (qrow < Nq) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    uint16_t* orow = a.o + ((size_t)bh * Nq + qrow) * D;
#pragma unroll
    for (int od = 0; od < OD; ++od)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 out;
        out[0] = pack2<T>(oacc[od][4 * g + 0] * inv, oacc[od][4 * g + 1] * inv);
        out[1] = pack2<T>(oacc[od][4 * g + 2] * inv, oacc[od][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + od * 32 + g * 8 + h * 4) = out;
      }
    if (h == 0)
      a.lse[(size_t)bh * Nq + qrow] = l > 0.0f ? (m_run + __log2f(l)) * LN2 : -INFINITY;
  }
}

template <typename T, int D>
hipError_t launch_typed(const Problem& p, const FwdPtrs& t, hipStream_t stream) {
  FwdArgs a;
  a.q = static_cast<const uint16_t*>(t.q);
  a.k = static_cast<const uint16_t*>(t.k);
  a.v = static_cast<const uint16_t*>(t.v);
  a.o = static_cast<uint16_t*>(t.o);
  a.lse = t.lse;
  a.Hq = p.Hq;
  a.G = p.G;
  a.Nq = p.Nq;
  a.Nkv = p.Nkv;
  a.n_qtiles = (p.Nq + BR - 1) / BR;
  a.n_bh = p.B * p.Hq;
  a.scale_log2 = p.scale * LOG2E;
  dim3 grid(a.n_qtiles * a.n_bh);
  if (p.causal)
    hipLaunchKernelGGL((fwd_mfma_kernel<T, D, true>), grid, dim3(NT), 0, stream, a);
  else
    hipLaunchKernelGGL((fwd_mfma_kernel<T, D, false>), grid, dim3(NT), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_mfma(const Problem& p, const FwdPtrs& t, hipStream_t stream) {
  if (p.dt == FA_BF16) {
    return p.d == 64 ? launch_typed<BF16, 64>(p, t, stream) : launch_typed<BF16, 128>(p, t, stream);
  }
  return p.d == 64 ? launch_typed<F16, 64>(p, t, stream) : launch_typed<F16, 128>(p, t, stream);
}

}  // namespace fa
