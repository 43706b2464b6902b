// Decode forward (N_q == 1): split-KV attention for small-batch generation.
//
// [KB] "FlashAttention：为什么少搬数据，反而算得更快" §09: in decode the score
// row is 1 x history, so there is no query tile to parallelise over; the work
// is streaming K and V once from HBM. Parallelism comes instead from the key
// range, cut into splits: each workgroup folds one split of the keys into the
// online-softmax state (m, l, U) of [KB] §04 for all query heads that share a
// key/value head (the G heads of a group form the matrix-core columns, so K
// and V are read once per group), and writes the split's normalised partial
// output O_s = U / l and LSE_s = m + ln l to the workspace. A second kernel
// merges the splits with the same rescaling rule: with M = max_s LSE_s,
//   O = sum_s exp(LSE_s - M) O_s / sum_s exp(LSE_s - M),
//   LSE = M + ln sum_s exp(LSE_s - M).
//
// Causal masking has no effect here: with the bottom-right alignment the one
// query row sees every key.
#include <math.h>

#include "fa_device.h"
#include "fa_internal.h"
#include "fa_tile.h"

namespace fa {
namespace {

constexpr float LN2 = 0.69314718055994530942f;
constexpr float LOG2E = 1.44269504088896340736f;

struct DecArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  float* part_o;    // [B*Hq][splits][D]
  float* part_lse;  // [B*Hq][splits]
  int Hq, Hkv, G, Nkv, splits, keys_per_split, n_qgroups;
  float scale_log2;
};

// One workgroup per (b, kv head, group of 32 query heads, split). All waves
// compute the same 32-key x 32-head score tiles (cheap next to the stream of
// K and V); wave w owns output dims [32w, 32w + 32).
template <typename T, int D>
__global__ __launch_bounds__(NT) void decode_split_kernel(DecArgs a) {
  using L = KVTileLds<D>;
  using V8 = typename T::vec8;
  constexpr int KC = D / 16;

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * L::STAGE];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int h = lane >> 5;
  const int c = lane & 31;

  const int split = blockIdx.x % a.splits;
  const int rest = blockIdx.x / a.splits;
  const int qg = rest % a.n_qgroups;
  const int bk = rest / a.n_qgroups;  // b * Hkv + hkv
  const int b = bk / a.Hkv;
  const int hkv = bk % a.Hkv;
  const int gi = qg * 32 + c;         // index of this lane's head in the group
  const bool has_head = gi < a.G;
  const int hq = hkv * a.G + gi;
  const size_t row = (size_t)b * a.Hq + hq;  // (b, hq) row of Q, O, LSE

  const int key_begin = split * a.keys_per_split;
  const int key_end = min(a.Nkv, key_begin + a.keys_per_split);
  const int n_tiles = key_end > key_begin ? (key_end - key_begin + BC - 1) / BC : 0;

  // Buffer resources over this split's keys: reads past key_end return zero.
  const size_t split_off = ((size_t)bk * a.Nkv + key_begin) * D;
  const uint32_t split_bytes = (uint32_t)max(key_end - key_begin, 0) * D * 2u;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(a.k + split_off, split_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(a.v + split_off, split_bytes);

  V8 qf[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
    qf[kc] = as_vec8<T>(has_head ? ld16(a.q + row * D + kc * 16 + h * 8) : zero_u32x4());

  f32x16 oacc = zero16();
  float m_run = -INFINITY;
  float l_run = 0.0f;
  const bool owns_dims = wave < D / 32;

  KVTileRegs<D> regs;
  if (n_tiles > 0) {
    load_kv_tile<D>(regs, krs, vrs, 0, 0, tid);
    store_kv_tile<D>(regs, smem, smem + L::K_ELEMS, tid);
  }
  __syncthreads();

  int stage = 0;
  for (int j = 0; j < n_tiles; ++j) {
    const bool more = j + 1 < n_tiles;
    const int key0 = key_begin + j * BC;
    if (more) load_kv_tile<D>(regs, krs, vrs, (j + 1) * BC, (j + 1) * BC, tid);

    const uint16_t* ks = smem + stage * L::STAGE;
    const uint16_t* vt = ks + L::K_ELEMS;

    if (owns_dims) {
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = zero16();
        const uint16_t* krow = ks + (kb * 32 + row_perm(c)) * L::RSK + h * 8;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc)
          s[kb] = T::mfma(as_vec8<T>(*reinterpret_cast<const u32x4*>(krow + kc * 16)), qf[kc], s[kb]);
      }
      if (key0 + BC > key_end) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (key0 + kb * 32 + acc_key(h, r) >= key_end) s[kb][r] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = fmaxf(mx, swap_halves(mx));
      const float m_new = fmaxf(m_run, mx * a.scale_log2);
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      float psum = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][r], a.scale_log2, -m_use));
          s[kb][r] = p;
          psum += p;
        }
      l_run = fmaf(alpha, l_run, psum);
      m_run = m_new;
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[r] *= alpha;
#pragma unroll
      for (int ch = 0; ch < 4; ++ch) {
        float pv[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) pv[t] = s[ch >> 1][(ch & 1) * 8 + t];
        const V8 va = load_vt_operand<T, L::RSV>(vt, h, c, ch * 16, wave * 32);
        oacc = T::mfma(va, pack8<T>(pv), oacc);
      }
    }

    if (more) {
      uint16_t* nks = smem + (stage ^ 1) * L::STAGE;
      store_kv_tile<D>(regs, nks, nks + L::K_ELEMS, tid);
    }
    __syncthreads();
    stage ^= 1;
  }

  if (!owns_dims || !has_head) return;
  const float l = l_run + swap_halves(l_run);
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  float* po = a.part_o + (row * a.splits + split) * D + wave * 32;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    f32x4 out;
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = oacc[4 * g + i] * inv;
    *reinterpret_cast<f32x4*>(po + g * 8 + h * 4) = out;
  }
  if (wave == 0 && h == 0)
    a.part_lse[row * a.splits + split] = l > 0.0f ? (m_run + __log2f(l)) * LN2 : -INFINITY;
}

// Merge the splits of one (b, q head) row; one wave per row.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(const float* __restrict__ part_o,
                                                             const float* __restrict__ part_lse,
                                                             uint16_t* __restrict__ o,
                                                             float* __restrict__ lse, int rows,
                                                             int splits) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const float* pl = part_lse + (size_t)row * splits;
  float m = -INFINITY;
  for (int s = 0; s < splits; ++s) m = fmaxf(m, pl[s]);
  constexpr int PER = D / 64;
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.0f;
  float sum = 0.0f;
  if (m != -INFINITY) {
    for (int s = 0; s < splits; ++s) {
      const float w = __expf(pl[s] - m);
      sum += w;
      const float* po = part_o + ((size_t)row * splits + s) * D;
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] = fmaf(w, po[lane + 64 * i], acc[i]);
    }
  }
  const float inv = sum > 0.0f ? 1.0f / sum : 0.0f;
#pragma unroll
  for (int i = 0; i < PER; ++i) o[(size_t)row * D + lane + 64 * i] = T::from_float(acc[i] * inv);
  if (lane == 0) lse[row] = sum > 0.0f ? m + logf(sum) : -INFINITY;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

template <typename T, int D>
hipError_t launch_typed(const Problem& p, const FwdPtrs& t, hipStream_t stream) {
  const DecodeSplit sp = decode_split(p);
  const size_t rows = (size_t)p.B * p.Hq;
  DecArgs a;
  a.q = static_cast<const uint16_t*>(t.q);
  a.k = static_cast<const uint16_t*>(t.k);
  a.v = static_cast<const uint16_t*>(t.v);
  a.part_o = static_cast<float*>(t.ws);
  a.part_lse = reinterpret_cast<float*>(static_cast<char*>(t.ws) +
                                        align256(rows * sp.splits * D * sizeof(float)));
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.G = p.G;
  a.Nkv = p.Nkv;
  a.splits = sp.splits;
  a.keys_per_split = sp.keys_per_split;
  a.n_qgroups = (p.G + 31) / 32;
  a.scale_log2 = p.scale * LOG2E;
  dim3 grid((unsigned)((size_t)p.B * p.Hkv * a.n_qgroups * sp.splits));
  hipLaunchKernelGGL((decode_split_kernel<T, D>), grid, dim3(NT), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 cgrid((unsigned)((rows + 3) / 4));
  hipLaunchKernelGGL((decode_combine_kernel<T, D>), cgrid, dim3(256), 0, stream, a.part_o,
                     a.part_lse, static_cast<uint16_t*>(t.o), t.lse, (int)rows, sp.splits);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const Problem& p, const FwdPtrs& t, hipStream_t stream) {
  if (p.dt == FA_BF16)
    return p.d == 64 ? launch_typed<BF16, 64>(p, t, stream) : launch_typed<BF16, 128>(p, t, stream);
  return p.d == 64 ? launch_typed<F16, 64>(p, t, stream) : launch_typed<F16, 128>(p, t, stream);
}

}  // namespace fa
