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
  const uint16_t* k;   // [B, Hkv, Nkv, D], or the K page pool [num_pages, Hkv, page_size, D]
  const uint16_t* v;   // likewise
  float* part_o;    // [B*Hq][splits][D]
  float* part_lse;  // [B*Hq][splits]
  int Hq, Hkv, G, Nkv, splits, keys_per_split, n_qgroups;
  int q_rows;        // rows of Q (B * Hq)
  float scale_log2;
  // Paged K/V: page_table [B, max_pages] (physical page of each logical
  // page), seq_lens [B]; Nkv = max_pages * page_size.
  const int* page_table;
  const int* seq_lens;
  int page_size, max_pages, num_pages;
};

// Copy `blocks` 1 KiB blocks starting at byte `src` of a flat array (`bytes`
// long; reads past the end fill zeros) to LDS at dst, block i of this wave
// at dst + (wave * blocks + i) KiB, 16 bytes per lane. Issued from inline
// assembly so that the compiler adds no waits of its own for them: the
// caller waits on vmcnt before the barrier that precedes any read.
//
// Decode reads every byte of Q, K and V exactly once, so these copies are
// non-temporal (`nt`): the lines they bring in are not kept in the caches.
// With ordinary loads the stream displaces whatever the caches hold, and
// when that is data written by earlier work (dirty lines) every displaced
// line costs an extra write to HBM: on a cache full of such lines that
// halves the decode's read rate.
__device__ __forceinline__ void copy_blocks_async(uint8_t* dst, const void* base, uint32_t bytes,
                                                  uint32_t src, int wave, int lane, int blocks) {
  for (int i = 0; i < blocks; ++i) {
    const uint32_t start = src + (uint32_t)(wave * blocks + i) * 1024u;
    const uint32_t left = bytes - __builtin_amdgcn_readfirstlane(min(bytes, start));
    const uint64_t addr = reinterpret_cast<uint64_t>(static_cast<const uint8_t*>(base) + start);
    u32x4 rsrc;  // base, stride 0, size, raw access with zero fill out of range
    rsrc[0] = __builtin_amdgcn_readfirstlane((uint32_t)addr);
    rsrc[1] = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32) & 0xffffu);
    rsrc[2] = __builtin_amdgcn_readfirstlane(left);
    rsrc[3] = 0x00020000u;
    const uint32_t lds = (uint32_t)reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) uint8_t*)(dst + (wave * blocks + i) * 1024));
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen nt lds"
        :
        : "s"(lds), "v"((uint32_t)lane * 16u), "s"(rsrc)
        : "memory", "m0");
  }
}

// The same for one K or V tile in the blocked LDS layouts of fa_tile.h
// (lane_src: k_dma_src or v_dma_src; step: K_STEP or V_STEP).
template <int D>
__device__ __forceinline__ void copy_tile_async(uint8_t* tile, const uint16_t* head,
                                                uint32_t head_bytes, int key0, int wave,
                                                uint32_t lane_src, int step) {
  using DT = DmaTile<D, 4>;
#pragma unroll
  for (int i = 0; i < DT::PER_WAVE; ++i) {
    const uint32_t start = (uint32_t)key0 * DT::RB + (uint32_t)(i * step);
    const uint32_t left = head_bytes - __builtin_amdgcn_readfirstlane(min(head_bytes, start));
    const uint64_t addr = reinterpret_cast<uint64_t>(reinterpret_cast<const uint8_t*>(head) + start);
    u32x4 rsrc;
    rsrc[0] = __builtin_amdgcn_readfirstlane((uint32_t)addr);
    rsrc[1] = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32) & 0xffffu);
    rsrc[2] = __builtin_amdgcn_readfirstlane(left);
    rsrc[3] = 0x00020000u;
    const uint32_t lds = (uint32_t)reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) uint8_t*)(tile + (wave * DT::PER_WAVE + i) * 1024));
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen nt lds"
        :
        : "s"(lds), "v"(lane_src), "s"(rsrc)
        : "memory", "m0");
  }
}

// Wait until at most N of this wave's copies are in flight and its LDS
// reads have returned.
template <int N>
__device__ __forceinline__ void wait_copies() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
  asm volatile("" ::: "memory");
}

// One workgroup per (b, kv head, group of 32 query heads, split); the 32
// heads are the matrix-core columns, so K and V are read once per group.
// Each wave takes every fourth 64-key tile of the split and runs its own
// online softmax over them ([KB] §04) in private LDS buffers: a K buffer
// and a V buffer, each refilled with the wave's next tile as soon as its
// products are issued, so a wave has a load in flight while it computes and
// the waves need no barrier inside the loop. At the end the four partial
// states are merged with the same rescaling rule and written as the split's
// O_s = U / l and LSE_s.
template <typename T, int D, bool PAGED>
__global__ __launch_bounds__(NT, 1) void decode_split_kernel(DecArgs a) {
  using V8 = typename T::vec8;
  using DT = DmaTile<D, 4>;
  constexpr int KC = D / 16;
  constexpr int OD = D / 32;
  constexpr int TB = DT::BYTES;
  constexpr int QB = 32 * DT::RB;        // the group's 32 query rows
  constexpr int QBLK = QB / 1024 / 4;    // 1 KiB Q blocks per wave
  constexpr int CPT = 4 * DT::PER_WAVE;  // copies per K (or V) tile, one wave
  static_assert(QBLK >= 1, "Q blocks");
  static_assert(4 * OD * 16 * 64 * 4 <= 4 * TB, "merge fits in the K buffers");

  __shared__ __attribute__((aligned(1024))) uint8_t kbuf[4][TB];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf[4][TB];
  __shared__ __attribute__((aligned(1024))) uint8_t qbuf[QB];
  __shared__ float mbuf[4][32], lbuf[4][32];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  // Keys of this sequence (paged: its own length, read as a scalar).
  int n_keys = a.Nkv;
  if constexpr (PAGED) {
    const auto* lens = (const __attribute__((address_space(4))) int*)a.seq_lens;
    n_keys = min(max(lens[b], 0), a.Nkv);
  }
  const int key_begin = split * a.keys_per_split;
  const int key_end = min(n_keys, key_begin + a.keys_per_split);
  const int n_tiles = key_end > key_begin ? (key_end - key_begin + BC - 1) / BC : 0;

  // Where tile j of the split comes from: a base pointer, the bytes that may
  // be read from it (reads past them fill zeros) and the tile's first key
  // relative to the base. Contiguous: the split's range. Paged: the tile's
  // page (a page holds a whole number of 64-key tiles); the table is read
  // only for tiles before the sequence's end, and a tile whose entry is out
  // of [0, num_pages) is not read at all (its keys are masked out below).
  struct Src {
    const uint16_t* k;
    const uint16_t* v;
    uint32_t bytes;
    int key0;
  };
  // Paged: the pool page of tile j, or -1 when the tile lies past the
  // sequence's end or its table entry is out of range (uniform scalar).
  auto tile_page = [&](int j) __attribute__((always_inline)) -> int {
    const int key0 = key_begin + j * BC;  // key of the sequence
    if (key0 >= key_end) return -1;
    const int pg = __builtin_amdgcn_readfirstlane(key0 / a.page_size);  // < max_pages
    const auto* table = (const __attribute__((address_space(4))) int*)a.page_table;
    const int phys = table[(size_t)b * a.max_pages + pg];
    return (phys >= 0 && phys < a.num_pages) ? phys : -1;
  };
  auto tile_src = [&](int j) __attribute__((always_inline)) -> Src {
    Src r;
    if constexpr (!PAGED) {
      const size_t split_off = ((size_t)bk * a.Nkv + key_begin) * D;
      r.k = a.k + split_off;
      r.v = a.v + split_off;
      r.bytes = (uint32_t)max(key_end - key_begin, 0) * D * 2u;
      r.key0 = j * BC;
    } else {
      const int key0 = key_begin + j * BC;  // key of the sequence
      const int phys = tile_page(j);
      const bool ok = phys >= 0;
      const size_t off = (((size_t)(ok ? phys : 0) * a.Hkv + hkv) * a.page_size + key0 % a.page_size) * D;
      r.k = a.k + off;
      r.v = a.v + off;
      r.bytes = ok ? (uint32_t)min(key_end - key0, BC) * D * 2u : 0u;
      r.key0 = 0;
    }
    return r;
  };
  uint8_t* const ks = kbuf[wave];
  uint8_t* const vs = vbuf[wave];
  // The whole tile by this wave: the four quarters the 4-wave copy layout
  // assigns to waves 0..3.
  auto load_k = [&](int j) __attribute__((always_inline)) {
    const Src t = tile_src(j);
#pragma unroll
    for (int w = 0; w < 4; ++w)
      copy_tile_async<D>(ks, t.k, t.bytes, t.key0, w, k_dma_src<D, 4>(w, lane), DT::K_STEP);
  };
  auto load_v = [&](int j) __attribute__((always_inline)) {
    const Src t = tile_src(j);
#pragma unroll
    for (int w = 0; w < 4; ++w)
      copy_tile_async<D>(vs, t.v, t.bytes, t.key0, w, v_dma_src<D, 4>(w, lane), DT::V_STEP);
  };

  // The group's Q rows (rows past the group's heads are loaded but unused),
  // copied by all waves; then each wave's first tile.
  // The copy's buffer resource starts at the group's first row (64-bit
  // address arithmetic) and spans at most its 32 rows, so its 32-bit range
  // never depends on B * Hq.
  const size_t q_row0 = (size_t)b * a.Hq + hkv * a.G + qg * 32;
  const uint32_t q_left = (uint32_t)min((size_t)32, (size_t)a.q_rows - q_row0) * DT::RB;
  copy_blocks_async(qbuf, a.q + q_row0 * D, q_left, 0u, wave, lane, QBLK);
  const int my_tiles = n_tiles > wave ? (n_tiles - wave + 3) / 4 : 0;
  load_k(wave);
  load_v(wave);
  FA_STAGE_WAIT();
  wait_copies<2 * CPT>();  // this wave's Q blocks
  __syncthreads();         // everyone's Q blocks

  const uint32_t kr0 = k_read_base<D>(h, c, 0);
  const uint32_t kr1 = k_read_base<D>(h, c, 1);
  const uint32_t vr = v_read_base<D>(h, c);
  V8 qf[KC];
#pragma unroll
  for (int kc = 0; kc < KC; ++kc)
    qf[kc] = as_vec8<T>(*reinterpret_cast<const u32x4*>(qbuf + c * DT::RB + (16 * kc + 8 * h) * 2));

  f32x16 oacc[OD];
#pragma unroll
  for (int od = 0; od < OD; ++od) oacc[od] = zero16();
  float m_run = -INFINITY;
  float l_run = 0.0f;

  for (int n = 0; n < my_tiles; ++n) {
    const int j = wave + 4 * n;  // tile of the split
    const int key0 = key_begin + j * BC;
    wait_copies<CPT>();  // K tile j (its V may still be in flight)
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = zero16();
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) {
        const uint8_t* p = ks + ((kc & 1) ? kr1 : kr0) + kb * 32 * DT::RB + (kc >> 1) * 1024;
        s[kb] = T::mfma(as_vec8<T>(*reinterpret_cast<const u32x4*>(p)), qf[kc], s[kb]);
      }
    }
    // The K buffer is free once its reads returned: refill it (tiles past
    // the split fill zeros, so every pass issues the same copies).
    wait_copies<CPT>();
    load_k(j + 4);
    FA_STAGE_WAIT();
    // Keys past the end and, paged, every key of a tile whose table entry
    // is out of range: such keys are dropped, not read as zeros.
    const int key_lim = (PAGED && tile_page(j) < 0) ? key0 : key_end;
    if (key0 + BC > key_lim) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (key0 + kb * 32 + acc_key(h, r) >= key_lim) s[kb][r] = -INFINITY;
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
    uint32_t pk[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s[i >> 3][2 * (i & 7)], a.scale_log2, -m_use));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(s[i >> 3][2 * (i & 7) + 1], a.scale_log2, -m_use));
      pk[i] = pack2<T>(p0, p1);
      psum += p0 + p1;
    }
    l_run = fmaf(alpha, l_run, psum);
    m_run = m_new;
#pragma unroll
    for (int od = 0; od < OD; ++od)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[od][r] *= alpha;
    wait_copies<CPT>();  // V tile j (the K copies just issued may be in flight)
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
      u32x4 w;
      w[0] = pk[4 * ch + 0];
      w[1] = pk[4 * ch + 1];
      w[2] = pk[4 * ch + 2];
      w[3] = pk[4 * ch + 3];
#pragma unroll
      for (int od = 0; od < OD; ++od)
        oacc[od] = T::mfma(load_vt_dma<T, D>(vs, vr, ch, od), as_vec8<T>(w), oacc[od]);
    }
    wait_copies<CPT>();
    load_v(j + 4);
    FA_STAGE_WAIT();
  }
  // Copies past the split may still be in flight.
  wait_copies<0>();
  __syncthreads();

  // Merge the four waves' states: wave w leaves m, l and U in LDS (the K
  // buffers), then wave v combines output dims [32v, 32v + 32).
  const float l_tot = l_run + swap_halves(l_run);
  if (h == 0) {
    mbuf[wave][c] = m_run;
    lbuf[wave][c] = l_tot;
  }
  float* ubuf = reinterpret_cast<float*>(&kbuf[0][0]);
#pragma unroll
  for (int od = 0; od < OD; ++od)
#pragma unroll
    for (int r = 0; r < 16; ++r) ubuf[((wave * OD + od) * 16 + r) * 64 + lane] = oacc[od][r];
  __syncthreads();
  if (wave >= OD || !has_head) return;
  float mw[4], M = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    mw[w] = mbuf[w][c];
    M = fmaxf(M, mw[w]);
  }
  const float M_use = (M == -INFINITY) ? 0.0f : M;
  float L = 0.0f;
  f32x16 u = zero16();
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float f = __builtin_amdgcn_exp2f(mw[w] - M_use);
    L = fmaf(f, lbuf[w][c], L);
#pragma unroll
    for (int r = 0; r < 16; ++r) u[r] = fmaf(f, ubuf[((w * OD + wave) * 16 + r) * 64 + lane], u[r]);
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  float* po = a.part_o + (row * a.splits + split) * D + wave * 32;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    f32x4 out;
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = u[4 * g + i] * inv;
    *reinterpret_cast<f32x4*>(po + g * 8 + h * 4) = out;
  }
  if (wave == 0 && h == 0)
    a.part_lse[row * a.splits + split] = L > 0.0f ? (M + __log2f(L)) * LN2 : -INFINITY;
}

// Merge the splits of one (b, q head) row with the [KB] §04 rescaling rule
// (O = sum_s w_s O_s / sum_s w_s, w_s = exp(LSE_s - max LSE), LSE = max +
// ln sum_s w_s); one wave per row. Lane l holds the LSE and weight of split
// 64 r + l in round r; the partial outputs are read sixteen splits at a
// time, the first sixteen while the LSEs are reduced, and added in split
// order.
template <typename T, int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(const float* __restrict__ part_o,
                                                             const float* __restrict__ part_lse,
                                                             uint16_t* __restrict__ o,
                                                             float* __restrict__ lse, int rows,
                                                             int splits) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  constexpr int PER = D / 64;
  constexpr int U = 16;  // splits whose partial outputs are loaded together
  const float* pl = part_lse + (size_t)row * splits;
  const float* po = part_o + (size_t)row * splits * D + lane;
  float x[U][PER];
  auto load_group = [&](int s0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = min(s0 + u, splits - 1);  // past the last split: reread it, weight 0
#pragma unroll
      for (int i = 0; i < PER; ++i) x[u][i] = po[(size_t)s * D + 64 * i];
    }
  };
  const float l0 = lane < splits ? pl[lane] : -INFINITY;
  load_group(0);
  float m = l0;
  for (int s = lane + 64; s < splits; s += 64) m = fmaxf(m, pl[s]);
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) m = fmaxf(m, __shfl_xor(m, k, 64));
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.0f;
  float sum = 0.0f;
  if (m != -INFINITY) {
    float w_lane = 0.0f;
    for (int s0 = 0; s0 < splits; s0 += U) {
      if ((s0 & 63) == 0) {
        const int s = s0 + lane;
        const float l = s0 == 0 ? l0 : (s < splits ? pl[s] : -INFINITY);
        w_lane = s < splits ? __expf(l - m) : 0.0f;
        sum += w_lane;
      }
      if (s0 > 0) load_group(s0);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float w = __shfl(w_lane, (s0 & 63) + u, 64);  // 0 past the last split
#pragma unroll
        for (int i = 0; i < PER; ++i) acc[i] = fmaf(w, x[u][i], acc[i]);
      }
    }
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) sum += __shfl_xor(sum, k, 64);
  }
  const float inv = sum > 0.0f ? 1.0f / sum : 0.0f;
#pragma unroll
  for (int i = 0; i < PER; ++i) o[(size_t)row * D + lane + 64 * i] = T::from_float(acc[i] * inv);
  if (lane == 0) lse[row] = sum > 0.0f ? m + logf(sum) : -INFINITY;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

template <typename T, int D, bool PAGED>
hipError_t launch_typed(const Problem& p, const FwdPtrs& t, const PagedPtrs* pg,
                        hipStream_t stream) {
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
  a.q_rows = p.B * p.Hq;
  a.scale_log2 = p.scale * LOG2E;
  a.page_table = PAGED ? pg->page_table : nullptr;
  a.seq_lens = PAGED ? pg->seq_lens : nullptr;
  a.page_size = PAGED ? pg->page_size : 0;
  a.max_pages = PAGED ? pg->max_pages : 0;
  a.num_pages = PAGED ? pg->num_pages : 0;
  dim3 grid((unsigned)((size_t)p.B * p.Hkv * a.n_qgroups * sp.splits));
  hipLaunchKernelGGL((decode_split_kernel<T, D, PAGED>), grid, dim3(NT), 0, stream, a);
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
    return p.d == 64 ? launch_typed<BF16, 64, false>(p, t, nullptr, stream)
                     : launch_typed<BF16, 128, false>(p, t, nullptr, stream);
  return p.d == 64 ? launch_typed<F16, 64, false>(p, t, nullptr, stream)
                   : launch_typed<F16, 128, false>(p, t, nullptr, stream);
}

hipError_t launch_decode_paged(const Problem& p, const FwdPtrs& t, const PagedPtrs& pg,
                               hipStream_t stream) {
  if (p.dt == FA_BF16)
    return p.d == 64 ? launch_typed<BF16, 64, true>(p, t, &pg, stream)
                     : launch_typed<BF16, 128, true>(p, t, &pg, stream);
  return p.d == 64 ? launch_typed<F16, 64, true>(p, t, &pg, stream)
                   : launch_typed<F16, 128, true>(p, t, &pg, stream);
}

}  // namespace fa
