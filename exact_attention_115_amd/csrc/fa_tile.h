// K / V tile staging for the 16-bit forward, decode and backward kernels: a
// tile of BC = 64 keys (or query rows) is copied from global memory straight
// into LDS by buffer loads with an LDS destination (no register staging), in
// blocked layouts chosen so that the matrix-core operand reads are free of
// LDS bank conflicts:
// * K rows are read 16 bytes per lane, 16 consecutive rows per access group
//   (the A operand of S^T = K Q^T);
// * V is consumed as the A operand of O^T += V^T P^T, i.e. eight consecutive
//   KEYS of one dim per lane, a column of the row-major tile. gfx950's
//   transposed LDS read (ds_read_b64_tr_b16) delivers exactly that: within
//   each group of 16 lanes, the lanes' 4-element row chunks form a 16 x 4
//   matrix M (row = source lane) and result lane i receives M[4k + i/4][i % 4],
//   k = 0..3.
// The layouts and the per-lane read offsets are below (DmaTile, k_read_base,
// v_read_base, kt_read_base). Global reads go through a buffer resource whose
// size is the head's K (or V) extent: reads past the last key return zero
// without a branch, and the caller masks those keys to -inf.
#pragma once

#include "fa_device.h"

namespace fa {

constexpr int BC = 64;   // keys per tile
constexpr int NT = 256;  // threads per decode workgroup

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Buffer resource over `bytes` bytes at `base` (raw, unswizzled; reads at or
// past `bytes` return zero).
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// ---------------------------------------------------------------------------
// Direct global -> LDS staging (gfx950 buffer_load ... lds): a 16-byte load
// per lane, written by the hardware to LDS at M0 + 16 * lane, so one wave
// instruction fills 1 KiB of LDS and no VGPRs hold the tile in between. Each
// lane chooses which 16-byte chunk of the tile it fetches; the layouts below
// keep every fetch a whole 64-byte run of a key row (coalesced) and every
// matrix-core operand read below free of LDS bank conflicts.
//
// K tile: rows r = 16 m + u (u < 16), 16-byte chunks q of a row. Chunk q of
// row r lives at byte
//   m * 16 RB + (q / 4) * 1024 + u * 64 + ((q % 4) ^ (u / 4)) * 16,
// i.e. each 64-byte run of a row in its own 64-byte slot, its four chunks
// permuted by u / 4. The operand read (16 lanes read the same chunk of 16
// rows u = 0..15) then touches every 16-byte bank group of a 256-byte bank
// line exactly once.
//
// V tile: rows r = 4 R4 + t (t < 4). Chunk q of row r lives at byte
//   R4 * 4 RB + (q / 4) * 256 + t * 64 + (q % 4) * 16,
// i.e. 4 rows x 64 bytes per 256-byte block. A transposed read (16 lanes:
// 4 consecutive rows x 32 bytes; 32 lanes: 4 rows x 64 bytes) stays inside
// one such block and touches each bank once.
template <int D, int NW = 4>
struct DmaTile {
  static constexpr int RB = 2 * D;                   // bytes per key row
  static constexpr int BYTES = BC * RB;              // bytes per tile
  static constexpr int PER_WAVE = BYTES / 1024 / NW;  // 1 KiB DMA blocks per wave (NW waves)
  static constexpr int K_STEP = 64;                  // source step between a wave's K blocks
  static constexpr int V_STEP = 1024;                // source step between a wave's V blocks
  static_assert((RB / 64) % PER_WAVE == 0, "a wave's K blocks share one 16-row group");
};

// Tile-relative source byte of lane l's chunk in the wave's first K block
// (block i of the wave adds i * K_STEP).
template <int D, int NW>
__device__ inline uint32_t k_dma_src(int wave, int l) {
  using T = DmaTile<D, NW>;
  const int g = wave * T::PER_WAVE;  // first 1 KiB block: 16-row group m, 64-byte run G
  const int m = g / (T::RB / 64), G = g % (T::RB / 64);
  const int u = l >> 2, slot = l & 3;
  return (uint32_t)((16 * m + u) * T::RB + (4 * G + (slot ^ (u >> 2))) * 16);
}

// Same for V (block i adds i * V_STEP).
template <int D, int NW>
__device__ inline uint32_t v_dma_src(int wave, int l) {
  using T = DmaTile<D, NW>;
  const int b = (T::PER_WAVE * wave) * 1024 + 16 * l;  // LDS byte of the wave's first block
  const int r4 = b / (4 * T::RB), rem = b % (4 * T::RB);
  const int q = 4 * (rem >> 8) + ((rem >> 4) & 3);
  const int t = (rem >> 6) & 3;
  return (uint32_t)((4 * r4 + t) * T::RB + q * 16);
}

// Issue this wave's DMA loads of one K (or V) tile: `tile` is the tile's LDS
// base, `head` the global base of the head's K (or V), `head_bytes` its size,
// `key0` the tile's first key; block i of the wave reads from STEP * i bytes
// past the lane's source (K_STEP or V_STEP). One buffer resource covers the
// tile: it starts at the tile and ends at the head's end, so reads past the
// end fill zeros; the blocks differ only in the instruction's offset field.
template <int D, int NW, int STEP, int I = 0>
__device__ __forceinline__ void dma_blocks(__amdgpu_buffer_rsrc_t r, uint8_t* tile, int wave,
                                           uint32_t lane_src) {
  using T = DmaTile<D, NW>;
  if constexpr (I < T::PER_WAVE) {
    // The offset field is added to the LDS address as well as to the
    // memory address: the LDS base is lowered by as much.
    static_assert(I * STEP < 4096 && I * STEP <= I * 1024, "offset field is 12 bits");
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r,
        (__attribute__((address_space(3))) void*)(tile + (wave * T::PER_WAVE + I) * 1024 - I * STEP),
        16, lane_src, 0, I * STEP, 0);
    dma_blocks<D, NW, STEP, I + 1>(r, tile, wave, lane_src);
  }
}

template <int D, int NW, int STEP>
__device__ inline void dma_tile(uint8_t* tile, const uint16_t* head, uint32_t head_bytes, int key0,
                                int wave, uint32_t lane_src) {
  using T = DmaTile<D, NW>;
  const uint32_t start = (uint32_t)key0 * T::RB;
  // Scalar arithmetic (min then subtract) keeps the resource in SGPRs.
  const uint32_t left = head_bytes - __builtin_amdgcn_readfirstlane(min(head_bytes, start));
  const __amdgpu_buffer_rsrc_t r = make_rsrc(reinterpret_cast<const uint8_t*>(head) + start, left);
  dma_blocks<D, NW, STEP>(r, tile, wave, lane_src);
}

// Per-lane byte offsets of the matrix-core operand reads.
// K (A operand of S^T = K Q^T, lane (h, c) reads row kb * 32 + row_perm(c),
// chunk 2 kc + h): byte = k_read_base(h, c, kc % 2) + kb * 32 RB + (kc / 2) * 1024.
template <int D>
__device__ inline uint32_t k_read_base(int h, int c, int parity) {
  using T = DmaTile<D>;
  const int u = row_perm(c) & 15;
  return (uint32_t)((c >> 4) * 16 * T::RB + u * 64 + (((2 * parity + h) ^ (u >> 2)) << 4));
}

// V (transposed read of rows ch * 16 + 8h + 4s + j / 4, element columns
// od * 32 + 16 (c / 16) + 4 (j % 4), j = c % 16):
// byte = v_read_base(h, c) + (4 ch + s) * 4 RB + od * 256.
template <int D>
__device__ inline uint32_t v_read_base(int h, int c) {
  using T = DmaTile<D>;
  const int j = c & 15;
  return (uint32_t)(8 * h * T::RB + (j >> 2) * 64 + (2 * (c >> 4) + ((j >> 1) & 1)) * 16 + 8 * (j & 1));
}

__device__ inline s16x4 ds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
}

// The A operand V^T[dim0 + c][key0 + 8h .. +7] (dim0 = 32 od, key0 = 16 ch)
// from a DMA-staged V tile (vt: its LDS base, vb: v_read_base).
template <typename T, int D>
__device__ inline typename T::vec8 load_vt_dma(const uint8_t* vt, uint32_t vb, int ch, int od) {
  constexpr int RB = DmaTile<D>::RB;
  const s16x4 lo = ds_read_tr16(reinterpret_cast<const uint16_t*>(vt + vb + (4 * ch) * 4 * RB + od * 256));
  const s16x4 hi = ds_read_tr16(reinterpret_cast<const uint16_t*>(vt + vb + (4 * ch + 1) * 4 * RB + od * 256));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 x;
  x[0] = lo[0]; x[1] = lo[1]; x[2] = lo[2]; x[3] = lo[3];
  x[4] = hi[0]; x[5] = hi[1]; x[6] = hi[2]; x[7] = hi[3];
  return __builtin_bit_cast(typename T::vec8, x);
}

// Transposed reads from a K-layout tile (the layout supports both 16-byte
// row reads and transposed reads without bank conflicts: a transposed read
// touches 4 consecutive rows of one 16-row group, which sit in distinct
// 64-byte slots). The A operand X^T[dim0 + c][key0 + 8h .. +7] with
// dim0 = 32 od, key0 = 16 ch: lane (h, c), j = c % 16, reads row
// 16 ch + 8h + 4s + j / 4 at element column 32 od + 16 (c / 16) + 4 (j % 4),
// i.e. byte kt_read_base(h, c, s) + ch * 16 RB + od * 1024.
template <int D>
__device__ inline uint32_t kt_read_base(int h, int c, int s) {
  const int j = c & 15;
  const int q3 = 2 * (c >> 4) + ((j >> 1) & 1);  // chunk within the 64-byte run
  return (uint32_t)((8 * h + 4 * s + (j >> 2)) * 64 + ((q3 ^ (2 * h + s)) << 4) + 8 * (j & 1));
}

template <typename T, int D>
__device__ inline typename T::vec8 load_kt_dma(const uint8_t* kt, uint32_t b0, uint32_t b1, int ch,
                                               int od) {
  constexpr int RB = DmaTile<D>::RB;
  const s16x4 lo = ds_read_tr16(reinterpret_cast<const uint16_t*>(kt + b0 + ch * 16 * RB + od * 1024));
  const s16x4 hi = ds_read_tr16(reinterpret_cast<const uint16_t*>(kt + b1 + ch * 16 * RB + od * 1024));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 x;
  x[0] = lo[0]; x[1] = lo[1]; x[2] = lo[2]; x[3] = lo[3];
  x[4] = hi[0]; x[5] = hi[1]; x[6] = hi[2]; x[7] = hi[3];
  return __builtin_bit_cast(typename T::vec8, x);
}

struct TileId {
  int qt, b, hq;
};

// Workgroup w -> (query tile, batch, query head). Heaviest (last, under the
// causal mask) query tiles go first. Workgroups are handed to the 8 XCDs
// round-robin (w % 8); when the key/value heads divide evenly over the XCDs,
// every query tile of the query heads sharing one key/value head is kept on
// one XCD so that head's K and V are reused from that XCD's L2.
__device__ __forceinline__ TileId tile_of(int w, int B, int Hq, int Hkv, int G, int n_qtiles) {
  TileId t;
  const int units = B * Hkv;
  if ((units & 7) == 0) {
    const int xcd = w & 7;
    const int j = w >> 3;
    const int per_level = (units >> 3) * G;  // workgroups per tile row, per XCD
    t.qt = n_qtiles - 1 - j / per_level;
    const int rem = j % per_level;
    const int u = xcd + 8 * (rem / G);
    t.b = u / Hkv;
    t.hq = (u % Hkv) * G + rem % G;
  } else {
    const int n_bh = B * Hq;
    t.qt = n_qtiles - 1 - w / n_bh;
    const int bh = w % n_bh;
    t.b = bh / Hq;
    t.hq = bh % Hq;
  }
  return t;
}

}  // namespace fa
