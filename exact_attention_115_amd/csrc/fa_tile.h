// K / V tile staging for the forward and decode kernels: a tile of BC = 64
// keys is read from global memory with 16-byte loads into registers, then
// written to LDS row-major, K[key][dim] and V[key][dim], each row padded by
// 32 bytes. The pad puts consecutive rows 8 banks apart, so neither the
// 16-byte row reads of K nor the transposed 8-byte reads of V (below) hit the
// same bank twice in one access group.
//
// V is consumed as the A operand of O^T += V^T P^T, i.e. eight consecutive
// KEYS of one dim per lane, which is a column of the row-major tile. gfx950's
// transposed LDS read (ds_read_b64_tr_b16) delivers exactly that: within each
// group of 16 lanes, the lanes' 4-element row chunks form a 16 x 4 matrix M
// (row = source lane) and result lane i receives M[4k + i/4][i % 4], k = 0..3.
// vt_addr() gives each lane the row chunk to point at so that lane (h, c)
// receives V[key0 + 8h + 4s + k][dim0 + c], k = 0..3, for half s = 0, 1.
#pragma once

#include "fa_device.h"

namespace fa {

constexpr int BC = 64;   // keys per tile
constexpr int NT = 256;  // threads per workgroup that stage a tile

typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int D>
struct KVTileLds {
  static constexpr int RS = D + 16;  // row stride (elements) of both K and V
  static constexpr int K_ELEMS = BC * RS;
  static constexpr int V_ELEMS = BC * RS;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
};

// Global loads of one K/V tile held in registers between issue and LDS write.
template <int D>
struct KVTileRegs {
  static constexpr int CH = (BC * D / 8) / NT;  // 16-byte chunks per thread, per tensor
  u32x4 k[CH];
  u32x4 v[CH];
};

template <int D>
__device__ inline void load_kv_tile(KVTileRegs<D>& r, const uint16_t* __restrict__ kbase,
                                    const uint16_t* __restrict__ vbase, int key0, int key_end,
                                    int tid) {
#pragma unroll
  for (int i = 0; i < KVTileRegs<D>::CH; ++i) {
    const int id = tid + NT * i;
    const int key = id / (D / 8), dc = id % (D / 8);
    const bool in = key0 + key < key_end;
    const size_t off = (size_t)(key0 + key) * D + dc * 8;
    r.k[i] = in ? ld16(kbase + off) : zero_u32x4();
    r.v[i] = in ? ld16(vbase + off) : zero_u32x4();
  }
}

template <int D>
__device__ inline void store_kv_tile(const KVTileRegs<D>& r, uint16_t* ks, uint16_t* vs, int tid) {
  using L = KVTileLds<D>;
#pragma unroll
  for (int i = 0; i < KVTileRegs<D>::CH; ++i) {
    const int id = tid + NT * i;
    const int key = id / (D / 8), dc = id % (D / 8);
    *reinterpret_cast<u32x4*>(ks + key * L::RS + dc * 8) = r.k[i];
    *reinterpret_cast<u32x4*>(vs + key * L::RS + dc * 8) = r.v[i];
  }
}

// Element offset, inside a V tile, of the 4-element row chunk lane (h, c)
// points at so that the transposed read returns V[key0 + 8h + 4s + k][dim0 + c]
// (k = 0..3). Lane (h, c) sits in 16-lane group 2h + c/16 at position
// j = c % 16; it supplies row key0 + 8h + 4s + j/4, columns
// dim0 + 16 (c/16) + 4 (j % 4) .. +3.
template <int RS>
__device__ inline int vt_addr(int h, int c, int key0, int dim0, int s) {
  const int j = c & 15;
  return (key0 + 8 * h + 4 * s + (j >> 2)) * RS + dim0 + 16 * (c >> 4) + 4 * (j & 3);
}

__device__ inline s16x4 ds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
}

// The A operand V^T[dim0 + c][key0 + 8h .. +7] from the row-major V tile.
template <typename T, int RS>
__device__ inline typename T::vec8 load_vt_operand(const uint16_t* vs, int h, int c, int key0,
                                                   int dim0) {
  const s16x4 lo = ds_read_tr16(vs + vt_addr<RS>(h, c, key0, dim0, 0));
  const s16x4 hi = ds_read_tr16(vs + vt_addr<RS>(h, c, key0, dim0, 1));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 x;
  x[0] = lo[0]; x[1] = lo[1]; x[2] = lo[2]; x[3] = lo[3];
  x[4] = hi[0]; x[5] = hi[1]; x[6] = hi[2]; x[7] = hi[3];
  return __builtin_bit_cast(typename T::vec8, x);
}

}  // namespace fa
