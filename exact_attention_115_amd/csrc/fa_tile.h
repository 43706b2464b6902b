// K / V tile staging for the forward and decode kernels: a tile of BC = 64
// keys is read from global memory with 16-byte loads into registers, then
// written to LDS as K[key][dim] (row-major, padded) and V^T[dim][key] (the
// transpose the P V product needs, formed in registers: each thread holds a
// 4-key x 8-dim block and writes 8 runs of 4 keys).
#pragma once

#include "fa_device.h"

namespace fa {

constexpr int BC = 64;   // keys per tile
constexpr int NT = 256;  // threads per workgroup that stage a tile

template <int D>
struct KVTileLds {
  static constexpr int KS = D + 8;    // K tile row stride (elements), +16 B pad
  static constexpr int VS = BC + 8;   // V^T tile row stride (elements)
  static constexpr int K_ELEMS = BC * KS;
  static constexpr int V_ELEMS = D * VS;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int BYTES = 2 * STAGE * 2;
};

// Global loads of one K/V tile held in registers between issue and LDS write.
template <int D>
struct KVTileRegs {
  static constexpr int KCH = (BC * D / 8) / NT;      // 16-byte K chunks per thread
  static constexpr int V_ITEMS = (BC / 4) * (D / 8);  // 4-key x 8-dim V blocks
  u32x4 k[KCH];
  u32x4 v[4];
};

template <int D>
__device__ inline void load_kv_tile(KVTileRegs<D>& r, const uint16_t* __restrict__ kbase,
                                 const uint16_t* __restrict__ vbase, int key0, int Nkv, int tid) {
#pragma unroll
  for (int i = 0; i < KVTileRegs<D>::KCH; ++i) {
    const int id = tid + NT * i;
    const int key = id / (D / 8), dc = id % (D / 8);
    r.k[i] = (key0 + key < Nkv) ? ld16(kbase + (size_t)(key0 + key) * D + dc * 8) : zero_u32x4();
  }
  if (tid < KVTileRegs<D>::V_ITEMS) {
    const int kg = tid / (D / 8), dc = tid % (D / 8);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int key = key0 + kg * 4 + rr;
      r.v[rr] = key < Nkv ? ld16(vbase + (size_t)key * D + dc * 8) : zero_u32x4();
    }
  }
}

template <int D>
__device__ inline void store_kv_tile(const KVTileRegs<D>& r, uint16_t* ks, uint16_t* vt, int tid) {
  using L = KVTileLds<D>;
#pragma unroll
  for (int i = 0; i < KVTileRegs<D>::KCH; ++i) {
    const int id = tid + NT * i;
    const int key = id / (D / 8), dc = id % (D / 8);
    *reinterpret_cast<u32x4*>(ks + key * L::KS + dc * 8) = r.k[i];
  }
  if (tid < KVTileRegs<D>::V_ITEMS) {
    const int kg = tid / (D / 8), dc = tid % (D / 8);
    // Element e of the 8 dims, for the 4 keys, packed as 4 x 16 bit.
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int w = e >> 1;
      const int sh = (e & 1) * 16;
      const uint32_t x0 = (r.v[0][w] >> sh) & 0xffffu;
      const uint32_t x1 = (r.v[1][w] >> sh) & 0xffffu;
      const uint32_t x2 = (r.v[2][w] >> sh) & 0xffffu;
      const uint32_t x3 = (r.v[3][w] >> sh) & 0xffffu;
      u32x2 out;
      out[0] = x0 | (x1 << 16);
      out[1] = x2 | (x3 << 16);
      *reinterpret_cast<u32x2*>(vt + (dc * 8 + e) * L::VS + kg * 4) = out;
    }
  }
}

}  // namespace fa
