// bwd_common.h -- LDS tile helpers shared by the backward kernels
// (attn_bwd_dkdv.hip, attn_bwd_dq.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernel_common.h"

namespace attn {

// Per-lane LDS byte offsets of the two read patterns over a tile of rows of
// D 16-bit elements (row stride 2 D bytes):
//   row reads  (A/B operand, 8 consecutive elements of row key_perm(l % 32)):
//              koff(kk) = koff0 ^ (kk << 5), +32 rows per 32-row block;
//   transposed (A operand: 32 columns x 16 rows, ds_read_b64_tr_b16 pairs):
//              voff(db) = voff0 ^ (db << 6), + 16 rows per chunk, second
//              read + 4 rows.
template <int D>
struct TileReads {
  static constexpr int ROW = 2 * D;
  int koff0;
  uint32_t voff0;
  __device__ __forceinline__ TileReads(int lane) {
    const int h = lane >> 5, l32 = lane & 31;
    const int r0 = key_perm(l32);
    koff0 = r0 * ROW + ((h ^ swz_k<D>(r0)) << 4);
    const int G = lane >> 4, i16 = lane & 15;
    const int r = 8 * h + (i16 >> 2);
    const int dd = 16 * (G & 1) + 4 * (i16 & 3);
    voff0 = r * ROW + (((dd >> 3) ^ swz_v<D>(r)) << 4) + ((dd & 7) << 1);
  }
  __device__ __forceinline__ int koff(int kk) const { return koff0 ^ (kk << 5); }
  __device__ __forceinline__ uint32_t voff(int db) const { return voff0 ^ (uint32_t)(db << 6); }
};

// DMA offsets of the copy of a tile of ROWS rows (row stride `stride`
// elements in global memory) by NW waves, for either swizzle.
template <int D, int ROWS, int NW>
struct TileCopy {
  static constexpr int CPR = D / 8;
  static constexpr int LOADS = ROWS * CPR / (NW * 64);
  static_assert(LOADS >= 1 && ROWS * CPR % (NW * 64) == 0, "tile copy shape");
  uint32_t k[LOADS], v[LOADS];
  __device__ __forceinline__ TileCopy(int wave, int lane, int stride) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int pos = (wave * LOADS + i) * 64 + lane;
      const int row = pos / CPR, phys = pos % CPR;
      k[i] = (uint32_t)(row * stride * 2 + ((phys ^ swz_k<D>(row)) << 4));
      v[i] = (uint32_t)(row * stride * 2 + ((phys ^ swz_v<D>(row)) << 4));
    }
  }
};

// Eight transposed reads (ds_read_b64_tr_b16): the A operands of two 16-row
// chunks at each of the addresses a0 and a1 (r[2 c], r[2 c + 1] = chunk c of
// a0; r[4 + 2 c], r[5 + 2 c] = chunk c of a1, c = 0, 1).  Wait for them with
// lds_wait; pair j is complete once at most 6 - 2 j reads issued after it
// are outstanding.
template <int D>
__device__ __forceinline__ void tr_issue8(uint32_t a0, uint32_t a1, i16x4 (&r)[8]) {
  constexpr int R = 2 * D;
  r[0] = lds_tr16<0>(a0);
  r[1] = lds_tr16<4 * R>(a0);
  r[2] = lds_tr16<16 * R>(a0);
  r[3] = lds_tr16<20 * R>(a0);
  r[4] = lds_tr16<0>(a1);
  r[5] = lds_tr16<4 * R>(a1);
  r[6] = lds_tr16<16 * R>(a1);
  r[7] = lds_tr16<20 * R>(a1);
}

template <typename V>
__device__ __forceinline__ V tr_pair(const i16x4 (&r)[8], int j) {
  const i16x8 w = __builtin_shufflevector(r[2 * j], r[2 * j + 1], 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(V, w);
}

}  // namespace attn
