// 32-row LDS tiles for gfx950 (MI355X): layout, direct-to-LDS tile loads and
// MFMA operand fragments, shared by the backward and the small-head forward.
#pragma once
#include "attn_common.h"

namespace attn {

// A 32-row tile of D elements in LDS, 2*D bytes per row, its 16-byte chunks
// XOR-swizzled per row (chunk c of row r sits at c ^ sw(r)) so that both read
// patterns touch distinct banks (64 banks of 4 bytes):
//  - row reads (ds_read_b128): 16 lanes read one chunk column of 16 rows;
//  - transposed reads (ds_read_b64_tr_b16): 32 lanes read 64 bytes of each of 4
//    rows r = 4m .. 4m + 3.
// sw(r) takes distinct values over 16 consecutive rows that share a bank
// position, and for D >= 64 moves the 4 rows of a transposed read to disjoint
// 64-byte bank groups.
template <int D> struct BTile {
  static constexpr int RS = D * 2;       // bytes per row
  static constexpr int BYTES = 32 * RS;
  static constexpr int NCH = D / 8;      // 16-byte chunks per row
  static constexpr int CHUNKS = 32 * NCH;
  static __device__ __forceinline__ int sw(int r) {
    if constexpr (D == 128) return 4 * (r % 4) + (r / 4) % 4;
    else if constexpr (D == 64) return 4 * ((r / 2) % 2) + (r / 4) % 4;
    else if constexpr (D == 32) return (r / 4) % 4;
    else return (r / 8) % 2;
  }
  // byte offset of element (r, col) (col a multiple of 4 here)
  static __device__ __forceinline__ int at(int r, int col) {
    return r * RS + 16 * ((col / 8) ^ sw(r)) + 2 * (col % 8);
  }
};

// global -> LDS copy of one 32-row tile by the NTH threads of a work-group with
// direct-to-LDS loads: load i of wave w fills the 16-byte slots NTH*i + 64*w +
// lane, slot x being row x / NCH, physical chunk x % NCH, which receives the
// logical chunk the swizzle maps there.  Rows at or past `nrows` re-read row
// nrows - 1 (finite data; the kernels mask or discard what those rows produce).
// The caller waits for the loads (s_waitcnt) before the barrier that publishes
// the tile.  TileOffs holds each load's element offset from the tile's first
// row (row * rs + column), computed once, so that a tile lying inside the
// sequence costs one 64-bit add per load.
template <int D, int NTH> struct TileOffs {
  static constexpr int N = BTile<D>::CHUNKS / NTH;
  static_assert(BTile<D>::CHUNKS % NTH == 0, "whole tiles per load round");
  int64_t off[N];
  __device__ __forceinline__ TileOffs(int64_t rs, int tid) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int x = NTH * i + tid;
      const int row = x / BTile<D>::NCH;
      off[i] = (int64_t)row * rs + ((x % BTile<D>::NCH) ^ BTile<D>::sw(row)) * 8;
    }
  }
};

template <int D, int NTH>
__device__ __forceinline__ void dma_tile(const TileOffs<D, NTH>& o, const unsigned short* __restrict__ G, int64_t rs,
                                         int row0, int nrows, int tid, int wave, char* lds) {
  if (row0 + 32 <= nrows) {  // wave-uniform
    const unsigned short* B = G + (int64_t)row0 * rs;
#pragma unroll
    for (int i = 0; i < TileOffs<D, NTH>::N; ++i) lds_dma16<false>(B + o.off[i], lds + (NTH * i + 64 * wave) * 16);
  } else {
#pragma unroll
    for (int i = 0; i < TileOffs<D, NTH>::N; ++i) {
      const int x = NTH * i + tid;
      const int row = x / BTile<D>::NCH;
      const int col = ((x % BTile<D>::NCH) ^ BTile<D>::sw(row)) * 8;
      const int64_t r = min(row0 + row, nrows - 1);
      lds_dma16<false>(G + r * rs + col, lds + (NTH * i + 64 * wave) * 16);
    }
  }
}

// Row-major fragment of a 32-row LDS tile: lane (l32, hi) gets elements
// [8*hi + 16*kk, +8) of row l32, the A (or B) operand layout of the 32x32x16
// product along D.
template <int D>
__device__ __forceinline__ u32x4_t frag_rows(const char* t, int l32, int hi, int kk) {
  return *(const u32x4_t*)(t + BTile<D>::at(l32, 8 * (hi + 2 * kk)));
}

// Transposed fragment of a 32-row LDS tile: the A operand of a product whose
// M index is the tile's column (cb*32 + l32) and whose K index runs over the
// tile's rows.  For K chunk t16 the lane holds rows 16*t16 + 4*hi + {0..3} and
// 16*t16 + 8 + 4*hi + {0..3}, the rows that lane owns in an accumulator block
// of the 32x32 product (element r at row (r/4)*8 + 4*hi + r%4), so an
// accumulator converted in place is the matching B operand.  Each half comes
// from one ds_read_b64_tr_b16, in which lane x of a 16-lane group fetches 4
// columns of row x/4 and receives column x of the 4 rows.  At D = 16 the upper
// 16 columns repeat the lower ones.
template <int D>
__device__ __forceinline__ u32x4_t frag_cols(const char* t, int lane, int hi, int cb, int t16) {
  const int g16 = (lane >> 4) & 1, xr = (lane & 15) >> 2, xq = lane & 3;
  const int col = (cb * 32 + g16 * 16 + xq * 4) & (D >= 32 ? 0x7fffffff : D - 1);
  u32x4_t f;
#pragma unroll
  for (int rd = 0; rd < 2; ++rd) {
    const int row = 16 * t16 + 8 * rd + 4 * hi + xr;
    const char* a = t + BTile<D>::at(row, col);
    const u32x2_t y = bitcast<u32x2_t>(__builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4_t*)(a)));
    f[2 * rd] = y[0];
    f[2 * rd + 1] = y[1];
  }
  return f;
}

// Store a lane's accumulated column: element r of block cb is d = cb*32 +
// (r/4)*8 + 4*hi + r%4, times `mul`, rounded to the storage type.
template <int T_, int D, int CB>
__device__ __forceinline__ void store_cols(unsigned short* __restrict__ dst, const f32x16_t (&acc)[CB], int hi,
                                           float mul) {
  using Tt = Ty<T_>;
#pragma unroll
  for (int cb = 0; cb < CB; ++cb)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int col = cb * 32 + r4 * 8 + hi * 4;
      if (col >= D) continue;
      u32x2_t x = {Tt::pack2(acc[cb][4 * r4] * mul, acc[cb][4 * r4 + 1] * mul),
                   Tt::pack2(acc[cb][4 * r4 + 2] * mul, acc[cb][4 * r4 + 3] * mul)};
      *(u32x2_t*)(dst + col) = x;
    }
}

}  // namespace attn
