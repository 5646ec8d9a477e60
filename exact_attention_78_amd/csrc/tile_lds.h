// LDS tiles of 16-bit rows shared by the backward and decode kernels: one chunk swizzle
// that serves both row reads and transpose reads, the per-lane addresses of both read
// patterns for 32x32x16 MFMA operands, direct global->LDS tile loads, packing of fp32
// accumulators into the 16-bit B operand of the next contraction, and row stores through
// LDS.
#pragma once

#include "device_common.h"

namespace attn {

// Chunk swizzle of the LDS tiles: 16-byte chunk c of tile row r is stored at chunk
// c ^ f(r). The tiles here are read both by rows (32 rows x one chunk per ds_read_b128)
// and by transpose reads (4 rows x 2 chunks per 16 lanes), and f spreads both patterns
// over distinct banks: 16 consecutive rows get 16 (d = 128) or, paired with the row
// parity, 8 (d = 64) distinct values, and rows 4a..4a+3 move a chunk pair {2g, 2g+1}
// to four disjoint places. f depends on row bits 0..3 only.
template <int D> struct BSwz;
template <> struct BSwz<128> {
  static __device__ __forceinline__ int f(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
};
template <> struct BSwz<64> {
  static __device__ __forceinline__ int f(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }
};

// Per-lane LDS byte offsets inside a tile of rows of D 16-bit elements.
template <int D>
struct TileAddr {
  static constexpr int ROW = D * 2;
  static constexpr int NSTEP = D / 16;
  static constexpr int NDB = D / 32;
  uint32_t row[NSTEP];       // row read: row l32, head-dim step s (16 elements)
  uint32_t tr[2][NDB];       // transpose read: rows tr_row (+8), head-dim block db
  __device__ __forceinline__ void init(int lane) {
    const int half = lane / 32, l32 = lane % 32;
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) row[s] = l32 * ROW + (((2 * s + half) ^ BSwz<D>::f(l32)) << 4);
    const int g16 = lane / 16, i16 = lane % 16;
    const int tr_row = (g16 / 2) * 4 + i16 / 4;
    const int tr_col = 16 * (g16 % 2) + 4 * (i16 % 4);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int r = tr_row + 8 * j, col = db * 32 + tr_col;
        tr[j][db] = r * ROW + (((col >> 3) ^ BSwz<D>::f(r)) << 4) + ((col & 7) << 1);
      }
  }
};

// A-operand fragment of rows [r0, r0 + 32) of a tile, head-dim step s (row reads).
template <int D>
__device__ __forceinline__ u32x4 row_frag(const uint8_t* tile, const TileAddr<D>& a, int r0, int s) {
  return *(const u32x4*)(tile + r0 * TileAddr<D>::ROW + a.row[s]);
}
// A-operand fragment of the transpose of rows [r0, r0 + 16) (the contraction index),
// head-dim block db: the 8 rows each half of the wave supplies follow the order of the
// 32x32 accumulator rows (8 * (r / 4) + 4 * half + r % 4) that the B operand comes from.
template <int D>
__device__ __forceinline__ u32x4 tr_frag(const uint8_t* tile, const TileAddr<D>& a, int r0, int db) {
  const uint8_t* base = tile + r0 * TileAddr<D>::ROW;
  const u32x2 v1 = lds_read_tr16((const uint16_t*)(base + a.tr[0][db]));
  const u32x2 v2 = lds_read_tr16((const uint16_t*)(base + a.tr[1][db]));
  return u32x4{v1[0], v1[1], v2[0], v2[1]};
}

// Direct global -> LDS load of a tile of R rows starting at row r0 (rows past N re-read
// row N-1, whose results are masked). Wave w of W fills 1 KiB pieces w, w + W, ...
template <int D, int R, int W>
__device__ __forceinline__ void load_rows(const uint16_t* src, int r0, int N, uint8_t* dst, int wave, int lane) {
  constexpr int ROW = D * 2, TB = R * ROW, LPW = TB / 1024 / W;
  static_assert(LPW >= 1 && LPW * 1024 * W == TB, "tile must split into whole 1 KiB loads per wave");
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int slot = (wave * LPW + i) * 1024 + lane * 16;
    const int r = slot / ROW, phys = (slot % ROW) / 16;
    const int row = min(r0 + r, N - 1);
    dma_load16((const uint8_t*)(src + (int64_t)row * D) + ((phys ^ BSwz<D>::f(r)) << 4),
               lds_u32(dst) + (wave * LPW + i) * 1024);
  }
}

// load_rows with a wave-uniform base: each lane's byte offsets within the tile (row and
// source chunk of its 1 KiB pieces) are set once, then a tile whose rows all lie before N
// loads from base src + r0 * D; a tile that reaches past N re-reads row N-1 as load_rows
// does.
template <int D, int R, int W>
struct RowPieces {
  static constexpr int ROW = D * 2, TB = R * ROW, LPW = TB / 1024 / W;
  static_assert(LPW >= 1 && LPW * 1024 * W == TB, "tile must split into whole 1 KiB loads per wave");
  static_assert((ROW & (ROW - 1)) == 0, "row length a power of two");
  uint32_t off[LPW];
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int slot = (wave * LPW + i) * 1024 + lane * 16;
      const int r = slot / ROW, phys = (slot % ROW) / 16;
      off[i] = r * ROW + ((phys ^ BSwz<D>::f(r)) << 4);
    }
  }
  __device__ __forceinline__ void load(const uint16_t* src, int r0, int N, uint8_t* dst, int wave) const {
    if (r0 + R <= N) {
      const uint16_t* base = src + (int64_t)r0 * D;
#pragma unroll
      for (int i = 0; i < LPW; ++i) dma_load16_s(base, off[i], lds_u32(dst) + (wave * LPW + i) * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < LPW; ++i) {
        const int row = min(r0 + (int)(off[i] / ROW), N - 1);
        dma_load16((const uint8_t*)(src + (int64_t)row * D) + (off[i] % ROW), lds_u32(dst) + (wave * LPW + i) * 1024);
      }
    }
  }
};

// B operand of the next contraction: 16 fp32 accumulator values -> two groups of 8
// 16-bit values (accumulator rows 0..7 and 8..15).
template <typename Tag>
__device__ __forceinline__ void pack16(const float (&x)[16], u32x4 (&p)[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h)
    p[h] = u32x4{pack2(Tag{}, x[h * 8 + 0], x[h * 8 + 1]), pack2(Tag{}, x[h * 8 + 2], x[h * 8 + 3]),
                 pack2(Tag{}, x[h * 8 + 4], x[h * 8 + 5]), pack2(Tag{}, x[h * 8 + 6], x[h * 8 + 7])};
}

// Store 32 x D accumulators (lane pair l32, l32 + 32: one row of the result; head dims
// 8 * (r / 4) + 4 * half + r % 4 of each block) times `mul` as 16-bit values, through LDS
// so that the stores write whole rows: the wave's 32 rows are staged in stg (32 * D * 2
// bytes, 16-byte chunk c of row r at chunk c ^ (r mod chunks per row)), then written with
// 16-byte stores, 1 KiB of consecutive rows per instruction, to dst0 (the first of the 32
// rows, which are contiguous); rows from nvalid on are not written. The caller makes stg
// free for this wave (a barrier).
template <typename Tag, int D>
__device__ __forceinline__ void store_rows_staged(uint16_t* dst0, int nvalid, const f32x16 (&acc)[D / 32], int lane,
                                                  float mul, uint8_t* stg) {
  constexpr int ROW = D * 2, NCH = ROW / 16;
  const int half = lane / 32, l32 = lane % 32;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x16 a = acc[db];
      *(u32x2*)(stg + l32 * ROW + (((db * 4 + g) ^ (l32 % NCH)) << 4) + half * 8) =
          u32x2{pack2(Tag{}, a[g * 4 + 0] * mul, a[g * 4 + 1] * mul), pack2(Tag{}, a[g * 4 + 2] * mul, a[g * 4 + 3] * mul)};
    }
#pragma unroll
  for (int i = 0; i < 32 * ROW / 1024; ++i) {
    const int off = i * 1024 + lane * 16, r = off / ROW, ch = (off % ROW) / 16;
    const u32x4 x = *(const u32x4*)(stg + r * ROW + ((ch ^ (r % NCH)) << 4));
    if (r < nvalid) *(u32x4*)((uint8_t*)dst0 + off) = x;
  }
}

// B-operand fragments of one row (this lane's) of a [N, D] tensor: head-dim step s holds
// elements s * 16 + half * 8 .. + 7; zero past the end of the sequence.
template <int D>
__device__ __forceinline__ void load_row_operand(const uint16_t* base, int row, int N, int half, u32x4 (&r)[D / 16]) {
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    r[s] = row < N ? *(const u32x4*)(base + (int64_t)row * D + s * 16 + half * 8) : u32x4{0, 0, 0, 0};
}

}  // namespace attn
