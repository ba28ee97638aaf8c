// LDS tile layouts of the backward kernels (gfx950) and the operand read that uses them.
// Both backward kernels stage Q / dO rows (read row-wise and, in the key-tile kernel,
// transposed) and K / V rows (read row-wise for the score products and transposed for
// the dQ product); the swizzles below keep those access shapes on distinct LDS banks.
#pragma once
#include "common.h"

namespace tri {

// Element offset of (row, col) in the LDS tiles.  D = 32: unpadded 64-byte rows.  Q, dO
// (and V): row r at row position pq(r) (row bit 4 copied into bit 2), its 16-byte chunks
// XORed with 2 where row bit 3 is set, so that the score-product reads (rows
// 8(c/4) + 4e + c%4 of a 32-row tile, one chunk per lane group), the transposing reads and
// 16 consecutive rows all touch distinct banks per half-wave; K: chunk XOR by row bits 2-3.
// D = 16: Q / dO rows padded to 24 elements.
template <int D> struct Lay;
template <> struct Lay<32> {
  static constexpr int kRowElems = 32;
  static constexpr int kKVRowElems = 32;
  __device__ static __forceinline__ int pq(int row) { return row ^ (((row >> 4) & 1) << 2); }
  __device__ static __forceinline__ int swq(int row) { return ((row >> 3) & 1) << 1; }
  __device__ static __forceinline__ int swk(int row) { return (row >> 2) & 3; }
  __device__ static __forceinline__ int q(int row, int col) {
    return pq(row) * 32 + ((((col >> 3) ^ swq(row)) & 3) << 3) + (col & 7);
  }
  __device__ static __forceinline__ int k(int row, int col) {
    return row * 32 + ((((col >> 3) ^ swk(row)) & 3) << 3) + (col & 7);
  }
  __device__ static __forceinline__ int v(int row, int col) { return q(row, col); }
  // logical row stored at row position `prow` (pq is an involution), and the logical chunk
  // stored in physical slot `pchunk` of logical row `row`
  __device__ static __forceinline__ int q_src_row(int prow) { return pq(prow); }
  __device__ static __forceinline__ int q_src_chunk(int row, int pchunk) { return (pchunk ^ swq(row)) & 3; }
  static constexpr int kSlotsPerRow = 4;
};
template <> struct Lay<16> {
  static constexpr int kRowElems = 24;       // Q / dO rows padded to 48 bytes
  static constexpr int kKVRowElems = 16;     // K / V rows unpadded (32 bytes)
  __device__ static __forceinline__ int q(int row, int col) { return row * 24 + col; }
  // K and V: in every 16-row group rows 8..11 and 12..15 trade places (row bit 2
  // flipped where bit 3 is set) and the four 8-byte units of those rows are
  // permuted by an XOR with 2, so that both the row reads (16 rows x 2 units per
  // half-wave) and the transposing reads (rows 0..3 and 8..11 of a 16-row group)
  // touch 64 distinct banks
  __device__ static __forceinline__ int k(int row, int col) {
    const int hi = (row >> 3) & 1;
    return (row ^ (hi << 2)) * 16 + ((((col >> 2) ^ (hi << 1)) & 3) << 2) + (col & 3);
  }
  __device__ static __forceinline__ int v(int row, int col) { return k(row, col); }
  __device__ static __forceinline__ int q_src_row(int prow) { return prow; }
  __device__ static __forceinline__ int q_src_chunk(int row, int pchunk) { return pchunk < 2 ? pchunk : 0; }
  static constexpr int kSlotsPerRow = 3;     // two data chunks and one padding chunk
};

// D = 64: unpadded 128-byte rows of eight 16-byte chunks, the chunk index XORed with a
// row-dependent value.  Per half-wave, the score-product row reads touch four rows of
// equal (row mod 4) at two chunks each (Q / dO: rows differing in bits 3-4; K / V: bits
// 2-3) and the transposing reads four rows of equal parity at two chunks each (bits 1
// and 3); the XOR values below give every such set eight distinct 16-byte positions
// (and distinct 8-byte units for the transposing reads).
template <> struct Lay<64> {
  static constexpr int kRowElems = 64;
  static constexpr int kKVRowElems = 64;
  __device__ static __forceinline__ int swq(int row) {
    return (((row >> 1) & 1) * 2) ^ (((row >> 3) & 1) * 5) ^ (((row >> 4) & 1) * 4);
  }
  __device__ static __forceinline__ int swk(int row) {
    return (((row >> 1) & 1) * 2) ^ (((row >> 2) & 1) * 4) ^ (((row >> 3) & 1) * 5);
  }
  __device__ static __forceinline__ int q(int row, int col) {
    return row * 64 + ((((col >> 3) ^ swq(row)) & 7) << 3) + (col & 7);
  }
  __device__ static __forceinline__ int k(int row, int col) {
    return row * 64 + ((((col >> 3) ^ swk(row)) & 7) << 3) + (col & 7);
  }
  __device__ static __forceinline__ int v(int row, int col) { return k(row, col); }
  __device__ static __forceinline__ int q_src_row(int prow) { return prow; }
  __device__ static __forceinline__ int q_src_chunk(int row, int pchunk) { return (pchunk ^ swq(row)) & 7; }
  static constexpr int kSlotsPerRow = 8;
};

// One lane's contraction operand (DOp<D>::T) from an LDS tile: D / 4 elements from
// column col of row row; with D = 64 its two 16-byte chunks sit at their own swizzled
// positions.
template <int D, typename F>
__device__ __forceinline__ typename DOp<D>::T ld_op(const uint16_t* t, int row, int col, F at) {
  if constexpr (D == 64) {
    typename DOp<D>::T r;
    r.x[0] = ld_shared<u32x4>(&t[at(row, col)]);
    r.x[1] = ld_shared<u32x4>(&t[at(row, col + 8)]);
    return r;
  } else {
    return ld_shared<typename DOp<D>::T>(&t[at(row, col)]);
  }
}

}  // namespace tri
