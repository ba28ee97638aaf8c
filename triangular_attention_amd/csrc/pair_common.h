// Device helpers shared by the pair-feature kernels (triangle-attention block and triangle
// multiplicative update): swizzled LDS tiles of 128-element rows, 16-lane DPP sums, the
// LayerNorm forms every kernel must share bit for bit, pair indexing and bf16 packing.
#pragma once
#include "common.h"

namespace tri {
namespace pair {

// Chunk swizzle of a 256-byte row (16 chunks of 16 bytes).  gfx950 serves an LDS access as two
// 32-lane halves; a half is conflict-free when its 16-byte slots are distinct modulo 512 bytes
// (16-byte accesses) or its 8-byte units distinct modulo 256 bytes (8-byte accesses).  The XOR
// mask below, a linear map of the row's low four bits, makes every access shape of the pair
// kernels conflict-free under that rule (checked exhaustively on the host): MFMA operand reads
// (16 consecutive rows, chunks 2k and 2k + 1 in a half), transposing reads (rows 8g + 0..3 and
// + 4, two adjacent chunks, both 8-byte halves), 8-byte reads of one chunk of 16 rows, and
// stores of 8 rows x 4 chunks, 16 rows x 2 chunks or 2 rows x 16 chunks.
__device__ __forceinline__ int swz(int r) { return ((r & 7) << 1) ^ (-((r >> 3) & 1) & 11); }
// element offset of logical 16-byte chunk j (0..15) of row r in a [rows][128] bf16 tile
__device__ __forceinline__ int toff(int r, int j) { return r * 128 + ((j ^ swz(r)) << 3); }

// Transposing read of an 8-slot MFMA operand from a swizzled [rows][128] tile:
// the lane receives column col0 + (lane & 15) of rows row0 + 0..7.
__device__ __forceinline__ u32x4 tr8_swz(const uint16_t* tile, int row0, int col0, int lane) {
  const int kk = (lane & 15) >> 2, a = lane & 3;
  const int col = col0 + 4 * a, j = col >> 3, half = (col >> 2) & 1;
  const int r0 = row0 + kk, r1 = r0 + 4;
  return ds_read_tr8_at(tile, toff(r0, j) + 4 * half, toff(r1, j) + 4 * half);
}

// Sum over the 16 lanes of a row with DPP; every lane ends with the same value.
template <int CTRL> __device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum16(float x) {
  x += dpp_mov<0xB1>(x);    // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);    // quad_perm [2,3,0,1]
  x += dpp_mov<0x141>(x);   // row_half_mirror
  x += dpp_mov<0x140>(x);   // row_mirror
  return x;
}

// The normalised feature exactly as every kernel forms it (forward and backward
// must agree bit for bit): xhat = (z - mean) * rstd, zln = xhat * gamma + beta (one FMA).
__device__ __forceinline__ float ln_xhat(float z, float mean, float rstd) { return (z - mean) * rstd; }
__device__ __forceinline__ float ln_out(float xh, float gm, float bt) { return __builtin_fmaf(xh, gm, bt); }
__device__ __forceinline__ float sigm(float x) { return 1.f / (1.f + __expf(-x)); }

struct PairIx { int b, x, y; };
__device__ __forceinline__ PairIx pair_ix(int r, int N) {
  const int nn = N * N;
  PairIx p;
  p.b = r / nn;
  const int rem = r - p.b * nn;
  p.x = rem / N;
  p.y = rem - p.x * N;
  return p;
}
// Element offset of the pair's 128-feature row in Z / dZ / Y / dY.
__device__ __forceinline__ int zrow(const PairIx& p, int N, int ending) {
  return ((p.b * N + (ending ? p.y : p.x)) * N + (ending ? p.x : p.y)) * 128;
}
// Element offset of (pair, head h, feature d) in a [B, N, H, N, D] tensor.
template <int H, int D>
__device__ __forceinline__ int hm_off(const PairIx& p, int N, int h, int d) {
  return ((p.b * N + p.x) * H + h) * N * D + p.y * D + d;
}

// The pairs of one tile, r0 = tile * TP .. r0 + TP - 1, where pair r = (b N + x) N + y.  When they
// all lie in one row (b, x) of the pair grid and inside the problem (always so when TP divides N),
// pair l of the tile is (b, x, y0 + l) and its offsets need no division: one division pair per
// tile replaces one per pair and load (each an integer-division sequence of some twenty vector
// instructions).  Otherwise (rows shorter than a tile, the last tile) every pair is divided out.
// The struct depends only on the tile, so `one` is the same for the whole workgroup.  The fast
// forms use 24-bit products, so they are also limited to B N < 2^23 rows.
struct TileRows {
  int r0, b, x, y0;
  bool one;
};
__device__ __forceinline__ TileRows tile_rows(int tile, int TP, int N, int total) {
  TileRows t;
  t.r0 = tile * TP;
  const PairIx p = pair_ix(t.r0 < total ? t.r0 : 0, N);
  t.b = p.b;
  t.x = p.x;
  t.y0 = p.y;
  t.one = t.r0 + TP <= total && p.y + TP <= N && (total >> 23) < N;
  return t;
}
// Pair l (< TP) of the tile is inside the problem.
__device__ __forceinline__ bool tile_ok(const TileRows& t, int l, int total) { return t.one || t.r0 + l < total; }
// zrow of pair l of the tile (the pair must be inside the problem)
__device__ __forceinline__ int zrow_t(const TileRows& t, int l, int N, int ending) {
  if (t.one) return ending ? (__mul24(t.b * N + t.y0 + l, N) + t.x) * 128 : (t.r0 + l) * 128;
  return zrow(pair_ix(t.r0 + l, N), N, ending);
}
// hm_off of pair l of the tile (the pair must be inside the problem)
template <int H, int D>
__device__ __forceinline__ int hm_off_t(const TileRows& t, int l, int N, int h, int d) {
  if (t.one) return (t.b * N + t.x) * (H * N * D) + __mul24(h, N * D) + (t.y0 + l) * D + d;
  return hm_off<H, D>(pair_ix(t.r0 + l, N), N, h, d);
}
// Element offset of pair l's entry of head h in a [B, H, N, N] tensor (the pair bias)
template <int H>
__device__ __forceinline__ int bias_off_t(const TileRows& t, int l, int N, int h) {
  if (t.one) return (t.b * H * N + t.x) * N + t.y0 + l + h * (N * N);
  const PairIx p = pair_ix(t.r0 + l, N);
  return ((p.b * H + h) * N + p.x) * N + p.y;
}

__device__ __forceinline__ void unpack8(u32x4 v, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) { f[2 * i] = bf_lo(v[i]); f[2 * i + 1] = bf_hi(v[i]); }
}
__device__ __forceinline__ u32x4 pack8(const float* f) {
  return u32x4{pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]), pack_bf16(f[4], f[5]), pack_bf16(f[6], f[7])};
}
__device__ __forceinline__ void st_lds16(uint16_t* tile, int off, u32x4 v) {
  *reinterpret_cast<u32x4*>(tile + off) = v;
}
__device__ __forceinline__ u32x4 ld_lds16(const uint16_t* tile, int off) {
  return *reinterpret_cast<const u32x4*>(tile + off);
}

}  // namespace pair
}  // namespace tri
