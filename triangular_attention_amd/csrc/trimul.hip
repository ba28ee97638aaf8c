// Triangle multiplicative update (outgoing and incoming) for gfx950.
//
// "TurboPairFormer: Fast and Stable Protein Folding Model Training with an
// Optimized Triangle Attention Kernel", Figure 12: an input step normalises the
// pair features and forms five projections (two branch values, two branch gates,
// the output gate logits) and gates the branch values; one contraction per
// channel; an output step normalises the contraction, projects it back to the
// pair features and multiplies by the sigmoid of the saved gate logits.
//
// The incoming form contracts over the first token index (x[i,j] = sum_k a[k,i]
// b[k,j]).  Here the input kernels read Z with its token axes swapped for it and
// write the branch operands transposed, so both forms share one contraction
// x[c] = A[c] B[c]^T and the backward products dA = dX B, dB = dX^T A.
//
// Kernels (persistent on a grid fixed by the problem size, except the products):
//   tm_in_fwd    LayerNorm + the 4c + 128 projections; gated branch operands written
//                channel-major through an LDS tile (16-byte stores), gate logits pair-major
//   tm_gemm      one N x N x N product per (example, channel) on MFMA, 128 x 128 tiles,
//                operands staged in LDS (row or transposing reads per orientation)
//   tm_out_fwd   LayerNorm over the channels (two-pass FP32 statistics), projection, gate
//   tm_out_bwd   gate / projection / LayerNorm backward; d w_o and d gamma_o / d beta_o partials
//   tm_in_bwd    recomputes the branch projections and forms their gradients (dproj)
//   tm_in_dz     dZ through the input projections and the LayerNorm; d gamma / d beta partials
//   tm_in_dw     d w_in partials (128 rows per workgroup, the workgroups of one tile group
//                on one XCD so that the shared Z tiles come from its L2)
// All products are bf16 MFMA (v_mfma_f32_16x16x32_bf16) with FP32 accumulation; no MFMA
// sits in a lane-masked branch (the matrix cores ignore EXEC).
#include <type_traits>

#include "common.h"
#include "pair_common.h"
#include "trimul_kernels.h"

namespace tri {
namespace {

using namespace pair;
constexpr int C = kTmC;
constexpr int NT = 512;

// channel-major element offset of (kernel pair r, channel ch) in [B, c, N, N]
__device__ __forceinline__ int cm_off(int r, int ch, int nn, int c) {
  const int b = r / nn;
  return (b * c + ch) * nn + (r - b * nn);
}
// the same for pair l of a tile (TileRows: no division when the tile lies in one row)
__device__ __forceinline__ int cm_off_t(const TileRows& t, int l, int ch, int nn, int c) {
  if (t.one) return t.b * (c - 1) * nn + t.r0 + l + ch * nn;
  return cm_off(t.r0 + l, ch, nn, c);
}

// [channel][pair] LDS tiles: rows of 128 pairs padded to 144 elements (row stride 8 banks), so
// the transposing reads of 4 rows are conflict-free and a pair-block offset is a constant
// (an XOR swizzle would make every pair block a separate address register).
constexpr int CP = 144;
__device__ __forceinline__ int coff(int ch, int p) { return ch * CP + p; }
__device__ __forceinline__ u32x4 tr8_pad(const uint16_t* tile, int row0, int col0, int lane) {
  const int kk = (lane & 15) >> 2, a = lane & 3;
  const int o = (row0 + kk) * CP + col0 + 4 * a;
  return ds_read_tr8_at(tile, o, o + 4 * CP);
}

// Wave w's branch items: (kind 0 = a / 1 = b, 16-channel block).  c = 128: both kinds of block w;
// c = 64: kind w & 1 of block w >> 1.
template <int CH> __device__ __forceinline__ int item_kind(int it, int w) { return CH == 128 ? it : (w & 1); }
template <int CH> __device__ __forceinline__ int item_cb(int it, int w) { return CH == 128 ? w : (w >> 1); }

// LayerNorm of 4 pair rows per lane (16 lanes per pair, 8 features per lane) into a Zln tile.
struct LnRows {
  float gm[8], bt[8];
  __device__ __forceinline__ void init(const float* gamma, const float* beta, int c) {
#pragma unroll
    for (int i = 0; i < 8; ++i) { gm[i] = gamma[8 * c + i]; bt[i] = beta[8 * c + i]; }
  }
};

// ----------------------------------------------------------------------------------------------
// Input step, forward.  Tile = 128 pairs.
template <int CH>
__global__ __launch_bounds__(NT) void tm_in_fwd_kernel(TmInArgs a) {
  constexpr int TP = kTmTileIn;
  constexpr int NIT = CH / 64;
  constexpr int NSTORE = CH * TP / 8 / NT;
  __shared__ __align__(16) uint16_t sZ[2][TP * C];
  __shared__ __align__(16) uint16_t sAB[2][CH * CP];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
  const int t = threadIdx.x;
  const int N = a.s.N, inc = a.s.incoming, nn = N * N;
  const int total = a.s.B * nn;
  const int ntiles = (total + TP - 1) / TP;
  const uint32_t zbytes = (uint32_t)total * C * 2;
  const auto zr = make_rsrc(a.z, zbytes);

  LnRows ln;
  ln.init(a.gamma, a.beta, c);
  u32x4 wv[NIT][4], wq[NIT][4], wo[4];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int kind = item_kind<CH>(it, w), cb = item_cb<CH>(it, w);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      wv[it][s] = ld_global<u32x4>(a.w_in + (kind * 2 * CH + cb * 16 + c) * C + 32 * s + 8 * g);
      wq[it][s] = ld_global<u32x4>(a.w_in + (kind * 2 * CH + CH + cb * 16 + c) * C + 32 * s + 8 * g);
    }
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) wo[s] = ld_global<u32x4>(a.w_in + (4 * CH + 16 * w + c) * C + 32 * s + 8 * g);

  u32x4 zv[4];
  auto load_z = [&](int tile) {
    const TileRows tr = tile_rows(tile, TP, N, total);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int l = 16 * w + 4 * s + g;
      zv[s] = buf_ld16(zr, tile_ok(tr, l, total) ? (uint32_t)zrow_t(tr, l, N, inc) * 2 + 16 * c : zbytes);
    }
  };
  if ((int)blockIdx.x < ntiles) load_z(blockIdx.x);
  int iter = 0;
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x, ++iter) {
    uint16_t* buf = sZ[iter & 1];
    const TileRows tr = tile_rows(tile, TP, N, total);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float x[8];
      unpack8(zv[s], x);
      float sum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) sum += x[i];
      const float mean = sum16(sum) * (1.f / C);
      float sq = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) { x[i] -= mean; sq += x[i] * x[i]; }
      const float rstd = 1.f / sqrtf(sum16(sq) * (1.f / C) + a.s.eps);
      float y[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = ln_out(x[i] * rstd, ln.gm[i], ln.bt[i]);
      const int rl = 16 * w + 4 * s + g;
      st_lds16(buf, toff(rl, c), pack8(y));
      const int r = tile * TP + rl;
      if (c == 0 && r < total) *reinterpret_cast<f32x2*>(a.stats + 2 * (size_t)r) = f32x2{mean, rstd};
    }
    const int nt = tile + gridDim.x;
    if (nt < ntiles) load_z(nt);
    lds_barrier();
#pragma unroll 2
    for (int pb = 0; pb < TP / 16; ++pb) {
      const int rl = 16 * pb + c;
      u32x4 bf[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) bf[s] = ld_lds16(buf, toff(rl, 4 * s + g));
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int kind = item_kind<CH>(it, w), cb = item_cb<CH>(it, w);
        // pairs as rows: lane (g, c) gets pairs 16pb + 4g + 0..3 of channel cb*16 + c, written
        // to the [channel][pair] tile as one 8-byte word
        f32x4 av = {0.f, 0.f, 0.f, 0.f}, ag = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          av = mfma_k32(bf[s], wv[it][s], av);
          ag = mfma_k32(bf[s], wq[it][s], ag);
        }
        float ab[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ab[i] = sigm(ag[i]) * av[i];
        *reinterpret_cast<u32x2*>(&sAB[kind][coff(cb * 16 + c, 16 * pb + 4 * g)]) =
            u32x2{pack_bf16(ab[0], ab[1]), pack_bf16(ab[2], ab[3])};
      }
      f32x4 go = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) go = mfma_k32(wo[s], bf[s], go);
      if (tile_ok(tr, rl, total))
        *reinterpret_cast<u32x2*>(a.g + zrow_t(tr, rl, N, inc) + 16 * w + 4 * g) =
            u32x2{pack_bf16(go[0], go[1]), pack_bf16(go[2], go[3])};
    }
    lds_barrier();
    // channel-major stores: 8 consecutive pairs of one channel per 16 bytes
#pragma unroll
    for (int kd = 0; kd < 2; ++kd) {
      uint16_t* dst = kd ? a.b : a.a;
#pragma unroll
      for (int k = 0; k < NSTORE; ++k) {
        const int q = t + NT * k, ch = q >> 4, seg = q & 15;
        if (tr.r0 + 8 * seg < total)
          *reinterpret_cast<u32x4*>(dst + cm_off_t(tr, 8 * seg, ch, nn, CH)) = ld_lds16(sAB[kd], coff(ch, 8 * seg));
      }
    }
  }
}

// ----------------------------------------------------------------------------------------------
// Input step, backward part 1: recompute the four branch projections exactly as the forward did
// (Zln from Z and the saved statistics) and form their gradients from da, db.
template <int CH>
__global__ __launch_bounds__(NT) void tm_in_bwd_kernel(TmInArgs a) {
  constexpr int TP = kTmTileIn;
  constexpr int NIT = CH / 64;
  constexpr int NLD = CH * TP / 8 / NT;
  __shared__ __align__(16) uint16_t sZ[TP * C];
  __shared__ __align__(16) uint16_t sD[2][CH * CP];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
  const int t = threadIdx.x;
  const int N = a.s.N, inc = a.s.incoming, nn = N * N;
  const int total = a.s.B * nn;
  const int ntiles = (total + TP - 1) / TP;
  const uint32_t zbytes = (uint32_t)total * C * 2, cbytes = (uint32_t)total * CH * 2;
  const auto zr = make_rsrc(a.z, zbytes);
  const auto sr = make_rsrc(a.stats, (uint32_t)total * 8);
  const auto dar = make_rsrc(a.da, cbytes), dbr = make_rsrc(a.db, cbytes);

  LnRows ln;
  ln.init(a.gamma, a.beta, c);
  u32x4 wv[NIT][4], wq[NIT][4];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int kind = item_kind<CH>(it, w), cb = item_cb<CH>(it, w);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      wv[it][s] = ld_global<u32x4>(a.w_in + (kind * 2 * CH + cb * 16 + c) * C + 32 * s + 8 * g);
      wq[it][s] = ld_global<u32x4>(a.w_in + (kind * 2 * CH + CH + cb * 16 + c) * C + 32 * s + 8 * g);
    }
  }
  u32x4 zv[4], dv[2][NLD];
  f32x2 st[4];
  auto load = [&](int tile) {
    const TileRows tr = tile_rows(tile, TP, N, total);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int l = 16 * w + 4 * s + g, r = tr.r0 + l;
      const bool ok = tile_ok(tr, l, total);
      zv[s] = buf_ld16(zr, ok ? (uint32_t)zrow_t(tr, l, N, inc) * 2 + 16 * c : zbytes);
      st[s] = __builtin_bit_cast(f32x2, buf_ld8(sr, ok ? (uint32_t)r * 8 : (uint32_t)total * 8));
    }
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      const int q = t + NT * k, ch = q >> 4, seg = q & 15;
      const uint32_t off = tr.r0 + 8 * seg < total ? (uint32_t)cm_off_t(tr, 8 * seg, ch, nn, CH) * 2 : cbytes;
      dv[0][k] = buf_ld16(dar, off);
      dv[1][k] = buf_ld16(dbr, off);
    }
  };
  if ((int)blockIdx.x < ntiles) load(blockIdx.x);
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    lds_barrier();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float x[8], y[8];
      unpack8(zv[s], x);
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = ln_out(ln_xhat(x[i], st[s][0], st[s][1]), ln.gm[i], ln.bt[i]);
      st_lds16(sZ, toff(16 * w + 4 * s + g, c), pack8(y));
    }
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      const int q = t + NT * k, ch = q >> 4, seg = q & 15;
      st_lds16(sD[0], coff(ch, 8 * seg), dv[0][k]);
      st_lds16(sD[1], coff(ch, 8 * seg), dv[1][k]);
    }
    const int nt = tile + gridDim.x;
    if (nt < ntiles) load(nt);
    lds_barrier();
#pragma unroll 2
    for (int pb = 0; pb < TP / 16; ++pb) {
      const int rl = 16 * pb + c;
      const int r = tile * TP + rl;
      u32x4 bf[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) bf[s] = ld_lds16(sZ, toff(rl, 4 * s + g));
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int kind = item_kind<CH>(it, w), cb = item_cb<CH>(it, w);
        f32x4 av = {0.f, 0.f, 0.f, 0.f}, ag = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          av = mfma_k32(wv[it][s], bf[s], av);
          ag = mfma_k32(wq[it][s], bf[s], ag);
        }
        float gv[4], gg[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ch = cb * 16 + 4 * g + i;
          const float d = bf_to_f(sD[kind][coff(ch, rl)]);
          const float sg = sigm(ag[i]);
          gv[i] = d * sg;
          gg[i] = d * av[i] * (sg * (1.f - sg));
        }
        if (r < total) {
          uint16_t* row = a.dproj + (size_t)r * 4 * CH + kind * 2 * CH + cb * 16 + 4 * g;
          *reinterpret_cast<u32x2*>(row) = u32x2{pack_bf16(gv[0], gv[1]), pack_bf16(gv[2], gv[3])};
          *reinterpret_cast<u32x2*>(row + CH) = u32x2{pack_bf16(gg[0], gg[1]), pack_bf16(gg[2], gg[3])};
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------------------------
// The per-channel products.  C[b] = opA(b) opB(b) with M = N = K = n for every b (an example
// and channel).  TA: A stored [k][m] (else [m][k]); TB: B stored [k][n] (else [n][k]).  The MFMA
// forms C^T = opB^T opA^T so that a lane's four results are four consecutive n of one m.
// 256 threads, MT x MT tile, waves 2 x 2 of MT/2 x MT/2, k step 32, operand tiles double-buffered.
// MT = 192 when 192 divides n (4 x 4 tiles per matrix at n = 768: with two workgroups per CU the
// 2048 tiles of 128 channels are exactly 4 rounds of the 256 CUs, where 128 x 128 tiles left the
// last of 4.5 rounds half empty); 128 otherwise.
template <bool TA, bool TB, int MT>
__global__ __launch_bounds__(256) void tm_gemm_kernel(TmGemmArgs p) {
  constexpr int TK = 32;
  constexpr int MB = MT / 32;          // 16-row blocks of a wave in m (a wave holds MT / 2 rows)
  constexpr int LA = MT / 64;          // A-tile loads per thread
  constexpr int NTT = MT;              // n rows of the tile (the B tile)
  constexpr int NBB = NTT / 32;        // 16-column blocks of a wave in n
  constexpr int LB = NTT / 64;
  static_assert(MT == 128 || MT == 192, "tiles of 128 or 192");
  constexpr int CPR = MT / 8;          // 16-byte chunks per row of a transposed ([k][m]) tile
  __shared__ __align__(16) uint16_t sA[2][MT * TK];
  __shared__ __align__(16) uint16_t sB[2][NTT * TK];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
  const int t = threadIdx.x;
  const int N = p.N, ntm = (N + MT - 1) / MT, nt = (N + NTT - 1) / NTT, ntile = ntm * nt;
  // all tiles of one matrix on one XCD (blocks are dealt round-robin over 8 XCDs)
  const int xcd = blockIdx.x & 7, kx = blockIdx.x >> 3;
  const int bt = (kx / ntile) * 8 + xcd;
  if (bt >= p.batch) return;
  const int tile = kx % ntile, m0 = (tile / nt) * MT, n0 = (tile % nt) * NTT;
  const uint32_t bytes = (uint32_t)p.batch * N * N * 2;
  const auto ar = make_rsrc(p.A, bytes), br = make_rsrc(p.B, bytes);
  const int base = bt * N * N;
  const int wm = w >> 1, wn = w & 1;

  // row-major [MT][32] tiles: 16-byte chunk kc of row r stored at kc ^ ((r >> 1) & 3); an LDS probe
  // of the operand reads (16 rows, chunk g per lane group) measured no bank conflicts for this
  // mask, 3.8 conflict cycles per read for kc ^ ((r >> 2) & 3)
  auto off32 = [](int r, int kc) { return r * 32 + ((kc ^ ((r >> 1) & 3)) << 3); };
  // transposed tiles [32 k][MT]: 128-wide rows use the pair-tile swizzle (toff); 192-wide rows
  // XOR the chunk (within its aligned group of 8) with 2 (row bit 1) and 4 (row bit 3), which
  // keeps the transposing reads of rows 8g + 0..3 (+4) and the row-major stores conflict-free
  auto offT = [](int r, int j) {
    if constexpr (MT == 128) return toff(r, j);
    else return r * MT + ((j ^ ((((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2))) << 3);
  };
  auto trT = [&](const uint16_t* tile, int row0, int col0) {
    const int kk = (lane & 15) >> 2, a4 = lane & 3;
    const int col = col0 + 4 * a4, j = col >> 3, half = (col >> 2) & 1;
    const int r0 = row0 + kk, r1 = r0 + 4;
    return ds_read_tr8_at(tile, offT(r0, j) + 4 * half, offT(r1, j) + 4 * half);
  };
  u32x4 la[LA], lb[LB];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int q = t + 256 * i;
      if constexpr (!TA) {
        const int row = q >> 2, kc = q & 3, k = k0 + 8 * kc;
        la[i] = buf_ld16(ar, k < N ? (uint32_t)(base + (m0 + row) * N + k) * 2 : bytes);
      } else {
        const int row = q / CPR, mc = q % CPR, k = k0 + row;
        la[i] = buf_ld16(ar, k < N ? (uint32_t)(base + k * N + m0 + 8 * mc) * 2 : bytes);
      }
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int q = t + 256 * i;
      if constexpr (!TB) {
        const int row = q >> 2, kc = q & 3, k = k0 + 8 * kc;
        lb[i] = buf_ld16(br, k < N ? (uint32_t)(base + (n0 + row) * N + k) * 2 : bytes);
      } else {
        const int row = q / CPR, nc = q % CPR, k = k0 + row;
        lb[i] = buf_ld16(br, k < N ? (uint32_t)(base + k * N + n0 + 8 * nc) * 2 : bytes);
      }
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      const int q = t + 256 * i;
      if constexpr (!TA) st_lds16(sA[buf], off32(q >> 2, q & 3), la[i]);
      else st_lds16(sA[buf], offT(q / CPR, q % CPR), la[i]);
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int q = t + 256 * i;
      if constexpr (!TB) st_lds16(sB[buf], off32(q >> 2, q & 3), lb[i]);
      else st_lds16(sB[buf], offT(q / CPR, q % CPR), lb[i]);
    }
  };

  f32x4 acc[NBB][MB];
#pragma unroll
  for (int i = 0; i < NBB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  load(0);
  for (int k0 = 0, step = 0; k0 < N; k0 += TK, ++step) {
    const int buf = step & 1;
    stash(buf);
    if (k0 + TK < N) load(k0 + TK);
    lds_barrier();
    u32x4 fa[NBB], fb[MB];
#pragma unroll
    for (int nb = 0; nb < NBB; ++nb) {
      const int n = wn * (NTT / 2) + nb * 16;
      if constexpr (!TB) fa[nb] = ld_lds16(sB[buf], off32(n + c, g));
      else fa[nb] = trT(sB[buf], 8 * g, n);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = wm * (MT / 2) + mb * 16;
      if constexpr (!TA) fb[mb] = ld_lds16(sA[buf], off32(m + c, g));
      else fb[mb] = trT(sA[buf], 8 * g, m);
    }
#pragma unroll
    for (int nb = 0; nb < NBB; ++nb)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[nb][mb] = mfma_k32(fa[nb], fb[mb], acc[nb][mb]);
  }
#pragma unroll
  for (int nb = 0; nb < NBB; ++nb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int m = m0 + wm * (MT / 2) + mb * 16 + c, n = n0 + wn * (NTT / 2) + nb * 16 + 4 * g;
      if (m < N && n < N)
        *reinterpret_cast<u32x2*>(p.C + base + m * N + n) =
            u32x2{pack_bf16(acc[nb][mb][0], acc[nb][mb][1]), pack_bf16(acc[nb][mb][2], acc[nb][mb][3])};
    }
}

// ----------------------------------------------------------------------------------------------
// Output step.  Tile = 128 update pairs; the contraction tile is staged [channel][pair].
// c = 64: two workgroups per CU (at most 128 VGPRs); c = 128 keeps one (it would spill)
template <int CH>
__global__ __launch_bounds__(NT, CH == 64 ? 4 : 2) void tm_out_fwd_kernel(TmOutArgs a) {
  constexpr int TP = kTmTileOut;
  constexpr int NQ = CH / 4;                 // channels per thread in the statistics passes
  constexpr int NLD = CH * TP / 8 / NT;      // 16-byte chunks per thread of a contraction tile
  __shared__ __align__(16) uint16_t sX[CH * CP];
  __shared__ __align__(16) float sRed[4][TP];
  __shared__ float sGam[CH], sBet[CH];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
  const int t = threadIdx.x;
  const int N = a.s.N, nn = N * N;
  const int total = a.s.B * nn;
  const int ntiles = (total + TP - 1) / TP;
  const uint32_t xbytes = (uint32_t)total * CH * 2;
  const auto xr = make_rsrc(a.x, xbytes);
  for (int i = t; i < CH; i += NT) { sGam[i] = a.gamma_o[i]; sBet[i] = a.beta_o[i]; }
  u32x4 wo[CH / 32];
#pragma unroll
  for (int s = 0; s < CH / 32; ++s) wo[s] = ld_global<u32x4>(a.w_o + (16 * w + c) * CH + 32 * s + 8 * g);
  const int pp = t & (TP - 1), qq = t >> 7;    // statistics: pair pp, channel quarter qq

  const uint32_t gbytes = (uint32_t)total * C * 2;
  const auto gr = make_rsrc(a.g, gbytes);
  u32x4 xv[NLD];
  u32x2 gv[TP / 16];        // this lane's gate logits of the tile (4 features of one pair per block)
  auto load = [&](int tile) {
    const TileRows tr = tile_rows(tile, TP, N, total);
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      const int q = t + NT * k, ch = q >> 4, seg = q & 15;
      xv[k] = buf_ld16(xr, tr.r0 + 8 * seg < total ? (uint32_t)cm_off_t(tr, 8 * seg, ch, nn, CH) * 2 : xbytes);
    }
#pragma unroll
    for (int pb = 0; pb < TP / 16; ++pb) {
      const int r = tile * TP + 16 * pb + c;
      gv[pb] = buf_ld8(gr, r < total ? (uint32_t)(r * C + 16 * w + 4 * g) * 2 : gbytes);
    }
  };
  if ((int)blockIdx.x < ntiles) load(blockIdx.x);
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    lds_barrier();
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      const int q = t + NT * k;
      st_lds16(sX, coff(q >> 4, 8 * (q & 15)), xv[k]);
    }
    u32x2 gc[TP / 16];
#pragma unroll
    for (int pb = 0; pb < TP / 16; ++pb) gc[pb] = gv[pb];
    const int nt = tile + gridDim.x;
    if (nt < ntiles) load(nt);
    lds_barrier();
    float v[NQ];
    float s1 = 0.f;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      v[j] = bf_to_f(sX[coff(qq * NQ + j, pp)]);
      s1 += v[j];
    }
    sRed[qq][pp] = s1;
    lds_barrier();
    const float mean = ((sRed[0][pp] + sRed[1][pp]) + (sRed[2][pp] + sRed[3][pp])) * (1.f / CH);
    float s2 = 0.f;
#pragma unroll
    for (int j = 0; j < NQ; ++j) { v[j] -= mean; s2 += v[j] * v[j]; }
    lds_barrier();
    sRed[qq][pp] = s2;
    lds_barrier();
    const float rstd = 1.f / sqrtf(((sRed[0][pp] + sRed[1][pp]) + (sRed[2][pp] + sRed[3][pp])) * (1.f / CH) +
                                   a.s.eps);
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const int ch = qq * NQ + j;
      sX[coff(ch, pp)] = f_to_bf(ln_out(v[j] * rstd, sGam[ch], sBet[ch]));
    }
    const int rp = tile * TP + pp;
    if (qq == 0 && rp < total) *reinterpret_cast<f32x2*>(a.stats_o + 2 * (size_t)rp) = f32x2{mean, rstd};
    lds_barrier();
#pragma unroll
    for (int pb = 0; pb < TP / 16; ++pb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < CH / 32; ++s) acc = mfma_k32(wo[s], tr8_pad(sX, 32 * s + 8 * g, 16 * pb, lane), acc);
      const int r = tile * TP + 16 * pb + c;
      if (r < total) {
        const size_t o = (size_t)r * C + 16 * w + 4 * g;
        const u32x2 gl = gc[pb];
        const float gf[4] = {bf_lo(gl[0]), bf_hi(gl[0]), bf_lo(gl[1]), bf_hi(gl[1])};
        float ov[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ov[i] = sigm(gf[i]) * acc[i];
        *reinterpret_cast<u32x2*>(a.out + o) = u32x2{pack_bf16(ov[0], ov[1]), pack_bf16(ov[2], ov[3])};
      }
    }
  }
}

// Output step, backward.  Tile = 128 update pairs.
//   p = LN(x) w_o^T (recomputed), dp = dout * sigmoid(g), d g = dout * p * sigmoid'(g)
//   dxln = dp w_o (waves own 16-channel blocks), dx by the LayerNorm backward
//   d w_o += dp^T LN(x) (wave w: output features 16w..16w+15 x all channels)
template <int CH>
__global__ __launch_bounds__(NT) void tm_out_bwd_kernel(TmOutArgs a) {
  constexpr int TP = kTmTileOutBwd;
  constexpr int SEGS = TP / 8;                          // 16-byte chunks per channel row of a tile
  constexpr int NLD = CH * TP / 8 / NT;
  constexpr int NPB = CH == 128 ? TP / 16 : TP / 32;   // pair blocks of a wave in the dx product
  constexpr int KC = NPB < 4 ? NPB : 4;                 // pair blocks per chunk of the dx phase
  constexpr int NH = 128 / CH;                          // waves sharing one channel block
  __shared__ __align__(16) uint16_t sX[CH * CP];        // x
  __shared__ __align__(16) uint16_t sXL[CH * CP];       // LN(x), then (last phase) dx
  __shared__ __align__(16) uint16_t sDP[TP * C];        // dp [pair][feature]
  __shared__ __align__(16) uint16_t sWT[CH * C];        // w_o^T
  __shared__ __align__(16) float sRed[8][TP][2];
  __shared__ __align__(16) float sSt[TP][2];
  __shared__ float sGam[CH], sBet[CH];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
  const int t = threadIdx.x;
  const int N = a.s.N, nn = N * N;
  const int total = a.s.B * nn;
  const int ntiles = (total + TP - 1) / TP;
  const uint32_t xbytes = (uint32_t)total * CH * 2, pbytes = (uint32_t)total * C * 2;
  const auto xr = make_rsrc(a.x, xbytes);
  const auto dr = make_rsrc(a.dout, pbytes), gr = make_rsrc(a.g, pbytes);
  for (int i = t; i < CH; i += NT) { sGam[i] = a.gamma_o[i]; sBet[i] = a.beta_o[i]; }
  u32x4 wo[CH / 32];
#pragma unroll
  for (int s = 0; s < CH / 32; ++s) wo[s] = ld_global<u32x4>(a.w_o + (16 * w + c) * CH + 32 * s + 8 * g);
  // w_o^T in LDS ([channel][output feature], swizzled rows), the A operand of dxln = dp w_o:
  // row = channel chb*16 + c, slots = output features 32s + 8g + j
  const int chb = CH == 128 ? w : (w & 3), pb0 = CH == 128 ? 0 : (w >> 2) * NPB;
  for (int i = t; i < CH * C / 8; i += NT) {
    const int ch = i >> 4, j = i & 15;
    uint16_t e[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) e[u] = a.w_o[(8 * j + u) * CH + ch];
    u32x4 v;
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = (uint32_t)e[2 * u] | ((uint32_t)e[2 * u + 1] << 16);
    st_lds16(sWT, toff(ch, j), v);
  }
  f32x4 accw[CH / 16];
#pragma unroll
  for (int k = 0; k < CH / 16; ++k) accw[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  float gm[4], dgam[4], dbet[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { gm[i] = a.gamma_o[chb * 16 + 4 * g + i]; dgam[i] = 0.f; dbet[i] = 0.f; }
  const int pp = t & (TP - 1), qq = t / TP;

  const auto sr = make_rsrc(a.stats_o, (uint32_t)total * 8);
  u32x4 xv[NLD];
  f32x2 stv;                // statistics of this thread's pair pp
  // this lane's incoming gradient and gate logits (4 features of one pair per block)
  u32x2 dln[TP / 16], gln[TP / 16];
  auto load = [&](int tile) {
    const TileRows tr = tile_rows(tile, TP, N, total);
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      const int q = t + NT * k, ch = q / SEGS, seg = q % SEGS;
      xv[k] = buf_ld16(xr, tr.r0 + 8 * seg < total ? (uint32_t)cm_off_t(tr, 8 * seg, ch, nn, CH) * 2 : xbytes);
    }
    const int rp = tile * TP + pp;
    stv = __builtin_bit_cast(f32x2, buf_ld8(sr, rp < total ? (uint32_t)rp * 8 : (uint32_t)total * 8));
#pragma unroll
    for (int pb = 0; pb < TP / 16; ++pb) {
      const int r = tile * TP + 16 * pb + c;
      const uint32_t o = r < total ? (uint32_t)(r * C + 16 * w + 4 * g) * 2 : pbytes;
      dln[pb] = buf_ld8(dr, o);
      gln[pb] = buf_ld8(gr, o);
    }
  };
  // everything a tile reads from memory is requested one tile ahead
  if ((int)blockIdx.x < ntiles) load(blockIdx.x);
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    lds_barrier();
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      const int q = t + NT * k;
      st_lds16(sX, coff(q / SEGS, 8 * (q % SEGS)), xv[k]);
    }
    const f32x2 s = stv;
    u32x2 dlv[TP / 16], glv[TP / 16];
#pragma unroll
    for (int pb = 0; pb < TP / 16; ++pb) { dlv[pb] = dln[pb]; glv[pb] = gln[pb]; }
    const int nt = tile + gridDim.x;
    if (nt < ntiles) load(nt);
    {
      if (qq == 0) { sSt[pp][0] = s[0]; sSt[pp][1] = s[1]; }
      lds_barrier();
      // LN(x) 8 pairs of one channel at a time (the chunks this thread staged)
#pragma unroll
      for (int k = 0; k < NLD; ++k) {
        const int q = t + NT * k, ch = q / SEGS, seg = q % SEGS;
        float xf[8], y[8];
        unpack8(ld_lds16(sX, coff(ch, 8 * seg)), xf);
        const float gmv = sGam[ch], btv = sBet[ch];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int pq = 8 * seg + e;
          y[e] = ln_out(ln_xhat(xf[e], sSt[pq][0], sSt[pq][1]), gmv, btv);
        }
        st_lds16(sXL, coff(ch, 8 * seg), pack8(y));
      }
    }
    lds_barrier();
    // p, dp, d gate
#pragma unroll 1
    for (int pb = 0; pb < TP / 16; ++pb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < CH / 32; ++s) acc = mfma_k32(wo[s], tr8_pad(sXL, 32 * s + 8 * g, 16 * pb, lane), acc);
      const int rl = 16 * pb + c, r = tile * TP + rl;
      const size_t o = (size_t)(r < total ? r : 0) * C + 16 * w + 4 * g;
      const u32x2 dl = dlv[pb], gl = glv[pb];
      const float df[4] = {bf_lo(dl[0]), bf_hi(dl[0]), bf_lo(dl[1]), bf_hi(dl[1])};
      const float gf[4] = {bf_lo(gl[0]), bf_hi(gl[0]), bf_lo(gl[1]), bf_hi(gl[1])};
      float dp[4], dg[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float sg = sigm(gf[i]);
        dp[i] = df[i] * sg;
        dg[i] = df[i] * acc[i] * (sg * (1.f - sg));
      }
      *reinterpret_cast<u32x2*>(sDP + toff(rl, (16 * w + 4 * g) >> 3) + (4 * g & 4)) =
          u32x2{pack_bf16(dp[0], dp[1]), pack_bf16(dp[2], dp[3])};
      if (r < total)
        *reinterpret_cast<u32x2*>(a.dg + o) = u32x2{pack_bf16(dg[0], dg[1]), pack_bf16(dg[2], dg[3])};
    }
    lds_barrier();
    // dxln = dp w_o, LayerNorm backward partial sums
    // (x-hat is recomputed from the x tile where needed rather than kept in registers)
    auto xhat4 = [&](int rl, float* xh) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xh[i] = ln_xhat(bf_to_f(sX[coff(chb * 16 + 4 * g + i, rl)]), sSt[rl][0], sSt[rl][1]);
    };
    // d w_o += dp^T LN(x): contraction over the tile's pairs (before any dx overwrites LN(x))
#pragma unroll
    for (int ks = 0; ks < TP / 32; ++ks) {
      const u32x4 A = tr8_swz(sDP, 32 * ks + 8 * g, 16 * w, lane);
#pragma unroll
      for (int cb = 0; cb < CH / 16; ++cb)
        accw[cb] = mfma_k32(A, ld_lds16(sXL, coff(16 * cb + c, 32 * ks + 8 * g)), accw[cb]);
    }
    // the wave's pair blocks in chunks of 4 (fewer live accumulators): products and partial sums,
    // barrier, then dx into the LN(x) tile
#pragma unroll
    for (int h = 0; h < NPB / KC; ++h) {
      f32x4 acc2[KC];
      float xhk[KC][4];
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        const int rl = 16 * (pb0 + KC * h + k) + c;
        f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
          s4 = mfma_k32(ld_lds16(sWT, toff(chb * 16 + c, 4 * s + g)), ld_lds16(sDP, toff(rl, 4 * s + g)), s4);
        acc2[k] = s4;
        float* xh = xhk[k];
        xhat4(rl, xh);
        float p1 = 0.f, p2 = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float dx = gm[i] * s4[i];
          p1 += dx;
          p2 += dx * xh[i];
          dgam[i] += s4[i] * xh[i];
          dbet[i] += s4[i];
        }
        p1 = wave_sum_groups(p1);
        p2 = wave_sum_groups(p2);
        if (g == 0) { sRed[w][rl][0] = p1; sRed[w][rl][1] = p2; }
      }
      lds_barrier();
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        const int rl = 16 * (pb0 + KC * h + k) + c;
        const int w0 = CH == 128 ? 0 : 4 * (w >> 2);
        float m1 = 0.f, m2 = 0.f;
#pragma unroll
        for (int v = 0; v < CH / 16; ++v) { m1 += sRed[w0 + v][rl][0]; m2 += sRed[w0 + v][rl][1]; }
        m1 *= 1.f / CH;
        m2 *= 1.f / CH;
        const float* xh = xhk[k];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ch = chb * 16 + 4 * g + i;
          sXL[coff(ch, rl)] = f_to_bf(sSt[rl][1] * (gm[i] * acc2[k][i] - m1 - xh[i] * m2));
        }
      }
    }
    lds_barrier();
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      const int q = t + NT * k, ch = q / SEGS, seg = q % SEGS;
      const TileRows tr = tile_rows(tile, TP, N, total);
      if (tr.r0 + 8 * seg < total)
        *reinterpret_cast<u32x4*>(a.dx + cm_off_t(tr, 8 * seg, ch, nn, CH)) = ld_lds16(sXL, coff(ch, 8 * seg));
    }
  }
  // partials: d w_o [C][CH]; d gamma_o / d beta_o per (workgroup, wave half)
  float* dst = a.wo_partial + (size_t)blockIdx.x * C * CH;
#pragma unroll
  for (int cb = 0; cb < CH / 16; ++cb)
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[(16 * w + 4 * g + i) * CH + 16 * cb + c] = accw[cb][i];
  float* lp = a.lno_partial + ((size_t)blockIdx.x * NH + (CH == 128 ? 0 : (w >> 2))) * 2 * CH;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float sg = sum16(dgam[i]), sb = sum16(dbet[i]);
    if (c == 0) { lp[chb * 16 + 4 * g + i] = sg; lp[CH + chb * 16 + 4 * g + i] = sb; }
  }
}

// ----------------------------------------------------------------------------------------------
// Input step, backward part 2: dZln = [dproj | d gate] w_in (K = 4c + 128), LayerNorm backward.
// Tile = 32 pairs, staged as 128-column segments (the last one from the gate-logit gradient).
template <int CH>
__global__ __launch_bounds__(NT) void tm_in_dz_kernel(TmInGradArgs a) {
  constexpr int TP = kTmTileDz;
  constexpr int NS = (4 * CH + C) / 128;
  constexpr int KS = 4 * NS;
  __shared__ __align__(16) uint16_t sP[NS][TP * 128];
  __shared__ __align__(16) float sRed[8][TP][2];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
  const int t = threadIdx.x;
  const int N = a.s.N, inc = a.s.incoming;
  const int total = a.s.B * N * N;
  const int ntiles = (total + TP - 1) / TP;
  const uint32_t zbytes = (uint32_t)total * C * 2, pbytes = (uint32_t)total * 4 * CH * 2;
  const auto zr = make_rsrc(a.z, zbytes), gr = make_rsrc(a.dg, zbytes), pr = make_rsrc(a.dproj, pbytes);
  const auto sr = make_rsrc(a.stats, (uint32_t)total * 8);
  // w_in^T: row = pair feature 16w + c, slots = projected features 32s + 8g + j
  u32x4 wt[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    uint16_t e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = a.w_in[(32 * s + 8 * g + j) * C + 16 * w + c];
#pragma unroll
    for (int j = 0; j < 4; ++j) wt[s][j] = (uint32_t)e[2 * j] | ((uint32_t)e[2 * j + 1] << 16);
  }
  const int c0 = 16 * w + 4 * g;
  float gm[4], dgam[4], dbet[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { gm[i] = a.gamma[c0 + i]; dgam[i] = 0.f; dbet[i] = 0.f; }

  // loader: one chunk per segment per thread (pair t >> 4, chunk t & 15).  Two register
  // sets: the loads of a tile are issued two tiles ahead (set K serves every other tile).
  const int lp = t >> 4, lj = t & 15;
  u32x4 pv[2][NS];
  u32x2 zq[2][TP / 16];
  f32x2 st[2][TP / 16];
  auto load = [&](int tile, auto k_c) {
    constexpr int K = decltype(k_c)::value;
    const TileRows tr = tile_rows(tile, TP, N, total);
    const int r = tr.r0 + lp;
    const bool ok = tile_ok(tr, lp, total);
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
      pv[K][s] = buf_ld16(pr, ok ? (uint32_t)((size_t)r * 4 * CH + 128 * s + 8 * lj) * 2 : pbytes);
    pv[K][NS - 1] = buf_ld16(gr, ok ? (uint32_t)(zrow_t(tr, lp, N, inc) + 8 * lj) * 2 : zbytes);
#pragma unroll
    for (int pb = 0; pb < TP / 16; ++pb) {
      const int l = 16 * pb + c, rr = tr.r0 + l;
      const bool ok2 = tile_ok(tr, l, total);
      zq[K][pb] = buf_ld8(zr, ok2 ? (uint32_t)(zrow_t(tr, l, N, inc) + c0) * 2 : zbytes);
      st[K][pb] = __builtin_bit_cast(f32x2, buf_ld8(sr, ok2 ? (uint32_t)rr * 8 : (uint32_t)total * 8));
    }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  const int gs = gridDim.x;
  if ((int)blockIdx.x < ntiles) load(blockIdx.x, S0{});
  if ((int)blockIdx.x + gs < ntiles) load(blockIdx.x + gs, S1{});
  auto body = [&](int tile, auto k_c) {
    constexpr int K = decltype(k_c)::value;
    const TileRows trs = tile_rows(tile, TP, N, total);
    lds_barrier();
#pragma unroll
    for (int s = 0; s < NS; ++s) st_lds16(sP[s], toff(lp, lj), pv[K][s]);
    u32x2 zc[TP / 16];
    f32x2 sc[TP / 16];
#pragma unroll
    for (int pb = 0; pb < TP / 16; ++pb) { zc[pb] = zq[K][pb]; sc[pb] = st[K][pb]; }
    const int nt = tile + 2 * gs;
    if (nt < ntiles) load(nt, k_c);
    lds_barrier();
    f32x4 acc[TP / 16];
    float xh[TP / 16][4];
#pragma unroll
    for (int pb = 0; pb < TP / 16; ++pb) {
      const int rl = 16 * pb + c;
      f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) s4 = mfma_k32(wt[s], ld_lds16(sP[s >> 2], toff(rl, 4 * (s & 3) + g)), s4);
      acc[pb] = s4;
      const float zf[4] = {bf_lo(zc[pb][0]), bf_hi(zc[pb][0]), bf_lo(zc[pb][1]), bf_hi(zc[pb][1])};
      float p1 = 0.f, p2 = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xh[pb][i] = ln_xhat(zf[i], sc[pb][0], sc[pb][1]);
        const float dx = gm[i] * s4[i];
        p1 += dx;
        p2 += dx * xh[pb][i];
        dgam[i] += s4[i] * xh[pb][i];
        dbet[i] += s4[i];
      }
      p1 = wave_sum_groups(p1);
      p2 = wave_sum_groups(p2);
      if (g == 0) { sRed[w][rl][0] = p1; sRed[w][rl][1] = p2; }
    }
    lds_barrier();
#pragma unroll
    for (int pb = 0; pb < TP / 16; ++pb) {
      const int rl = 16 * pb + c;
      float m1 = 0.f, m2 = 0.f;
#pragma unroll
      for (int v = 0; v < 8; ++v) { m1 += sRed[v][rl][0]; m2 += sRed[v][rl][1]; }
      m1 *= 1.f / C;
      m2 *= 1.f / C;
      float dz[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) dz[i] = sc[pb][1] * (gm[i] * acc[pb][i] - m1 - xh[pb][i] * m2);
      if (tile_ok(trs, rl, total))
        *reinterpret_cast<u32x2*>(a.dz + zrow_t(trs, rl, N, inc) + c0) =
            u32x2{pack_bf16(dz[0], dz[1]), pack_bf16(dz[2], dz[3])};
    }
  };
  for (int tile = blockIdx.x; tile < ntiles; tile += 2 * gs) {
    body(tile, S0{});
    if (tile + gs < ntiles) body(tile + gs, S1{});
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float sg = sum16(dgam[i]), sb = sum16(dbet[i]);
    if (c == 0) {
      a.ln_partial[(size_t)blockIdx.x * 2 * C + c0 + i] = sg;
      a.ln_partial[(size_t)blockIdx.x * 2 * C + C + c0 + i] = sb;
    }
  }
}

// Input step, backward part 3: d w_in = [dproj | d gate]^T Zln.  Workgroup (group, split) takes
// rows 128 split .. +127 of d w_in over the group's tiles; wave w owns rows 16w..16w+15 of that
// slice x all 128 pair features.  Partial layout [groups][4c + 128][128].
template <int CH>
__global__ __launch_bounds__(NT) void tm_in_dw_kernel(TmInGradArgs a) {
  constexpr int TP = kTmTileDw;
  constexpr int NSPLIT = (4 * CH + C) / 128;
  __shared__ __align__(16) uint16_t sP[TP * 128];
  __shared__ __align__(16) uint16_t sZ[TP * C];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
  const int t = threadIdx.x;
  const int N = a.s.N, inc = a.s.incoming;
  const int total = a.s.B * N * N;
  const int ntiles = (total + TP - 1) / TP;
  const int cap = 8 * (kTmDwMaxWG / (8 * NSPLIT));
  const int groups = ntiles < cap ? ntiles : cap;
  const int bx = blockIdx.x, kx = bx >> 3;
  const int split = kx % NSPLIT, grp = (kx / NSPLIT) * 8 + (bx & 7);
  if (grp >= groups) return;
  const uint32_t zbytes = (uint32_t)total * C * 2, pbytes = (uint32_t)total * 4 * CH * 2;
  const auto zr = make_rsrc(a.z, zbytes), sr = make_rsrc(a.stats, (uint32_t)total * 8);
  const bool from_gate = split == NSPLIT - 1;
  const auto pr = from_gate ? make_rsrc(a.dg, zbytes) : make_rsrc(a.dproj, pbytes);

  const int zj = t & 15;
  float gmv[8], btv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) { gmv[i] = a.gamma[8 * zj + i]; btv[i] = a.beta[8 * zj + i]; }
  u32x4 pv[2], zv[2];
  f32x2 st[2];
  auto load = [&](int tile) {
    const TileRows tr = tile_rows(tile, TP, N, total);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int pl = (t >> 4) + 32 * i, r = tr.r0 + pl;
      const bool ok = tile_ok(tr, pl, total);
      const int zo = ok ? zrow_t(tr, pl, N, inc) : 0;
      const uint32_t poff = from_gate ? (uint32_t)(zo + 8 * zj) * 2
                                      : (uint32_t)((size_t)r * 4 * CH + 128 * split + 8 * zj) * 2;
      pv[i] = buf_ld16(pr, ok ? poff : (from_gate ? zbytes : pbytes));
      zv[i] = buf_ld16(zr, ok ? (uint32_t)zo * 2 + 16 * zj : zbytes);
      st[i] = __builtin_bit_cast(f32x2, buf_ld8(sr, ok ? (uint32_t)r * 8 : (uint32_t)total * 8));
    }
  };
  f32x4 acc[8];
#pragma unroll
  for (int cb = 0; cb < 8; ++cb) acc[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  load(grp);
  for (int tile = grp; tile < ntiles; tile += groups) {
    lds_barrier();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int pl = (t >> 4) + 32 * i, r = tile * TP + pl;
      st_lds16(sP, toff(pl, zj), pv[i]);
      float x[8], y[8];
      unpack8(zv[i], x);
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = r < total ? ln_out(ln_xhat(x[e], st[i][0], st[i][1]), gmv[e], btv[e]) : 0.f;
      st_lds16(sZ, toff(pl, zj), pack8(y));
    }
    const int nt = tile + groups;
    if (nt < ntiles) load(nt);
    lds_barrier();
#pragma unroll
    for (int ks = 0; ks < TP / 32; ++ks) {
      const int row0 = 32 * ks + 8 * g;
      const u32x4 A = tr8_swz(sP, row0, 16 * w, lane);
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) acc[cb] = mfma_k32(A, tr8_swz(sZ, row0, 16 * cb, lane), acc[cb]);
    }
  }
  float* dst = a.w_partial + (size_t)grp * (4 * CH + C) * C;
#pragma unroll
  for (int cb = 0; cb < 8; ++cb)
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[(128 * split + 16 * w + 4 * g + i) * C + 16 * cb + c] = acc[cb][i];
}

template <typename Args, typename K64, typename K128>
hipError_t launch_pairs(const Args& a, int tile, K64 k64, K128 k128, hipStream_t st, int cap = kTmMaxWG) {
  const int64_t pairs = (int64_t)a.s.B * a.s.N * a.s.N;
  const int grid = (int)tm_grid(pairs, tile, cap);
  if (grid == 0) return hipSuccess;
  if (a.s.c == 128) hipLaunchKernelGGL(k128, dim3(grid), dim3(NT), 0, st, a);
  else hipLaunchKernelGGL(k64, dim3(grid), dim3(NT), 0, st, a);
  return hipGetLastError();
}

template <bool TA, bool TB, int MT>
hipError_t launch_gemm_t(const TmGemmArgs& a, hipStream_t st) {
  const int ntm = (a.N + MT - 1) / MT, nt = ntm;
  const int grid = (a.batch + 7) / 8 * 8 * ntm * nt;
  hipLaunchKernelGGL((tm_gemm_kernel<TA, TB, MT>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}
template <bool TA, bool TB>
hipError_t launch_gemm(const TmGemmArgs& a, hipStream_t st) {
  if (a.batch == 0 || a.N == 0) return hipSuccess;
  if (a.N % 192 == 0) return launch_gemm_t<TA, TB, 192>(a, st);
  return launch_gemm_t<TA, TB, 128>(a, st);
}

}  // namespace

hipError_t launch_tm_in_fwd(const TmInArgs& a, hipStream_t st) {
  return launch_pairs(a, kTmTileIn, tm_in_fwd_kernel<64>, tm_in_fwd_kernel<128>, st);
}
hipError_t launch_tm_in_bwd(const TmInArgs& a, hipStream_t st) {
  return launch_pairs(a, kTmTileIn, tm_in_bwd_kernel<64>, tm_in_bwd_kernel<128>, st);
}
hipError_t launch_tm_out_fwd(const TmOutArgs& a, hipStream_t st) {
  return launch_pairs(a, kTmTileOut, tm_out_fwd_kernel<64>, tm_out_fwd_kernel<128>, st,
                      a.s.c == 64 ? kTmOutMaxWG : kTmMaxWG);
}
hipError_t launch_tm_out_bwd(const TmOutArgs& a, hipStream_t st) {
  return launch_pairs(a, kTmTileOutBwd, tm_out_bwd_kernel<64>, tm_out_bwd_kernel<128>, st);
}
hipError_t launch_tm_in_dz(const TmInGradArgs& a, hipStream_t st) {
  return launch_pairs(a, kTmTileDz, tm_in_dz_kernel<64>, tm_in_dz_kernel<128>, st);
}
hipError_t launch_tm_in_dw(const TmInGradArgs& a, hipStream_t st) {
  const int64_t pairs = (int64_t)a.s.B * a.s.N * a.s.N;
  const int64_t groups = tm_dw_groups(pairs, a.s.c);
  if (groups == 0) return hipSuccess;
  const int grid = (int)((groups + 7) / 8 * 8 * tm_dw_splits(a.s.c));
  if (a.s.c == 128) hipLaunchKernelGGL(tm_in_dw_kernel<128>, dim3(grid), dim3(NT), 0, st, a);
  else hipLaunchKernelGGL(tm_in_dw_kernel<64>, dim3(grid), dim3(NT), 0, st, a);
  return hipGetLastError();
}
hipError_t launch_tm_gemm_nt(const TmGemmArgs& a, hipStream_t st) { return launch_gemm<false, false>(a, st); }
hipError_t launch_tm_gemm_nn(const TmGemmArgs& a, hipStream_t st) { return launch_gemm<false, true>(a, st); }
hipError_t launch_tm_gemm_tn(const TmGemmArgs& a, hipStream_t st) { return launch_gemm<true, true>(a, st); }

}  // namespace tri
