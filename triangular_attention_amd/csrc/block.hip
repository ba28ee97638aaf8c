// Triangle-attention block around the attention core, for gfx950.
//
// "TurboPairFormer: Fast and Stable Protein Folding Model Training with an
// Optimized Triangle Attention Kernel", Table 1 and Figure 6: slice o of the
// attention is row o of the pair tensor Z; pair (o, q) gives query q, pair
// (o, k) key and value k, pair (q, k) the bias of (q, k); the output updates
// pair (o, q); a normalisation precedes the projections.  The rest of the block
// (gate, output projection) follows the common Pairformer form: LayerNorm, Q /
// K / V / gate / bias projections without additive terms, sigmoid gate on the
// attention output, output projection.  The ending node is the same block on Z
// with its two token axes swapped: only the Z / dZ / Y / dY addresses change.
//
// Kernels (all persistent: workgroup i takes tiles i, i + grid, ...; the grid
// is fixed by the problem size, so every partial buffer is deterministic):
//   ln_proj      LayerNorm (FP32 statistics) + the 4 * 128 + H projections
//   gate_out     sigmoid(gate) * O -> output projection
//   gate_out_bwd dO, d gate, and d w_o partials
//   proj_dz      dZ through the projections and the LayerNorm, d gamma / d beta partials
//   proj_dw      d w_qkvg and d w_b partials
//   reduce       fixed-order sum of partials
// Every product is a bf16 MFMA with FP32 accumulation (v_mfma_f32_16x16x32_bf16);
// operand conventions as in common.h.  LDS tiles of 128-feature rows use an XOR
// swizzle of the 16-byte chunks that keeps both the row reads of MFMA operands
// (16 rows, one chunk each) and the transposing reads (4 rows x 4 column chunks)
// free of bank conflicts.
#include "block_kernels.h"
#include "common.h"
#include "pair_common.h"

namespace tri {
namespace {

using namespace pair;

constexpr int C = kBlkC;
constexpr int F = kBlkF;
constexpr int NT = 512;      // threads per workgroup: 8 waves

// ----------------------------------------------------------------------------------------------
// LayerNorm + projections.  Tile = 128 pairs.  Wave w normalises pairs 16w..16w+15 of the tile
// (16 lanes per pair, 8 features per lane) and owns projected features 64w..64w+63 (4 blocks of
// 16; waves 2p, 2p+1 write projection p of Q, K, V, gate) plus the bias block of pair block w.
// No MFMA sits in a lane-masked branch anywhere in this file: the matrix cores ignore EXEC.
template <int H, int D>
__global__ __launch_bounds__(NT) void ln_proj_kernel(BlkLnProjArgs a) {
  constexpr int TP = kBlkTileFwd;
  static_assert(H * D == F, "H * D must be 128");
  __shared__ __align__(16) uint16_t sZ[2][TP * C];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
  const int N = a.s.N, ending = a.s.ending;
  const int total = a.s.B * N * N;
  const int ntiles = (total + TP - 1) / TP;
  const uint32_t zbytes = (uint32_t)total * C * 2;
  const auto zr = make_rsrc(a.z, zbytes);

  float gm[8], bt[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) { gm[i] = a.gamma[8 * c + i]; bt[i] = a.beta[8 * c + i]; }
  u32x4 wf[4][4], wb[4];
#pragma unroll
  for (int fb = 0; fb < 4; ++fb)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      wf[fb][s] = ld_global<u32x4>(a.w_qkvg + (64 * w + 16 * fb + c) * C + 32 * s + 8 * g);
#pragma unroll
  for (int s = 0; s < 4; ++s)
    wb[s] = c < H ? ld_global<u32x4>(a.w_b + c * C + 32 * s + 8 * g) : u32x4{0, 0, 0, 0};
  uint16_t* outp = w < 2 ? a.q : w < 4 ? a.k : w < 6 ? a.v : a.g;

  u32x4 zv[4];
  auto load_z = [&](int tile) {
    const TileRows tr = tile_rows(tile, TP, N, total);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int l = 16 * w + 4 * s + g;
      const uint32_t off = tile_ok(tr, l, total) ? (uint32_t)zrow_t(tr, l, N, ending) * 2 + 16 * c : zbytes;
      zv[s] = buf_ld16(zr, off);
    }
  };
  if ((int)blockIdx.x < ntiles) load_z(blockIdx.x);
  int it = 0;
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x, ++it) {
    uint16_t* buf = sZ[it & 1];
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
      for (int i = 0; i < 8; ++i) y[i] = ln_out(x[i] * rstd, gm[i], bt[i]);
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
      f32x4 acc[4];
#pragma unroll
      for (int fb = 0; fb < 4; ++fb) acc[fb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int fb = 0; fb < 4; ++fb) acc[fb] = mfma_k32(wf[fb][s], bf[s], acc[fb]);
      const bool ok = tile_ok(tr, rl, total);
#pragma unroll
      for (int fb = 0; fb < 4; ++fb) {
        const int hd0 = 64 * (w & 1) + 16 * fb;
        const int h = hd0 / D, d0 = hd0 % D + 4 * g;
        if (ok)
          *reinterpret_cast<u32x2*>(outp + hm_off_t<H, D>(tr, rl, N, h, d0)) =
              u32x2{pack_bf16(acc[fb][0], acc[fb][1]), pack_bf16(acc[fb][2], acc[fb][3])};
      }
    }
    // the bias block of pair block w (outside the loop: an MFMA executes whatever the EXEC mask,
    // so it must not sit in a lane-masked branch)
    {
      const int rl = 16 * w + c;
      f32x4 ab = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) ab = mfma_k32(wb[s], ld_lds16(buf, toff(rl, 4 * s + g)), ab);
      if (tile_ok(tr, rl, total)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int h = 4 * g + i;
          if (h < H) a.bias[bias_off_t<H>(tr, rl, N, h)] = f_to_bf(ab[i]);
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------------------------
// Loader of a tile of O and gate logits (head-major rows of D features): 128 pairs x 16 chunks of
// 16 bytes each; thread t takes chunks t + 512 i.  Returns the pair (tile-local) and the logical
// chunk (feature / 8) of load i.
template <int H, int D>
__device__ __forceinline__ void hm_chunk(int t, int i, int TP, int& p, int& h, int& dc) {
  constexpr int CPR = D / 8;                 // chunks per (pair, head)
  const int q = t + NT * i;
  h = q / (TP * CPR);
  const int v = q - h * TP * CPR;
  p = v / CPR;
  dc = v - p * CPR;
}

// Gate times output, rounded to bf16 once: the output-projection operand (forward and backward).
__device__ __forceinline__ u32x4 gate_mul8(u32x4 gv, u32x4 ov) {
  float gf[8], of[8], r[8];
  unpack8(gv, gf);
  unpack8(ov, of);
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = sigm(gf[i]) * of[i];
  return pack8(r);
}

// Gate + output projection.  Tile = 128 pairs; wave w owns output features 16w..16w+15.
template <int H, int D>
__global__ __launch_bounds__(NT) void gate_out_kernel(BlkGateOutArgs a) {
  constexpr int TP = kBlkTileFwd;
  static_assert(H * D == F, "H * D must be 128");
  __shared__ __align__(16) uint16_t sGO[2][TP * F];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
  const int t = threadIdx.x;
  const int N = a.s.N, ending = a.s.ending;
  const int total = a.s.B * N * N;
  const int ntiles = (total + TP - 1) / TP;
  const uint32_t hbytes = (uint32_t)total * F * 2;
  const auto orr = make_rsrc(a.o, hbytes), grr = make_rsrc(a.g, hbytes);
  u32x4 wo[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) wo[s] = ld_global<u32x4>(a.w_o + (16 * w + c) * F + 32 * s + 8 * g);

  u32x4 ov[4], gv[4];
  auto load = [&](int tile) {
    const TileRows tr = tile_rows(tile, TP, N, total);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int p, h, dc;
      hm_chunk<H, D>(t, i, TP, p, h, dc);
      const uint32_t off = tile_ok(tr, p, total) ? (uint32_t)hm_off_t<H, D>(tr, p, N, h, 8 * dc) * 2 : hbytes;
      ov[i] = buf_ld16(orr, off);
      gv[i] = buf_ld16(grr, off);
    }
  };
  if ((int)blockIdx.x < ntiles) load(blockIdx.x);
  int it = 0;
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x, ++it) {
    uint16_t* buf = sGO[it & 1];
    const TileRows tr = tile_rows(tile, TP, N, total);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int p, h, dc;
      hm_chunk<H, D>(t, i, TP, p, h, dc);
      st_lds16(buf, toff(p, h * (D / 8) + dc), gate_mul8(gv[i], ov[i]));
    }
    const int nt = tile + gridDim.x;
    if (nt < ntiles) load(nt);
    lds_barrier();
#pragma unroll 2
    for (int pb = 0; pb < TP / 16; ++pb) {
      const int rl = 16 * pb + c;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) acc = mfma_k32(wo[s], ld_lds16(buf, toff(rl, 4 * s + g)), acc);
      if (tile_ok(tr, rl, total))
        *reinterpret_cast<u32x2*>(a.y + zrow_t(tr, rl, N, ending) + 16 * w + 4 * g) =
            u32x2{pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3])};
    }
  }
}

// Backward of gate + output projection.  Tile = 128 pairs.
//   dGO = dY w_o (wave w: gate/output features 16w..16w+15), dO = dGO * s, d gate = dGO * O * s(1-s)
//   d w_o += dY^T GO (wave w: output features 16w..16w+15 x all 128 GO features)
template <int H, int D>
__global__ __launch_bounds__(NT) void gate_out_bwd_kernel(BlkGateOutArgs a) {
  constexpr int TP = kBlkTileOutBwd;
  static_assert(H * D == F, "H * D must be 128");
  __shared__ __align__(16) uint16_t sDY[TP * C];
  __shared__ __align__(16) uint16_t sGO[TP * F];
  __shared__ __align__(16) uint16_t sO[TP * F];
  __shared__ __align__(16) uint16_t sG[TP * F];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
  const int t = threadIdx.x;
  const int N = a.s.N, ending = a.s.ending;
  const int total = a.s.B * N * N;
  const int ntiles = (total + TP - 1) / TP;
  const uint32_t hbytes = (uint32_t)total * F * 2, ybytes = (uint32_t)total * C * 2;
  const auto orr = make_rsrc(a.o, hbytes), grr = make_rsrc(a.g, hbytes), yr = make_rsrc(a.dy, ybytes);

  // w_o^T as the A operand: row = GO feature 16w + c, slots = output features 32s + 8g + 0..7
  u32x4 wt[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    uint16_t e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = a.w_o[(32 * s + 8 * g + j) * F + 16 * w + c];
#pragma unroll
    for (int j = 0; j < 4; ++j) wt[s][j] = (uint32_t)e[2 * j] | ((uint32_t)e[2 * j + 1] << 16);
  }
  f32x4 accw[8];
#pragma unroll
  for (int fb = 0; fb < 8; ++fb) accw[fb] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 yv[4], ov[4], gv[4];
  auto load = [&](int tile) {
    const TileRows tr = tile_rows(tile, TP, N, total);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = t + NT * i, p = q >> 4, j = q & 15;
      yv[i] = buf_ld16(yr, tile_ok(tr, p, total) ? (uint32_t)zrow_t(tr, p, N, ending) * 2 + 16 * j : ybytes);
      int ph, h, dc;
      hm_chunk<H, D>(t, i, TP, ph, h, dc);
      const uint32_t off = tile_ok(tr, ph, total) ? (uint32_t)hm_off_t<H, D>(tr, ph, N, h, 8 * dc) * 2 : hbytes;
      ov[i] = buf_ld16(orr, off);
      gv[i] = buf_ld16(grr, off);
    }
  };
  auto stash = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = t + NT * i, p = q >> 4, j = q & 15;
      st_lds16(sDY, toff(p, j), yv[i]);
      int ph, h, dc;
      hm_chunk<H, D>(t, i, TP, ph, h, dc);
      const int o = toff(ph, h * (D / 8) + dc);
      st_lds16(sO, o, ov[i]);
      st_lds16(sG, o, gv[i]);
      st_lds16(sGO, o, gate_mul8(gv[i], ov[i]));
    }
  };
  if ((int)blockIdx.x < ntiles) load(blockIdx.x);
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const TileRows tr = tile_rows(tile, TP, N, total);
    lds_barrier();            // the previous tile's reads are done
    stash();
    const int nt = tile + gridDim.x;
    if (nt < ntiles) load(nt);
    lds_barrier();
    // dGO, dO, d gate
    const int f0 = 16 * w + 4 * g;                 // this lane's 4 GO features
    const int h = f0 / D, d0 = f0 % D;
#pragma unroll 2
    for (int pb = 0; pb < TP / 16; ++pb) {
      const int rl = 16 * pb + c;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) acc = mfma_k32(wt[s], ld_lds16(sDY, toff(rl, 4 * s + g)), acc);
      const int eo = toff(rl, f0 >> 3) + (f0 & 4);
      const u32x2 o2 = *reinterpret_cast<const u32x2*>(sO + eo);
      const u32x2 g2 = *reinterpret_cast<const u32x2*>(sG + eo);
      const float of[4] = {bf_lo(o2[0]), bf_hi(o2[0]), bf_lo(o2[1]), bf_hi(o2[1])};
      const float gf[4] = {bf_lo(g2[0]), bf_hi(g2[0]), bf_lo(g2[1]), bf_hi(g2[1])};
      float dov[4], dgv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float sg = sigm(gf[i]);
        dov[i] = acc[i] * sg;
        dgv[i] = acc[i] * of[i] * (sg * (1.f - sg));
      }
      if (tile_ok(tr, rl, total)) {
        const int off = hm_off_t<H, D>(tr, rl, N, h, d0);
        *reinterpret_cast<u32x2*>(a.d_o + off) = u32x2{pack_bf16(dov[0], dov[1]), pack_bf16(dov[2], dov[3])};
        *reinterpret_cast<u32x2*>(a.d_g + off) = u32x2{pack_bf16(dgv[0], dgv[1]), pack_bf16(dgv[2], dgv[3])};
      }
    }
    // d w_o: contraction over the tile's pairs (rows beyond the problem are zero in dY)
#pragma unroll
    for (int ks = 0; ks < TP / 32; ++ks) {
      const int row0 = 32 * ks + 8 * g;
      const u32x4 A = tr8_swz(sDY, row0, 16 * w, lane);
#pragma unroll
      for (int fb = 0; fb < 8; ++fb) accw[fb] = mfma_k32(A, tr8_swz(sGO, row0, 16 * fb, lane), accw[fb]);
    }
  }
  // partial [C][F]: lane holds rows 16w + 4g + i, column 16 fb + c
  float* dst = a.wo_partial + (size_t)blockIdx.x * C * F;
#pragma unroll
  for (int fb = 0; fb < 8; ++fb)
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[(16 * w + 4 * g + i) * F + 16 * fb + c] = accw[fb][i];
}

// ----------------------------------------------------------------------------------------------
// Backward of the projections.  The four head-major gradients (dQ, dK, dV, d gate) of a tile are
// staged as four swizzled [64 pairs][128] tiles (segment = projection), the bias gradient as a
// [64][16] tile (heads in columns 0..H-1, zeros after).  Loader: thread t takes chunks t + 512 i
// of the 4 x 64 x 16 chunk space (8 per thread).
template <int H, int D, int NSEG>
struct ProjTileLoader {
  static constexpr int TP = kBlkTileProjBwd;
  u32x4 v[2 * NSEG];
  uint16_t bv;
  // rs: buffer descriptors of the NSEG head-major gradients staged as segments 0..NSEG-1
  __device__ __forceinline__ void load(const BlkProjBwdArgs& a, int tile, int t, int total,
                                       const __amdgpu_buffer_rsrc_t* rs, uint32_t hbytes) {
    const int N = a.s.N;
    const TileRows tr = tile_rows(tile, TP, N, total);
#pragma unroll
    for (int i = 0; i < 2 * NSEG; ++i) {
      const int seg = i >> 1;                       // 1024 chunks per segment = 2 per thread
      int p, h, dc;
      hm_chunk<H, D>(t, i & 1, TP, p, h, dc);
      const uint32_t off = tile_ok(tr, p, total) ? (uint32_t)hm_off_t<H, D>(tr, p, N, h, 8 * dc) * 2 : hbytes;
      v[i] = buf_ld16(rs[seg], off);
    }
    bv = 0;
    if (t < TP * H) {
      const int p = t % TP, h = t / TP;
      if (tile_ok(tr, p, total)) bv = a.dbias[bias_off_t<H>(tr, p, N, h)];
    }
  }
  __device__ __forceinline__ void stash(uint16_t* sP, uint16_t* sB, int t) const {
#pragma unroll
    for (int i = 0; i < 2 * NSEG; ++i) {
      const int seg = i >> 1;
      int p, h, dc;
      hm_chunk<H, D>(t, i & 1, TP, p, h, dc);
      st_lds16(sP + seg * TP * F, toff(p, h * (D / 8) + dc), v[i]);
    }
    if (t < TP * H) sB[(t % TP) * 16 + t / TP] = bv;
  }
};

// dZ: dZln = [dQ dK dV dG] w_qkvg + dbias w_b (wave w: pair features 16w..16w+15), then the
// LayerNorm backward per pair (cross-wave sums through LDS, fixed order); d gamma / d beta partials.
template <int H, int D>
__global__ __launch_bounds__(NT) void proj_dz_kernel(BlkProjBwdArgs a) {
  constexpr int TP = kBlkTileProjBwd;
  static_assert(H * D == F && H <= 16, "H * D must be 128");
  __shared__ __align__(16) uint16_t sP[4 * TP * F];
  __shared__ __align__(16) uint16_t sB[TP * 16];
  __shared__ __align__(16) float sRed[8][TP][2];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
  const int t = threadIdx.x;
  const int N = a.s.N, ending = a.s.ending;
  const int total = a.s.B * N * N;
  const int ntiles = (total + TP - 1) / TP;
  const uint32_t hbytes = (uint32_t)total * F * 2, zbytes = (uint32_t)total * C * 2;
  const __amdgpu_buffer_rsrc_t rs[4] = {make_rsrc(a.dq, hbytes), make_rsrc(a.dk, hbytes),
                                        make_rsrc(a.dv, hbytes), make_rsrc(a.dg, hbytes)};
  const auto zr = make_rsrc(a.z, zbytes);
  const auto sr = make_rsrc(a.stats, (uint32_t)total * 8);

  // w_qkvg^T as the A operand: row = pair feature 16w + c, slots = projected features 32s + 8g + j
  u32x4 wt[16];
#pragma unroll
  for (int s = 0; s < 16; ++s) {
    uint16_t e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = a.w_qkvg[(32 * s + 8 * g + j) * C + 16 * w + c];
#pragma unroll
    for (int j = 0; j < 4; ++j) wt[s][j] = (uint32_t)e[2 * j] | ((uint32_t)e[2 * j + 1] << 16);
  }
  // w_b^T: slots (g, j) = head 8g + j (zero past H; H <= 16 heads fill lane groups 0 and 1).
  // One 16x16x32 product: its result is read by the VALU right away, which the compiler
  // schedules correctly for this form (not for the 16x16x16 form on this target).
  u32x4 wbt;
  {
    uint16_t e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = (8 * g + j < H) ? a.w_b[(8 * g + j) * C + 16 * w + c] : (uint16_t)0;
#pragma unroll
    for (int j = 0; j < 4; ++j) wbt[j] = (uint32_t)e[2 * j] | ((uint32_t)e[2 * j + 1] << 16);
  }
  const int c0 = 16 * w + 4 * g;   // this lane's 4 pair features
  float gm[4], dgam[4], dbet[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) { gm[i] = a.gamma[c0 + i]; dgam[i] = 0.f; dbet[i] = 0.f; }
  for (int i = t; i < TP * 16; i += NT) sB[i] = 0;

  ProjTileLoader<H, D, 4> ld;
  u32x2 zq[TP / 16];
  f32x2 st[TP / 16];
  auto load_own = [&](int tile) {      // this lane's Z features and statistics of its 4 pairs
    const TileRows tr = tile_rows(tile, TP, N, total);
#pragma unroll
    for (int pb = 0; pb < TP / 16; ++pb) {
      const int l = 16 * pb + c, r = tr.r0 + l;
      const bool ok = tile_ok(tr, l, total);
      zq[pb] = buf_ld8(zr, ok ? (uint32_t)(zrow_t(tr, l, N, ending) + c0) * 2 : zbytes);
      st[pb] = __builtin_bit_cast(f32x2, buf_ld8(sr, ok ? (uint32_t)r * 8 : (uint32_t)total * 8));
    }
  };
  if ((int)blockIdx.x < ntiles) { ld.load(a, blockIdx.x, t, total, rs, hbytes); load_own(blockIdx.x); }
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const TileRows tr = tile_rows(tile, TP, N, total);
    lds_barrier();
    ld.stash(sP, sB, t);
    u32x2 zc[TP / 16];
    f32x2 sc[TP / 16];
#pragma unroll
    for (int pb = 0; pb < TP / 16; ++pb) { zc[pb] = zq[pb]; sc[pb] = st[pb]; }
    const int nt = tile + gridDim.x;
    if (nt < ntiles) { ld.load(a, nt, t, total, rs, hbytes); load_own(nt); }
    lds_barrier();
    f32x4 acc[TP / 16];
    float xh[TP / 16][4];
#pragma unroll
    for (int pb = 0; pb < TP / 16; ++pb) {
      const int rl = 16 * pb + c;
      f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 16; ++s)
        s4 = mfma_k32(wt[s], ld_lds16(sP + (s >> 2) * TP * F, toff(rl, 4 * (s & 3) + g)), s4);
      const u32x4 bb = g < 2 ? ld_lds16(sB, rl * 16 + 8 * g) : u32x4{0, 0, 0, 0};
      s4 = mfma_k32(wbt, bb, s4);
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
      if (tile_ok(tr, rl, total))
        *reinterpret_cast<u32x2*>(a.dz + zrow_t(tr, rl, N, ending) + c0) =
            u32x2{pack_bf16(dz[0], dz[1]), pack_bf16(dz[2], dz[3])};
    }
  }
  // d gamma / d beta of this workgroup: sum over the 16 lanes (pairs) of each feature
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float sg = sum16(dgam[i]), sb = sum16(dbet[i]);
    if (c == 0) {
      a.ln_partial[(size_t)blockIdx.x * 2 * C + c0 + i] = sg;
      a.ln_partial[(size_t)blockIdx.x * 2 * C + C + c0 + i] = sb;
    }
  }
}

// d w_qkvg / d w_b: contraction over pairs of [dQ dK dV dG | dbias]^T and Zln (recomputed from Z
// and the statistics exactly as in the forward).  The 528 x 128 FP32 accumulators of one tile
// group do not fit one workgroup's registers, so two workgroups share each group of tiles:
// half 0 takes the Q and K rows, half 1 the V and gate rows and the bias rows.  Blocks b and b + 8
// (the same XCD, as blocks are dealt round-robin over 8 XCDs) are the two halves of one group,
// so the group's Z tiles are fetched from HBM once into that XCD's L2.  In a half, wave w owns
// projected features 32(w & 3) .. +31 of segment w / 4 x all 128 pair features; in half 1 also
// the bias rows x pair features 16w..16w+15.  Partial layout: [groups][4F + H][C].
template <int H, int D>
__global__ __launch_bounds__(NT) void proj_dw_kernel(BlkProjBwdArgs a) {
  constexpr int TP = kBlkTileProjBwd;
  static_assert(H * D == F && H <= 16, "H * D must be 128");
  __shared__ __align__(16) uint16_t sP[2 * TP * F];
  __shared__ __align__(16) uint16_t sB[TP * 16];
  __shared__ __align__(16) uint16_t sZ[TP * C];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane >> 4, c = lane & 15;
  const int t = threadIdx.x;
  const int N = a.s.N, ending = a.s.ending;
  const int total = a.s.B * N * N;
  const int ntiles = (total + TP - 1) / TP;
  const int ngroups = ntiles < kBlkMaxWG / 2 ? ntiles : kBlkMaxWG / 2;
  const int bx = blockIdx.x;
  const int half = (bx >> 3) & 1, grp = (bx >> 4) * 8 + (bx & 7);
  if (grp >= ngroups) return;
  const uint32_t hbytes = (uint32_t)total * F * 2, zbytes = (uint32_t)total * C * 2;
  const __amdgpu_buffer_rsrc_t rs[2] = {make_rsrc(half ? a.dv : a.dq, hbytes),
                                        make_rsrc(half ? a.dg : a.dk, hbytes)};
  const auto zr = make_rsrc(a.z, zbytes);
  const auto sr = make_rsrc(a.stats, (uint32_t)total * 8);
  for (int i = t; i < TP * 16; i += NT) sB[i] = 0;

  // Z loader: pair t / 16 + 32 i, chunk t % 16 (i = 0, 1)
  const int zj = t & 15;
  float gm[8], bt[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) { gm[i] = a.gamma[8 * zj + i]; bt[i] = a.beta[8 * zj + i]; }
  ProjTileLoader<H, D, 2> ld;
  u32x4 zv[2];
  f32x2 st[2];
  auto load_z = [&](int tile) {
    const TileRows tr = tile_rows(tile, TP, N, total);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int l = (t >> 4) + 32 * i, r = tr.r0 + l;
      const bool ok = tile_ok(tr, l, total);
      zv[i] = buf_ld16(zr, ok ? (uint32_t)zrow_t(tr, l, N, ending) * 2 + 16 * zj : zbytes);
      st[i] = __builtin_bit_cast(f32x2, buf_ld8(sr, ok ? (uint32_t)r * 8 : (uint32_t)total * 8));
    }
  };

  const int sl = w >> 2, nb0 = (w & 3) * 2;     // local segment, first 16-feature block
  f32x4 acc[2][8], accb;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) acc[nb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};
  accb = f32x4{0.f, 0.f, 0.f, 0.f};

  ld.load(a, grp, t, total, rs, hbytes);
  load_z(grp);
  for (int tile = grp; tile < ntiles; tile += ngroups) {
    lds_barrier();
    ld.stash(sP, sB, t);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float x[8], y[8];
      unpack8(zv[i], x);
      const int r = tile * TP + (t >> 4) + 32 * i;
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = r < total ? ln_out(ln_xhat(x[e], st[i][0], st[i][1]), gm[e], bt[e]) : 0.f;
      st_lds16(sZ, toff((t >> 4) + 32 * i, zj), pack8(y));
    }
    const int nt = tile + ngroups;
    if (nt < ntiles) { ld.load(a, nt, t, total, rs, hbytes); load_z(nt); }
    lds_barrier();
    const uint16_t* P = sP + sl * TP * F;
#pragma unroll
    for (int ks = 0; ks < TP / 32; ++ks) {
      const int row0 = 32 * ks + 8 * g;
      u32x4 A[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) A[nb] = tr8_swz(P, row0, 16 * (nb0 + nb), lane);
      const int kk = (lane & 15) >> 2, aa = lane & 3;
      const u32x4 Ab = ds_read_tr8_at(sB, (row0 + kk) * 16 + 4 * aa, (row0 + kk + 4) * 16 + 4 * aa);
#pragma unroll
      for (int cb = 0; cb < 8; ++cb) {
        const u32x4 Bz = tr8_swz(sZ, row0, 16 * cb, lane);
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[nb][cb] = mfma_k32(A[nb], Bz, acc[nb][cb]);
      }
      // bias rows x pair features 16w..16w+15, outside any lane-masked branch: an MFMA
      // executes whatever the EXEC mask (half 0 computes and discards it)
      accb = mfma_k32(Ab, tr8_swz(sZ, row0, 16 * w, lane), accb);
    }
  }
  // acc[nb][cb]: lane (g, c) holds rows (2 half + sl) * 128 + 16 (nb0 + nb) + 4g + i, column 16cb + c
  float* dst = a.w_partial + (size_t)grp * (4 * F + H) * C;
  const int row_base = (2 * half + sl) * F + 16 * nb0 + 4 * g;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb)
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(row_base + 16 * nb + i) * C + 16 * cb + c] = acc[nb][cb][i];
  if (half) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * g + i < H) dst[(4 * F + 4 * g + i) * C + 16 * w + c] = accb[i];
  }
}

// Fixed-order sum of partial buffers, out[e] = sum over i of partial[i][e], for elems % 4 == 0.
// Lane l of a wave owns elements 4 (l mod 16) .. +3 of the wave's 64-element chunk and the
// partials i = l / 16 (mod 4), added in ascending i; the four lane sums are then combined as
// (s0 + s1) + (s2 + s3).  The tree depends only on n, so every call gives the same bits.
// Loads are 16 bytes, 8 partials in flight per lane.
__global__ __launch_bounds__(256) void blk_reduce_kernel(BlkReduceArgs a) {
  constexpr int U = 8;
  const int lane = threadIdx.x & 63, j = lane >> 4;
  const int64_t e0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 64 + 4 * (lane & 15);
  if (e0 >= a.elems) return;   // the four lanes of a chunk leave together
  const float* p = a.partial + e0;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  int i = j;
  for (; i + 4 * (U - 1) < a.n; i += 4 * U) {
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + (size_t)(i + 4 * u) * a.elems));
#pragma unroll
    for (int u = 0; u < U; ++u) s += v[u];
  }
  for (; i < a.n; i += 4) s += *reinterpret_cast<const f32x4*>(p + (size_t)i * a.elems);
#pragma unroll
  for (int m = 16; m <= 32; m <<= 1) {
    f32x4 o;
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = __shfl_xor(s[k], m);
    s = s + o;
  }
  if (j == 0) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t e = e0 + k;
      if (e < a.split) a.out0[e] = s[k];
      else a.out1[e - a.split] = s[k];
    }
  }
}

}  // namespace

#define TRI_BLK_LAUNCH(KERNEL, ARGS, TILE, CAP)                                              \
  {                                                                                            \
    const int64_t pairs = (int64_t)(ARGS).s.B * (ARGS).s.N * (ARGS).s.N;                       \
    const int grid = (int)blk_grid(pairs, TILE, CAP);                                          \
    if (grid == 0) return hipSuccess;                                                          \
    if ((ARGS).s.D == 32)                                                                      \
      hipLaunchKernelGGL((KERNEL<4, 32>), dim3(grid), dim3(NT), 0, st, ARGS);                  \
    else                                                                                       \
      hipLaunchKernelGGL((KERNEL<8, 16>), dim3(grid), dim3(NT), 0, st, ARGS);                  \
    return hipGetLastError();                                                                  \
  }

hipError_t launch_blk_ln_proj(const BlkLnProjArgs& a, hipStream_t st)
    TRI_BLK_LAUNCH(ln_proj_kernel, a, kBlkTileFwd, kBlkMaxWG)
hipError_t launch_blk_gate_out(const BlkGateOutArgs& a, hipStream_t st)
    TRI_BLK_LAUNCH(gate_out_kernel, a, kBlkTileFwd, 2 * kBlkMaxWG)   // 88 VGPRs, 64 KB LDS: two per CU
hipError_t launch_blk_gate_out_bwd(const BlkGateOutArgs& a, hipStream_t st)
    TRI_BLK_LAUNCH(gate_out_bwd_kernel, a, kBlkTileOutBwd, kBlkMaxWG)
hipError_t launch_blk_proj_dz(const BlkProjBwdArgs& a, hipStream_t st)
    TRI_BLK_LAUNCH(proj_dz_kernel, a, kBlkTileProjBwd, kBlkMaxWG)
hipError_t launch_blk_proj_dw(const BlkProjBwdArgs& a, hipStream_t st) {
  const int64_t pairs = (int64_t)a.s.B * a.s.N * a.s.N;
  const int64_t groups = blk_dw_groups(pairs);
  if (groups == 0) return hipSuccess;
  const int grid = (int)((2 * groups + 15) / 16 * 16);
  if (a.s.D == 32) hipLaunchKernelGGL((proj_dw_kernel<4, 32>), dim3(grid), dim3(NT), 0, st, a);
  else hipLaunchKernelGGL((proj_dw_kernel<8, 16>), dim3(grid), dim3(NT), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_blk_reduce(const BlkReduceArgs& a, hipStream_t st) {
  if (a.elems == 0) return hipSuccess;
  if (a.elems % 4 != 0) return hipErrorInvalidValue;   // every weight shape here is a multiple of 4
  const int64_t blocks = (a.elems + 255) / 256;   // one lane per element (4 lanes per 4 elements)
  hipLaunchKernelGGL(blk_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace tri
