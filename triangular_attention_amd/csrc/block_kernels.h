// Argument blocks and launchers of the triangle-attention block kernels (internal).
//
// The block around the attention core: LayerNorm of the pair features and the
// projections to Q, K, V, the gate and the pair bias; the gated output
// projection; and their backward with fixed-order weight-gradient partials.
// C_z = 128 pair features and H * D = 128 projected features.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tri {

constexpr int kBlkC = 128;          // pair features C_z
constexpr int kBlkF = 128;          // projected features H * D
constexpr int kBlkMaxWG = 256;      // persistent grid: at most one workgroup per compute unit
constexpr int kBlkTileFwd = 128;    // pairs per tile: LayerNorm + projections, gate + output
constexpr int kBlkTileOutBwd = 128; // pairs per tile: backward of gate + output projection
constexpr int kBlkTileProjBwd = 64; // pairs per tile: backward of the projections

// Workgroups (= partial buffers) of a persistent launch over `pairs` pairs in tiles of `tile`.
inline int64_t blk_grid(int64_t pairs, int tile, int cap = kBlkMaxWG) {
  const int64_t t = (pairs + tile - 1) / tile;
  return t < cap ? t : cap;
}

// Tile groups (= partial buffers) of the weight-gradient kernel: two workgroups per group.
inline int64_t blk_dw_groups(int64_t pairs) {
  const int64_t t = (pairs + kBlkTileProjBwd - 1) / kBlkTileProjBwd;
  return t < kBlkMaxWG / 2 ? t : kBlkMaxWG / 2;
}

struct BlkShape {
  int B, N, H, D;
  int ending;        // 0: pair (x, y) of the block is Z[b, x, y]; 1: it is Z[b, y, x]
  float eps;
};

struct BlkLnProjArgs {
  BlkShape s;
  const uint16_t* z;        // [B, N, N, C] bf16
  const float* gamma;       // [C]
  const float* beta;        // [C]
  const uint16_t* w_qkvg;   // [4F, C] bf16 (rows: Q, K, V, gate features)
  const uint16_t* w_b;      // [H, C] bf16
  uint16_t* q; uint16_t* k; uint16_t* v; uint16_t* g;   // [B, N, H, N, D] bf16
  uint16_t* bias;           // [B, H, N, N] bf16
  float* stats;             // [B * N * N, 2]: mean, 1 / sqrt(var + eps) per pair
};

struct BlkGateOutArgs {
  BlkShape s;
  const uint16_t* o;        // [B, N, H, N, D] bf16 attention output
  const uint16_t* g;        // [B, N, H, N, D] bf16 gate logits
  const uint16_t* w_o;      // [C, F] bf16
  uint16_t* y;              // [B, N, N, C] bf16 (forward)
  const uint16_t* dy;       // [B, N, N, C] bf16 (backward)
  uint16_t* d_o;            // [B, N, H, N, D] bf16 (backward)
  uint16_t* d_g;            // [B, N, H, N, D] bf16 (backward)
  float* wo_partial;        // [grid, C, F] FP32 (backward)
};

struct BlkProjBwdArgs {
  BlkShape s;
  const uint16_t* z;
  const float* stats;
  const float* gamma;
  const float* beta;
  const uint16_t* w_qkvg;
  const uint16_t* w_b;
  const uint16_t* dq; const uint16_t* dk; const uint16_t* dv; const uint16_t* dg;
  const uint16_t* dbias;    // [B, H, N, N] bf16
  uint16_t* dz;             // [B, N, N, C] bf16
  float* ln_partial;        // [grid, 2C] FP32: dgamma then dbeta
  float* w_partial;         // [grid, 4F + H, C] FP32: d w_qkvg rows then d w_b rows
};

struct BlkReduceArgs {
  const float* partial;     // [n, elems]
  float* out0;              // elements [0, split)
  float* out1;              // elements [split, elems)
  int64_t elems, split;
  int n;
};

hipError_t launch_blk_ln_proj(const BlkLnProjArgs& a, hipStream_t st);
hipError_t launch_blk_gate_out(const BlkGateOutArgs& a, hipStream_t st);
hipError_t launch_blk_gate_out_bwd(const BlkGateOutArgs& a, hipStream_t st);
hipError_t launch_blk_proj_dz(const BlkProjBwdArgs& a, hipStream_t st);
hipError_t launch_blk_proj_dw(const BlkProjBwdArgs& a, hipStream_t st);
hipError_t launch_blk_reduce(const BlkReduceArgs& a, hipStream_t st);

}  // namespace tri
