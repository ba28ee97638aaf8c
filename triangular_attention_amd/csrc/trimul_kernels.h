// Argument blocks and launchers of the triangle-multiplicative-update kernels (internal).
//
// Pair features C = 128, branch channels c in {64, 128}; N % 8 == 0.  The branch operands
// and the contraction live channel-major ([B, c, N, N], one N x N matrix per channel); the
// gate logits, the update and the input/output gradients pair-major ([B, N, N, 128]).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tri {

constexpr int kTmC = 128;
constexpr int kTmTileIn = 128;     // pairs per tile: input kernels
constexpr int kTmTileOut = 128;    // pairs per tile: output step, forward
constexpr int kTmTileOutBwd = 64;  // pairs per tile: output step, backward
constexpr int kTmTileDz = 32;      // pairs per tile: dZ of the input projections
constexpr int kTmTileDw = 64;      // pairs per tile: weight gradient of the input projections
constexpr int kTmMaxWG = 256;
constexpr int kTmDwMaxWG = 512;    // the input weight-gradient kernel fits two workgroups per CU
constexpr int kTmOutMaxWG = 512;   // so does the output step's forward with c = 64 (no partials)

inline int64_t tm_grid(int64_t pairs, int tile, int cap = kTmMaxWG) {
  const int64_t t = (pairs + tile - 1) / tile;
  return t < cap ? t : cap;
}
// Workgroups per tile group of the input weight gradient (128 rows of d w_in each) and the
// number of tile groups (= partial buffers).
inline int tm_dw_splits(int c) { return (4 * c + kTmC) / 128; }
inline int64_t tm_dw_groups(int64_t pairs, int c) {
  const int64_t t = (pairs + kTmTileDw - 1) / kTmTileDw;
  const int64_t cap = 8 * (kTmDwMaxWG / (8 * tm_dw_splits(c)));
  return t < cap ? t : cap;
}

struct TmShape {
  int B, N, c;
  int incoming;      // 0: outgoing; 1: incoming (the input kernels read Z with its token axes swapped)
  float eps;
};

struct TmInArgs {
  TmShape s;
  const uint16_t* z;        // [B, N, N, C]
  const float* gamma;
  const float* beta;
  const uint16_t* w_in;     // [4c + C, C]: value a, gate a, value b, gate b, output gate
  uint16_t* a;              // [B, c, N, N] (forward)
  uint16_t* b;
  uint16_t* g;              // [B, N, N, C] output gate logits (forward)
  float* stats;             // [B * N * N, 2] LayerNorm mean, 1/sigma (forward writes, backward reads)
  const uint16_t* da;       // [B, c, N, N] (backward)
  const uint16_t* db;
  uint16_t* dproj;          // [B * N * N, 4c] gradients of the four branch projections (backward)
};

struct TmGemmArgs {
  const uint16_t* A;        // [batch, N, N]
  const uint16_t* B;
  uint16_t* C;
  int batch, N;
};

struct TmOutArgs {
  TmShape s;
  const uint16_t* x;        // [B, c, N, N]
  const uint16_t* g;        // [B, N, N, C]
  const float* gamma_o;     // [c]
  const float* beta_o;
  const uint16_t* w_o;      // [C, c]
  uint16_t* out;            // [B, N, N, C] (forward)
  float* stats_o;           // [B * N * N, 2] (forward writes, backward reads)
  const uint16_t* dout;     // (backward)
  uint16_t* dx;             // [B, c, N, N]
  uint16_t* dg;             // [B, N, N, C]
  float* wo_partial;        // [grid, C, c]
  float* lno_partial;       // [grid, 2c]
};

struct TmInGradArgs {
  TmShape s;
  const uint16_t* z;
  const float* stats;
  const float* gamma;
  const float* beta;
  const uint16_t* w_in;
  const uint16_t* dproj;    // [B * N * N, 4c] (input-kernel pair order)
  const uint16_t* dg;       // [B, N, N, C] (update pair order)
  uint16_t* dz;             // [B, N, N, C]
  float* ln_partial;        // [grid, 2C]
  float* w_partial;         // [groups, 4c + C, C]
};

hipError_t launch_tm_in_fwd(const TmInArgs& a, hipStream_t st);
hipError_t launch_tm_in_bwd(const TmInArgs& a, hipStream_t st);
// C[i] = A[i] B[i]^T (forward), dA = dX B, dB = dX^T A (backward); all [batch, N, N] bf16
hipError_t launch_tm_gemm_nt(const TmGemmArgs& a, hipStream_t st);
hipError_t launch_tm_gemm_nn(const TmGemmArgs& a, hipStream_t st);
hipError_t launch_tm_gemm_tn(const TmGemmArgs& a, hipStream_t st);
hipError_t launch_tm_out_fwd(const TmOutArgs& a, hipStream_t st);
hipError_t launch_tm_out_bwd(const TmOutArgs& a, hipStream_t st);
hipError_t launch_tm_in_dz(const TmInGradArgs& a, hipStream_t st);
hipError_t launch_tm_in_dw(const TmInGradArgs& a, hipStream_t st);

}  // namespace tri
