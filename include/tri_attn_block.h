/*
 * tri_attn_block.h -- C ABI of the triangle-attention block around the attention core.
 *
 * The block of "TurboPairFormer: Fast and Stable Protein Folding Model Training
 * with an Optimized Triangle Attention Kernel" (Table 1; worked example,
 * Figure 6): slice o of the attention is row o of the pair tensor Z; pair
 * (o, q) is projected to query q, pair (o, k) to key k and value k, pair (q, k)
 * to the bias of (q, k), shared by every slice; the attention output updates
 * pair (o, q); a normalisation precedes the projections.  Where the pages stop,
 * this library takes the plain Pairformer form:
 *
 *   Zln  = LayerNorm(Z) over C_z (biased variance, eps inside the root, scale gamma, shift beta)
 *   Q, K, V, G = Zln w_q^T, Zln w_k^T, Zln w_v^T, Zln w_g^T   (C_z -> H*D, no additive terms)
 *   bias = Zln w_b^T                                          (C_z -> H)
 *   O    = triangular attention (tri_attn.h) with scale 1/sqrt(D), no mask
 *   Y    = (sigmoid(G) * O) w_o^T                             (H*D -> C_z)
 *
 * The ending node is the same block applied to Z with its two token axes
 * swapped (pair (x, y) of the block is Z[b, y, x]); Y and dZ are swapped back.
 * Seven calls, in order: tri_block_ln_proj, tri_attn_fwd, tri_block_gate_out
 * (forward); tri_block_gate_out_bwd, tri_attn_bwd_delta, tri_attn_bwd,
 * tri_attn_reduce_dbias, tri_attn_reduce_dq, tri_block_proj_bwd_dz,
 * tri_block_proj_bwd_dw, tri_block_reduce_wgrad (backward).  The attention
 * calls take tri_attn_dims {B, N_o = N, H, N, D, scale = 1/sqrt(D)}.
 *
 * Supported: C_z = 128, H * D = 128 with D = 32 (H = 4) or D = 16 (H = 8),
 * N >= 1, B * N * N * 128 * 2 bytes < 2^31.
 *
 * Layouts (dense, row-major, every pointer a DEVICE pointer owned by the caller,
 * 16-byte aligned):
 *   z, dz, y, dy          [B, N, N, C_z]        bf16
 *   q, k, v, g (and grads), o, d_o  [B, N, H, N, D]  bf16 (g = gate logits)
 *   bias, dbias           [B, H, N, N]          bf16
 *   ln_stats              [B, N, N, 2]          fp32 (mean, 1/sqrt(var + eps)) per pair,
 *                                               in the block's pair order (x, y)
 *   gamma, beta           [C_z]                 fp32
 *   w_qkvg                [4*H*D, C_z]          bf16, rows: Q, K, V, gate features (h*D + d)
 *   w_b                   [H, C_z]              bf16
 *   w_o                   [C_z, H*D]            bf16
 *   dw_qkvg, dw_b, dw_o, dgamma, dbeta           fp32, same shapes as the weights
 *   wo_partial            [n_out, C_z, H*D]     fp32 (n_out from tri_block_workspace)
 *   w_partial             [n_w, 4*H*D + H, C_z] fp32
 *   ln_partial            [n_ln, 2 * C_z]       fp32
 *
 * Rounding: Zln, the projections, the gated output sigmoid(G) * O and every
 * gradient that leaves a kernel are rounded once to bf16 (nearest even); all
 * products accumulate in FP32; LayerNorm statistics are FP32.  Weight-gradient
 * partials are FP32, one per workgroup of a fixed-size grid, summed in a fixed
 * order: every output is bitwise reproducible.
 *
 * Errors: as in tri_attn.h (checked on the host before any launch; nothing is
 * enqueued on error except for TRI_ATTN_ERR_LAUNCH).  The library allocates,
 * frees and synchronises nothing.
 */
#ifndef TRI_ATTN_BLOCK_H
#define TRI_ATTN_BLOCK_H

#include "tri_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int64_t B, N, C_z, H, D;
  int32_t ending; /* 0: starting node, 1: ending node */
  float eps;      /* LayerNorm epsilon (> 0) */
} tri_block_dims;

/* Partial-buffer counts of the backward (host only; any pointer may be NULL). */
tri_attn_status tri_block_workspace(const tri_block_dims* d, int64_t* n_out, int64_t* n_w,
                                    int64_t* n_ln);

/*
 * Forward, part 1 (Figure 6 steps 1-3 and the normalisation before the projections):
 * LayerNorm + the Q, K, V, gate and bias projections; writes ln_stats for the backward.
 */
tri_attn_status tri_block_ln_proj(const tri_block_dims* d, const tri_bf16* z, const float* gamma,
                                  const float* beta, const tri_bf16* w_qkvg, const tri_bf16* w_b,
                                  tri_bf16* q, tri_bf16* k, tri_bf16* v, tri_bf16* g,
                                  tri_bf16* bias, float* ln_stats, tri_attn_stream stream);

/* Forward, part 3 (Figure 6 step 4, the update of pair (o, q)): Y = (sigmoid(G) * O) w_o^T. */
tri_attn_status tri_block_gate_out(const tri_block_dims* d, const tri_bf16* o, const tri_bf16* g,
                                   const tri_bf16* w_o, tri_bf16* y, tri_attn_stream stream);

/*
 * Backward of the gated output projection: dGO = dY w_o, d_o = dGO * sigmoid(G),
 * d_g = dGO * O * sigmoid(G) (1 - sigmoid(G)); wo_partial[i] = this workgroup's sum of
 * dY^T (sigmoid(G) * O).
 */
tri_attn_status tri_block_gate_out_bwd(const tri_block_dims* d, const tri_bf16* dy,
                                       const tri_bf16* o, const tri_bf16* g, const tri_bf16* w_o,
                                       tri_bf16* d_o, tri_bf16* d_g, float* wo_partial,
                                       tri_attn_stream stream);

/*
 * Backward of the projections and the LayerNorm, part 1:
 * dZln = [dQ dK dV dG] w_qkvg + dbias^T w_b, dZ = LayerNorm backward of dZln;
 * ln_partial[i] = this workgroup's (sum dZln * xhat, sum dZln) per feature.
 */
tri_attn_status tri_block_proj_bwd_dz(const tri_block_dims* d, const tri_bf16* z,
                                      const float* ln_stats, const float* gamma,
                                      const tri_bf16* w_qkvg, const tri_bf16* w_b,
                                      const tri_bf16* dq, const tri_bf16* dk, const tri_bf16* dv,
                                      const tri_bf16* dg, const tri_bf16* dbias, tri_bf16* dz,
                                      float* ln_partial, tri_attn_stream stream);

/*
 * Backward of the projections, part 2: w_partial[i] = this tile group's
 * [dQ dK dV dG | dbias]^T Zln (Zln recomputed from z and ln_stats).
 */
tri_attn_status tri_block_proj_bwd_dw(const tri_block_dims* d, const tri_bf16* z,
                                      const float* ln_stats, const float* gamma, const float* beta,
                                      const tri_bf16* dq, const tri_bf16* dk, const tri_bf16* dv,
                                      const tri_bf16* dg, const tri_bf16* dbias, float* w_partial,
                                      tri_attn_stream stream);

/* Fixed-order sums of the three partial sets into the FP32 weight gradients. */
tri_attn_status tri_block_reduce_wgrad(const tri_block_dims* d, const float* w_partial,
                                       const float* wo_partial, const float* ln_partial,
                                       float* dw_qkvg, float* dw_b, float* dw_o, float* dgamma,
                                       float* dbeta, tri_attn_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* TRI_ATTN_BLOCK_H */
