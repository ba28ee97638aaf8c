/*
 * tri_mul.h -- C ABI of the triangle multiplicative update (outgoing and incoming).
 *
 * The update of "TurboPairFormer: Fast and Stable Protein Folding Model Training
 * with an Optimized Triangle Attention Kernel", Figure 12 (times in Table 10): an
 * input step normalises the pair features and forms five projections -- two branch
 * values, two branch gates and the output gate logits -- and gates the branch
 * values; one contraction per channel; an output step normalises the contraction,
 * projects it back to the pair features and multiplies by the sigmoid of the saved
 * gate logits.  In formulas (no additive terms in any projection, no pair mask):
 *
 *   Zln = LayerNorm(Z)                                    over C_z, FP32 statistics
 *   a   = sigmoid(Zln w_ag^T) * (Zln w_ap^T),  b likewise  C_z -> c channels
 *   G   = Zln w_g^T                                        C_z -> C_z (gate logits)
 *   outgoing  x[i,j,ch] = sum_k a[i,k,ch] b[j,k,ch]
 *   incoming  x[i,j,ch] = sum_k a[k,i,ch] b[k,j,ch]
 *   out = sigmoid(G) * (LayerNorm_c(x) w_o^T)             c -> C_z
 *
 * Calls: forward tri_mul_in_fwd, tri_mul_contract, tri_mul_out_fwd; backward
 * tri_mul_out_bwd, tri_mul_contract_bwd, tri_mul_in_bwd, tri_mul_in_bwd_dz,
 * tri_mul_in_bwd_dw, tri_mul_reduce_wgrad.
 *
 * Supported: C_z = 128, c in {64, 128}, N >= 8 with N % 8 == 0, and
 * B * N * N * 4c * 2 bytes < 2^31.
 *
 * Layouts (dense, row-major; every pointer a DEVICE pointer owned by the caller,
 * 16-byte aligned):
 *   z, dz, out, dout, g, dg   [B, N, N, C_z]     bf16 (g = gate logits)
 *   a, b, da, db              [B, c, N, N]       bf16, one N x N matrix per channel; for the
 *                                                incoming form a[., ch, i, k] holds a[k, i, ch]
 *   x, dx                     [B, c, N, N]       bf16, x[., ch, i, j]
 *   stats, stats_o            [B * N * N, 2]     fp32 (mean, 1/sqrt(var + eps)) per pair
 *   dproj                     [B * N * N, 4c]    bf16 gradients of the four branch projections
 *   gamma, beta [C_z]; gamma_o, beta_o [c]       fp32
 *   w_in   [4c + C_z, C_z]    bf16, rows: value a, gate a, value b, gate b, output gate
 *   w_o    [C_z, c]           bf16
 *   dw_in, dw_o, dgamma, dbeta, dgamma_o, dbeta_o  fp32, shapes of the parameters
 *   w_partial [n_w, 4c + C_z, C_z], wo_partial [n_out, C_z, c], ln_partial [n_ln, 2 C_z],
 *   lno_partial [n_lno, 2c]   fp32 (counts from tri_mul_workspace)
 *
 * Rounding: Zln, a, b, G, x, LayerNorm_c(x), out and every gradient that leaves a kernel are
 * rounded once to bf16 (nearest even); products accumulate in FP32.  Weight gradients are
 * FP32 partials, one per workgroup of a fixed grid, summed in a fixed order: every output is
 * bitwise reproducible.  Errors as in tri_attn.h; the library allocates, frees and
 * synchronises nothing.
 */
#ifndef TRI_MUL_H
#define TRI_MUL_H

#include "tri_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int64_t B, N, C_z, c;
  int32_t incoming; /* 0: outgoing, 1: incoming */
  float eps;        /* LayerNorm epsilon of both normalisations (> 0) */
} tri_mul_dims;

/* Partial-buffer counts of the backward (host only; any pointer may be NULL). */
tri_attn_status tri_mul_workspace(const tri_mul_dims* d, int64_t* n_w, int64_t* n_out, int64_t* n_ln,
                                  int64_t* n_lno);

/* Input step (Figure 12, fused input kernel): LayerNorm, five projections, gated branch operands. */
tri_attn_status tri_mul_in_fwd(const tri_mul_dims* d, const tri_bf16* z, const float* gamma,
                               const float* beta, const tri_bf16* w_in, tri_bf16* a, tri_bf16* b,
                               tri_bf16* g, float* stats, tri_attn_stream stream);

/* The per-channel contraction (Figure 12, batched product): x[ch] = a[ch] b[ch]^T. */
tri_attn_status tri_mul_contract(const tri_mul_dims* d, const tri_bf16* a, const tri_bf16* b,
                                 tri_bf16* x, tri_attn_stream stream);

/* Output step (Figure 12, fused output kernel): LayerNorm over channels, projection, gate. */
tri_attn_status tri_mul_out_fwd(const tri_mul_dims* d, const tri_bf16* x, const tri_bf16* g,
                                const float* gamma_o, const float* beta_o, const tri_bf16* w_o,
                                tri_bf16* out, float* stats_o, tri_attn_stream stream);

/* Backward of the output step: dx, d gate logits, d w_o and d gamma_o / d beta_o partials. */
tri_attn_status tri_mul_out_bwd(const tri_mul_dims* d, const tri_bf16* dout, const tri_bf16* x,
                                const tri_bf16* g, const float* stats_o, const float* gamma_o,
                                const float* beta_o, const tri_bf16* w_o, tri_bf16* dx,
                                tri_bf16* dg, float* wo_partial, float* lno_partial,
                                tri_attn_stream stream);

/* Backward of the contraction: da[ch] = dx[ch] b[ch], db[ch] = dx[ch]^T a[ch]. */
tri_attn_status tri_mul_contract_bwd(const tri_mul_dims* d, const tri_bf16* dx, const tri_bf16* a,
                                     const tri_bf16* b, tri_bf16* da, tri_bf16* db,
                                     tri_attn_stream stream);

/* Backward of the input step, part 1: the branch projections recomputed, their gradients
 * (value and gate of a and b) from da, db. */
tri_attn_status tri_mul_in_bwd(const tri_mul_dims* d, const tri_bf16* z, const float* stats,
                               const float* gamma, const float* beta, const tri_bf16* w_in,
                               const tri_bf16* da, const tri_bf16* db, tri_bf16* dproj,
                               tri_attn_stream stream);

/* Backward of the input step, part 2: dZ through the projections and the LayerNorm;
 * d gamma / d beta partials. */
tri_attn_status tri_mul_in_bwd_dz(const tri_mul_dims* d, const tri_bf16* z, const float* stats,
                                  const float* gamma, const tri_bf16* w_in, const tri_bf16* dproj,
                                  const tri_bf16* dg, tri_bf16* dz, float* ln_partial,
                                  tri_attn_stream stream);

/* Backward of the input step, part 3: d w_in partials ([dproj | dg]^T Zln). */
tri_attn_status tri_mul_in_bwd_dw(const tri_mul_dims* d, const tri_bf16* z, const float* stats,
                                  const float* gamma, const float* beta, const tri_bf16* dproj,
                                  const tri_bf16* dg, float* w_partial, tri_attn_stream stream);

/* Fixed-order sums of the four partial sets into the FP32 parameter gradients. */
tri_attn_status tri_mul_reduce_wgrad(const tri_mul_dims* d, const float* w_partial,
                                     const float* wo_partial, const float* ln_partial,
                                     const float* lno_partial, float* dw_in, float* dw_o,
                                     float* dgamma, float* dbeta, float* dgamma_o,
                                     float* dbeta_o, tri_attn_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* TRI_MUL_H */
