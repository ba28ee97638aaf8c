// C ABI of the triangle-attention block: argument validation and launch.
// See include/tri_attn_block.h for the contract of each entry point.
#include <cmath>
#include <cstdint>

#include "../../include/tri_attn_block.h"
#include "block_kernels.h"

namespace {

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

tri_attn_status check(const tri_block_dims* d) {
  if (!d) return TRI_ATTN_ERR_NULL;
  if (d->B < 1 || d->N < 1 || d->C_z < 1 || d->H < 1 || d->D < 1) return TRI_ATTN_ERR_SHAPE;
  if (!(d->eps > 0.f) || !std::isfinite(d->eps)) return TRI_ATTN_ERR_SHAPE;
  if (d->ending != 0 && d->ending != 1) return TRI_ATTN_ERR_SHAPE;
  if (d->C_z != tri::kBlkC || d->H * d->D != tri::kBlkF || (d->D != 32 && d->D != 16))
    return TRI_ATTN_ERR_UNSUPPORTED;
  // 32-bit element offsets: every pair tensor [B, N, N, 128] must stay below 2^31 bytes
  // (B and N are capped first, so the product below cannot overflow int64)
  if (d->N > 32767 || d->B > 65535 || d->B * d->N * d->N * tri::kBlkC * 2 >= (int64_t(1) << 31))
    return TRI_ATTN_ERR_SHAPE;
  return TRI_ATTN_OK;
}

int64_t pairs(const tri_block_dims* d) { return d->B * d->N * d->N; }

tri::BlkShape shape(const tri_block_dims* d) {
  tri::BlkShape s;
  s.B = (int)d->B; s.N = (int)d->N; s.H = (int)d->H; s.D = (int)d->D;
  s.ending = d->ending; s.eps = d->eps;
  return s;
}

tri_attn_status launched(hipError_t e) { return e == hipSuccess ? TRI_ATTN_OK : TRI_ATTN_ERR_LAUNCH; }

}  // namespace

extern "C" {

tri_attn_status tri_block_workspace(const tri_block_dims* d, int64_t* n_out, int64_t* n_w, int64_t* n_ln) {
  const tri_attn_status st = check(d);
  if (st != TRI_ATTN_OK) return st;
  if (n_out) *n_out = tri::blk_grid(pairs(d), tri::kBlkTileOutBwd);
  if (n_w) *n_w = tri::blk_dw_groups(pairs(d));
  if (n_ln) *n_ln = tri::blk_grid(pairs(d), tri::kBlkTileProjBwd);
  return TRI_ATTN_OK;
}

tri_attn_status tri_block_ln_proj(const tri_block_dims* d, const tri_bf16* z, const float* gamma,
                                  const float* beta, const tri_bf16* w_qkvg, const tri_bf16* w_b,
                                  tri_bf16* q, tri_bf16* k, tri_bf16* v, tri_bf16* g,
                                  tri_bf16* bias, float* ln_stats, tri_attn_stream stream) {
  const tri_attn_status st = check(d);
  if (st != TRI_ATTN_OK) return st;
  if (!z || !gamma || !beta || !w_qkvg || !w_b || !q || !k || !v || !g || !bias || !ln_stats)
    return TRI_ATTN_ERR_NULL;
  if (!al16(z) || !al16(gamma) || !al16(beta) || !al16(w_qkvg) || !al16(w_b) || !al16(q) ||
      !al16(k) || !al16(v) || !al16(g) || !al16(bias) || !al16(ln_stats))
    return TRI_ATTN_ERR_ALIGN;
  tri::BlkLnProjArgs a;
  a.s = shape(d);
  a.z = z; a.gamma = gamma; a.beta = beta; a.w_qkvg = w_qkvg; a.w_b = w_b;
  a.q = q; a.k = k; a.v = v; a.g = g; a.bias = bias; a.stats = ln_stats;
  return launched(tri::launch_blk_ln_proj(a, (hipStream_t)stream));
}

tri_attn_status tri_block_gate_out(const tri_block_dims* d, const tri_bf16* o, const tri_bf16* g,
                                   const tri_bf16* w_o, tri_bf16* y, tri_attn_stream stream) {
  const tri_attn_status st = check(d);
  if (st != TRI_ATTN_OK) return st;
  if (!o || !g || !w_o || !y) return TRI_ATTN_ERR_NULL;
  if (!al16(o) || !al16(g) || !al16(w_o) || !al16(y)) return TRI_ATTN_ERR_ALIGN;
  tri::BlkGateOutArgs a = {};
  a.s = shape(d);
  a.o = o; a.g = g; a.w_o = w_o; a.y = y;
  return launched(tri::launch_blk_gate_out(a, (hipStream_t)stream));
}

tri_attn_status tri_block_gate_out_bwd(const tri_block_dims* d, const tri_bf16* dy,
                                       const tri_bf16* o, const tri_bf16* g, const tri_bf16* w_o,
                                       tri_bf16* d_o, tri_bf16* d_g, float* wo_partial,
                                       tri_attn_stream stream) {
  const tri_attn_status st = check(d);
  if (st != TRI_ATTN_OK) return st;
  if (!dy || !o || !g || !w_o || !d_o || !d_g || !wo_partial) return TRI_ATTN_ERR_NULL;
  if (!al16(dy) || !al16(o) || !al16(g) || !al16(w_o) || !al16(d_o) || !al16(d_g) || !al16(wo_partial))
    return TRI_ATTN_ERR_ALIGN;
  tri::BlkGateOutArgs a = {};
  a.s = shape(d);
  a.o = o; a.g = g; a.w_o = w_o; a.dy = dy; a.d_o = d_o; a.d_g = d_g; a.wo_partial = wo_partial;
  return launched(tri::launch_blk_gate_out_bwd(a, (hipStream_t)stream));
}

tri_attn_status tri_block_proj_bwd_dz(const tri_block_dims* d, const tri_bf16* z,
                                      const float* ln_stats, const float* gamma,
                                      const tri_bf16* w_qkvg, const tri_bf16* w_b,
                                      const tri_bf16* dq, const tri_bf16* dk, const tri_bf16* dv,
                                      const tri_bf16* dg, const tri_bf16* dbias, tri_bf16* dz,
                                      float* ln_partial, tri_attn_stream stream) {
  const tri_attn_status st = check(d);
  if (st != TRI_ATTN_OK) return st;
  if (!z || !ln_stats || !gamma || !w_qkvg || !w_b || !dq || !dk || !dv || !dg || !dbias || !dz ||
      !ln_partial)
    return TRI_ATTN_ERR_NULL;
  if (!al16(z) || !al16(ln_stats) || !al16(gamma) || !al16(w_qkvg) || !al16(w_b) || !al16(dq) ||
      !al16(dk) || !al16(dv) || !al16(dg) || !al16(dbias) || !al16(dz) || !al16(ln_partial))
    return TRI_ATTN_ERR_ALIGN;
  tri::BlkProjBwdArgs a = {};
  a.s = shape(d);
  a.z = z; a.stats = ln_stats; a.gamma = gamma; a.w_qkvg = w_qkvg; a.w_b = w_b;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbias = dbias; a.dz = dz; a.ln_partial = ln_partial;
  return launched(tri::launch_blk_proj_dz(a, (hipStream_t)stream));
}

tri_attn_status tri_block_proj_bwd_dw(const tri_block_dims* d, const tri_bf16* z,
                                      const float* ln_stats, const float* gamma, const float* beta,
                                      const tri_bf16* dq, const tri_bf16* dk, const tri_bf16* dv,
                                      const tri_bf16* dg, const tri_bf16* dbias, float* w_partial,
                                      tri_attn_stream stream) {
  const tri_attn_status st = check(d);
  if (st != TRI_ATTN_OK) return st;
  if (!z || !ln_stats || !gamma || !beta || !dq || !dk || !dv || !dg || !dbias || !w_partial)
    return TRI_ATTN_ERR_NULL;
  if (!al16(z) || !al16(ln_stats) || !al16(gamma) || !al16(beta) || !al16(dq) || !al16(dk) ||
      !al16(dv) || !al16(dg) || !al16(dbias) || !al16(w_partial))
    return TRI_ATTN_ERR_ALIGN;
  tri::BlkProjBwdArgs a = {};
  a.s = shape(d);
  a.z = z; a.stats = ln_stats; a.gamma = gamma; a.beta = beta;
  a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbias = dbias; a.w_partial = w_partial;
  return launched(tri::launch_blk_proj_dw(a, (hipStream_t)stream));
}

tri_attn_status tri_block_reduce_wgrad(const tri_block_dims* d, const float* w_partial,
                                       const float* wo_partial, const float* ln_partial,
                                       float* dw_qkvg, float* dw_b, float* dw_o, float* dgamma,
                                       float* dbeta, tri_attn_stream stream) {
  const tri_attn_status st = check(d);
  if (st != TRI_ATTN_OK) return st;
  if (!w_partial || !wo_partial || !ln_partial || !dw_qkvg || !dw_b || !dw_o || !dgamma || !dbeta)
    return TRI_ATTN_ERR_NULL;
  if (!al16(w_partial) || !al16(wo_partial) || !al16(ln_partial) || !al16(dw_qkvg) || !al16(dw_b) ||
      !al16(dw_o) || !al16(dgamma) || !al16(dbeta))
    return TRI_ATTN_ERR_ALIGN;
  const int64_t C = tri::kBlkC, F = tri::kBlkF, H = d->H;
  tri::BlkReduceArgs r;
  r.partial = w_partial; r.out0 = dw_qkvg; r.out1 = dw_b;
  r.elems = (4 * F + H) * C; r.split = 4 * F * C;
  r.n = (int)tri::blk_dw_groups(pairs(d));
  hipError_t e = tri::launch_blk_reduce(r, (hipStream_t)stream);
  if (e != hipSuccess) return TRI_ATTN_ERR_LAUNCH;
  r.partial = wo_partial; r.out0 = dw_o; r.out1 = nullptr;
  r.elems = C * F; r.split = C * F;
  r.n = (int)tri::blk_grid(pairs(d), tri::kBlkTileOutBwd);
  e = tri::launch_blk_reduce(r, (hipStream_t)stream);
  if (e != hipSuccess) return TRI_ATTN_ERR_LAUNCH;
  r.partial = ln_partial; r.out0 = dgamma; r.out1 = dbeta;
  r.elems = 2 * C; r.split = C;
  r.n = (int)tri::blk_grid(pairs(d), tri::kBlkTileProjBwd);
  return launched(tri::launch_blk_reduce(r, (hipStream_t)stream));
}

}  // extern "C"
