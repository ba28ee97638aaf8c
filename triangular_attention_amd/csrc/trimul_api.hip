// C ABI of the triangle multiplicative update: argument validation and launch.
// See include/tri_mul.h for the contract of each entry point.
#include <cmath>
#include <cstdint>

#include "../../include/tri_mul.h"
#include "block_kernels.h"
#include "trimul_kernels.h"

namespace {

bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

tri_attn_status check(const tri_mul_dims* d) {
  if (!d) return TRI_ATTN_ERR_NULL;
  if (d->B < 1 || d->N < 1 || d->C_z < 1 || d->c < 1) return TRI_ATTN_ERR_SHAPE;
  if (!(d->eps > 0.f) || !std::isfinite(d->eps)) return TRI_ATTN_ERR_SHAPE;
  if (d->incoming != 0 && d->incoming != 1) return TRI_ATTN_ERR_SHAPE;
  if (d->C_z != tri::kTmC || (d->c != 64 && d->c != 128)) return TRI_ATTN_ERR_UNSUPPORTED;
  if (d->N % 8 != 0) return TRI_ATTN_ERR_SHAPE;
  // 32-bit offsets: the largest pair tensor (dproj, [B * N * N, 4c] bf16) stays below 2^31 bytes
  // (B and N are capped first, so the product below cannot overflow int64)
  if (d->N > 32767 || d->B > 65535 || d->B * d->N * d->N * 4 * d->c * 2 >= (int64_t(1) << 31))
    return TRI_ATTN_ERR_SHAPE;
  return TRI_ATTN_OK;
}

int64_t pairs(const tri_mul_dims* d) { return d->B * d->N * d->N; }

tri::TmShape shape(const tri_mul_dims* d) {
  tri::TmShape s;
  s.B = (int)d->B; s.N = (int)d->N; s.c = (int)d->c;
  s.incoming = d->incoming; s.eps = d->eps;
  return s;
}

tri_attn_status launched(hipError_t e) { return e == hipSuccess ? TRI_ATTN_OK : TRI_ATTN_ERR_LAUNCH; }

int64_t n_out(const tri_mul_dims* d) { return tri::tm_grid(pairs(d), tri::kTmTileOutBwd); }
int64_t n_lno(const tri_mul_dims* d) { return n_out(d) * (128 / d->c); }

}  // namespace

extern "C" {

tri_attn_status tri_mul_workspace(const tri_mul_dims* d, int64_t* n_w, int64_t* n_out_cnt, int64_t* n_ln,
                                  int64_t* n_lno_out) {
  const tri_attn_status st = check(d);
  if (st != TRI_ATTN_OK) return st;
  if (n_w) *n_w = tri::tm_dw_groups(pairs(d), (int)d->c);
  if (n_out_cnt) *n_out_cnt = n_out(d);
  if (n_ln) *n_ln = tri::tm_grid(pairs(d), tri::kTmTileDz);
  if (n_lno_out) *n_lno_out = n_lno(d);
  return TRI_ATTN_OK;
}

tri_attn_status tri_mul_in_fwd(const tri_mul_dims* d, const tri_bf16* z, const float* gamma,
                               const float* beta, const tri_bf16* w_in, tri_bf16* a, tri_bf16* b,
                               tri_bf16* g, float* stats, tri_attn_stream stream) {
  const tri_attn_status st = check(d);
  if (st != TRI_ATTN_OK) return st;
  if (!z || !gamma || !beta || !w_in || !a || !b || !g || !stats) return TRI_ATTN_ERR_NULL;
  if (!al16(z) || !al16(gamma) || !al16(beta) || !al16(w_in) || !al16(a) || !al16(b) || !al16(g) ||
      !al16(stats))
    return TRI_ATTN_ERR_ALIGN;
  tri::TmInArgs p = {};
  p.s = shape(d);
  p.z = z; p.gamma = gamma; p.beta = beta; p.w_in = w_in; p.a = a; p.b = b; p.g = g; p.stats = stats;
  return launched(tri::launch_tm_in_fwd(p, (hipStream_t)stream));
}

tri_attn_status tri_mul_contract(const tri_mul_dims* d, const tri_bf16* a, const tri_bf16* b,
                                 tri_bf16* x, tri_attn_stream stream) {
  const tri_attn_status st = check(d);
  if (st != TRI_ATTN_OK) return st;
  if (!a || !b || !x) return TRI_ATTN_ERR_NULL;
  if (!al16(a) || !al16(b) || !al16(x)) return TRI_ATTN_ERR_ALIGN;
  tri::TmGemmArgs p;
  p.A = a; p.B = b; p.C = x; p.batch = (int)(d->B * d->c); p.N = (int)d->N;
  return launched(tri::launch_tm_gemm_nt(p, (hipStream_t)stream));
}

tri_attn_status tri_mul_out_fwd(const tri_mul_dims* d, const tri_bf16* x, const tri_bf16* g,
                                const float* gamma_o, const float* beta_o, const tri_bf16* w_o,
                                tri_bf16* out, float* stats_o, tri_attn_stream stream) {
  const tri_attn_status st = check(d);
  if (st != TRI_ATTN_OK) return st;
  if (!x || !g || !gamma_o || !beta_o || !w_o || !out || !stats_o) return TRI_ATTN_ERR_NULL;
  if (!al16(x) || !al16(g) || !al16(gamma_o) || !al16(beta_o) || !al16(w_o) || !al16(out) || !al16(stats_o))
    return TRI_ATTN_ERR_ALIGN;
  tri::TmOutArgs p = {};
  p.s = shape(d);
  p.x = x; p.g = g; p.gamma_o = gamma_o; p.beta_o = beta_o; p.w_o = w_o; p.out = out; p.stats_o = stats_o;
  return launched(tri::launch_tm_out_fwd(p, (hipStream_t)stream));
}

tri_attn_status tri_mul_out_bwd(const tri_mul_dims* d, const tri_bf16* dout, const tri_bf16* x,
                                const tri_bf16* g, const float* stats_o, const float* gamma_o,
                                const float* beta_o, const tri_bf16* w_o, tri_bf16* dx,
                                tri_bf16* dg, float* wo_partial, float* lno_partial,
                                tri_attn_stream stream) {
  const tri_attn_status st = check(d);
  if (st != TRI_ATTN_OK) return st;
  if (!dout || !x || !g || !stats_o || !gamma_o || !beta_o || !w_o || !dx || !dg || !wo_partial || !lno_partial)
    return TRI_ATTN_ERR_NULL;
  if (!al16(dout) || !al16(x) || !al16(g) || !al16(stats_o) || !al16(gamma_o) || !al16(beta_o) ||
      !al16(w_o) || !al16(dx) || !al16(dg) || !al16(wo_partial) || !al16(lno_partial))
    return TRI_ATTN_ERR_ALIGN;
  tri::TmOutArgs p = {};
  p.s = shape(d);
  p.x = x; p.g = g; p.gamma_o = gamma_o; p.beta_o = beta_o; p.w_o = w_o; p.stats_o = const_cast<float*>(stats_o);
  p.dout = dout; p.dx = dx; p.dg = dg; p.wo_partial = wo_partial; p.lno_partial = lno_partial;
  return launched(tri::launch_tm_out_bwd(p, (hipStream_t)stream));
}

tri_attn_status tri_mul_contract_bwd(const tri_mul_dims* d, const tri_bf16* dx, const tri_bf16* a,
                                     const tri_bf16* b, tri_bf16* da, tri_bf16* db,
                                     tri_attn_stream stream) {
  const tri_attn_status st = check(d);
  if (st != TRI_ATTN_OK) return st;
  if (!dx || !a || !b || !da || !db) return TRI_ATTN_ERR_NULL;
  if (!al16(dx) || !al16(a) || !al16(b) || !al16(da) || !al16(db)) return TRI_ATTN_ERR_ALIGN;
  tri::TmGemmArgs p;
  p.batch = (int)(d->B * d->c); p.N = (int)d->N;
  p.A = dx; p.B = b; p.C = da;
  if (tri::launch_tm_gemm_nn(p, (hipStream_t)stream) != hipSuccess) return TRI_ATTN_ERR_LAUNCH;
  p.A = dx; p.B = a; p.C = db;
  return launched(tri::launch_tm_gemm_tn(p, (hipStream_t)stream));
}

tri_attn_status tri_mul_in_bwd(const tri_mul_dims* d, const tri_bf16* z, const float* stats,
                               const float* gamma, const float* beta, const tri_bf16* w_in,
                               const tri_bf16* da, const tri_bf16* db, tri_bf16* dproj,
                               tri_attn_stream stream) {
  const tri_attn_status st = check(d);
  if (st != TRI_ATTN_OK) return st;
  if (!z || !stats || !gamma || !beta || !w_in || !da || !db || !dproj) return TRI_ATTN_ERR_NULL;
  if (!al16(z) || !al16(stats) || !al16(gamma) || !al16(beta) || !al16(w_in) || !al16(da) || !al16(db) ||
      !al16(dproj))
    return TRI_ATTN_ERR_ALIGN;
  tri::TmInArgs p = {};
  p.s = shape(d);
  p.z = z; p.stats = const_cast<float*>(stats); p.gamma = gamma; p.beta = beta; p.w_in = w_in;
  p.da = da; p.db = db; p.dproj = dproj;
  return launched(tri::launch_tm_in_bwd(p, (hipStream_t)stream));
}

tri_attn_status tri_mul_in_bwd_dz(const tri_mul_dims* d, const tri_bf16* z, const float* stats,
                                  const float* gamma, const tri_bf16* w_in, const tri_bf16* dproj,
                                  const tri_bf16* dg, tri_bf16* dz, float* ln_partial,
                                  tri_attn_stream stream) {
  const tri_attn_status st = check(d);
  if (st != TRI_ATTN_OK) return st;
  if (!z || !stats || !gamma || !w_in || !dproj || !dg || !dz || !ln_partial) return TRI_ATTN_ERR_NULL;
  if (!al16(z) || !al16(stats) || !al16(gamma) || !al16(w_in) || !al16(dproj) || !al16(dg) || !al16(dz) ||
      !al16(ln_partial))
    return TRI_ATTN_ERR_ALIGN;
  tri::TmInGradArgs p = {};
  p.s = shape(d);
  p.z = z; p.stats = stats; p.gamma = gamma; p.w_in = w_in; p.dproj = dproj; p.dg = dg; p.dz = dz;
  p.ln_partial = ln_partial;
  return launched(tri::launch_tm_in_dz(p, (hipStream_t)stream));
}

tri_attn_status tri_mul_in_bwd_dw(const tri_mul_dims* d, const tri_bf16* z, const float* stats,
                                  const float* gamma, const float* beta, const tri_bf16* dproj,
                                  const tri_bf16* dg, float* w_partial, tri_attn_stream stream) {
  const tri_attn_status st = check(d);
  if (st != TRI_ATTN_OK) return st;
  if (!z || !stats || !gamma || !beta || !dproj || !dg || !w_partial) return TRI_ATTN_ERR_NULL;
  if (!al16(z) || !al16(stats) || !al16(gamma) || !al16(beta) || !al16(dproj) || !al16(dg) || !al16(w_partial))
    return TRI_ATTN_ERR_ALIGN;
  tri::TmInGradArgs p = {};
  p.s = shape(d);
  p.z = z; p.stats = stats; p.gamma = gamma; p.beta = beta; p.dproj = dproj; p.dg = dg; p.w_partial = w_partial;
  return launched(tri::launch_tm_in_dw(p, (hipStream_t)stream));
}

tri_attn_status tri_mul_reduce_wgrad(const tri_mul_dims* d, const float* w_partial,
                                     const float* wo_partial, const float* ln_partial,
                                     const float* lno_partial, float* dw_in, float* dw_o,
                                     float* dgamma, float* dbeta, float* dgamma_o,
                                     float* dbeta_o, tri_attn_stream stream) {
  const tri_attn_status st = check(d);
  if (st != TRI_ATTN_OK) return st;
  if (!w_partial || !wo_partial || !ln_partial || !lno_partial || !dw_in || !dw_o || !dgamma || !dbeta ||
      !dgamma_o || !dbeta_o)
    return TRI_ATTN_ERR_NULL;
  if (!al16(w_partial) || !al16(wo_partial) || !al16(ln_partial) || !al16(lno_partial) || !al16(dw_in) ||
      !al16(dw_o) || !al16(dgamma) || !al16(dbeta) || !al16(dgamma_o) || !al16(dbeta_o))
    return TRI_ATTN_ERR_ALIGN;
  const int64_t C = tri::kTmC, c = d->c;
  hipStream_t s = (hipStream_t)stream;
  tri::BlkReduceArgs r;
  r.partial = w_partial; r.out0 = dw_in; r.out1 = nullptr;
  r.elems = (4 * c + C) * C; r.split = r.elems; r.n = (int)tri::tm_dw_groups(pairs(d), (int)c);
  if (tri::launch_blk_reduce(r, s) != hipSuccess) return TRI_ATTN_ERR_LAUNCH;
  r.partial = wo_partial; r.out0 = dw_o; r.out1 = nullptr;
  r.elems = C * c; r.split = r.elems; r.n = (int)n_out(d);
  if (tri::launch_blk_reduce(r, s) != hipSuccess) return TRI_ATTN_ERR_LAUNCH;
  r.partial = ln_partial; r.out0 = dgamma; r.out1 = dbeta;
  r.elems = 2 * C; r.split = C; r.n = (int)tri::tm_grid(pairs(d), tri::kTmTileDz);
  if (tri::launch_blk_reduce(r, s) != hipSuccess) return TRI_ATTN_ERR_LAUNCH;
  r.partial = lno_partial; r.out0 = dgamma_o; r.out1 = dbeta_o;
  r.elems = 2 * c; r.split = c; r.n = (int)n_lno(d);
  return launched(tri::launch_blk_reduce(r, s));
}

}  // extern "C"
