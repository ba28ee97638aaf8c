// C ABI of the triangular-attention library: argument validation and launch.
// See include/tri_attn.h for the contract of each entry point.
#include <cmath>
#include <cstdint>

#include "../../include/tri_attn.h"
#include "kernels.h"

namespace {

constexpr int64_t kMaxGridZ = 65535;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

tri_attn_status check_dims(const tri_attn_dims* d) {
  if (!d) return TRI_ATTN_ERR_NULL;
  if (d->B < 1 || d->N_o < 1 || d->H < 1 || d->N < 1 || d->D < 1) return TRI_ATTN_ERR_SHAPE;
  // the backward forms -lse / scale in FP32: |scale| >= 2^-64 keeps it finite for any
  // |lse| < 2^63 (zero and subnormal scales are rejected)
  if (!std::isfinite(d->scale) || std::fabs(d->scale) < 0x1p-64f) return TRI_ATTN_ERR_SHAPE;
  if (d->D != 16 && d->D != 32 && d->D != 64) return TRI_ATTN_ERR_UNSUPPORTED;
  // each dimension is capped before any product is formed (no int64 overflow); then the
  // 32-bit index limits of the kernels: every per-tensor row count fits in int32 and the
  // byte size of one FP32 N x N plane (4*N*N) fits in uint32
  if (d->N > (1 << 15) - 1 || d->B > kMaxGridZ || d->N_o > kMaxGridZ || d->H > kMaxGridZ)
    return TRI_ATTN_ERR_SHAPE;
  if (d->B * d->N_o > kMaxGridZ) return TRI_ATTN_ERR_SHAPE;
  const int64_t rows = d->B * d->N_o * d->H * d->N;     // < 2^16 * 2^16 * 2^15
  if (rows > (int64_t(1) << 31) / 64) return TRI_ATTN_ERR_SHAPE;
  return TRI_ATTN_OK;
}

int64_t n_key_tiles(const tri_attn_dims* d) { return (d->N + tri::kBwdKeyTile - 1) / tri::kBwdKeyTile; }
int64_t group_size(const tri_attn_dims* d) { return tri::bwd_group((int)d->D, tri::bias_load_width((int)d->N) != 0); }
int64_t n_groups(const tri_attn_dims* d) { return (d->N_o + group_size(d) - 1) / group_size(d); }
int64_t x_elems(const tri_attn_dims* d) { return d->B * d->N_o * d->H * d->N * d->D; }
int64_t y_elems(const tri_attn_dims* d) { return d->B * d->H * d->N * d->N; }

tri_attn_status launched(hipError_t e) { return e == hipSuccess ? TRI_ATTN_OK : TRI_ATTN_ERR_LAUNCH; }

}  // namespace

extern "C" {

const char* tri_attn_status_string(tri_attn_status s) {
  switch (s) {
    case TRI_ATTN_OK: return "ok";
    case TRI_ATTN_ERR_NULL: return "null pointer argument";
    case TRI_ATTN_ERR_SHAPE: return "invalid dimensions or scale";
    case TRI_ATTN_ERR_UNSUPPORTED: return "unsupported head dimension (D must be 16, 32 or 64)";
    case TRI_ATTN_ERR_ALIGN: return "pointer not 16-byte aligned";
    case TRI_ATTN_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

const char* tri_attn_version(void) { return "0.1.0"; }

tri_attn_status tri_attn_workspace(const tri_attn_dims* d, int64_t* dq_partial_elems,
                                   int64_t* dbias_partial_elems, int64_t* j_k, int64_t* l,
                                   int64_t* key_tile, int64_t* outer_group) {
  tri_attn_status st = check_dims(d);
  if (st != TRI_ATTN_OK) return st;
  if (dq_partial_elems) *dq_partial_elems = n_key_tiles(d) * x_elems(d);
  if (dbias_partial_elems) *dbias_partial_elems = n_groups(d) * y_elems(d);
  if (j_k) *j_k = n_key_tiles(d);
  if (l) *l = n_groups(d);
  if (key_tile) *key_tile = tri::kBwdKeyTile;
  if (outer_group) *outer_group = group_size(d);
  return TRI_ATTN_OK;
}

tri_attn_status tri_attn_fwd(const tri_attn_dims* d, const tri_bf16* q, const tri_bf16* k,
                             const tri_bf16* v, const tri_bf16* bias, const float* mask,
                             tri_bf16* o, tri_bf16* o_res, float* lse, tri_attn_stream stream) {
  tri_attn_status st = check_dims(d);
  if (st != TRI_ATTN_OK) return st;
  if (!q || !k || !v || !bias || !o || !lse) return TRI_ATTN_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(bias) || !aligned16(o) ||
      !aligned16(lse) || (mask && !aligned16(mask)) || (o_res && !aligned16(o_res)))
    return TRI_ATTN_ERR_ALIGN;
  tri::FwdArgs a;
  a.q = q; a.k = k; a.v = v; a.bias = bias; a.mask = mask;
  a.o = o; a.o_res = o_res; a.lse = lse;
  a.B = (int)d->B; a.N_o = (int)d->N_o; a.H = (int)d->H; a.N = (int)d->N;
  a.scale = d->scale;
  return launched(tri::launch_fwd(a, (int)d->D, (hipStream_t)stream));
}

tri_attn_status tri_attn_bwd_delta(const tri_attn_dims* d, const tri_bf16* o,
                                   const tri_bf16* o_res, const tri_bf16* d_o, float* delta,
                                   tri_attn_stream stream) {
  tri_attn_status st = check_dims(d);
  if (st != TRI_ATTN_OK) return st;
  if (!o || !d_o || !delta) return TRI_ATTN_ERR_NULL;
  if (!aligned16(o) || !aligned16(d_o) || !aligned16(delta) || (o_res && !aligned16(o_res)))
    return TRI_ATTN_ERR_ALIGN;
  tri::DeltaArgs a;
  a.o = o; a.o_res = o_res; a.d_o = d_o; a.delta = delta;
  a.rows = d->B * d->N_o * d->H * d->N;
  return launched(tri::launch_delta(a, (int)d->D, (hipStream_t)stream));
}

}  // extern "C"

namespace {

tri_attn_status bwd_impl(const tri_attn_dims* d, const tri_bf16* q, const tri_bf16* k,
                         const tri_bf16* v, const tri_bf16* bias, const float* mask,
                         const tri_bf16* d_o, const float* lse, const float* delta, tri_bf16* dk,
                         tri_bf16* dv, void* dq_partial, void* dbias_partial, int bf16_partials,
                         tri_attn_stream stream) {
  tri_attn_status st = check_dims(d);
  if (st != TRI_ATTN_OK) return st;
  if (!q || !k || !v || !bias || !d_o || !lse || !delta || !dk || !dv || !dq_partial ||
      !dbias_partial)
    return TRI_ATTN_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(bias) || !aligned16(d_o) ||
      !aligned16(lse) || !aligned16(delta) || !aligned16(dk) || !aligned16(dv) ||
      !aligned16(dq_partial) || !aligned16(dbias_partial) || (mask && !aligned16(mask)))
    return TRI_ATTN_ERR_ALIGN;
  tri::BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.bias = bias; a.mask = mask; a.d_o = d_o;
  a.lse = lse; a.delta = delta; a.dk = dk; a.dv = dv;
  a.dq_partial = dq_partial; a.dbias_partial = dbias_partial;
  a.bf16_partials = bf16_partials;
  a.B = (int)d->B; a.N_o = (int)d->N_o; a.H = (int)d->H; a.N = (int)d->N;
  a.n_key_tiles = (int)n_key_tiles(d);
  a.n_groups = (int)n_groups(d);
  a.scale = d->scale;
  const int64_t nblk = n_key_tiles(d) * d->H * n_groups(d) * d->B;
  if (nblk > 0x7fffffff) return TRI_ATTN_ERR_SHAPE;
  return launched(tri::launch_bwd(a, (int)d->D, (hipStream_t)stream));
}

tri_attn_status reduce_impl(const tri_attn_dims* d, const void* partial, tri_bf16* out, bool dq,
                            int bf16_partials, tri_attn_stream stream) {
  tri_attn_status st = check_dims(d);
  if (st != TRI_ATTN_OK) return st;
  if (!partial || !out) return TRI_ATTN_ERR_NULL;
  if (!aligned16(partial) || !aligned16(out)) return TRI_ATTN_ERR_ALIGN;
  tri::ReduceArgs a;
  a.partial = partial; a.out = out;
  a.elems = dq ? x_elems(d) : y_elems(d);
  a.n_partials = (int)(dq ? n_key_tiles(d) : n_groups(d));
  a.bf16_partials = bf16_partials;
  return launched(tri::launch_reduce(a, (hipStream_t)stream));
}

}  // namespace

extern "C" {

tri_attn_status tri_attn_bwd(const tri_attn_dims* d, const tri_bf16* q, const tri_bf16* k,
                             const tri_bf16* v, const tri_bf16* bias, const float* mask,
                             const tri_bf16* d_o, const float* lse, const float* delta,
                             tri_bf16* dk, tri_bf16* dv, float* dq_partial, float* dbias_partial,
                             tri_attn_stream stream) {
  return bwd_impl(d, q, k, v, bias, mask, d_o, lse, delta, dk, dv, dq_partial, dbias_partial, 0, stream);
}

tri_attn_status tri_attn_bwd_bf16p(const tri_attn_dims* d, const tri_bf16* q, const tri_bf16* k,
                                   const tri_bf16* v, const tri_bf16* bias, const float* mask,
                                   const tri_bf16* d_o, const float* lse, const float* delta,
                                   tri_bf16* dk, tri_bf16* dv, tri_bf16* dq_partial,
                                   tri_bf16* dbias_partial, tri_attn_stream stream) {
  return bwd_impl(d, q, k, v, bias, mask, d_o, lse, delta, dk, dv, dq_partial, dbias_partial, 1, stream);
}

tri_attn_status tri_attn_reduce_dq(const tri_attn_dims* d, const float* dq_partial,
                                   tri_bf16* dq, tri_attn_stream stream) {
  return reduce_impl(d, dq_partial, dq, true, 0, stream);
}

tri_attn_status tri_attn_reduce_dbias(const tri_attn_dims* d, const float* dbias_partial,
                                      tri_bf16* dbias, tri_attn_stream stream) {
  return reduce_impl(d, dbias_partial, dbias, false, 0, stream);
}

tri_attn_status tri_attn_reduce_dq_bf16p(const tri_attn_dims* d, const tri_bf16* dq_partial,
                                         tri_bf16* dq, tri_attn_stream stream) {
  return reduce_impl(d, dq_partial, dq, true, 1, stream);
}

tri_attn_status tri_attn_reduce_dbias_bf16p(const tri_attn_dims* d, const tri_bf16* dbias_partial,
                                            tri_bf16* dbias, tri_attn_stream stream) {
  return reduce_impl(d, dbias_partial, dbias, false, 1, stream);
}

}  // extern "C"
