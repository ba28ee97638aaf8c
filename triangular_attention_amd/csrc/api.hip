// C ABI of the triangular-attention library: argument validation and launch.
// See include/tri_attn.h for the contract of each entry point.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

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

// The default FP32 backward runs as two kernels (the key-tile kernel for dK, dV and the
// query-tile kernel for dQ, dbias) for D = 32, and for D = 16 past N = 640: below that the
// single-pass kernel's partials are small enough that the second evaluation of the scores
// does not pay (D = 16, measured at N = 384 / 640 / 768: 0.291 / 1.171 / 1.913 ms per step
// single-pass against 0.300 / 1.171 / 1.788 ms with two kernels).  D = 64, the bf16-partial
// variant and the chunked backward use the single-pass key-tile kernel.  Partial counts of
// each design:
bool two_kernel(const tri_attn_dims* d) { return d->D == 32 || (d->D == 16 && d->N > 640); }
tri::BwdQPlan q_plan(const tri_attn_dims* d) { return tri::bwdq_plan(d->B, d->N_o, d->H, d->N); }
int64_t dq_parts(const tri_attn_dims* d) { return two_kernel(d) ? q_plan(d).n_ranges : n_key_tiles(d); }
int64_t db_parts(const tri_attn_dims* d) { return two_kernel(d) ? q_plan(d).n_groups : n_groups(d); }

tri_attn_status launched(hipError_t e) { return e == hipSuccess ? TRI_ATTN_OK : TRI_ATTN_ERR_LAUNCH; }

}  // namespace

extern "C" {

const char* tri_attn_status_string(int status) {
  // an int, not the enum: any code a caller passes is a defined value here
  switch (status) {
    case TRI_ATTN_OK: return "ok";
    case TRI_ATTN_ERR_NULL: return "null pointer argument";
    case TRI_ATTN_ERR_SHAPE: return "invalid dimensions or scale";
    case TRI_ATTN_ERR_UNSUPPORTED: return "unsupported head dimension (D must be 16, 32 or 64)";
    case TRI_ATTN_ERR_ALIGN: return "pointer not 16-byte aligned";
    case TRI_ATTN_ERR_LAUNCH: return "kernel launch failed";
    case TRI_ATTN_ERR_WORKSPACE: return "workspace too small for the partials of one outer group";
  }
  return "unknown status";
}

const char* tri_attn_version(void) { return "0.1.0"; }

tri_attn_status tri_attn_workspace(const tri_attn_dims* d, int64_t* dq_partial_elems,
                                   int64_t* dbias_partial_elems, int64_t* j_k, int64_t* l,
                                   int64_t* key_tile, int64_t* outer_group) {
  tri_attn_status st = check_dims(d);
  if (st != TRI_ATTN_OK) return st;
  const bool two = two_kernel(d);
  const tri::BwdQPlan p = two ? q_plan(d) : tri::BwdQPlan();
  if (dq_partial_elems) *dq_partial_elems = dq_parts(d) * x_elems(d);
  if (dbias_partial_elems) *dbias_partial_elems = db_parts(d) * y_elems(d);
  if (j_k) *j_k = dq_parts(d);
  if (l) *l = db_parts(d);
  if (key_tile) *key_tile = two ? p.kr : tri::kBwdKeyTile;
  if (outer_group) *outer_group = two ? p.gs : group_size(d);
  return TRI_ATTN_OK;
}

tri_attn_status tri_attn_workspace_single_pass(const tri_attn_dims* d, int64_t* dq_partial_elems,
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

// Arguments of the backward kernel over every outer group (no partial buffers yet).
tri::BwdArgs bwd_args(const tri_attn_dims* d, const tri_bf16* q, const tri_bf16* k, const tri_bf16* v,
                      const tri_bf16* bias, const float* mask, const tri_bf16* d_o, const float* lse,
                      const float* delta, tri_bf16* dk, tri_bf16* dv) {
  tri::BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.bias = bias; a.mask = mask; a.d_o = d_o;
  a.lse = lse; a.delta = delta; a.dk = dk; a.dv = dv;
  a.dq_partial = nullptr; a.dbias_partial = nullptr;
  a.bf16_partials = 0;
  a.kv_only = 0;
  a.B = (int)d->B; a.N_o = (int)d->N_o; a.H = (int)d->H; a.N = (int)d->N;
  a.n_key_tiles = (int)n_key_tiles(d);
  a.g0 = 0;
  a.n_groups = (int)n_groups(d);
  a.part_slices = (int)d->N_o;
  a.scale = d->scale;
  return a;
}

tri_attn_status check_bwd_inputs(const tri_attn_dims* d, const tri_bf16* q, const tri_bf16* k,
                                 const tri_bf16* v, const tri_bf16* bias, const float* mask,
                                 const tri_bf16* d_o, const float* lse, const float* delta) {
  if (!q || !k || !v || !bias || !d_o || !lse || !delta) return TRI_ATTN_ERR_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(bias) || !aligned16(d_o) ||
      !aligned16(lse) || !aligned16(delta) || (mask && !aligned16(mask)))
    return TRI_ATTN_ERR_ALIGN;
  // a launch has 8 * ceil(B * L * H / 8) * J_K workgroups (32-bit grid), the query-tile
  // kernel 8 * ceil(B * H * J * L / 8) * ceil(N / 32)
  if (n_key_tiles(d) * (d->H * n_groups(d) * d->B + 7) > 0x7fffffff) return TRI_ATTN_ERR_SHAPE;
  if (two_kernel(d)) {
    const tri::BwdQPlan p = q_plan(d);
    if ((d->B * d->H * p.n_ranges * p.n_groups + 7) * p.n_qt > 0x7fffffff) return TRI_ATTN_ERR_SHAPE;
  }
  return TRI_ATTN_OK;
}

tri_attn_status bwd_impl(const tri_attn_dims* d, const tri_bf16* q, const tri_bf16* k,
                         const tri_bf16* v, const tri_bf16* bias, const float* mask,
                         const tri_bf16* d_o, const float* lse, const float* delta, tri_bf16* dk,
                         tri_bf16* dv, void* dq_partial, void* dbias_partial, int bf16_partials,
                         tri_attn_stream stream) {
  tri_attn_status st = check_dims(d);
  if (st != TRI_ATTN_OK) return st;
  if (!dk || !dv || !dq_partial || !dbias_partial) return TRI_ATTN_ERR_NULL;
  st = check_bwd_inputs(d, q, k, v, bias, mask, d_o, lse, delta);
  if (st != TRI_ATTN_OK) return st;
  if (!aligned16(dk) || !aligned16(dv) || !aligned16(dq_partial) || !aligned16(dbias_partial))
    return TRI_ATTN_ERR_ALIGN;
  tri::BwdArgs a = bwd_args(d, q, k, v, bias, mask, d_o, lse, delta, dk, dv);
  if (!bf16_partials && two_kernel(d)) {
    // dK, dV from the key-tile kernel; dQ and dbias partials from the query-tile kernel
    a.kv_only = 1;
    hipError_t e = tri::launch_bwd(a, (int)d->D, (hipStream_t)stream);
    if (e != hipSuccess) return TRI_ATTN_ERR_LAUNCH;
    tri::BwdQArgs qa;
    qa.q = q; qa.k = k; qa.v = v; qa.bias = bias; qa.mask = mask; qa.d_o = d_o;
    qa.lse = lse; qa.delta = delta;
    qa.dq_partial = static_cast<float*>(dq_partial);
    qa.dbias_partial = static_cast<float*>(dbias_partial);
    qa.B = (int)d->B; qa.N_o = (int)d->N_o; qa.H = (int)d->H; qa.N = (int)d->N;
    qa.p = q_plan(d);
    qa.scale = d->scale;
    return launched(tri::launch_bwdq(qa, (int)d->D, (hipStream_t)stream));
  }
  a.dq_partial = dq_partial; a.dbias_partial = dbias_partial;
  a.bf16_partials = bf16_partials;
  return launched(tri::launch_bwd(a, (int)d->D, (hipStream_t)stream));
}

int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

// Buffers of the chunked backward for chunks of C outer groups, as byte offsets into the
// workspace: the chunk's dQ partials [J_K, B, PS, H, N, D] (PS = min(C * G, N_o) slices per
// example), its dbias partials [C, B, H, N, N], and the FP32 running dbias sum [B, H, N, N]
// (only with more than one chunk).
struct ChunkPlan {
  int64_t C = 0, n_chunks = 0, part_slices = 0;
  int64_t dq_off = 0, db_off = 0, acc_off = 0, bytes = 0;
};

ChunkPlan chunk_plan(const tri_attn_dims* d, int64_t C) {
  const int64_t L = n_groups(d), G = group_size(d);
  ChunkPlan p;
  p.C = std::max<int64_t>(1, std::min(C, L));
  p.n_chunks = (L + p.C - 1) / p.C;
  p.part_slices = std::min(p.C * G, d->N_o);
  const int64_t dq = 4 * n_key_tiles(d) * d->B * p.part_slices * d->H * d->N * d->D;
  const int64_t db = 4 * p.C * y_elems(d);
  const int64_t acc = p.n_chunks > 1 ? 4 * y_elems(d) : 0;
  p.dq_off = 0;
  p.db_off = align256(dq);
  p.acc_off = p.db_off + align256(db);
  p.bytes = p.acc_off + align256(acc);
  return p;
}

// The largest chunk whose buffers fit in `bytes` (C = 0: not even one outer group fits).
ChunkPlan chunk_plan_for(const tri_attn_dims* d, int64_t bytes) {
  for (int64_t C = n_groups(d); C >= 1; --C) {
    const ChunkPlan p = chunk_plan(d, C);
    if (p.bytes <= bytes) return p;
  }
  return ChunkPlan();
}

// Backward over chunks of outer groups (see tri_attn_bwd_chunked): per chunk, the main
// backward writes the chunk's partials, then one launch of the segmented reduction forms the
// chunk's dQ rows and carries the dbias sum on; the next chunk reuses the buffers.
tri_attn_status chunked_impl(const tri_attn_dims* d, const tri_bf16* q, const tri_bf16* k,
                             const tri_bf16* v, const tri_bf16* bias, const float* mask,
                             const tri_bf16* d_o, const float* lse, const float* delta, tri_bf16* dq,
                             tri_bf16* dk, tri_bf16* dv, tri_bf16* dbias, void* workspace,
                             int64_t workspace_bytes, hipStream_t stream) {
  tri_attn_status st = check_dims(d);
  if (st != TRI_ATTN_OK) return st;
  if (!dq || !dk || !dv || !dbias || !workspace) return TRI_ATTN_ERR_NULL;
  st = check_bwd_inputs(d, q, k, v, bias, mask, d_o, lse, delta);
  if (st != TRI_ATTN_OK) return st;
  if (!aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(dbias) || !aligned16(workspace))
    return TRI_ATTN_ERR_ALIGN;
  const ChunkPlan plan = chunk_plan_for(d, workspace_bytes);
  if (plan.C == 0) return TRI_ATTN_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  float* dqp = reinterpret_cast<float*>(ws + plan.dq_off);
  float* dbp = reinterpret_cast<float*>(ws + plan.db_off);
  float* acc = reinterpret_cast<float*>(ws + plan.acc_off);
  tri::BwdArgs a = bwd_args(d, q, k, v, bias, mask, d_o, lse, delta, dk, dv);
  a.dq_partial = dqp;
  a.dbias_partial = dbp;
  a.part_slices = (int)plan.part_slices;
  const int64_t L = n_groups(d), G = group_size(d), PS = plan.part_slices;
  const int64_t slice = d->H * d->N * d->D;     // elements of one outer slice of Q
  for (int64_t c = 0; c < plan.n_chunks; ++c) {
    const int64_t g0 = c * plan.C, ng = std::min(plan.C, L - g0);
    a.g0 = (int)g0;
    a.n_groups = (int)ng;
    hipError_t e = tri::launch_bwd(a, (int)d->D, stream);
    if (e != hipSuccess) return TRI_ATTN_ERR_LAUNCH;
    const int64_t s0 = g0 * G, ns = std::min(d->N_o, (g0 + ng) * G) - s0;
    tri::SegReduceArgs r;
    r.njobs = 2;
    // the dbias job first: its blocks each add a chunk's worth of partials and run longest,
    // so they start first and the short dQ blocks fill in behind them
    tri::SegReduceJob& jq = r.job[1];     // the chunk's dQ rows: sum over key tiles
    jq.partial = dqp;
    jq.pstride = d->B * PS * slice;
    jq.sstride = PS * slice;
    jq.seg_len = ns * slice;
    jq.nseg = (int)d->B;
    jq.n_partials = (int)n_key_tiles(d);
    jq.acc_in = nullptr;
    jq.acc_out = nullptr;
    jq.out = dq + s0 * slice;
    jq.ostride = d->N_o * slice;
    tri::SegReduceJob& jb = r.job[0];     // dbias: the running sum over outer groups
    jb.partial = dbp;
    jb.pstride = y_elems(d);
    jb.sstride = 0;
    jb.seg_len = y_elems(d);
    jb.nseg = 1;
    jb.n_partials = (int)ng;
    jb.acc_in = c > 0 ? acc : nullptr;
    jb.acc_out = c + 1 < plan.n_chunks ? acc : nullptr;
    jb.out = dbias;
    jb.ostride = 0;
    e = tri::launch_seg_reduce(r, stream);
    if (e != hipSuccess) return TRI_ATTN_ERR_LAUNCH;
  }
  return TRI_ATTN_OK;
}

// Device memory of the allocation-free backward: one array per GPU, held by the loaded code
// object until the process ends.  Host code never uses the array's name as an address (it is
// a host-side stand-in); the device address comes from hipGetSymbolAddress, once per device.
constexpr int64_t kScratchBytes = int64_t(128) << 20;
constexpr int kMaxDevices = 64;
static __device__ __attribute__((used)) __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch address on the current device (looked up on the first call on that device).
tri_attn_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TRI_ATTN_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TRI_ATTN_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TRI_ATTN_OK;
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
  // FP32 partials: the default design's counts; bf16 partials: the single-pass kernel's
  if (bf16_partials) a.n_partials = (int)(dq ? n_key_tiles(d) : n_groups(d));
  else a.n_partials = (int)(dq ? dq_parts(d) : db_parts(d));
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

tri_attn_status tri_attn_bwd_chunked_workspace(const tri_attn_dims* d, int64_t groups_per_chunk,
                                               int64_t* workspace_bytes, int64_t* groups_used) {
  tri_attn_status st = check_dims(d);
  if (st != TRI_ATTN_OK) return st;
  if (groups_per_chunk < 1) return TRI_ATTN_ERR_SHAPE;
  const ChunkPlan p = chunk_plan(d, groups_per_chunk);
  if (workspace_bytes) *workspace_bytes = p.bytes;
  if (groups_used) *groups_used = p.C;
  return TRI_ATTN_OK;
}

tri_attn_status tri_attn_bwd_chunked(const tri_attn_dims* d, const tri_bf16* q, const tri_bf16* k,
                                     const tri_bf16* v, const tri_bf16* bias, const float* mask,
                                     const tri_bf16* d_o, const float* lse, const float* delta,
                                     tri_bf16* dq, tri_bf16* dk, tri_bf16* dv, tri_bf16* dbias,
                                     void* workspace, int64_t workspace_bytes, tri_attn_stream stream) {
  return chunked_impl(d, q, k, v, bias, mask, d_o, lse, delta, dq, dk, dv, dbias, workspace, workspace_bytes,
                      (hipStream_t)stream);
}

tri_attn_status tri_attn_bwd_chunked_noalloc(const tri_attn_dims* d, const tri_bf16* q, const tri_bf16* k,
                                             const tri_bf16* v, const tri_bf16* bias, const float* mask,
                                             const tri_bf16* d_o, const float* lse, const float* delta,
                                             tri_bf16* dq, tri_bf16* dk, tri_bf16* dv, tri_bf16* dbias,
                                             tri_attn_stream stream) {
  // validate everything before the scratch lookup touches the device
  tri_attn_status st = check_dims(d);
  if (st != TRI_ATTN_OK) return st;
  if (!dq || !dk || !dv || !dbias) return TRI_ATTN_ERR_NULL;
  st = check_bwd_inputs(d, q, k, v, bias, mask, d_o, lse, delta);
  if (st != TRI_ATTN_OK) return st;
  if (!aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(dbias)) return TRI_ATTN_ERR_ALIGN;
  if (chunk_plan(d, 1).bytes > kScratchBytes) return TRI_ATTN_ERR_WORKSPACE;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != TRI_ATTN_OK) return st;
  return chunked_impl(d, q, k, v, bias, mask, d_o, lse, delta, dq, dk, dv, dbias, ws, kScratchBytes,
                      (hipStream_t)stream);
}

int64_t tri_attn_noalloc_scratch_bytes(void) { return kScratchBytes; }

}  // extern "C"
