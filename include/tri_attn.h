/*
 * tri_attn.h -- C ABI of the MI355X (gfx950) triangular-attention library.
 *
 * Operation: triangular attention with a pair bias shared by every outer slice,
 * as defined in "TurboPairFormer: Fast and Stable Protein Folding Model
 * Training with an Optimized Triangle Attention Kernel" (notation table,
 * Table 1; Figure 1(a); worked example, Figure 6).  For example b, outer slice
 * o and head h, with N x D matrices Q, K, V taken from the pairs (o, .):
 *
 *   s[q,k]  = scale * <Q[q], K[k]> + bias[b,h,q,k] + mask[b,o,k]
 *   P[q,:]  = softmax_k(s[q,:]),  O[q] = sum_k P[q,k] V[k]
 *
 * The bias is the same for every o; scale multiplies the dot product only.
 * The backward produces dQ, dK, dV and dbias = sum_o dS_o (three reduction
 * axes: keys, queries, outer slices; Figure 1(a)).
 *
 * Data layout (all tensors dense, row-major, no strides):
 *   Q, K, V, O, E, dO, dQ, dK, dV  [B, N_o, H, N, D]   bf16 (bit patterns)
 *   bias, dbias                    [B, H, N, N]        bf16, indexed [query, key]
 *   mask                           [B, N_o, N]         fp32 additive (0 keeps a key,
 *                                                      -1e9 removes it), or NULL
 *   lse, delta                     [B, N_o, H, N]      fp32 (lse in natural log)
 *   dq_partial                     [J_K, B, N_o, H, N, D] fp32
 *   dbias_partial                  [L,   B, H, N, N]      fp32
 * with J_K = ceil(N / key tile) and L = ceil(N_o / outer group) as reported by
 * tri_attn_workspace() (the bf16-partial calls: tri_attn_workspace_single_pass()).
 *
 * Ownership: every pointer is a DEVICE pointer owned by the caller.  The
 * library allocates nothing, frees nothing and never synchronises; each call
 * only enqueues kernels on `stream` and returns.  Inputs may alias each other
 * read-only; outputs must not alias any other argument.  The library holds no
 * mutable global state, so calls on distinct buffers may run concurrently.
 *
 * Errors: arguments are checked on the host before any launch.  A null
 * required pointer gives TRI_ATTN_ERR_NULL, a bad dimension or scale
 * TRI_ATTN_ERR_SHAPE, an unsupported head dimension TRI_ATTN_ERR_UNSUPPORTED,
 * a pointer not 16-byte aligned TRI_ATTN_ERR_ALIGN, a workspace too small for
 * the chunked backward TRI_ATTN_ERR_WORKSPACE, and a failed launch
 * TRI_ATTN_ERR_LAUNCH; in every error case nothing has been enqueued except
 * for TRI_ATTN_ERR_LAUNCH.  Device faults surface at the caller's next
 * synchronisation, as for any HIP call.  NaN and Inf inputs propagate; bias
 * entries must be finite (the forward adds the bias with an exact identity
 * matrix product, where an infinite entry also turns the other scores of its
 * 16 x 16 score block into NaN), so keys are removed through the mask.
 *
 * Determinism: for fixed dimensions and build, every output is bitwise
 * reproducible across calls on the same GPU model.  No float atomics are
 * used; every sum has a fixed order.
 */
#ifndef TRI_ATTN_H
#define TRI_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TRI_ATTN_OK = 0,
  TRI_ATTN_ERR_NULL = 1,
  TRI_ATTN_ERR_SHAPE = 2,
  TRI_ATTN_ERR_UNSUPPORTED = 3,
  TRI_ATTN_ERR_ALIGN = 4,
  TRI_ATTN_ERR_LAUNCH = 5,
  TRI_ATTN_ERR_WORKSPACE = 6
} tri_attn_status;

/* Problem dimensions.  D must be 16, 32 or 64 (the method is measured at 16 and 32;
 * 64 is a wider head run by the same kernels); 1 <= B, N_o, H <= 65535 with
 * B * N_o <= 65535; 1 <= N <= 32767; B * N_o * H * N <= 2^25; scale finite with
 * |scale| >= 2^-64 (the backward divides the log-sum-exp by it in FP32). */
typedef struct {
  int64_t B, N_o, H, N, D;
  float scale;
} tri_attn_dims;

typedef uint16_t tri_bf16; /* bfloat16 bit pattern */

/* Opaque HIP stream (hipStream_t); NULL is the default stream. */
typedef void* tri_attn_stream;

/*
 * Forward (Figure 6 steps 1-4; online softmax over key tiles).
 * Writes O = bf16(O32) with O32 the FP32 normalised output, the output
 * residual E = bf16(O32 - O) when o_res is not NULL (the saved BF16
 * approximation of the output-rounding residual: Abstract, Figure 7(b)), and
 * lse = max_k s + log(sum_k exp(s - max)) per row.  O is bitwise the same
 * whether or not o_res is given.
 */
tri_attn_status tri_attn_fwd(const tri_attn_dims* d,
                             const tri_bf16* q, const tri_bf16* k, const tri_bf16* v,
                             const tri_bf16* bias, const float* mask /* may be NULL */,
                             tri_bf16* o, tri_bf16* o_res /* may be NULL */, float* lse,
                             tri_attn_stream stream);

/*
 * Softmax correction (Figure 7(b)): delta[row] = sum_d dO[row,d] * (O[row,d] + E[row,d])
 * in FP32 with a fixed order; with o_res == NULL it is sum_d dO * O (no compensation).
 */
tri_attn_status tri_attn_bwd_delta(const tri_attn_dims* d, const tri_bf16* o,
                                   const tri_bf16* o_res /* may be NULL */,
                                   const tri_bf16* d_o, float* delta,
                                   tri_attn_stream stream);

/*
 * Main backward (Figure 2).  dK and dV (scaled by `scale` for dK) are finished here;
 * dQ (already scaled) leaves as J_K FP32 partials and dbias as L FP32 partials, each
 * element written by exactly one workgroup (Figure 11(a), materialised partials), with
 * J_K and L as reported by tri_attn_workspace.
 *   D = 64, and D = 16 with N <= 640: the single-pass key-tile kernel (Figure 7(c)):
 *     one workgroup owns one 128-key tile of one head for one outer group of G slices
 *     and visits every query tile, evaluating S, P, dP and dS once; one dQ partial per
 *     key tile, one dbias partial per outer group.
 *   D = 32, and D = 16 with N > 640: two kernels.  The key-tile kernel forms dK and dV
 *     only; a query-tile kernel then evaluates S, P, dP and dS again per (32 queries,
 *     range of up to 384 keys, outer group of up to N_o / L slices), sums each slice's
 *     dQ over the key range and the dbias of its (query, key) block over the whole outer
 *     group inside the workgroup: J_K = ceil(N / 384) dQ partials and L <= 64 dbias
 *     partials (L = 8 at N = 768), a small fraction of the single-pass kernel's partial
 *     bytes.
 * Either way every sum has a fixed order, so results are bitwise reproducible.
 */
tri_attn_status tri_attn_bwd(const tri_attn_dims* d,
                             const tri_bf16* q, const tri_bf16* k, const tri_bf16* v,
                             const tri_bf16* bias, const float* mask /* may be NULL */,
                             const tri_bf16* d_o, const float* lse, const float* delta,
                             tri_bf16* dk, tri_bf16* dv,
                             float* dq_partial, float* dbias_partial,
                             tri_attn_stream stream);

/* dQ = bf16(sum_{t=0..J_K-1} dq_partial[t]), summed in ascending t in FP32 (Figure 7(d)). */
tri_attn_status tri_attn_reduce_dq(const tri_attn_dims* d, const float* dq_partial,
                                   tri_bf16* dq, tri_attn_stream stream);

/* dbias = bf16(sum_{l=0..L-1} dbias_partial[l]), summed in ascending l in FP32 (Figure 7(d)). */
tri_attn_status tri_attn_reduce_dbias(const tri_attn_dims* d, const float* dbias_partial,
                                      tri_bf16* dbias, tri_attn_stream stream);

/*
 * BF16-partial variant (the pages size the partials in BF16, Table 2): the three calls
 * of the single-pass key-tile kernel (at every D) with the dQ and dbias partials stored
 * as bf16 — each partial element is the FP32 value rounded once to bf16 (round to
 * nearest even) before it is stored; the reductions add the partials in FP32 in a fixed
 * order.  Half the single-pass kernel's partial bytes, at the cost of one bf16 rounding
 * per partial.  Buffers hold the element counts of tri_attn_workspace_single_pass, 2
 * bytes each, 16-byte aligned.  The FP32 calls above remain the reference path.  Errors
 * as for those calls.
 */
tri_attn_status tri_attn_bwd_bf16p(const tri_attn_dims* d,
                                   const tri_bf16* q, const tri_bf16* k, const tri_bf16* v,
                                   const tri_bf16* bias, const float* mask /* may be NULL */,
                                   const tri_bf16* d_o, const float* lse, const float* delta,
                                   tri_bf16* dk, tri_bf16* dv,
                                   tri_bf16* dq_partial, tri_bf16* dbias_partial,
                                   tri_attn_stream stream);
tri_attn_status tri_attn_reduce_dq_bf16p(const tri_attn_dims* d, const tri_bf16* dq_partial,
                                         tri_bf16* dq, tri_attn_stream stream);
tri_attn_status tri_attn_reduce_dbias_bf16p(const tri_attn_dims* d, const tri_bf16* dbias_partial,
                                            tri_bf16* dbias, tri_attn_stream stream);

/*
 * Chunked backward with bounded partial memory (Figure 7(d): the pair-bias partial
 * buffers are reused once consumed; Table 2, column W_bias,res), on the single-pass
 * key-tile kernel at every D.  Does what that kernel and the two reductions do together,
 * over chunks of C consecutive outer groups (outer groups, key tiles and partial counts
 * of tri_attn_workspace_single_pass): the main backward of a chunk writes the chunk's dQ
 * and dbias partials into `workspace`, then one reduction kernel sums the chunk's dQ
 * partials into its rows of dq and adds its dbias partials, in ascending group order, to
 * an FP32 running sum carried from chunk to chunk (rounded to bf16 into dbias after the
 * last chunk); the next chunk reuses the same buffers.  Every sum keeps the order of the
 * unchunked single-pass kernel and reductions, so results are bitwise the same for every
 * chunk size, and, for D = 16 and 64 (where tri_attn_bwd is that kernel), bitwise those
 * of the three calls; for D = 32 they equal the three calls up to summation order.
 *
 * C is the largest number of outer groups whose buffers fit in workspace_bytes (all
 * groups: a single chunk).  tri_attn_bwd_chunked_workspace gives the bytes a chunk of
 * groups_per_chunk groups needs (clamped to 1..L) and the clamped count.  Buffers of one
 * chunk: dQ partials J_K * B * min(C * G, N_o) * H * N * D FP32, dbias partials
 * C * B * H * N * N FP32, and with more than one chunk the running sum B * H * N * N FP32
 * (each rounded up to 256 bytes).
 *
 * Inputs and dq, dk, dv, dbias as for the three calls; `workspace` is caller-owned device
 * memory, 16-byte aligned, whose contents on entry do not matter and which no other call
 * may use until this call's kernels have finished.  Errors as for tri_attn_bwd, plus
 * TRI_ATTN_ERR_NULL for a null workspace and TRI_ATTN_ERR_WORKSPACE when not even one
 * outer group's buffers fit in workspace_bytes.
 */
tri_attn_status tri_attn_bwd_chunked_workspace(const tri_attn_dims* d, int64_t groups_per_chunk,
                                               int64_t* workspace_bytes, int64_t* groups_used);
tri_attn_status tri_attn_bwd_chunked(const tri_attn_dims* d,
                                     const tri_bf16* q, const tri_bf16* k, const tri_bf16* v,
                                     const tri_bf16* bias, const float* mask /* may be NULL */,
                                     const tri_bf16* d_o, const float* lse, const float* delta,
                                     tri_bf16* dq, tri_bf16* dk, tri_bf16* dv, tri_bf16* dbias,
                                     void* workspace, int64_t workspace_bytes,
                                     tri_attn_stream stream);

/*
 * Allocation-free variant of tri_attn_bwd_chunked, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments without the workspace: the chunk buffers live in a
 * static device array of tri_attn_noalloc_scratch_bytes() bytes (128 MiB) that the
 * library holds on every GPU it runs on until the process ends; its address is looked up
 * once per device, on the first call on that device.  The call allocates and frees
 * nothing.  Results are bitwise those of tri_attn_bwd_chunked (and of the unchunked
 * calls).  Shapes for which not even one outer group's buffers fit in the scratch array
 * (e.g. N = 4096, H = 4, where the FP32 running dbias sum alone is 256 MiB) return
 * TRI_ATTN_ERR_WORKSPACE before anything is enqueued.  Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (concurrent streams, or host threads
 * enqueueing at once) race on it and give undefined results; serialise them.  The array
 * needs no clearing: each chunk writes every element it later reads.
 */
tri_attn_status tri_attn_bwd_chunked_noalloc(const tri_attn_dims* d,
                                             const tri_bf16* q, const tri_bf16* k, const tri_bf16* v,
                                             const tri_bf16* bias, const float* mask /* may be NULL */,
                                             const tri_bf16* d_o, const float* lse, const float* delta,
                                             tri_bf16* dq, tri_bf16* dk, tri_bf16* dv, tri_bf16* dbias,
                                             tri_attn_stream stream);
/* Size in bytes of the scratch array behind tri_attn_bwd_chunked_noalloc. */
int64_t tri_attn_noalloc_scratch_bytes(void);

/*
 * Partial-buffer sizes of tri_attn_bwd for these dimensions (elements, FP32), the number
 * of dQ partials J_K and of dbias partials L, and the key-tile / outer-group sizes behind
 * them.  Single-pass kernel (D = 64; D = 16 with N <= 640): key tile 128; group G = 6 for
 * D = 16 with N even, 4 with N odd, 2 for D = 64.  Two kernels (D = 32; D = 16 with
 * N > 640): the key range of the query-tile kernel (128, 256 or 384 keys;
 * J_K = ceil(N / 384) ranges) and its outer group (L <= 64 groups).  Any output pointer may be NULL.  Host-only arithmetic;
 * no device access.
 */
tri_attn_status tri_attn_workspace(const tri_attn_dims* d, int64_t* dq_partial_elems,
                                   int64_t* dbias_partial_elems, int64_t* j_k, int64_t* l,
                                   int64_t* key_tile, int64_t* outer_group);

/*
 * The same sizes for the single-pass key-tile kernel that tri_attn_bwd_bf16p (and its two
 * reductions) and the chunked backward use at every D: key tile 128, outer group G = 4 for
 * D = 32, otherwise as above.
 */
tri_attn_status tri_attn_workspace_single_pass(const tri_attn_dims* d, int64_t* dq_partial_elems,
                                               int64_t* dbias_partial_elems, int64_t* j_k, int64_t* l,
                                               int64_t* key_tile, int64_t* outer_group);

/* Human-readable name of a status code (static string). */
const char* tri_attn_status_string(int status);   /* any int; unknown codes -> "unknown status" */

/* Library version, e.g. "0.1.0". */
const char* tri_attn_version(void);

#ifdef __cplusplus
}
#endif
#endif /* TRI_ATTN_H */
