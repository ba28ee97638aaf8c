// Argument blocks and launchers of the gfx950 kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tri {

// Tile constants of the key-tile backward.  J_K = ceil(N / kBwdKeyTile) dQ
// partials and L = ceil(N_o / G) dbias partials, G = bwd_group(D, N % 8 == 0)
// outer slices per workgroup: dK and dV of G slices stay in registers, so G is
// 4 for D = 32, 6 for D = 16 (half the accumulator registers per slice; 8
// spills; the register-staged path for odd N has no room and keeps 4) and 2 for
// D = 64 (twice the registers per slice).
constexpr int kBwdKeyTile = 128;
constexpr int bwd_group(int D, bool vec) { return D == 64 ? 2 : (D == 16 && vec) ? 6 : 4; }
// Width of the direct global->LDS loads of bias rows (N bf16 per row): 16 bytes when
// rows are 16-byte aligned, 4 bytes when they are 4-byte aligned, 0 = no direct loads
// (odd N: rows go through registers).  `vec` above means a nonzero width.
constexpr int bias_load_width(int N) { return N % 8 == 0 ? 16 : (N % 2 == 0 ? 4 : 0); }
// Queries per backward stage: 64, or 32 for D = 64 (its Q / dO stage buffers and
// dQ blocks per stage then match those of D = 32).
constexpr int bwd_query_tile(int D) { return D == 64 ? 32 : 64; }
constexpr int kFwdQueryTile = 128;
constexpr int kFwdKeyTile = 64;

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* bias;
  const float* mask;
  uint16_t* o;
  uint16_t* o_res;
  float* lse;
  int B, N_o, H, N;
  float scale;
};

struct DeltaArgs {
  const uint16_t* o;
  const uint16_t* o_res;
  const uint16_t* d_o;
  float* delta;
  int64_t rows;
};

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* bias;
  const float* mask;
  const uint16_t* d_o;
  const float* lse;
  const float* delta;
  uint16_t* dk;
  uint16_t* dv;
  void* dq_partial;      // FP32, or bf16 when bf16_partials
  void* dbias_partial;
  int B, N_o, H, N;
  int n_key_tiles;
  // outer groups g0 .. g0 + n_groups - 1 run in this launch (all groups, or one chunk of
  // the chunked backward); their dbias partials are planes 0 .. n_groups - 1 of
  // dbias_partial, and the dQ partials hold part_slices slices per example (N_o, or
  // n_groups * G), group g0 + i writing slices i * G ..
  int g0, n_groups, part_slices;
  float scale;
  int bf16_partials;     // 1: partials stored as bf16 (one RNE rounding each)
  int kv_only;           // 1: dK and dV only (dq_partial, dbias_partial unused)
};

struct ReduceArgs {
  const void* partial;   // FP32, or bf16 when bf16_partials
  uint16_t* out;
  int64_t elems;    // elements of one partial (== elements of the output)
  int n_partials;
  int bf16_partials;
};

// Segmented fixed-order sum of FP32 partials (the chunked backward's reductions).  Job j
// covers nseg segments of seg_len elements; element i of segment s is
//   x = (acc_in ? acc_in[s * seg_len + i] : first partial) + partials in ascending order,
// partial p at partial[p * pstride + s * sstride + i].  The sum goes to acc_out (FP32, dense
// [nseg, seg_len]) when acc_out is set, else rounded to bf16 into out[s * ostride + i].
struct SegReduceJob {
  const float* partial;
  int64_t pstride, sstride, seg_len, ostride;
  int n_partials, nseg;
  const float* acc_in;
  float* acc_out;
  uint16_t* out;
  int64_t blocks;        // workgroups of this job (set by the launcher)
  int vec;               // every length and stride a multiple of 4 (set by the launcher)
};
struct SegReduceArgs {
  SegReduceJob job[2];
  int njobs;
};

// Query-tile backward (dQ and dbias; bwd_q.hip).  A workgroup of nw waves owns 32 queries of
// one head, one range of kr = 32 * np * nw keys (wave w: keys 32 * np * w ..) and one outer
// group of gs consecutive slices, which it visits in ascending order: the dbias of its
// (query, key) block accumulates over the group in FP32 registers (one partial per group),
// and each slice's dQ over the range is complete in the workgroup (one partial per range).
constexpr int kBwdQQueries = 32;
// At most 384 keys per range (4 waves x 96 keys): two such workgroups (79 KB of LDS each) share
// a CU and their per-slice barriers fall at independent times; one 8-wave workgroup over 768
// keys (152 KB) measured 4% slower at N = 768 even with its single dQ partial.
constexpr int kBwdQMaxRange = 384;
constexpr int kDeviceCUs = 256;          // MI355X compute units
struct BwdQPlan {
  int nw, np;         // waves per workgroup, 32-key pairs per wave
  int n_ranges, kr;   // J key ranges of kr keys
  int n_groups, gs;   // L outer groups of gs slices
  int n_qt;           // 32-query tiles
};
inline BwdQPlan bwdq_plan(int64_t B, int64_t N_o, int64_t H, int64_t N) {
  BwdQPlan p;
  p.n_ranges = (int)((N + kBwdQMaxRange - 1) / kBwdQMaxRange);
  const int64_t need = (N + p.n_ranges - 1) / p.n_ranges;
  // smallest range that holds `need` keys: 128 (4 x 1), 256 (4 x 2), 384 (4 x 3)
  static const int opt[3][2] = {{4, 1}, {4, 2}, {4, 3}};
  int i = 0;
  while (i < 2 && 32 * opt[i][0] * opt[i][1] < need) ++i;
  p.nw = opt[i][0];
  p.np = opt[i][1];
  p.kr = 32 * p.nw * p.np;
  p.n_qt = (int)((N + kBwdQQueries - 1) / kBwdQQueries);
  // outer groups: fewest rounds of workgroups x slices per workgroup (plus a per-workgroup
  // start-up of about 1.5 slices); two workgroups per CU
  const int64_t slots = (int64_t)kDeviceCUs * 2;
  const int64_t units = B * H * p.n_ranges * p.n_qt;
  double best = 0;
  int bestL = 1;
  const int64_t maxL = N_o < 64 ? N_o : 64;
  for (int64_t L = 1; L <= maxL; ++L) {
    const int64_t gs = (N_o + L - 1) / L;
    const int64_t rounds = (units * L + slots - 1) / slots;
    const double cost = (double)rounds * ((double)gs + 1.5);
    if (L == 1 || cost < best) { best = cost; bestL = (int)L; }
  }
  p.gs = (int)((N_o + bestL - 1) / bestL);
  p.n_groups = (int)((N_o + p.gs - 1) / p.gs);
  return p;
}

struct BwdQArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* bias;
  const float* mask;
  const uint16_t* d_o;
  const float* lse;
  const float* delta;
  float* dq_partial;      // [n_ranges, B, N_o, H, N, D]
  float* dbias_partial;   // [n_groups, B, H, N, N]
  int B, N_o, H, N;
  BwdQPlan p;
  float scale;
};

hipError_t launch_fwd(const FwdArgs& a, int D, hipStream_t s);
hipError_t launch_bwdq(const BwdQArgs& a, int D, hipStream_t s);
hipError_t launch_delta(const DeltaArgs& a, int D, hipStream_t s);
hipError_t launch_bwd(const BwdArgs& a, int D, hipStream_t s);
hipError_t launch_reduce(const ReduceArgs& a, hipStream_t s);
hipError_t launch_seg_reduce(SegReduceArgs a, hipStream_t s);

}  // namespace tri
