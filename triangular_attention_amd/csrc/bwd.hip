// Key-tile-parallel backward of triangular attention on gfx950.
//
// Method: TurboPairFormer, Figure 2 and Figure 7(c): a workgroup owns one key
// tile of one head for one outer group of G slices and visits every query
// tile; for each query tile and slice it evaluates S, P, dP and dS exactly
// once.  dK and dV stay in FP32 registers for the whole kernel.  The score
// gradient goes through LDS to form one dQ partial per key tile, and the G
// slices' FP32 score gradients are added in a fixed order (slice 0, 1, ...)
// into one dbias partial per outer group.  Every partial element has exactly
// one writer (Figure 11(a), materialised partials); the reduction kernels sum
// them in ascending index order.
//
// Orientation: S = Q K^T with queries as MFMA rows and keys as columns; each
// wave owns 16 keys.  In this layout the bf16 P and dS blocks are directly the
// B operands of dV^T = dO^T P and dK^T = Q^T dS (contraction over queries);
// the dO^T and Q^T operands come from the row-major LDS tiles through the
// transposing LDS read.  dS is stored key-major in LDS and read back, also
// transposed, as the operand of dQ^T = K^T dS^T.  -lse/scale and -delta enter
// as the accumulator inputs of the S and dP products, so the exponent costs
// one FMA per score.
//
// Pipeline: one barrier per stage (query tile j, slice g); the dQ product of
// stage i runs in stage i+1, in the same straight-line block as that stage's
// score work, so every barrier interval mixes VALU-heavy and MFMA-heavy work.
// With N even the Q, dO and bias tiles go from memory straight into LDS:
// three stage buffers, loaded by two alternating sets of waves, so that each
// load has two stages to land and a wave waits on memory at every other
// barrier only.  With N odd the stages go through registers, double-buffered.
// Global reads are raw buffer loads with per-slice extents: rows past N read
// as zero, which makes their probabilities irrelevant (dO, Q and K are zero
// there) without per-load bounds checks.
//
// LDS layouts (bank conflicts of each access shape were measured on gfx950
// with probe kernels replaying the exact lane addresses).  D = 32: Q, dO and K
// tiles are unpadded 64-byte rows whose four 16-byte chunks are permuted by an
// XOR with a row-dependent value (Q, dO: row bits 3-4; K: row bits 2-3).  The
// transposing reads are conflict-free; the score-product row reads of Q, dO
// and K take two passes.  Swapping the two swizzles removes those conflicts
// but needs more address registers than the kernel has, and measured slower.
// D = 64 (outer group 2, 32-query stages): 128-byte rows whose eight 16-byte
// chunks are permuted by an XOR with row bits (Q/dO: bits 1, 3, 4; K/V: bits 1, 2,
// 3) so that both read shapes are conflict-free.  The dS^T tile is written 16
// bytes per lane and read transposed with a pitch of the stage's queries + 8;
// the bias tile has 256-byte rows whose 8-byte units are permuted by an XOR with
// the row's low bits (conflict-free transposing reads).
#include "common.h"
#include "kernels.h"
#include "bwd_layout.h"

namespace tri {

// LD: how the bias tile reaches LDS.  16: 16-byte direct loads (N % 8 == 0); 4: 4-byte
// direct loads, one per 256-byte bias row (N even); 0: through registers (N odd).
// BP: dQ and dbias partials stored as bf16 (one RNE rounding each) instead of FP32.
// KV: dK and dV only (no dQ product, no dbias tile, no partials); the query-tile
// kernel of bwd_q.hip computes dQ and dbias.
// TK: keys per workgroup, 16 per wave: 128 (8 waves, one workgroup per CU), or 64 for the
// dK/dV-only variant with D = 32 on the 16-byte load path.  That variant also takes outer
// groups of 2 slices and 32-query stages: without the dQ and dbias work it then needs 127
// VGPRs and 37 KB of LDS, so four workgroups (16 waves) share a CU and their stage barriers
// fall at independent times (at N = 768: 1.15 -> 0.87 ms against 8-wave workgroups).
template <int D, bool MASK, int LD, bool BP, int TK, bool KV>
__global__ __launch_bounds__(TK * 4, TK == 64 ? 3 : 1) void bwd_kernel(BwdArgs a) {
  constexpr bool VEC = LD != 0;   // direct global->LDS path
  constexpr int NW = TK / 16;     // waves; wave w owns keys 16w..16w+15 of the tile
  constexpr int NT = NW * 64;
  // 64-key tiles (dK/dV only): 32-query stages, 64 for D = 16 (its padded 48-byte Q rows
  // make whole-wave pieces only in 64-row tiles)
  constexpr int TQ = TK == 64 ? (D == 16 ? 64 : 32) : bwd_query_tile(D), G = TK == 64 ? 2 : bwd_group(D, VEC);
  constexpr int NQB = TQ / 16;    // 16-query blocks of a stage
  constexpr int NST = TQ / 32;    // 32-query halves of a stage (dV / dK contraction steps)
  static_assert(TQ % 32 == 0, "query tile must be whole 32-query halves");
  static_assert(G >= 2 && G % 2 == 0, "stage parity must repeat with every query tile");
  // Q / dO / -lse / -delta stage buffers: two on the register path, three on the
  // direct path (stage s uses buffer s % NB)
  constexpr int NB = VEC ? 3 : 2;
  constexpr int HW = NW / 2;      // waves per loader set (direct path)
  constexpr int RE = Lay<D>::kRowElems;   // LDS elements per Q / dO row
  constexpr int KRE = Lay<D>::kKVRowElems;  // LDS elements per K / V row
  constexpr int SP = TQ + 8;      // dS^T tile pitch (row = key)
  constexpr int CH = D / 8;       // 16-byte chunks per row in memory
  constexpr int NDB = D / 16;
  constexpr int NQCH = TQ * CH;   // chunks of one Q (or dO) tile
  static_assert(NQCH % 64 == 0, "a wave's register-path chunks lie in one of Q, dO");
  constexpr int NBCH = TQ * TK / 8;   // 16-byte chunks of one bias tile
  constexpr int NR = (2 * NQCH + NT - 1) / NT;
  constexpr int NRB = (NBCH + NT - 1) / NT;
  constexpr int NBLK = NQB * NDB; // dQ output blocks per stage
  static_assert(KV || NBLK <= NW, "one dQ block per wave at most");
  static_assert(TK == 128 || (TK == 64 && KV && LD == 16 && D != 64), "64-key tiles: dK/dV only, D = 16, 32, 16-byte loads");
  typedef typename DOp<D>::T QT;
  constexpr int QL = DOp<D>::kPerLane;

  __shared__ __align__(16) uint16_t sQ[NB][TQ * RE];
  __shared__ __align__(16) uint16_t sdO[NB][TQ * RE];
  __shared__ __align__(16) float sLD[2][NB][TQ];   // -lse / scale (0) and -delta (1) of the stage's rows
  __shared__ __align__(16) uint16_t sdS[KV ? 1 : 2][KV ? 8 : TK * SP];
  __shared__ __align__(16) uint16_t sK[G][TK * KRE];
  __shared__ __align__(16) uint16_t sV[G][TK * KRE];   // V rows of the key tile (row-read layout)
  __shared__ __align__(16) uint16_t sB[2][TQ * TK];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
  const int trk = (lane & 15) >> 2, tra = lane & 3;         // transposing-read row / chunk of the lane
  const int N = a.N, H = a.H, N_o = a.N_o;

  // XCD-aware order: blocks are dispatched round-robin over 8 XCDs; the key
  // tiles of one (example, group, head) unit run on the same XCD so that they
  // share its L2 for Q, dO and the bias rows.
  const int nunit = a.B * a.n_groups * H;     // groups of this launch (all, or one chunk)
  const int per_xcd = (nunit + 7) / 8;
  const int xcd = blockIdx.x % 8, kx = blockIdx.x / 8;
  const int unit = (kx / a.n_key_tiles) * 8 + xcd;
  if (kx / a.n_key_tiles >= per_xcd || unit >= nunit) return;
  const int t = kx % a.n_key_tiles;
  const int h = unit % H;
  const int grp_l = (unit / H) % a.n_groups;   // group index within the launch
  const int grp = a.g0 + grp_l;                 // outer group: slices grp*G ..
  const int b = unit / (H * a.n_groups);

  const float scale = a.scale;
  const float c1 = scale * kLog2e;
  const int key = t * TK + 16 * w + c;   // key column owned by this lane
  const bool kok = key < N;

  // Every group runs G stages per query tile.  When N_o is not a multiple of G
  // the last group's missing slices run as stages whose inputs all read as zero
  // (zero buffer extents); their dQ, dK and dV are not stored and their score
  // gradients are not added to the dbias tile.
  const int nsl = min(G, N_o - grp * G);
  const int nqt = (N + TQ - 1) / TQ;
  const int nst = G * nqt;        // stages

  // rows of slice (b, grp*G + gs, h) start at row0 + gs * ostride in the [B, N_o, H, N] row space
  const int64_t row0 = (((int64_t)b * N_o + grp * G) * H + h) * N;
  const int64_t ostride = (int64_t)H * N;
  // dQ partials hold a.part_slices slices per example (N_o, or the slices of one chunk);
  // the launch's group grp_l starts at slice grp_l * G of them
  const int64_t part_rows = (int64_t)a.B * a.part_slices * H * N;    // rows of one dQ partial
  const int64_t prow0 = (((int64_t)b * a.part_slices + grp_l * G) * H + h) * N;
  const uint32_t rowbytes = (uint32_t)N * D * 2;
  auto srow = [&](int gs) { return row0 + (gs < nsl ? gs : 0) * ostride; };
  const uint16_t* bias_plane = a.bias + ((int64_t)b * H + h) * N * N;

  // per-slice key mask, K and V tiles (LDS), accumulators
  float mk2[G];
  f32x4 dk_acc[G][NDB], dv_acc[G][NDB];
#pragma unroll
  for (int gs = 0; gs < G; ++gs) {
    mk2[gs] = -INFINITY;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      dk_acc[gs][db] = f32x4{0.f, 0.f, 0.f, 0.f};
      dv_acc[gs][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const bool live = gs < nsl;
    if (live && kok) mk2[gs] = MASK ? a.mask[((int64_t)b * N_o + grp * G + gs) * N + key] * kLog2e : 0.f;
    const int64_t sr = srow(gs);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k + sr * D, live ? rowbytes : 0u);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v + sr * D, live ? rowbytes : 0u);
    for (int ci = tid; ci < TK * CH; ci += NT) {
      const int r = ci / CH, ch = ci % CH;
      const uint32_t off = (uint32_t)((t * TK + r) * D + ch * 8) * 2;
      const u32x4 kv = buf_ld16(rk, off);
      const u32x4 vv = buf_ld16(rv, off);
      *reinterpret_cast<u32x4*>(&sK[gs][Lay<D>::k(r, ch * 8)]) = kv;
      *reinterpret_cast<u32x4*>(&sV[gs][Lay<D>::v(r, ch * 8)]) = vv;
    }
  }

  // ---- staging of one (query tile jj, slice gg) stage: Q, dO, -lse/scale, -delta.
  // The buffer descriptors start at the tile's first row and end at row N, so the
  // per-lane offsets do not depend on the stage and rows past N read as zero.
  //
  // Direct path (N even): stage s goes from memory straight into LDS buffer s % 3.
  // The waves form two loader sets (waves 0..NW/2-1 and NW/2..NW-1); set s % 2 loads
  // stage s right after the barrier that ends stage s - 3 and waits for it (vmcnt(0))
  // only at the end of stage s - 1, so every load has two stages of compute to land,
  // and each wave waits on its memory operations at every other barrier only.  Wave
  // ws < NQPIECE of a set fills Q piece ws and dO piece ws: lane l of a piece fills
  // 16-byte LDS slot l with the logical chunk that the layout stores there (padding
  // slots of the D = 16 layout reload chunk 0).
  // Register path: regs hold stage s+1 while stage s computes; buffers alternate.
  constexpr int SPR = Lay<D>::kSlotsPerRow;
  constexpr int NQPIECE = TQ * SPR / 64;
  static_assert(TQ * SPR % 64 == 0, "Q tile must be whole wave pieces");
  constexpr int NQPW = (NQPIECE + HW - 1) / HW;   // Q (and dO) pieces per wave of a loader set
  static_assert(!VEC || NQPW == 1 || TK == 64, "one Q and one dO piece per wave of a loader set");
  const int lset = w / HW, ws = w % HW;     // loader set of the wave, wave index within it
  uint32_t qoff[NQPW];                      // wave ws loads pieces ws, ws + HW, ..
#pragma unroll
  for (int k = 0; k < NQPW; ++k) {
    const int slot = (ws + k * HW) * 64 + lane, row = Lay<D>::q_src_row(slot / SPR);
    const int ch = Lay<D>::q_src_chunk(row, slot % SPR);
    qoff[k] = (uint32_t)(row * D + ch * 8) * 2;
  }
  // -lse/scale and -delta of a stage: lanes 0 .. TQ/4-1 of one wave fetch 4 lse values
  // each, the same lanes of the next wave 4 delta values (direct path: the first two waves
  // of the loading set; register path: waves 0 and 1).  One array per wave keeps each
  // wave's buffer descriptor uniform.
  static_assert(HW >= 2, "two waves per loader set");
  const int rls_w = VEC ? ws : w;            // 0: lse, 1: delta
  const bool rls_lane = rls_w < 2 && lane < TQ / 4;
  u32x4 rq[VEC ? 1 : NR];
  f32x4 rls = f32x4{0.f, 0.f, 0.f, 0.f};
  auto load_rls = [&](int64_t sr, int jj, bool live) {
    if (rls_lane) {
      const uint32_t lext = live ? (uint32_t)(N - jj * TQ) * 4 : 0u;
      const uint32_t q0 = 4 * lane;
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(uniform_ptr((rls_w == 0 ? a.lse : a.delta) + sr), lext);
      if (LD == 16) {     // rows of lse / delta 16-byte aligned (N % 4 == 0)
        rls = __builtin_bit_cast(f32x4, buf_ld16(rs, q0 * 4));
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) rls[i] = __uint_as_float(buf_ld4(rs, (q0 + i) * 4));
      }
    }
  };
  const float rls_f = rls_w == 0 ? -1.0f / scale : -1.0f;
  auto write_rls = [&](int buf) {
    if (rls_lane) *reinterpret_cast<f32x4*>(&sLD[rls_w & 1][buf][4 * lane]) = rls * rls_f;
  };
  auto load_stage_direct = [&](int jj, int gg, int buf) {
    const int64_t sr = srow(gg) + (int64_t)jj * TQ;     // first row of the tile
    const bool live = gg < nsl;
    const uint32_t ext = live ? (uint32_t)(N - jj * TQ) * D * 2 : 0u;
#pragma unroll
    for (int k = 0; k < NQPW; ++k) {
      const int piece = ws + k * HW;
      if (piece < NQPIECE) {
        dma16(make_rsrc_words(a.q + sr * D, ext), sQ[buf] + piece * 512, qoff[k]);
        dma16(make_rsrc_words(a.d_o + sr * D, ext), sdO[buf] + piece * 512, qoff[k]);
      }
    }
    load_rls(sr, jj, live);
  };
  auto load_stage_regs = [&](int jj, int gg) {
    const int64_t sr = srow(gg) + (int64_t)jj * TQ;
    const bool live = gg < nsl;
    const uint32_t ext = live ? (uint32_t)(N - jj * TQ) * D * 2 : 0u;
    const __amdgpu_buffer_rsrc_t rQ = make_rsrc(a.q + sr * D, ext);
    const __amdgpu_buffer_rsrc_t rO = make_rsrc(a.d_o + sr * D, ext);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int ci = tid + r * NT;
      if (ci < 2 * NQCH) {
        // Q or dO: the same for the whole wave (NQCH is a multiple of 64), so the choice of
        // descriptor stays uniform
        const int which = __builtin_amdgcn_readfirstlane(ci / NQCH), cc = ci % NQCH;
        const int row = cc / CH, ch = cc % CH;
        rq[r] = buf_ld16(which ? rO : rQ, (uint32_t)(row * D + ch * 8) * 2);
      }
    }
    load_rls(sr, jj, live);
  };
  auto stage_regs = [&](int buf) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int ci = tid + r * NT;
      if (ci < 2 * NQCH) {
        const int which = ci / NQCH, cc = ci % NQCH;
        const int row = cc / CH, ch = cc % CH;
        uint16_t* dst = which ? sdO[buf] : sQ[buf];
        *reinterpret_cast<u32x4*>(&dst[Lay<D>::q(row, ch * 8)]) = rq[r];
      }
    }
    write_rls(buf);
  };

  // ---- bias tile of (query tile j, key tile t), staged [query][key]: 256-byte rows,
  // 8-byte unit u of row r stored at unit position u ^ bsw(r) (bsw even, so 16-byte
  // chunks stay whole for the direct loads)
  // 64-key tiles: 128-byte rows, unit position u ^ bsw(r) with bsw from row bits 1 and 3,
  // so the transposing reads of a half-wave (rows r0 + 0..3 and r0 + 8..11, four units
  // each) cover all 64 banks
  auto bsw = [](int r) {
    return TK == 128 ? (((r & 3) << 2) | (((r >> 3) & 1) << 4)) : ((((r >> 1) & 1) << 2) | (((r >> 3) & 1) << 3));
  };
  auto b_at = [&](int r, int key) { return TK * r + 4 * ((key >> 2) ^ bsw(r)) + (key & 3); };
  constexpr int BCH = TK / 8;                    // 16-byte slots per bias row
  constexpr int NBPIECE = TQ * BCH / 64;
  static_assert(TQ * BCH % 64 == 0, "bias tile must be whole wave pieces");
  static_assert(NBPIECE % HW == 0, "bias pieces spread evenly over loader set 0");
  constexpr int BPW = NBPIECE / HW;              // bias pieces per wave of set 0
  static_assert(LD != 4 || HW == 4, "4-byte bias loads: row bits 0-1 select the wave of set 0");
  // direct path: the bias of a tile is loaded by set 0 (a tile starts at an even
  // stage).  LD 16: wave ws loads 1 KB pieces ws + k * NW/2.  LD 4: wave ws loads rows
  // ws + 4k, one 256-byte row per load; bsw of those rows takes two values (row bit 3),
  // so two lane offsets serve them all.  Keys past N get an offset past every extent
  // and land as zeros (a 16-byte chunk, or a 4-byte pair of keys, is entirely in or out).
  constexpr int NBOFF = LD == 4 ? 2 : BPW;
  uint32_t boff[NBOFF];
#pragma unroll
  for (int k = 0; k < NBOFF; ++k) {
    if (LD == 4) {
      const int unit = (lane >> 1) ^ ((ws << 2) | (k << 4));   // logical 8-byte unit of the lane's dword
      const int k0 = t * TK + 4 * unit + 2 * (lane & 1);
      boff[k] = k0 < N ? (uint32_t)k0 * 2 : 0xfffffff0u;
    } else {
      const int slot = (ws + k * HW) * 64 + lane, row = slot / BCH, ch = (slot % BCH) ^ (bsw(row) >> 1);
      const int k0 = t * TK + ch * 8;
      boff[k] = k0 < N ? (uint32_t)(row * N + k0) * 2 : 0xfffffff0u;
    }
  }
  auto load_bias_direct = [&](int j, int bbuf) {
    if (LD == 4) {
      // one descriptor per row, from that row to row N (extent zero past N)
#pragma unroll
      for (int k = 0; k < TQ / HW; ++k) {
        const int r = ws + k * HW, rows_left = N - j * TQ - r;
        const u32x4 rw = make_rsrc_words(bias_plane + ((int64_t)j * TQ + r) * N,
                                         rows_left > 0 ? (uint32_t)rows_left * N * 2 : 0u);
        dma4(rw, sB[bbuf] + r * TK, boff[(k >> 1) & 1]);
      }
    } else {
      // descriptor from row j*TQ to row N of the (b, h) bias plane
      const u32x4 rw = make_rsrc_words(bias_plane + (int64_t)j * TQ * N, (uint32_t)(N - j * TQ) * N * 2);
#pragma unroll
      for (int k = 0; k < BPW; ++k) dma16(rw, sB[bbuf] + (ws + k * HW) * 512, boff[k]);
    }
  };
  u32x4 rbt[VEC ? 1 : NRB];
  auto load_bias_regs = [&](int j) {
    // odd N: rows are only 2-byte aligned; the descriptor starts at the 4-byte boundary
    // at or below the tile's first row (extra bytes earlier), 8 keys are read as five
    // aligned dwords shifted into place, and keys past N are zeroed
    const uint16_t* rowp = bias_plane + (int64_t)j * TQ * N;
    const uint32_t extra = (uint32_t)((uintptr_t)rowp & 3u);
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc((const char*)rowp - extra, ((uint32_t)(N - j * TQ) * N * 2 + extra + 3u) & ~3u);
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      const int ci = tid + r * NT;
      if (ci < NBCH) {
        const int row = ci / (TK / 8), ch = ci % (TK / 8);
        const int k0 = t * TK + ch * 8;
        const uint32_t e0 = extra + (uint32_t)(row * N + k0) * 2;
        const uint32_t a0 = e0 & ~3u, sh = (e0 & 2u) << 3;
        uint32_t x[5];
#pragma unroll
        for (int p = 0; p < 5; ++p) x[p] = buf_ld4(rb, a0 + 4u * p);
        uint32_t wv[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int k_lo = k0 + 2 * p;
          const uint32_t wd = __builtin_amdgcn_alignbit(x[p + 1], x[p], sh);
          wv[p] = k_lo + 1 < N ? wd : (k_lo < N ? (wd & 0xffffu) : 0u);
        }
        rbt[r] = u32x4{wv[0], wv[1], wv[2], wv[3]};
      }
    }
  };
  auto stage_bias_regs = [&](int bbuf) {
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
      const int ci = tid + r * NT;
      if (ci < NBCH) {
        const int row = ci / (TK / 8), ch = ci % (TK / 8);
        *reinterpret_cast<u32x4*>(&sB[bbuf][b_at(row, ch * 8)]) = rbt[r];
      }
    }
  };

  // ---- dQ^T blocks (queries 16qb.., features 16db..) = K^T dS^T over the TK keys of a stage.
  // Each partial's descriptor starts at the tile's first row and ends at row N (extent zero
  // when nothing is to be stored), so rows past N are dropped.
  // Who computes them: on the direct path, the loader set that does not wait at the end of
  // the stage (wave ws of the set takes the DQB blocks of one query block starting at
  // feature block ws * DQB % NDB); its partial stores then have two stages to drain before
  // that set's next vmcnt(0), which on this hardware also waits for the wave's stores
  // (measured at N = 768: 1.63 -> 1.53 ms for D = 32, 1.18 -> 1.13 ms for D = 16, 3.50 ->
  // 3.46 ms for D = 64).  On the register path wave w takes block w.
  constexpr bool DSET = VEC;
  constexpr bool DEARLY = VEC && D == 64;   // dbias stores split around the last stage's barrier
  constexpr int DQB = DSET ? NBLK / HW : 1;     // dQ blocks per computing wave
  static_assert(KV || !DSET || (NBLK % HW == 0 && NDB % DQB == 0), "a wave's dQ blocks share one query block");
  auto dq_blocks = [&](int jj, int gg, int buf, bool store, int blk0) {
    const int qb = blk0 / NDB;
    const uint16_t* kt_tile = sK[gg];
    // the dS^T operand of the query block, shared by the wave's feature blocks
    u32x4 bs[TK / 32];
#pragma unroll
    for (int st = 0; st < TK / 32; ++st) {
      const int so = (32 * st + 8 * g + trk) * SP + 16 * qb + 4 * tra;
      bs[st] = ds_read_tr8_at(sdS[buf], so, so + 4 * SP);
    }
    const int64_t prow = t * part_rows + prow0 + (gg < nsl ? gg : 0) * ostride + (int64_t)jj * TQ;
#pragma unroll
    for (int bb = 0; bb < DQB; ++bb) {
      const int db = (blk0 + bb) % NDB;
      f32x4 dq0 = f32x4{0.f, 0.f, 0.f, 0.f}, dq1 = f32x4{0.f, 0.f, 0.f, 0.f};
      u32x4 ak[TK / 32];
#pragma unroll
      for (int st = 0; st < TK / 32; ++st) {
        const int kr = 32 * st + 8 * g + trk;
        const int kc = 16 * db + 4 * tra;
        ak[st] = ds_read_tr8_at(kt_tile, Lay<D>::k(kr, kc), Lay<D>::k(kr + 4, kc));
      }
#pragma unroll
      for (int st = 0; st < TK / 32; ++st) {
        if (st & 1) dq1 = mfma_k32(ak[st], bs[st], dq1);
        else dq0 = mfma_k32(ak[st], bs[st], dq0);
      }
      const f32x4 v = (dq0 + dq1) * scale;
      if constexpr (BP) {   // bf16 partials: one RNE rounding, 8 bytes per lane
        const uint32_t ext = __builtin_amdgcn_readfirstlane(store && gg < nsl ? (uint32_t)(N - jj * TQ) * D * 2 : 0u);
        const __amdgpu_buffer_rsrc_t rs = make_rsrc((uint16_t*)a.dq_partial + prow * D, ext);
        const uint32_t off = (uint32_t)((16 * qb + c) * D + 16 * db + 4 * g) * 2;
        __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])}, rs, off, 0, 0);
      } else {
        const uint32_t ext = __builtin_amdgcn_readfirstlane(store && gg < nsl ? (uint32_t)(N - jj * TQ) * D * 4 : 0u);
        const __amdgpu_buffer_rsrc_t rs = make_rsrc((float*)a.dq_partial + prow * D, ext);
        const uint32_t off = (uint32_t)((16 * qb + c) * D + 16 * db + 4 * g) * 4;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, off, 0, 0);
      }
    }
  };
  // dset: the loader set that does not wait at the end of the current stage
  auto dq_stage = [&](int jj, int gg, int buf, bool store, int dset) {
    if constexpr (KV) {
    } else if constexpr (DSET) {
      if (lset == dset) dq_blocks(jj, gg, buf, store, ws * DQB);
    } else {
      if (w < NBLK) dq_blocks(jj, gg, buf, store, w);
    }
  };

  // ---- prologue: the first stages and the first bias tile
  if (VEC) {
    if (lset == 0) {
      load_stage_direct(0, 0, 0);
      load_bias_direct(0, 0);
    } else {
      load_stage_direct(0, 1, 1);      // G >= 2: stage 1 is slice 1 of query tile 0
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    write_rls(lset);
    __syncthreads();                   // also publishes the K and V tiles
    if (lset == 0 && 2 < nst) {
      load_stage_direct(2 / G, 2 % G, 2);
      if (2 % G == 0) load_bias_direct(2 / G, (2 / G) & 1);   // G = 2: stage 2 starts query tile 1
    }
  } else {
    load_stage_regs(0, 0);
    load_bias_regs(0);
    stage_regs(0);
    stage_bias_regs(0);
    load_stage_regs(0, 1);
    if (nqt > 1) load_bias_regs(1);
    __syncthreads();
  }

  // one query tile: its G stages and its dbias tile.  FULL: all G slices of the group
  // exist (every group but a ragged last one), so every stage's dS enters the dbias tile.
  // R0: position of the tile's first stage in the cycle of direct-path buffers (stage s
  // uses buffer s % NB; with G % NB != 0 tiles come in triples, so R0 is 0, G or 2G).
  auto query_tile = [&](int j, auto full_c, auto r0_c) {
    constexpr bool FULL = decltype(full_c)::value;
    constexpr int R0 = decltype(r0_c)::value;
    // bias of the lane's (query, key) pairs: one transposing read per block gives rows
    // 32s + 8g + 4e + 0..3 of block qb = 2s + e at the lane's key column.  Without a mask
    // it is kept as bias * log2(e); with one as the bias itself, and each stage forms
    // bias * log2(e) + mask * log2(e) in one FMA (for a zero mask the same value)
    f32x4 bb[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int r0 = 32 * (qb >> 1) + 8 * g + 4 * (qb & 1);
      const u32x2 bw = ds_read_tr(&sB[j & 1][b_at(r0 + trk, 16 * w + 4 * tra)]);
      bb[qb] = f32x4{bf_lo(bw[0]), bf_hi(bw[0]), bf_lo(bw[1]), bf_hi(bw[1])};
      if constexpr (!MASK) bb[qb] *= kLog2e;
    }
    f32x4 dbacc[NQB];       // sum over the group's slices of the FP32 dS, in slice order
    // this group's dbias partial of query tile j (the FP32 sum over the group's slices)
    auto store_dbias = [&]() {
      if (kok) {
        // this group's dbias partial for (query tile j, key tile t); in the last query
        // tile rows past N go to an offset past the plane's extent and are dropped
        const int64_t plane = (((int64_t)grp_l * a.B + b) * H + h) * N * N;
        constexpr int EB = BP ? 2 : 4;         // bytes per partial element
        const __amdgpu_buffer_rsrc_t rs =
            BP ? make_rsrc((uint16_t*)a.dbias_partial + plane, (uint32_t)N * N * 2)
               : make_rsrc((float*)a.dbias_partial + plane, (uint32_t)N * N * 4);
        auto put = [&](float x, uint32_t voff, int soff) {
          if constexpr (BP) __builtin_amdgcn_raw_buffer_store_b16(f_to_bf(x), rs, voff, soff, 0);
          else __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), rs, voff, soff, 0);
        };
        if ((j + 1) * TQ <= N) {
          const uint32_t lane_off = (uint32_t)(8 * g * N + key) * EB;
  #pragma unroll
          for (int qb = 0; qb < NQB; ++qb)
  #pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int rr = j * TQ + 32 * (qb >> 1) + 4 * (qb & 1) + i;   // row of group g = 0
              put(dbacc[qb][i], lane_off, (int)((uint32_t)rr * N * EB));
            }
        } else {
  #pragma unroll
          for (int qb = 0; qb < NQB; ++qb)
  #pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int q = j * TQ + 32 * (qb >> 1) + 8 * g + 4 * (qb & 1) + i;
              put(dbacc[qb][i], q < N ? (uint32_t)(q * N + key) * EB : 0xFFFFF000u, 0);
            }
        }
      }
    };

#pragma unroll
    for (int gs = 0; gs < G; ++gs) {
      const int r = R0 + gs;                 // stage index modulo 3 * G
      const int s = G * j + gs;              // stage index
      const int buf = VEC ? r % NB : gs & 1;  // Q / dO / -lse / -delta buffer
      const int dsb = gs & 1;                // dS^T buffer
      const uint16_t* tq = sQ[buf];
      const uint16_t* tdo = sdO[buf];

      // dQ of the previous stage, (j, gs-1) or (j-1, G-1), whose dS^T tile was completed
      // at the previous barrier; before the first stage it runs on the idle buffer and
      // stores nothing
      // (the set waiting at the end of stage r is (r + 1) & 1, see below)
      if (gs > 0) dq_stage(j, gs - 1, dsb ^ 1, true, r & 1);
      else dq_stage(j > 0 ? j - 1 : 0, G - 1, dsb ^ 1, j > 0, r & 1);

      const auto lk = [](int r, int cc) { return Lay<D>::k(r, cc); };
      const auto lv = [](int r, int cc) { return Lay<D>::v(r, cc); };
      const auto lq = [](int r, int cc) { return Lay<D>::q(r, cc); };
      const QT kb = ld_op<D>(sK[gs], 16 * w + c, g * QL, lk);
      const QT vb = ld_op<D>(sV[gs], 16 * w + c, g * QL, lv);
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        u32x2 pP[2], pS[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int qb = 2 * st + e;
          const int ql = 32 * st + 8 * (c >> 2) + 4 * e + (c & 3);
          const int r0 = 32 * st + 8 * g + 4 * e;
          const QT qa = ld_op<D>(tq, ql, g * QL, lq);
          const QT da = ld_op<D>(tdo, ql, g * QL, lq);
          const f32x4 nl = *reinterpret_cast<const f32x4*>(&sLD[0][buf][r0]);
          const f32x4 nd = *reinterpret_cast<const f32x4*>(&sLD[1][buf][r0]);
          const f32x4 sv = DOp<D>::mma(qa, kb, nl);        // q.k - lse/scale
          const f32x4 dp = DOp<D>::mma(da, vb, nd);        // dP - delta
          float p[4], ds[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float bm = MASK ? fmaf(bb[qb][i], kLog2e, mk2[gs]) : bb[qb][i];
            const float x = fmaf(sv[i], c1, bm);
            p[i] = __builtin_amdgcn_exp2f(x);
            ds[i] = p[i] * dp[i];
          }
          if constexpr (!KV) {
            if (gs == 0) {
              dbacc[qb] = f32x4{ds[0], ds[1], ds[2], ds[3]};
            } else if (FULL || gs < nsl) {
              dbacc[qb] += f32x4{ds[0], ds[1], ds[2], ds[3]};
            }
          }
          pP[e] = u32x2{pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3])};
          pS[e] = u32x2{pack_bf16(ds[0], ds[1]), pack_bf16(ds[2], ds[3])};
        }
        // dV^T += dO^T P and dK^T += Q^T dS over the 32 queries of this half
        const u32x4 bp = u32x4{pP[0][0], pP[0][1], pP[1][0], pP[1][1]};
        const u32x4 bs = u32x4{pS[0][0], pS[0][1], pS[1][0], pS[1][1]};
        if constexpr (!KV) *reinterpret_cast<u32x4*>(&sdS[dsb][(16 * w + c) * SP + 32 * st + 8 * g]) = bs;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int qr = 32 * st + 8 * g + trk, qc = 16 * db + 4 * tra;
          const int olo = Lay<D>::q(qr, qc), ohi = Lay<D>::q(qr + 4, qc);
          const u32x4 ao = ds_read_tr8_at(tdo, olo, ohi);
          const u32x4 aq = ds_read_tr8_at(tq, olo, ohi);
          dv_acc[gs][db] = mfma_k32(ao, bp, dv_acc[gs][db]);
          dk_acc[gs][db] = mfma_k32(aq, bs, dk_acc[gs][db]);
        }
      }

      // the dbias partial: with D = 64 (two slices per group, 32-query stages) the set that
      // does not wait at the end of the tile's last stage stores it before that stage's
      // barrier, so its stores drain during the rest of this stage and all of the next before
      // that set's own vmcnt(0); the other set stores it after the barrier, two stages before
      // its wait (measured at N = 768: 3.44 -> 2.96 ms; no gain for D = 16 and 32, where a
      // tile has four stages, so the stores stay after the barrier there)
      if (!KV && DEARLY && gs == G - 1 && lset == (r & 1)) store_dbias();
      if (VEC) {
        // the set that loaded stage s+1 waits for it and stages its -lse/-delta; the
        // other set's loads (stage s+2) stay in flight across this barrier
        const bool mine = lset == ((r + 1) & 1);
        if (mine) {
          __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
          if (s + 1 < nst) write_rls((r + 1) % NB);
        }
        lds_barrier();          // this stage's dS^T complete; stage s+1 visible
        // the same set now loads stage s+3 into its buffer (last used by stage s+3-NB,
        // released by now), and with it the bias of the query tile that starts there
        if (mine && s + 3 < nst) {
          const int j3 = j + (gs + 3) / G, g3 = (gs + 3) % G;
          load_stage_direct(j3, g3, (r + 3) % NB);
          if (g3 == 0) load_bias_direct(j3, j3 & 1);
        }
      } else {
        if (s + 1 < nst) {
          stage_regs(buf ^ 1);
          if (gs == G - 1) stage_bias_regs((j + 1) & 1);
        }
        __syncthreads();        // this stage's dS^T complete; next stage's tiles visible
        // the stage two ahead: (j, gs + 2) or (j + 1, gs + 2 - G)
        const int j2 = gs + 2 < G ? j : j + 1, g2 = gs + 2 < G ? gs + 2 : gs + 2 - G;
        if (j2 < nqt) load_stage_regs(j2, g2);
        if (gs == G - 1 && j + 2 < nqt) load_bias_regs(j + 2);
      }
    }
    if (!KV && (!DEARLY || lset != ((R0 + G - 1) & 1))) store_dbias();

  };
  using R0a = std::integral_constant<int, 0>;
  using R0b = std::integral_constant<int, G>;
  using R0c = std::integral_constant<int, 2 * G>;
  auto run = [&](auto full_c) {
    if constexpr (VEC && G % NB != 0) {
      for (int j0 = 0; j0 < nqt; j0 += 3) {
        query_tile(j0, full_c, R0a{});
        if (j0 + 1 < nqt) query_tile(j0 + 1, full_c, R0b{});
        if (j0 + 2 < nqt) query_tile(j0 + 2, full_c, R0c{});
      }
    } else {
      for (int j = 0; j < nqt; ++j) query_tile(j, full_c, R0a{});
    }
  };
  if (nsl == G) run(std::true_type{});
  else run(std::false_type{});
  dq_stage(nqt - 1, G - 1, (G - 1) & 1, true, 0);

  // epilogue: dK = scale * dK^T^T, dV
  if (kok) {
#pragma unroll
    for (int gs = 0; gs < G; ++gs) {
      if (gs < nsl) {
        const int64_t row = row0 + gs * ostride + key;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const f32x4 k4 = dk_acc[gs][db] * scale;
          const f32x4 v4 = dv_acc[gs][db];
          *reinterpret_cast<u32x2*>(a.dk + row * D + 16 * db + 4 * g) =
              u32x2{pack_bf16(k4[0], k4[1]), pack_bf16(k4[2], k4[3])};
          *reinterpret_cast<u32x2*>(a.dv + row * D + 16 * db + 4 * g) =
              u32x2{pack_bf16(v4[0], v4[1]), pack_bf16(v4[2], v4[3])};
        }
      }
    }
  }
}

template <int D, bool MASK, int LD>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t s) {
  constexpr int TK = kBwdKeyTile;
  const int64_t nunit = (int64_t)a.B * a.n_groups * a.H;
  const int64_t nblk = 8 * ((nunit + 7) / 8) * a.n_key_tiles;
  if (a.kv_only) {
    // dK / dV only (the two-kernel backward, D = 16 and 32)
    if constexpr (D == 64) {
      return hipErrorInvalidValue;
    } else if constexpr (LD == 16) {
      // 64-key tiles over outer groups of 2 slices
      BwdArgs k = a;
      k.n_key_tiles = (a.N + 63) / 64;
      k.n_groups = (a.N_o + 1) / 2;
      const int64_t nu = (int64_t)a.B * k.n_groups * a.H;
      const int64_t nb = 8 * ((nu + 7) / 8) * k.n_key_tiles;
      hipLaunchKernelGGL((bwd_kernel<D, MASK, LD, false, 64, true>), dim3((unsigned)nb), dim3(256), 0, s, k);
    } else {
      hipLaunchKernelGGL((bwd_kernel<D, MASK, LD, false, TK, true>), dim3((unsigned)nblk), dim3(TK * 4), 0, s, a);
    }
  } else if (a.bf16_partials)
    hipLaunchKernelGGL((bwd_kernel<D, MASK, LD, true, TK, false>), dim3((unsigned)nblk), dim3(TK * 4), 0, s, a);
  else
    hipLaunchKernelGGL((bwd_kernel<D, MASK, LD, false, TK, false>), dim3((unsigned)nblk), dim3(TK * 4), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, int D, hipStream_t s) {
  const bool mask = a.mask != nullptr;
  const int ld = bias_load_width(a.N);
#define TRI_BWD_CASE(DD, MM, LL) \
  if (D == DD && mask == MM && ld == LL) return launch_bwd_t<DD, MM, LL>(a, s);
  TRI_BWD_CASE(32, false, 16)
  TRI_BWD_CASE(32, true, 16)
  TRI_BWD_CASE(32, false, 4)
  TRI_BWD_CASE(32, true, 4)
  TRI_BWD_CASE(32, false, 0)
  TRI_BWD_CASE(32, true, 0)
  TRI_BWD_CASE(16, false, 16)
  TRI_BWD_CASE(16, true, 16)
  TRI_BWD_CASE(16, false, 4)
  TRI_BWD_CASE(16, true, 4)
  TRI_BWD_CASE(16, false, 0)
  TRI_BWD_CASE(16, true, 0)
  TRI_BWD_CASE(64, false, 16)
  TRI_BWD_CASE(64, true, 16)
  TRI_BWD_CASE(64, false, 4)
  TRI_BWD_CASE(64, true, 4)
  TRI_BWD_CASE(64, false, 0)
  TRI_BWD_CASE(64, true, 0)
#undef TRI_BWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace tri
