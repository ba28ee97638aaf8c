// Query-tile backward of triangular attention on gfx950: dQ and dbias.
//
// Method: TurboPairFormer, Figure 2 (gradients of attention with a pair bias shared by
// the outer slices): per slice, P = softmax(scale q.k + bias + mask), dP = dO V^T,
// dS = P * (dP - delta) with delta the row sum of dO * O (compensated, Figure 3),
// dQ = scale dS K, and dbias = the sum over all outer slices of dS.
//
// Work split.  The key-tile kernel (bwd.hip, dK/dV-only variant) forms dK and dV; this
// kernel forms dQ and dbias and evaluates S, P, dP and dS a second time.  A workgroup owns
// 32 queries of one head, one range of up to 384 keys and one outer group of consecutive
// slices, which it visits in ascending order, so that
//  - dbias of its (query, key) block is summed over the whole group in FP32 registers and
//    written once per group: L = a few groups instead of N_o / 4, and
//  - each slice's dQ over the key range is summed inside the workgroup: one FP32 dQ
//    partial per key range (two for N = 768) instead of one per 128 keys.
// The partials of the single-pass design (TurboPairFormer, Figure 7(c)-(d)) cost
// 4 (J_K X + L Y) bytes written and read again; at N = 768, D = 32 that round trip is
// 7.2 GB, more than twice the time of this second evaluation of the scores.
//
// Orientation S^T = K Q^T: keys are MFMA rows, queries columns; wave w owns keys
// 32 np w .. 32 np (w + 1) - 1 of the range, in pairs of 16-key blocks.  Block e of pair p
// holds keys 32p + 8j + 4e + i at row 4j + i, so that lane (g, c) holds keys
// 32p + 8g + 4e + 0..3 at query c and its FP32 dS of the pair's two blocks, packed to bf16,
// is directly the B operand of dQ^T = K^T dS^T (slots 8g..8g+7 = keys 32p + 8g + 0..7);
// the K^T operand comes from the wave's K tile through the transposing LDS read.
// (bias + mask) / scale is the accumulator input of the S^T product: bias / scale sits in
// FP32 registers for the whole kernel (it does not depend on the slice; keys past N hold
// an infinity of the sign that makes their probability exactly zero) and the mask is added
// per slice by one FMA.  The exponent is one FMA with -lse log2(e) of the lane's query,
// and -delta is the accumulator input of the dP^T product.
//
// Staging per slice, one slice ahead: each wave loads its own K rows (and mask values)
// into a private double-buffered LDS tile by direct global->LDS loads; waves 0, 1 and 2
// load the shared Q, dO and lse / delta tiles the same way; V rows go to registers one key
// pair ahead.  The waves' dQ^T tiles over their keys meet in LDS and are summed in wave
// order.  Two barriers per slice: one publishes the staged tiles (after each wave's
// vmcnt(0), the wait invariant of common.h), one the waves' dQ^T tiles.
#include "bwd_layout.h"
#include "common.h"
#include "kernels.h"

namespace tri {

namespace {

// Q / dO tile element offset: D = 32 uses the swizzled 64-byte rows of the key-tile kernel,
// D = 16 plain 32-byte rows (only row reads here).
template <int D> __device__ __forceinline__ int q_at(int row, int col) {
  if constexpr (D == 32) return Lay<32>::q(row, col);
  else return row * 16 + col;
}
// Byte offset, relative to the tile's first row, of the 16 bytes that a direct load stores
// in physical 16-byte slot `slot` of a Q (or dO) tile ...
template <int D> __device__ __forceinline__ uint32_t q_src(int slot) {
  if constexpr (D == 32) {
    const int row = Lay<32>::q_src_row(slot >> 2);
    return (uint32_t)(row * 32 + Lay<32>::q_src_chunk(row, slot & 3) * 8) * 2;
  } else {
    return (uint32_t)slot * 16;
  }
}
// ... and of a K tile in the Lay<D>::k layouts (D = 32: 16-byte chunk XORed with row bits
// 2-3; D = 16: rows 8-11 and 12-15 of each 16-row group trade places and the two chunks of
// those rows swap)
template <int D> __device__ __forceinline__ uint32_t k_src(int slot) {
  if constexpr (D == 32) {
    const int row = slot >> 2;
    return (uint32_t)(row * 32 + ((slot & 3) ^ Lay<32>::swk(row)) * 8) * 2;
  } else {
    const int prow = slot >> 1, hi = (prow >> 3) & 1;
    return (uint32_t)((prow ^ (hi << 2)) * 16 + ((slot & 1) ^ hi) * 8) * 2;
  }
}

}  // namespace

template <int D, bool MASK, int NW, int NP>
__global__ __launch_bounds__(NW * 64, 2) void bwdq_kernel(BwdQArgs a) {
  constexpr int NT = NW * 64;
  constexpr int TQ = kBwdQQueries, NQB = TQ / 16;
  constexpr int KWP = 32 * NP;                 // keys per wave
  constexpr int NDB = D / 16;
  constexpr int QL = DOp<D>::kPerLane;
  typedef typename DOp<D>::T QT;
  constexpr int CH = D / 8;                    // 16-byte chunks per K / Q row
  constexpr int KDMA = KWP * CH / 64;          // direct loads per lane: the wave's K rows
  constexpr int QDMA = TQ * CH / 64;           // direct loads per lane: one Q (or dO) tile
  constexpr int MW = KWP <= 64 ? 64 : 128;     // mask floats per wave tile (4-byte loads of 64 lanes)
  constexpr int RP = D + 4;                    // row pitch (floats) of the dQ^T tiles in LDS
  constexpr int RED = TQ * D / 4;              // 16-byte items of one dQ tile
  static_assert(D == 16 || D == 32, "query-tile backward: D = 16 or 32");
  static_assert(KWP * CH % 64 == 0 && TQ * CH % 64 == 0 && NW >= 3 && RED <= NT, "tile shapes");

  __shared__ __align__(16) uint16_t sK[2][NW][KWP * D];
  __shared__ __align__(16) float sM[MASK ? 2 : 1][NW][MASK ? MW : 4];
  __shared__ __align__(16) uint16_t sQ[2][TQ * D];
  __shared__ __align__(16) uint16_t sdO[2][TQ * D];
  __shared__ __align__(16) float sLD[2][128];    // lse of the 32 queries at 0.., delta at 64..
  __shared__ __align__(16) float sRed[NW][TQ * RP];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int trk = (lane & 15) >> 2, tra = lane & 3;
  const int N = a.N, H = a.H, N_o = a.N_o;
  const BwdQPlan pl = a.p;

  // XCD-aware order: blocks are dispatched round-robin over 8 XCDs; the query tiles of one
  // (example, group, head) unit run on one XCD at the same pace, its key ranges interleaved
  // (range fastest), so each slice's K and V rows and each query tile's Q and dO rows are
  // fetched into that XCD's L2 once.
  const int nunit = a.B * pl.n_groups * H;
  const int xcd = blockIdx.x % 8, kx = blockIdx.x / 8;
  const int r = kx % pl.n_ranges;
  const int unit = (kx / (pl.n_ranges * pl.n_qt)) * 8 + xcd;
  if (unit >= nunit) return;
  const int qt = (kx / pl.n_ranges) % pl.n_qt;
  const int h = unit % H;
  const int l = (unit / H) % pl.n_groups;
  const int b = unit / (H * pl.n_groups);

  const int q0 = qt * TQ;
  const int kw0 = r * pl.kr + w * KWP;           // first key of this wave
  const int o0 = l * pl.gs;
  const int ns = min(pl.gs, N_o - o0);           // slices of this group
  const float scale = a.scale, inv_s = 1.0f / scale;
  const float c1 = scale * kLog2e;
  const float kill = scale > 0.f ? -INFINITY : INFINITY;   // (bias + mask) / scale of absent keys

  // Slice o's rows start at row ((b N_o + o) H + h) N of the [B, N_o, H, N] arrays; the
  // per-slice offsets below advance by a stride instead of being formed again per slice.
  const int64_t hn = (int64_t)H * N;
  const int64_t sr0 = (((int64_t)b * N_o + o0) * H + h) * N;
  const uint32_t kv_bytes = (uint32_t)N * D * 2;

  // ---- bias / scale of the lane's (key, query) pairs, for the whole kernel
  const uint16_t* bias_plane = a.bias + ((int64_t)b * H + h) * N * N;
  f32x4 bp[NP][2][NQB], dbacc[NP][2][NQB];
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const int q = q0 + 16 * qb + c;
        const int k = kw0 + 32 * p + 8 * g + 4 * e;
        f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
        if (q < N) {
          const uint16_t* row = bias_plane + (int64_t)q * N;
          if ((N & 3) == 0 && k + 3 < N) {
            const u32x2 wv = *reinterpret_cast<const u32x2*>(row + k);
            x = f32x4{bf_lo(wv[0]), bf_hi(wv[0]), bf_lo(wv[1]), bf_hi(wv[1])};
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = k + i < N ? bf_to_f(row[k + i]) : 0.f;
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) bp[p][e][qb][i] = k + i < N ? x[i] * inv_s : kill;
        dbacc[p][e][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }

  // ---- staging of slice o into buffer buf (direct loads; rows past N read as zero)
  auto stage = [&](int64_t sr, const float* mrow, int buf) {
    const u32x4 rk = make_rsrc_words(a.k + sr * D, kv_bytes);
#pragma unroll
    for (int i = 0; i < KDMA; ++i)
      dma16(rk, sK[buf][w] + 512 * i, (uint32_t)kw0 * D * 2 + k_src<D>(64 * i + lane));
    if constexpr (MASK) {
      const u32x4 rm = make_rsrc_words(mrow, (uint32_t)N * 4);
#pragma unroll
      for (int i = 0; i < MW / 64; ++i) dma4(rm, sM[buf][w] + 64 * i, (uint32_t)(kw0 + 64 * i + lane) * 4);
    }
    const uint32_t ext = (uint32_t)(N - q0) * D * 2;
    if (w == 0) {
      const u32x4 rq = make_rsrc_words(a.q + (sr + q0) * D, ext);
#pragma unroll
      for (int i = 0; i < QDMA; ++i) dma16(rq, sQ[buf] + 512 * i, q_src<D>(64 * i + lane));
    } else if (w == 1) {
      const u32x4 ro = make_rsrc_words(a.d_o + (sr + q0) * D, ext);
#pragma unroll
      for (int i = 0; i < QDMA; ++i) dma16(ro, sdO[buf] + 512 * i, q_src<D>(64 * i + lane));
    } else if (w == 2) {
      const uint32_t lext = (uint32_t)(N - q0) * 4;
      dma4(make_rsrc_words(a.lse + sr + q0, lext), sLD[buf], (uint32_t)lane * 4);
      dma4(make_rsrc_words(a.delta + sr + q0, lext), sLD[buf] + 64, (uint32_t)lane * 4);
    }
  };
  // V rows of pair p (blocks e = 0, 1) of slice o: the A operands of dP^T = V dO^T
  auto load_v = [&](int64_t sr, int p, QT (&vb)[2]) {
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v + sr * D, kv_bytes);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int key = kw0 + 32 * p + 8 * (c >> 2) + 4 * e + (c & 3);
      const uint32_t off = (uint32_t)(key * D + g * QL) * 2;
      if constexpr (D == 32) vb[e] = buf_ld16(rv, off);
      else vb[e] = buf_ld8(rv, off);
    }
  };
  // the workgroup's dQ rows of slice o: item tid of the summed tile, stored in the key
  // range's FP32 partial; rows past N fall outside the descriptor's extent
  const int64_t part_rows = (int64_t)a.B * N_o * H * N;
  auto store_dq = [&](int64_t sr, f32x4 v) {
    if (tid < RED) {
      const int row = tid / (D / 4), c4 = tid % (D / 4);
      const __amdgpu_buffer_rsrc_t rs =
          make_rsrc(a.dq_partial + (r * part_rows + sr + q0) * D, (uint32_t)(N - q0) * D * 4);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, (uint32_t)(row * D + 4 * c4) * 4,
                                             0, 0);
    }
  };

  // ---- prologue: slice o0 staged, V of its first pair in registers
  QT vcur[2], vnxt[2];
  const float* mrow = MASK ? a.mask + ((int64_t)b * N_o + o0) * N : nullptr;   // slice o0's mask row
  stage(sr0, mrow, 0);
  load_v(sr0, 0, vcur);
  __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
  lds_barrier();

  f32x4 red = f32x4{0.f, 0.f, 0.f, 0.f};
  int64_t sr = sr0;                              // slice o0 + s's row offset
  for (int s = 0; s < ns; ++s, sr += hn) {
    const int buf = s & 1;
    if (s > 0) {
      // slice o0 + s's tiles landed (each wave's own loads) and visible to all; every wave
      // has read the previous dQ^T tiles
      __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
      lds_barrier();
      store_dq(sr - hn, red);
    }
    if (MASK) mrow += N;
    if (s + 1 < ns) stage(sr + hn, mrow, buf ^ 1);

    // the slice's -lse log2(e) and -delta of the lane's queries
    float nl[NQB];
    f32x4 nd[NQB];
    const auto lq = [](int rr, int cc) { return q_at<D>(rr, cc); };
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      nl[qb] = -sLD[buf][16 * qb + c] * kLog2e;
      const float dl = -sLD[buf][64 + 16 * qb + c];
      nd[qb] = f32x4{dl, dl, dl, dl};
    }
    f32x4 dq[NDB][NQB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) dq[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};

    const uint16_t* kt = sK[buf][w];
    const auto lk = [](int rr, int cc) { return Lay<D>::k(rr, cc); };
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      // the query operands are read again for every pair (16 VGPRs fewer live across the
      // slice; the compiler barrier keeps them from being merged with the previous pair's)
      asm volatile("" ::: "memory");
      // V of the next pair, or of the next slice's first pair
      if (p + 1 < NP) load_v(sr, p + 1, vnxt);
      else if (s + 1 < ns) load_v(sr + hn, 0, vnxt);
      if (kw0 + 32 * p < N) {      // wave-uniform: the pair holds keys
        QT ka[2];
        f32x4 mk[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          ka[e] = ld_op<D>(kt, 32 * p + 8 * (c >> 2) + 4 * e + (c & 3), g * QL, lk);
          if constexpr (MASK) mk[e] = *reinterpret_cast<const f32x4*>(&sM[buf][w][32 * p + 8 * g + 4 * e]);
        }
        u32x4 kT[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const int kr = 32 * p + 8 * g + trk, kc = 16 * db + 4 * tra;
          kT[db] = ds_read_tr8_at(kt, Lay<D>::k(kr, kc), Lay<D>::k(kr + 4, kc));
        }
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          // B operands of the S^T and dP^T products: the query block's Q and dO rows
          const QT qa = ld_op<D>(sQ[buf], 16 * qb + c, g * QL, lq);
          const QT da = ld_op<D>(sdO[buf], 16 * qb + c, g * QL, lq);
          float ds[2][4];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            f32x4 cin = bp[p][e][qb];
            if constexpr (MASK) {
#pragma unroll
              for (int i = 0; i < 4; ++i) cin[i] = fmaf(mk[e][i], inv_s, cin[i]);
            }
            const f32x4 sv = DOp<D>::mma(ka[e], qa, cin);            // q.k + (bias + mask) / scale
            const f32x4 dp = DOp<D>::mma(vcur[e], da, nd[qb]);       // dP - delta
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float pr = __builtin_amdgcn_exp2f(fmaf(sv[i], c1, nl[qb]));
              ds[e][i] = pr * dp[i];
              dbacc[p][e][qb][i] += ds[e][i];
            }
          }
          const u32x4 bs = u32x4{pack_bf16(ds[0][0], ds[0][1]), pack_bf16(ds[0][2], ds[0][3]),
                                 pack_bf16(ds[1][0], ds[1][1]), pack_bf16(ds[1][2], ds[1][3])};
#pragma unroll
          for (int db = 0; db < NDB; ++db) dq[db][qb] = mfma_k32(kT[db], bs, dq[db][qb]);
        }
      }
      if (p + 1 < NP || s + 1 < ns) {
        vcur[0] = vnxt[0];
        vcur[1] = vnxt[1];
      }
    }

    // the waves' dQ^T tiles (d = 16db + 4g + i, query 16qb + c) meet in LDS, [query][d]
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
        *reinterpret_cast<f32x4*>(&sRed[w][(16 * qb + c) * RP + 16 * db + 4 * g]) = dq[db][qb];
    lds_barrier();
    if (tid < RED) {
      const int row = tid / (D / 4), c4 = tid % (D / 4);
      f32x4 acc = *reinterpret_cast<const f32x4*>(&sRed[0][row * RP + 4 * c4]);
#pragma unroll
      for (int ww = 1; ww < NW; ++ww) acc += *reinterpret_cast<const f32x4*>(&sRed[ww][row * RP + 4 * c4]);
      red = acc * scale;
    }
  }
  store_dq(sr0 + (ns - 1) * hn, red);

  // ---- this group's dbias partial of the (query, key) block: keys 32p + 8g + 4e + 0..3 of
  // the wave at query 16qb + c; entries past N fall outside the plane's extent
  float* plane = a.dbias_partial + (((int64_t)l * a.B + b) * H + h) * N * N;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(plane, (uint32_t)N * N * 4);
#pragma unroll
  for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const int q = q0 + 16 * qb + c;
        const int k = kw0 + 32 * p + 8 * g + 4 * e;
        if ((N & 3) == 0) {
          const uint32_t off = q < N && k < N ? (uint32_t)(q * N + k) * 4 : 0xFFFFF000u;
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, dbacc[p][e][qb]), rs, off, 0, 0);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t off = q < N && k + i < N ? (uint32_t)(q * N + k + i) * 4 : 0xFFFFF000u;
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dbacc[p][e][qb][i]), rs, off, 0, 0);
          }
        }
      }
}

template <int D, bool MASK, int NW, int NP>
static hipError_t launch_bwdq_t(const BwdQArgs& a, hipStream_t s) {
  const int64_t nunit = (int64_t)a.B * a.H * a.p.n_groups;
  const int64_t nblk = 8 * ((nunit + 7) / 8) * a.p.n_qt * a.p.n_ranges;
  hipLaunchKernelGGL((bwdq_kernel<D, MASK, NW, NP>), dim3((unsigned)nblk), dim3(NW * 64), 0, s, a);
  return hipGetLastError();
}

template <int D, bool MASK>
static hipError_t launch_bwdq_d(const BwdQArgs& a, hipStream_t s) {
  const int nw = a.p.nw, np = a.p.np;
  if (nw == 4 && np == 1) return launch_bwdq_t<D, MASK, 4, 1>(a, s);
  if (nw == 4 && np == 2) return launch_bwdq_t<D, MASK, 4, 2>(a, s);
  if (nw == 4 && np == 3) return launch_bwdq_t<D, MASK, 4, 3>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_bwdq(const BwdQArgs& a, int D, hipStream_t s) {
  const bool mask = a.mask != nullptr;
  if (D == 32) return mask ? launch_bwdq_d<32, true>(a, s) : launch_bwdq_d<32, false>(a, s);
  if (D == 16) return mask ? launch_bwdq_d<16, true>(a, s) : launch_bwdq_d<16, false>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace tri
