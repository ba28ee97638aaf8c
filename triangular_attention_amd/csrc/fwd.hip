// Forward of triangular attention on gfx950: online softmax over key tiles.
//
// Method: TurboPairFormer (Figure 6 steps 1-4; the forward visits keys in
// tiles and keeps a running row maximum and sum, Table 1's forward tile).
// Output residual: the abstract and Figure 7(b) keep a BF16 approximation of
// the rounding residual of O next to the BF16 output; here E = bf16(O32 - O).
//
// Work split: one workgroup = one (b, o, h) slice and 128 queries; four waves
// of 32 queries each.  Scores are computed transposed, S^T = K Q^T, so that a
// lane owns one query column: the row statistics (max, sum) of a query live
// in one lane plus its three partner lanes, the bias row of a query is read
// as contiguous 16-byte chunks, and the bf16 probability block is already the
// B operand of O^T = V^T P^T.  K and V tiles of 64 keys go from memory
// straight into LDS (row-major, double-buffered, shared by the four waves);
// the V^T operand is read with the LDS transposing read.  Bias and mask of the
// next tile are loaded into registers while the current tile is in flight.
//
// The running maximum is only moved when a tile raises it by more than 8 ln 2:
// until then the probabilities are taken relative to the old maximum (at most
// 2^8, exact in FP32 and bf16), and the accumulator rescale is skipped for the
// whole wave.
//
// Block order: all query tiles of a slice run on one XCD (blocks are dispatched
// round-robin over 8 XCDs), so K and V of the slice are fetched once into that
// XCD's L2; with H = 4 heads each XCD also sees a single head's bias.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace tri {

template <int D, bool MASK, bool VEC>
__global__ __launch_bounds__(256) void fwd_kernel(FwdArgs a) {
  constexpr int TQ = kFwdQueryTile, TK = kFwdKeyTile;
  constexpr int KP = D + 8;    // K / V tile pitch (bf16), one row per key
  constexpr int KCH = KP / 8;  // 16-byte slots per padded row
  constexpr int CH = D / 8;    // 16-byte chunks of data per row
  constexpr int NKPIECE = TK * KCH / 64;   // whole-wave 1 KB pieces per tile
  static_assert(TK * KCH % 64 == 0, "K/V tile must be whole wave pieces");
  constexpr int NDB = D / 16;  // 16-wide feature blocks of O
  constexpr float kRescale = 5.545177444479562f;   // 8 ln 2: growth that forces a rescale
  typedef typename DOp<D>::T QT;
  constexpr int QL = DOp<D>::kPerLane;

  __shared__ __align__(16) uint16_t sK[2][TK * KP];
  __shared__ __align__(16) uint16_t sV[2][TK * KP];

  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int N = a.N;
  const int nqt = (N + TQ - 1) / TQ;

  // XCD-aware unit order: unit = (b*N_o + o)*H + h; its nqt query tiles are
  // consecutive blocks of one XCD
  const int nunit = a.B * a.N_o * a.H;
  const int xcd = blockIdx.x % 8, kx = blockIdx.x / 8;
  const int unit = (kx / nqt) * 8 + xcd;
  if (unit >= nunit) return;
  const int qt = kx % nqt;
  const int h = unit % a.H, bo = unit / a.H;
  const int b = bo / a.N_o;

  const int64_t slice = ((int64_t)bo * a.H + h) * N;
  const uint32_t sbytes = (uint32_t)N * D * 2;
  const __amdgpu_buffer_rsrc_t rQ = make_rsrc(a.q + slice * D, sbytes);
  const __amdgpu_buffer_rsrc_t rK = make_rsrc(a.k + slice * D, sbytes);
  const __amdgpu_buffer_rsrc_t rV = make_rsrc(a.v + slice * D, sbytes);
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(a.bias + ((int64_t)b * a.H + h) * N * N, (uint32_t)N * N * 2);
  const __amdgpu_buffer_rsrc_t rM =
      make_rsrc(MASK ? (const void*)(a.mask + (int64_t)bo * N) : (const void*)a.q, MASK ? (uint32_t)N * 4 : 0u);
  const float scale = a.scale;

  // queries of this lane (rows past N read as zero and are never stored)
  int qrow[2];
  uint32_t boff[2];
  QT qop[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    qrow[qb] = qt * TQ + 32 * w + 16 * qb + c;
    const uint32_t qo = (uint32_t)(qrow[qb] * D + g * QL) * 2;
    if constexpr (D == 32) qop[qb] = buf_ld16(rQ, qo);
    else qop[qb] = buf_ld8(rQ, qo);
    boff[qb] = (uint32_t)qrow[qb] * N * 2;
  }

  const int nkt = (N + TK - 1) / TK;
  const bool ragged = (N % TK) != 0;

  // K and V tiles: whole-wave pieces, lane l of a piece fills 16-byte slot l of the padded
  // tile; padding slots reload the row's first chunk, rows past N read as zero
  auto load_kv = [&](int kt, int buf) {
    for (int pc = w; pc < 2 * NKPIECE; pc += 4) {
      const int which = pc / NKPIECE, piece = pc % NKPIECE;
      const int slot = piece * 64 + lane, row = slot / KCH, ch = slot % KCH;
      const uint32_t off = (uint32_t)((kt * TK + row) * D + (ch < CH ? ch : 0) * 8) * 2;
      buf_to_lds16(which ? rV : rK, (which ? sV[buf] : sK[buf]) + piece * 512, off);
    }
  };

  u32x4 rb[2][2];      // bias [qb][m]: keys 32m + 8g + 0..7 of the tile
  f32x4 rm[2][2];      // mask [m][e]: keys 32m + 8g + 4e + 0..3
  auto load_bm = [&](int kt) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int kk = kt * TK + 32 * m + 8 * g;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        if (VEC) {
          rb[qb][m] = buf_ld16(rB, boff[qb] + (uint32_t)kk * 2);
        } else {
          uint32_t wv[4];
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const uint32_t o2 = boff[qb] + (uint32_t)(kk + 2 * p) * 2;
            wv[p] = (uint32_t)buf_ld2(rB, o2) | ((uint32_t)buf_ld2(rB, o2 + 2) << 16);
          }
          rb[qb][m] = u32x4{wv[0], wv[1], wv[2], wv[3]};
        }
      }
      if (MASK) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          if (VEC) {
            rm[m][e] = __builtin_bit_cast(f32x4, buf_ld16(rM, (uint32_t)(kk + 4 * e) * 4));
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) rm[m][e][i] = __uint_as_float(buf_ld4(rM, (uint32_t)(kk + 4 * e + i) * 4));
          }
        }
      }
    }
  };

  float mref[2] = {-INFINITY, -INFINITY};   // reference maximum (natural units)
  float lsum[2] = {0.f, 0.f};
  f32x4 oacc[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) oacc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one key tile; TAIL = the last tile has keys past N (their scores become -inf)
  auto tile = [&](int kt, auto tail_tag) {
    constexpr bool TAIL = decltype(tail_tag)::value;
    const int cur = kt & 1;
    const bool more = kt + 1 < nkt;

    // S^T blocks: rows = keys 32m + 8(r/4) + 4e + (r%4), so that lane group g
    // holds keys 32m + 8g + 4e + 0..3 (contiguous bias/mask, and the V^T slots)
    f32x4 sacc[2][2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int kl = 32 * m + 8 * (c >> 2) + 4 * e + (c & 3);
        const QT ka = ld_shared<QT>(&sK[cur][kl * KP + g * QL]);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          sacc[qb][m][e] = DOp<D>::mma(ka, qop[qb], f32x4{0.f, 0.f, 0.f, 0.f});
      }

    // scores: s * scale + bias (+ mask)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t wd = rb[qb][m][2 * e + (i >> 1)];
            const float bv = (i & 1) ? bf_hi(wd) : bf_lo(wd);
            float x = fmaf(sacc[qb][m][e][i], scale, bv);
            if (MASK) x += rm[m][e][i];
            if (TAIL) {
              const int kx2 = kt * TK + 32 * m + 8 * g + 4 * e + i;
              x = kx2 < N ? x : -INFINITY;
            }
            sacc[qb][m][e][i] = x;
          }
    if (more) load_bm(kt + 1);

    u32x4 pp[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float tmax = -INFINITY;
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, sacc[qb][m][e][i]);
      tmax = wave_max_groups(tmax);
      if (__any(tmax > mref[qb] + kRescale)) {
        const float mnew = fmaxf(mref[qb], tmax);
        const float alpha = __builtin_amdgcn_exp2f((mref[qb] - mnew) * kLog2e);
        mref[qb] = mnew;
        lsum[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db][qb] *= alpha;
      }
      const float nm = -mref[qb] * kLog2e;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        float p[2][4];
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            p[e][i] = __builtin_amdgcn_exp2f(fmaf(sacc[qb][m][e][i], kLog2e, nm));
            lsum[qb] += p[e][i];
          }
        pp[qb][m] = u32x4{pack_bf16(p[0][0], p[0][1]), pack_bf16(p[0][2], p[0][3]),
                          pack_bf16(p[1][0], p[1][1]), pack_bf16(p[1][2], p[1][3])};
      }
    }

    // O^T += V^T P^T: contraction over the 32 keys of group m; V^T by transposing reads
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const u32x4 va = ds_read_tr8<KP>(&sV[cur][(32 * m + 8 * g) * KP + 16 * db], lane);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) oacc[db][qb] = mfma_k32(va, pp[qb][m], oacc[db][qb]);
      }

    // the next tile's direct loads were issued after the previous barrier
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    __syncthreads();
    if (kt + 2 < nkt) load_kv(kt + 2, cur);
  };

  load_kv(0, 0);
  load_bm(0);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  if (nkt > 1) load_kv(1, 1);

  const int nfull = ragged ? nkt - 1 : nkt;
  for (int kt = 0; kt < nfull; ++kt) tile(kt, std::integral_constant<bool, false>{});
  if (ragged) tile(nkt - 1, std::integral_constant<bool, true>{});

  // epilogue: O = bf16(O32), E = bf16(O32 - O), lse = m + log l
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l = wave_sum_groups(lsum[qb]);
    const float inv = 1.0f / l;
    if (qrow[qb] < N) {
      const int64_t row = slice + qrow[qb];
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const float o0 = oacc[db][qb][0] * inv, o1 = oacc[db][qb][1] * inv;
        const float o2 = oacc[db][qb][2] * inv, o3 = oacc[db][qb][3] * inv;
        const uint32_t w01 = pack_bf16(o0, o1), w23 = pack_bf16(o2, o3);
        *reinterpret_cast<u32x2*>(a.o + row * D + 16 * db + 4 * g) = u32x2{w01, w23};
        if (a.o_res) {
          const uint32_t r01 = pack_bf16(o0 - bf_lo(w01), o1 - bf_hi(w01));
          const uint32_t r23 = pack_bf16(o2 - bf_lo(w23), o3 - bf_hi(w23));
          *reinterpret_cast<u32x2*>(a.o_res + row * D + 16 * db + 4 * g) = u32x2{r01, r23};
        }
      }
      if (g == 0) a.lse[row] = mref[qb] + logf(l);
    }
  }
}

template <int D, bool MASK, bool VEC>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t s) {
  const int64_t nunit = (int64_t)a.B * a.N_o * a.H;
  const int64_t nqt = (a.N + kFwdQueryTile - 1) / kFwdQueryTile;
  const int64_t nblk = 8 * ((nunit + 7) / 8) * nqt;
  hipLaunchKernelGGL((fwd_kernel<D, MASK, VEC>), dim3((unsigned)nblk), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, int D, hipStream_t s) {
  const bool mask = a.mask != nullptr, vec = (a.N % 8) == 0;
#define TRI_FWD_CASE(DD, MM, VV) \
  if (D == DD && mask == MM && vec == VV) return launch_fwd_t<DD, MM, VV>(a, s);
  TRI_FWD_CASE(32, false, true)
  TRI_FWD_CASE(32, true, true)
  TRI_FWD_CASE(32, false, false)
  TRI_FWD_CASE(32, true, false)
  TRI_FWD_CASE(16, false, true)
  TRI_FWD_CASE(16, true, true)
  TRI_FWD_CASE(16, false, false)
  TRI_FWD_CASE(16, true, false)
#undef TRI_FWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace tri
