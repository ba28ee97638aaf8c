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
// operands of dV^T = dO^T P and dK^T = Q^T dS (contraction over queries), so
// only dS needs to be re-laid out (through LDS) for dQ^T = K^T dS^T.  The
// per-query softmax statistics (lse, delta) are per-register values; -delta
// is folded into the accumulator input of the dP product.
#include "common.h"
#include "kernels.h"

namespace tri {

template <int D, bool MASK, bool VEC>
__global__ __launch_bounds__(256) void bwd_kernel(BwdArgs a) {
  constexpr int TK = kBwdKeyTile, TQ = kBwdQueryTile, G = kBwdGroup;
  constexpr int QP = D + 8;     // row-major Q / dO tile pitch
  constexpr int TP = TQ + 8;    // transposed Q^T / dO^T tile pitch
  constexpr int SP = TK + 8;    // dS tile pitch (row = query)
  constexpr int KTP = TK + 8;   // K^T tile pitch (row = feature)
  constexpr int CH = D / 8;
  constexpr int NDB = D / 16;
  typedef typename DOp<D>::T QT;
  constexpr int QL = DOp<D>::kPerLane;

  __shared__ __align__(16) uint16_t sQ[TQ * QP];
  __shared__ __align__(16) uint16_t sdO[TQ * QP];
  __shared__ __align__(16) uint16_t sQt[D * TP];
  __shared__ __align__(16) uint16_t sdOt[D * TP];
  __shared__ __align__(16) uint16_t sdS[TQ * SP];
  __shared__ __align__(16) uint16_t sKt[G][D * KTP];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c = lane & 15;
  const int N = a.N, H = a.H, N_o = a.N_o;
  // blockIdx.x -> (key tile t fastest, then head, outer group, example)
  int bid = blockIdx.x;
  const int t = bid % a.n_key_tiles; bid /= a.n_key_tiles;
  const int h = bid % H; bid /= H;
  const int grp = bid % a.n_groups; bid /= a.n_groups;
  const int b = bid;
  const float scale = a.scale;

  const int key = t * TK + 16 * w + c;   // key column owned by this lane
  const bool kok = key < N;
  const uint16_t* __restrict__ Bs = a.bias + ((int64_t)b * H + h) * N * N;

  int nsl = N_o - grp * G;
  if (nsl > G) nsl = G;

  // per-slice key operands (registers) and K^T tile (LDS), staged once
  QT kB[G], vB[G];
  float mk[G];
  f32x4 dk_acc[G][NDB], dv_acc[G][NDB];
  const int srow = tid / CH, sch = tid % CH;
#pragma unroll
  for (int gs = 0; gs < G; ++gs) {
    QT z = {};
    kB[gs] = z;
    vB[gs] = z;
    mk[gs] = -INFINITY;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      dk_acc[gs][db] = f32x4{0.f, 0.f, 0.f, 0.f};
      dv_acc[gs][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (gs < nsl) {
      const int o = grp * G + gs;
      const int64_t slice = (((int64_t)b * N_o + o) * H + h) * N;
      if (kok) {
        kB[gs] = ld_global<QT>(a.k + (slice + key) * D + g * QL);
        vB[gs] = ld_global<QT>(a.v + (slice + key) * D + g * QL);
        mk[gs] = MASK ? a.mask[((int64_t)b * N_o + o) * N + key] : 0.f;
      }
      if (srow < TK) {
        const int kr = t * TK + srow;
        u32x4 kv = u32x4{0, 0, 0, 0};
        if (kr < N) kv = ld_global<u32x4>(a.k + (slice + kr) * D + sch * 8);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          sKt[gs][(sch * 8 + 2 * j) * KTP + srow] = (uint16_t)(kv[j] & 0xffffu);
          sKt[gs][(sch * 8 + 2 * j + 1) * KTP + srow] = (uint16_t)(kv[j] >> 16);
        }
      }
    }
  }

  const int nqt = (N + TQ - 1) / TQ;

  // register prefetch of the next (query tile, slice) stage
  u32x4 rq, rdo;
  auto prefetch = [&](int j, int gs) {
    const int o = grp * G + gs;
    const int64_t slice = (((int64_t)b * N_o + o) * H + h) * N;
    const int qr = j * TQ + srow;
    rq = u32x4{0, 0, 0, 0};
    rdo = u32x4{0, 0, 0, 0};
    if (srow < TQ && qr < N) {
      rq = ld_global<u32x4>(a.q + (slice + qr) * D + sch * 8);
      rdo = ld_global<u32x4>(a.d_o + (slice + qr) * D + sch * 8);
    }
  };
  auto stage = [&]() {
    if (srow < TQ) {
      *reinterpret_cast<u32x4*>(&sQ[srow * QP + sch * 8]) = rq;
      *reinterpret_cast<u32x4*>(&sdO[srow * QP + sch * 8]) = rdo;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sQt[(sch * 8 + 2 * j) * TP + srow] = (uint16_t)(rq[j] & 0xffffu);
        sQt[(sch * 8 + 2 * j + 1) * TP + srow] = (uint16_t)(rq[j] >> 16);
        sdOt[(sch * 8 + 2 * j) * TP + srow] = (uint16_t)(rdo[j] & 0xffffu);
        sdOt[(sch * 8 + 2 * j + 1) * TP + srow] = (uint16_t)(rdo[j] >> 16);
      }
    }
  };

  if (nsl > 0) prefetch(0, 0);
  for (int j = 0; j < nqt; ++j) {
    // bias of the lane's (query, key) pairs for query tile j, shared by the G slices
    float bb[4][4];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int q = j * TQ + 32 * (qb >> 1) + 8 * g + 4 * (qb & 1) + i;
        bb[qb][i] = (kok && q < N) ? bf_to_f(Bs[(int64_t)q * N + key]) : 0.f;
      }
    f32x4 dbacc[4];   // sum over the group's slices of the FP32 dS, in slice order

#pragma unroll
    for (int gs = 0; gs < G; ++gs) {
      if (gs >= nsl) break;
      const int o = grp * G + gs;
      const int64_t slice = (((int64_t)b * N_o + o) * H + h) * N;

      // per-register softmax statistics: rows 32s + 8g + 4e + 0..3 of block qb = 2s + e
      f32x4 nlse[4], ndel[4];
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        const int q0 = j * TQ + 32 * (qb >> 1) + 8 * g + 4 * (qb & 1);
        if (VEC) {
          if (q0 < N) {
            nlse[qb] = ld_global<f32x4>(a.lse + slice + q0);
            ndel[qb] = ld_global<f32x4>(a.delta + slice + q0);
          } else {
            nlse[qb] = f32x4{INFINITY, INFINITY, INFINITY, INFINITY};
            ndel[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const bool ok = q0 + i < N;
            nlse[qb][i] = ok ? a.lse[slice + q0 + i] : INFINITY;
            ndel[qb][i] = ok ? a.delta[slice + q0 + i] : 0.f;
          }
        }
        nlse[qb] = -nlse[qb] * kLog2e;
        ndel[qb] = -ndel[qb];
      }

      __syncthreads();          // previous stage's LDS readers are done
      stage();
      __syncthreads();          // Q, dO tiles of this stage visible
      if (gs + 1 < nsl) prefetch(j, gs + 1);
      else if (j + 1 < nqt) prefetch(j + 1, 0);

      u32x2 pP[4], pS[4];
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        const int ql = 32 * (qb >> 1) + 8 * (c >> 2) + 4 * (qb & 1) + (c & 3);
        const QT qa = ld_shared<QT>(&sQ[ql * QP + g * QL]);
        const QT da = ld_shared<QT>(&sdO[ql * QP + g * QL]);
        const f32x4 s = DOp<D>::mma(qa, kB[gs], f32x4{0.f, 0.f, 0.f, 0.f});
        const f32x4 dp = DOp<D>::mma(da, vB[gs], ndel[qb]);   // dP - delta
        float p[4], ds[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = fmaf(s[i], scale, bb[qb][i]);
          x += mk[gs];
          p[i] = __builtin_amdgcn_exp2f(fmaf(x, kLog2e, nlse[qb][i]));
          ds[i] = p[i] * dp[i];
        }
        if (gs == 0) {
          dbacc[qb] = f32x4{ds[0], ds[1], ds[2], ds[3]};
        } else {
          dbacc[qb] += f32x4{ds[0], ds[1], ds[2], ds[3]};
        }
        pP[qb] = u32x2{pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3])};
        pS[qb] = u32x2{pack_bf16(ds[0], ds[1]), pack_bf16(ds[2], ds[3])};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int qr = 32 * (qb >> 1) + 8 * g + 4 * (qb & 1) + i;
          const uint32_t wd = pS[qb][i >> 1];
          sdS[qr * SP + 16 * w + c] = (uint16_t)((i & 1) ? (wd >> 16) : (wd & 0xffffu));
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS, contracting over the 64 queries in two steps
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const u32x4 bp = u32x4{pP[2 * st][0], pP[2 * st][1], pP[2 * st + 1][0], pP[2 * st + 1][1]};
        const u32x4 bs = u32x4{pS[2 * st][0], pS[2 * st][1], pS[2 * st + 1][0], pS[2 * st + 1][1]};
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const u32x4 ao = ld_shared<u32x4>(&sdOt[(16 * db + c) * TP + 32 * st + 8 * g]);
          const u32x4 aq = ld_shared<u32x4>(&sQt[(16 * db + c) * TP + 32 * st + 8 * g]);
          dv_acc[gs][db] = mfma_k32(ao, bp, dv_acc[gs][db]);
          dk_acc[gs][db] = mfma_k32(aq, bs, dk_acc[gs][db]);
        }
      }
      __syncthreads();          // the whole dS tile is in LDS

      // dQ^T (queries 16w..16w+15 of the tile) = K^T dS^T over the 64 keys of this tile
      {
        f32x4 dq[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) dq[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const u32x4 bsd = ld_shared<u32x4>(&sdS[(16 * w + c) * SP + 32 * st + 8 * g]);
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const u32x4 ak = ld_shared<u32x4>(&sKt[gs][(16 * db + c) * KTP + 32 * st + 8 * g]);
            dq[db] = mfma_k32(ak, bsd, dq[db]);
          }
        }
        const int q = j * TQ + 16 * w + c;
        if (q < N) {
          float* dst = a.dq_partial + ((int64_t)t * a.B * N_o * H * N + slice + q) * D;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            *reinterpret_cast<f32x4*>(dst + 16 * db + 4 * g) = dq[db] * scale;
        }
      }
    }

    if (kok) {
      // this group's dbias partial for (query tile j, key tile t)
      float* dst = a.dbias_partial + (((int64_t)grp * a.B + b) * H + h) * N * N;
#pragma unroll
      for (int qb = 0; qb < 4; ++qb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int q = j * TQ + 32 * (qb >> 1) + 8 * g + 4 * (qb & 1) + i;
          if (q < N) dst[(int64_t)q * N + key] = dbacc[qb][i];
        }
    }
  }

  // epilogue: dK = scale * dK^T^T, dV
  if (kok) {
#pragma unroll
    for (int gs = 0; gs < G; ++gs) {
      if (gs < nsl) {
        const int o = grp * G + gs;
        const int64_t row = (((int64_t)b * N_o + o) * H + h) * N + key;
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

template <int D, bool MASK, bool VEC>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t s) {
  const int64_t nblk = (int64_t)a.n_key_tiles * a.H * a.n_groups * a.B;
  hipLaunchKernelGGL((bwd_kernel<D, MASK, VEC>), dim3((unsigned)nblk), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdArgs& a, int D, hipStream_t s) {
  const bool mask = a.mask != nullptr, vec = (a.N % 8) == 0;
#define TRI_BWD_CASE(DD, MM, VV) \
  if (D == DD && mask == MM && vec == VV) return launch_bwd_t<DD, MM, VV>(a, s);
  TRI_BWD_CASE(32, false, true)
  TRI_BWD_CASE(32, true, true)
  TRI_BWD_CASE(32, false, false)
  TRI_BWD_CASE(32, true, false)
  TRI_BWD_CASE(16, false, true)
  TRI_BWD_CASE(16, true, true)
  TRI_BWD_CASE(16, false, false)
  TRI_BWD_CASE(16, true, false)
#undef TRI_BWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace tri
