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
// B operand of O^T = V^T P^T.  K and V tiles of 64 keys are staged row-major
// in LDS (double-buffered, shared by the four waves); the V^T operand is read
// with the LDS transposing read.  Bias and mask of the next tile are loaded
// into registers while the current tile is in flight.
#include "common.h"
#include "kernels.h"

namespace tri {

template <int D, bool MASK, bool VEC>
__global__ __launch_bounds__(256) void fwd_kernel(FwdArgs a) {
  constexpr int TQ = kFwdQueryTile, TK = kFwdKeyTile;
  constexpr int KP = D + 8;    // K / V tile pitch (bf16), one row per key
  constexpr int CH = D / 8;    // 16-byte chunks per K/V row
  constexpr int NDB = D / 16;  // 16-wide feature blocks of O
  typedef typename DOp<D>::T QT;
  constexpr int QL = DOp<D>::kPerLane;

  __shared__ __align__(16) uint16_t sK[2][TK * KP];
  __shared__ __align__(16) uint16_t sV[2][TK * KP];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, c = lane & 15;
  const int N = a.N;
  const int qt = blockIdx.x, h = blockIdx.y, bo = blockIdx.z;
  const int b = bo / a.N_o;
  const int64_t slice = ((int64_t)bo * a.H + h) * N;
  const uint16_t* __restrict__ Qs = a.q + slice * D;
  const uint16_t* __restrict__ Ks = a.k + slice * D;
  const uint16_t* __restrict__ Vs = a.v + slice * D;
  const uint16_t* __restrict__ Bs = a.bias + ((int64_t)b * a.H + h) * N * N;
  const float* __restrict__ Ms = MASK ? a.mask + (int64_t)bo * N : nullptr;
  const float scale = a.scale;

  // queries of this lane; rows past N are clamped for loads and never stored
  int qrow[2];
  const uint16_t* brow[2];
  QT qop[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    qrow[qb] = qt * TQ + 32 * w + 16 * qb + c;
    const int ql = qrow[qb] < N ? qrow[qb] : N - 1;
    qop[qb] = ld_global<QT>(Qs + (int64_t)ql * D + g * QL);
    brow[qb] = Bs + (int64_t)ql * N;
  }

  const int srow = tid / CH, sch = tid % CH;   // staging: one 16-byte chunk of a K and a V row
  const bool sact = srow < TK;
  const int nkt = (N + TK - 1) / TK;
  const int nfull = N / TK;                    // tiles with every key in range

  u32x4 rk, rv;
  u32x4 rb[2][2];      // bias [qb][m]: keys 32m + 8g + 0..7 of the tile
  f32x4 rm[2][2];      // mask [m][e]: keys 32m + 8g + 4e + 0..3

  auto load_kv = [&](int kt) {
    const int kr = kt * TK + srow;
    rk = u32x4{0, 0, 0, 0};
    rv = u32x4{0, 0, 0, 0};
    if (sact && kr < N) {
      rk = ld_global<u32x4>(Ks + (int64_t)kr * D + sch * 8);
      rv = ld_global<u32x4>(Vs + (int64_t)kr * D + sch * 8);
    }
  };
  auto load_bm = [&](int kt) {
    const int k0 = kt * TK;
    if (kt < nfull) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int kk = k0 + 32 * m + 8 * g;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          if (VEC) {
            rb[qb][m] = ld_global<u32x4>(brow[qb] + kk);
          } else {
            uint32_t wv[4];
#pragma unroll
            for (int p = 0; p < 4; ++p)
              wv[p] = (uint32_t)brow[qb][kk + 2 * p] | ((uint32_t)brow[qb][kk + 2 * p + 1] << 16);
            rb[qb][m] = u32x4{wv[0], wv[1], wv[2], wv[3]};
          }
        }
        if (MASK) {
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            if (VEC) {
              rm[m][e] = ld_global<f32x4>(Ms + kk + 4 * e);
            } else {
#pragma unroll
              for (int i = 0; i < 4; ++i) rm[m][e][i] = Ms[kk + 4 * e + i];
            }
          }
        }
      }
    } else {
      // last, partial tile: keys past N get a -inf bias (bf16 0xff80)
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int kk = k0 + 32 * m + 8 * g;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          uint32_t wv[4];
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const int k_lo = kk + 2 * p, k_hi = kk + 2 * p + 1;
            const uint32_t lo = k_lo < N ? (uint32_t)brow[qb][k_lo] : 0xff80u;
            const uint32_t hi = k_hi < N ? (uint32_t)brow[qb][k_hi] : 0xff80u;
            wv[p] = lo | (hi << 16);
          }
          rb[qb][m] = u32x4{wv[0], wv[1], wv[2], wv[3]};
        }
        if (MASK) {
#pragma unroll
          for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int kx = kk + 4 * e + i;
              rm[m][e][i] = kx < N ? Ms[kx] : 0.f;
            }
        }
      }
    }
  };
  auto stage = [&](int buf) {
    if (sact) {
      *reinterpret_cast<u32x4*>(&sK[buf][srow * KP + sch * 8]) = rk;
      *reinterpret_cast<u32x4*>(&sV[buf][srow * KP + sch * 8]) = rv;
    }
  };

  float mrun[2] = {-INFINITY, -INFINITY};
  float lsum[2] = {0.f, 0.f};
  f32x4 oacc[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) oacc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};

  load_kv(0);
  load_bm(0);
  stage(0);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nkt;
    if (more) load_kv(kt + 1);

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

    // scores in natural units: s * scale + bias (+ mask)
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
      const float mnew = fmaxf(mrun[qb], tmax);
      const float alpha = __builtin_amdgcn_exp2f((mrun[qb] - mnew) * kLog2e);
      mrun[qb] = mnew;
      const float nm = -mnew * kLog2e;
      lsum[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db][qb] *= alpha;
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

    if (more) stage(cur ^ 1);
    __syncthreads();
  }

  // epilogue: O = bf16(O32), E = bf16(O32 - O), lse = m + log(l)
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
      if (g == 0) a.lse[row] = mrun[qb] + logf(l);
    }
  }
}

template <int D, bool MASK, bool VEC>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t s) {
  dim3 grid((a.N + kFwdQueryTile - 1) / kFwdQueryTile, a.H, a.B * a.N_o);
  hipLaunchKernelGGL((fwd_kernel<D, MASK, VEC>), grid, dim3(256), 0, s, a);
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
