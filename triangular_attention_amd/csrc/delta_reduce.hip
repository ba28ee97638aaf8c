// Streaming kernels: the compensated softmax correction and the fixed-order
// reductions of the dQ and dbias partials.
//
// Softmax correction: TurboPairFormer, Figure 7(b) -- a preprocessing kernel
// forms delta_hat = sum_d dO * (O + E) in FP32 from the BF16 output O and the
// BF16 output residual E and writes it to HBM.
// Reductions: Figure 7(d) and Figure 11(a) -- separate kernels add the
// single-writer partials in ascending index order in FP32.
// All three are HBM-bound: coalesced 16-byte loads, no LDS.
#include "common.h"
#include "kernels.h"

namespace tri {

// D/8 lanes per row; each lane accumulates its 8 features in order, then the
// lane partials are combined by a fixed butterfly.
template <int D, bool RES>
__global__ __launch_bounds__(256) void delta_kernel(DeltaArgs a) {
  constexpr int LPR = D / 8;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gid / LPR;
  const int part = (int)(gid % LPR);
  float acc = 0.f;
  if (row < a.rows) {
    const int64_t off = row * D + part * 8;
    const u32x4 o = ld_global<u32x4>(a.o + off);
    const u32x4 d = ld_global<u32x4>(a.d_o + off);
    u32x4 e = u32x4{0, 0, 0, 0};
    if (RES) e = ld_global<u32x4>(a.o_res + off);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x0 = RES ? bf_lo(o[j]) + bf_lo(e[j]) : bf_lo(o[j]);
      const float x1 = RES ? bf_hi(o[j]) + bf_hi(e[j]) : bf_hi(o[j]);
      acc = fmaf(bf_lo(d[j]), x0, acc);
      acc = fmaf(bf_hi(d[j]), x1, acc);
    }
  }
#pragma unroll
  for (int sh = 1; sh < LPR; sh <<= 1) acc = acc + __shfl_xor(acc, sh);
  if (row < a.rows && part == 0) a.delta[row] = acc;
}

// out[i] = bf16(sum_{p=0..P-1} partial[p][i]), p ascending.  Each thread owns 8
// consecutive elements and fetches up to 8 partials at a time (independent
// loads in flight), then adds them strictly in index order.  The partials are
// read once: nontemporal loads.
__global__ __launch_bounds__(256) void reduce_kernel(ReduceArgs a) {
  const int64_t i8 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (i8 >= a.elems) return;
  if (i8 + 8 <= a.elems && (a.elems % 4) == 0) {
    const f32x4* src = reinterpret_cast<const f32x4*>(a.partial + i8);
    const int64_t pstride = a.elems / 4;        // in f32x4 units
    f32x4 acc0 = __builtin_nontemporal_load(src), acc1 = __builtin_nontemporal_load(src + 1);
    int p = 1;
    for (; p + 8 <= a.n_partials; p += 8) {
      f32x4 x0[8], x1[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        x0[u] = __builtin_nontemporal_load(src + (p + u) * pstride);
        x1[u] = __builtin_nontemporal_load(src + (p + u) * pstride + 1);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        acc0 += x0[u];
        acc1 += x1[u];
      }
    }
    for (; p < a.n_partials; ++p) {
      acc0 += __builtin_nontemporal_load(src + p * pstride);
      acc1 += __builtin_nontemporal_load(src + p * pstride + 1);
    }
    *reinterpret_cast<u32x4*>(a.out + i8) = u32x4{pack_bf16(acc0[0], acc0[1]), pack_bf16(acc0[2], acc0[3]),
                                                  pack_bf16(acc1[0], acc1[1]), pack_bf16(acc1[2], acc1[3])};
  } else {
    for (int64_t i = i8; i < i8 + 8 && i < a.elems; ++i) {
      float acc = a.partial[i];
      for (int p = 1; p < a.n_partials; ++p) acc += a.partial[(int64_t)p * a.elems + i];
      a.out[i] = f_to_bf(acc);
    }
  }
}

template <int D, bool RES>
static hipError_t launch_delta_t(const DeltaArgs& a, hipStream_t s) {
  const int64_t threads = a.rows * (D / 8);
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL((delta_kernel<D, RES>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_delta(const DeltaArgs& a, int D, hipStream_t s) {
  const bool res = a.o_res != nullptr;
  if (D == 32) return res ? launch_delta_t<32, true>(a, s) : launch_delta_t<32, false>(a, s);
  if (D == 16) return res ? launch_delta_t<16, true>(a, s) : launch_delta_t<16, false>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_reduce(const ReduceArgs& a, hipStream_t s) {
  const int64_t threads = (a.elems + 7) / 8;
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace tri
