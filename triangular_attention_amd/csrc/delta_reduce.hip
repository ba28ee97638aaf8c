// Streaming kernels: the compensated softmax correction and the fixed-order
// reductions of the dQ and dbias partials.
//
// Softmax correction: TurboPairFormer, Figure 7(b) -- a preprocessing kernel
// forms delta_hat = sum_d dO * (O + E) in FP32 from the BF16 output O and the
// BF16 output residual E and writes it to HBM.
// Reductions: Figure 7(d) and Figure 11(a) -- separate kernels add the
// single-writer partials in ascending index order in FP32 (FP32 partials, or
// bf16 partials as the pages' Table 2 sizes them).
// All three are HBM-bound: coalesced 16-byte loads, no LDS.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace tri {

// D/8 lanes per row; each lane accumulates its 8 features in order, then the
// lane partials are combined by a fixed butterfly.  O, E and dO are read once
// here: nontemporal loads (measured 20% faster than plain loads).
template <int D, bool RES>
__global__ __launch_bounds__(256) void delta_kernel(DeltaArgs a) {
  constexpr int LPR = D / 8;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t row = gid / LPR;
  const int part = (int)(gid % LPR);
  float acc = 0.f;
  if (row < a.rows) {
    const int64_t off = row * D + part * 8;
    const u32x4 o = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.o + off));
    const u32x4 d = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.d_o + off));
    u32x4 e = u32x4{0, 0, 0, 0};
    if (RES) e = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.o_res + off));
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

// out[i] = bf16(sum_{p=0..P-1} partial[p][i]), p ascending.  Each thread owns EPT
// consecutive elements and fetches the partials in batches of 8 (all loads of a
// batch in flight, the ones past P predicated off), then adds them strictly in
// index order starting from partial 0 (no added zero, so -0 sums stay -0).  The
// partials are read once: nontemporal loads.  Four elements per thread keep
// enough workgroups in flight to stream near the HBM read rate.
template <int EPT>
__global__ __launch_bounds__(256) void reduce_kernel(ReduceArgs a) {
  constexpr int NV = EPT / 4;     // 16-byte vectors per thread and partial
  constexpr int U = 8;            // partials per batch
  const float* partial = static_cast<const float*>(a.partial);
  const int64_t i0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * EPT;
  if (i0 >= a.elems) return;
  if (i0 + EPT <= a.elems && (a.elems % 4) == 0) {
    const f32x4* src = reinterpret_cast<const f32x4*>(partial + i0);
    const int64_t pstride = a.elems / 4;        // in f32x4 units
    f32x4 acc[NV];
    for (int p = 0; p < a.n_partials; p += U) {
      f32x4 x[U][NV];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int v = 0; v < NV; ++v)
          x[u][v] = p + u < a.n_partials ? __builtin_nontemporal_load(src + (p + u) * pstride + v)
                                         : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          if (p + u == 0) acc[v] = x[u][v];
          else if (p + u < a.n_partials) acc[v] += x[u][v];
        }
    }
#pragma unroll
    for (int v = 0; v < NV; ++v)
      *reinterpret_cast<u32x2*>(a.out + i0 + 4 * v) = u32x2{pack_bf16(acc[v][0], acc[v][1]), pack_bf16(acc[v][2], acc[v][3])};
  } else {
    for (int64_t i = i0; i < i0 + EPT && i < a.elems; ++i) {
      float acc = partial[i];
      for (int p = 1; p < a.n_partials; ++p) acc += partial[(int64_t)p * a.elems + i];
      a.out[i] = f_to_bf(acc);
    }
  }
}

// The same sum over bf16 partials (each the RNE rounding of an FP32 partial): eight
// elements per thread, one 16-byte load per partial, FP32 accumulation in ascending
// partial order.
__global__ __launch_bounds__(256) void reduce_bf16_kernel(ReduceArgs a) {
  constexpr int U = 8;            // partials per batch
  const uint16_t* partial = static_cast<const uint16_t*>(a.partial);
  const int64_t i0 = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (i0 >= a.elems) return;
  if (i0 + 8 <= a.elems && (a.elems % 8) == 0) {
    const u32x4* src = reinterpret_cast<const u32x4*>(partial + i0);
    const int64_t pstride = a.elems / 8;        // in 16-byte units
    float acc[8];
    for (int p = 0; p < a.n_partials; p += U) {
      u32x4 x[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        x[u] = p + u < a.n_partials ? __builtin_nontemporal_load(src + (p + u) * pstride) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float y = (e & 1) ? bf_hi(x[u][e >> 1]) : bf_lo(x[u][e >> 1]);
          if (p + u == 0) acc[e] = y;
          else if (p + u < a.n_partials) acc[e] += y;
        }
      }
    }
    *reinterpret_cast<u32x4*>(a.out + i0) = u32x4{pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3]),
                                                   pack_bf16(acc[4], acc[5]), pack_bf16(acc[6], acc[7])};
  } else {
    for (int64_t i = i0; i < i0 + 8 && i < a.elems; ++i) {
      float acc = bf_to_f(partial[i]);
      for (int p = 1; p < a.n_partials; ++p) acc += bf_to_f(partial[(int64_t)p * a.elems + i]);
      a.out[i] = f_to_bf(acc);
    }
  }
}

// Segmented sums for the chunked backward: the same ascending order as reduce_kernel,
// optionally continuing an FP32 running sum carried over from earlier chunks, so that the
// chunked result is bitwise the unchunked one.  VEC: four consecutive elements per thread
// (16-byte loads); otherwise one element per thread.  Blocks [0, job[0].blocks) serve job 0,
// the rest job 1.
template <bool VEC>
__global__ __launch_bounds__(256) void seg_reduce_kernel(SegReduceArgs a) {
  constexpr int EPT = VEC ? 4 : 1;
  constexpr int U = 8;            // partials per batch of loads
  int64_t blk = blockIdx.x;
  const int j = blk < a.job[0].blocks ? 0 : 1;
  if (j == 1) blk -= a.job[0].blocks;
  const SegReduceJob jb = j == 0 ? a.job[0] : a.job[1];
  // whole blocks per segment: the segment and the offset in it come from the (uniform)
  // block index, no per-lane 64-bit division
  const int64_t bps = (jb.seg_len + 256 * EPT - 1) / (256 * EPT);
  const int64_t sg = blk / bps;
  const int64_t i = (blk - sg * bps) * 256 * EPT + threadIdx.x * EPT;
  if (i >= jb.seg_len) return;
  const int64_t e0 = sg * jb.seg_len + i;     // element of the dense running sum
  const float* src = jb.partial + sg * jb.sstride + i;
  typedef typename std::conditional<VEC, f32x4, float>::type V;
  auto ld = [&](const float* p) -> V {
    if constexpr (VEC) return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    else return __builtin_nontemporal_load(p);
  };
  V acc;
  const bool carry = jb.acc_in != nullptr;
  if (carry) {
    if constexpr (VEC) acc = *reinterpret_cast<const f32x4*>(jb.acc_in + e0);
    else acc = jb.acc_in[e0];
  }
  for (int p = 0; p < jb.n_partials; p += U) {
    V x[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (p + u < jb.n_partials) x[u] = ld(src + (int64_t)(p + u) * jb.pstride);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (p + u == 0 && !carry) acc = x[u];
      else if (p + u < jb.n_partials) acc += x[u];
    }
  }
  if (jb.acc_out) {
    if constexpr (VEC) *reinterpret_cast<f32x4*>(jb.acc_out + e0) = acc;
    else jb.acc_out[e0] = acc;
  } else {
    uint16_t* o = jb.out + sg * jb.ostride + i;
    if constexpr (VEC) *reinterpret_cast<u32x2*>(o) = u32x2{pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3])};
    else *o = f_to_bf(acc);
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
  if (D == 64) return res ? launch_delta_t<64, true>(a, s) : launch_delta_t<64, false>(a, s);
  return hipErrorInvalidValue;
}

hipError_t launch_reduce(const ReduceArgs& a, hipStream_t s) {
  if (a.bf16_partials) {
    const int64_t blocks = ((a.elems + 7) / 8 + 255) / 256;
    hipLaunchKernelGGL(reduce_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  constexpr int EPT = 4;   // measured: 4 elements per thread streams faster than 8 for both reductions
  const int64_t threads = (a.elems + EPT - 1) / EPT;
  const int64_t blocks = (threads + 255) / 256;
  hipLaunchKernelGGL(reduce_kernel<EPT>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_seg_reduce(SegReduceArgs a, hipStream_t s) {
  bool vec = true;
  for (int j = 0; j < a.njobs; ++j) {
    const SegReduceJob& jb = a.job[j];
    vec = vec && jb.seg_len % 4 == 0 && jb.pstride % 4 == 0 && jb.sstride % 4 == 0 && jb.ostride % 4 == 0;
  }
  int64_t total = 0;
  for (int j = 0; j < 2; ++j) {
    SegReduceJob& jb = a.job[j];
    jb.vec = vec;
    const int64_t per_block = 256 * (vec ? 4 : 1);
    jb.blocks = j < a.njobs ? jb.nseg * ((jb.seg_len + per_block - 1) / per_block) : 0;
    total += jb.blocks;
  }
  if (total == 0) return hipSuccess;
  if (vec) hipLaunchKernelGGL(seg_reduce_kernel<true>, dim3((unsigned)total), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(seg_reduce_kernel<false>, dim3((unsigned)total), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace tri
