// Shared device helpers for the gfx950 triangular-attention kernels.
//
// MFMA operand convention used by every kernel (v_mfma_f32_16x16x32_bf16):
// lane l = 16*g + c (g = lane group 0..3, c = 0..15).
//   A operand: lane (g, c) supplies row c of A and the contraction slots of group g.
//   B operand: lane (g, c) supplies column c of B and the slots of group g.
//   Result:    lane (g, c) holds rows 4g+0..3 of column c.
// The product sums A-slot (g, j) against B-slot (g, j) over all (g, j), so the
// kernels are free to assign any contraction index to a slot as long as A and
// B agree.  A 16x16 result block in bf16 therefore serves directly as the B
// operand (or, transposed, as the A operand) of a product that contracts over
// the block's rows: slots (g, 0..3) of one block and (g, 4..7) of a second.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tri {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf_to_f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Two floats -> two bf16 (round to nearest even, hardware v_cvt_pk_bf16_f32); a in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  f32x2 v = {a, b};
  bf16x2 r = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ uint16_t f_to_bf(float a) { return (uint16_t)(pack_bf16(a, 0.f) & 0xffffu); }

__device__ __forceinline__ f32x4 mfma_k32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Contraction over the head dimension D (16, 32 or 64) of one 16x16 block.
// For D = 32 each lane supplies 8 values (slots d = 8g..8g+7), for D = 16 four (d = 4g..4g+3),
// for D = 64 sixteen (d = 16g..16g+15: two 16x16x32 products, d = 16g..16g+7 in the first).
template <int D> struct DOp;
struct u32x4x2 {
  u32x4 x[2];
};
template <> struct DOp<64> {
  typedef u32x4x2 T;
  static constexpr int kPerLane = 16;
  __device__ static __forceinline__ f32x4 mma(T a, T b, f32x4 c) {
    return mfma_k32(a.x[1], b.x[1], mfma_k32(a.x[0], b.x[0], c));
  }
};
template <> struct DOp<32> {
  typedef u32x4 T;
  static constexpr int kPerLane = 8;
  __device__ static __forceinline__ f32x4 mma(T a, T b, f32x4 c) { return mfma_k32(a, b, c); }
};
// D = 16 runs as a 16x16x32 product with slots 8g+4..8g+7 zero: on gfx950 it takes as long as
// the 16x16x16 form, and the compiler's wait states after a 16x16x16 product are too short
// for a dependent read of its result.
template <> struct DOp<16> {
  typedef u32x2 T;
  static constexpr int kPerLane = 4;
  __device__ static __forceinline__ f32x4 mma(T a, T b, f32x4 c) {
    return mfma_k32(u32x4{a[0], a[1], 0u, 0u}, u32x4{b[0], b[1], 0u, 0u}, c);
  }
};

// Raw buffer access: 32-bit byte offsets from a uniform base; reads past
// `bytes` return zero, which gives free zero fill for ragged tails.
// A pointer that is the same in every lane, moved to scalar registers (the buffer
// descriptors built from it are then uniform without a per-value loop).
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
  const uint64_t x = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
  return (const T*)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ u32x2 buf_ld8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_ld4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint16_t buf_ld2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

// Buffer -> LDS direct load: lane l's 16 bytes at byte offset `off` land at
// LDS address `lds + 16 * l` (the LDS address must be wave-uniform).
__device__ __forceinline__ void buf_to_lds16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lds), 16, off, 0,
                                           0, 0);
}

// The same direct load issued as inline assembly, invisible to the compiler's
// wait-count bookkeeping.  The compiler tracks every direct load it knows of as a
// pending LDS write and waits for it (vmcnt(0)) before any LDS read it cannot prove
// disjoint, which would serialise a prefetch into one buffer with the reads of the
// other.  The compiler's own counted waits stay correct: a load it tracks cannot
// complete before the younger loads it also tracks, so untracked loads only make
// those waits stricter.
//
// Wait invariant that every caller of dma16 / dma4 keeps (the compiler cannot):
//  1. a wave's direct loads have landed in LDS only after that wave has executed
//     s_waitcnt vmcnt(0): they do not complete in order with register loads, so a
//     counted wait vmcnt(n > 0) is never used to cover them;
//  2. other waves may read the data only after the loading wave's vmcnt(0) is
//     followed by a workgroup barrier (lds_barrier) that the readers also pass;
//  3. a buffer is refilled only after a barrier that every wave reading its previous
//     contents passed after its last read of them (lds_barrier waits lgkmcnt(0), so
//     those reads have returned).
// Forward: each wave issues the loads of tile kt + 2 right after the barrier that
// ends tile kt (into the buffer tile kt used) and waits vmcnt(0) just before the
// barrier that ends tile kt + 1.  Backward: loader set s % 2 issues stage s right
// after the barrier that ends stage s - 3 (into the buffer stage s - 3 used) and
// waits vmcnt(0) just before the barrier that ends stage s - 1; the other set's
// loads stay in flight across that barrier and are waited for a stage later.
// rsrc: buffer descriptor words (wave-uniform); lds: wave-uniform LDS address (M0).
// The compiler does not insert hazard wait states in front of inline assembly, so the
// asm carries its own: on GFX9 a vector-memory instruction that reads an SGPR written
// by a VALU instruction (v_readlane restoring a spilled SGPR, v_readfirstlane) needs 5
// wait states after that write, which also covers the 1 a write of M0 needs before an
// LDS-DMA load.  Without them the load can read a stale descriptor word.
__device__ __forceinline__ u32x4 make_rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  return u32x4{(uint32_t)b, (uint32_t)(b >> 32) & 0xffffu, bytes, 0x00020000u};
}
__device__ __forceinline__ void dma16(u32x4 rsrc, const void* lds, uint32_t off) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)(lds);
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"{m0}"(m0), "v"(off), "s"(rsrc) : "memory");
}

// The 4-byte form (lane l's 4 bytes land at `lds + 4 * l`), for rows that are only
// 4-byte aligned in memory.
__device__ __forceinline__ void dma4(u32x4 rsrc, const void* lds, uint32_t off) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)(lds);
  asm volatile("s_nop 4\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"{m0}"(m0), "v"(off), "s"(rsrc) : "memory");
}

template <typename T> __device__ __forceinline__ T ld_shared(const uint16_t* p) {
  return *reinterpret_cast<const T*>(p);
}
template <typename T> __device__ __forceinline__ T ld_global(const void* p) {
  return *reinterpret_cast<const T*>(p);
}

// LDS transposing read (ds_read_b64_tr_b16).  Within each 16-lane group, lane
// 4k + a (k, a = 0..3) supplies the address of 4 consecutive bf16 of row k of a
// 4 x 16 block (its column chunk a); lane i of the group then receives column i
// of the block, i.e. the four rows' elements at column i.  With rows = the
// contraction index this yields 4 contraction slots of an MFMA operand whose
// row/column index is the lane's position in the group.
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
__device__ __forceinline__ u32x2 ds_read_tr(const uint16_t* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)((__attribute__((address_space(3))) uint16_t*)(p)));
  return __builtin_bit_cast(u32x2, v);
}
// Two transposing reads = one 8-slot operand: rows r0 + 0..3 then r0 + 4..7.
// `base` points at element (r0, col0) of a row-major bf16 tile with `pitch`
// elements per row; the lane's own row/column chunk is added here.
template <int PITCH>
__device__ __forceinline__ u32x4 ds_read_tr8(const uint16_t* base, int lane) {
  const int k = (lane & 15) >> 2, a = lane & 3;
  const uint16_t* p = base + k * PITCH + 4 * a;
  const u32x2 lo = ds_read_tr(p);
  const u32x2 hi = ds_read_tr(p + 4 * PITCH);
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// Cross-group exchange with VALU lane swaps (no LDS): v_permlane16_swap pairs
// rows 0<->1 and 2<->3 of 16 lanes, v_permlane32_swap pairs the two halves;
// with both operands equal to x the two results hold x of lane l and of lane
// l^16 (resp. l^32) in some order.
__device__ __forceinline__ float xor16_pair_max(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_pair_max(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor16_pair_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_pair_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Two transposing reads at explicit element offsets (rows r0 + 0..3 and
// r0 + 4..7 of the lane's column chunk), for tiles with a swizzled layout.
__device__ __forceinline__ u32x4 ds_read_tr8_at(const uint16_t* tile, int off_lo, int off_hi) {
  const u32x2 lo = ds_read_tr(tile + off_lo);
  const u32x2 hi = ds_read_tr(tile + off_hi);
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// Workgroup barrier for LDS tiles filled by direct global->LDS loads.
// __syncthreads() also orders global memory, which makes the compiler wait for
// every outstanding vector-memory load (register prefetches included) before
// the barrier.  Here the caller waits for its direct loads explicitly (vmcnt(0),
// see the wait invariant above), this wave's LDS reads are waited for
// (lgkmcnt(0)), and compiler barriers keep memory accesses on their side.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), other counters unconstrained
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// max over the 4 lane groups that share a column (lanes c, c+16, c+32, c+48)
__device__ __forceinline__ float wave_max_groups(float x) { return xor32_pair_max(xor16_pair_max(x)); }
// fixed order: every lane ends with (x0 + x1) + (x2 + x3) (group sums in row order)
__device__ __forceinline__ float wave_sum_groups(float x) { return xor32_pair_sum(xor16_pair_sum(x)); }

}  // namespace tri
