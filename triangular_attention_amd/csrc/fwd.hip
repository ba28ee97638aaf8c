// Forward of triangular attention on gfx950: online softmax over key tiles.
//
// Method: TurboPairFormer (Figure 6 steps 1-4; the forward visits keys in
// tiles and keeps a running row maximum and sum, Table 1's forward tile).
// Output residual: the abstract and Figure 7(b) keep a BF16 approximation of
// the rounding residual of O next to the BF16 output; here E = bf16(O32 - O).
//
// Work split: one workgroup = one (b, o, h) slice and 128 queries; four waves
// of 32 queries each.  Scores are computed transposed, S^T = K Q^T, so that a
// lane owns one query column, the bias row of a query is read as contiguous
// 16-byte chunks, and the bf16 probability block is already the B operand of
// O^T = V^T P^T; the V^T operand comes from the LDS transposing read.
//
// Data movement: everything a key tile needs (K, V, the 64 mask values and
// the block's 128 x 64 bias tile) is requested one tile ahead with direct
// global->LDS loads into double-buffered LDS, so the loop has no register
// prefetch and one wait (all loads done) plus one barrier per tile.  Per-lane
// 16-byte loads of mask and bias from every wave cost more address-unit time
// than the arithmetic they feed, so the per-key mask is loaded once per
// workgroup.  The loads and their wait remain the largest single cost; the
// exponentials and the matrix products follow.
//
// Score arithmetic, kept short:
//  * bias and mask enter through one exact matrix product per score block:
//    identity (bf16) times the bias block, accumulated onto the mask;
//  * the softmax scale is folded into Q once, as a pair of bf16 terms
//    (hi + lo, relative error about 2^-18), so Q K^T needs no per-score scaling;
//  * there is no per-tile maximum pass: probabilities are taken relative to
//    the running reference maximum, and only when a lane's tile sum reaches
//    2^64 (or at the first tile) is the tile's maximum formed, the
//    accumulators rescaled and the tile's probabilities recomputed.  FP32 and
//    bf16 hold values up to 2^64 with unchanged relative precision, and the
//    common factor cancels in O and in lse.
// Consequence for the inputs: bias entries must be finite (a 0 * inf in the
// identity product would spread NaN); masking goes through the mask.
//
// Block order: all query tiles of a slice run on one XCD (blocks are dispatched
// round-robin over 8 XCDs), so K and V of the slice are fetched once into that
// XCD's L2; with H = 4 heads each XCD also sees a single head's bias.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace tri {

// q * scale as a pair of bf16 terms per element, hi = bf16(x) and lo = bf16(x - hi).
template <typename V>
__device__ __forceinline__ void split_scaled(V q, float scale, V& hi, V& lo) {
  constexpr int n = sizeof(V) / 4;
#pragma unroll
  for (int j = 0; j < n; ++j) {
    const float x0 = bf_lo(q[j]) * scale, x1 = bf_hi(q[j]) * scale;
    const uint32_t hw = pack_bf16(x0, x1);
    hi[j] = hw;
    lo[j] = pack_bf16(x0 - bf_lo(hw), x1 - bf_hi(hw));
  }
}

// LD: width of the direct global->LDS loads of bias rows and mask values.  16: 16-byte
// loads (N % 8 == 0); 4: 4-byte loads (N even); 0: bias and mask through registers (N odd).
template <int D, bool MASK, int LD>
__global__ __launch_bounds__(256, D == 64 ? 2 : 3) void fwd_kernel(FwdArgs a) {
  constexpr int TQ = kFwdQueryTile, TK = kFwdKeyTile;
  constexpr int KP = D;        // K / V tile pitch (bf16), one row per key, 16-byte chunks swizzled
  constexpr int CH = D / 8;    // 16-byte chunks of data per row
  constexpr int NKPIECE = TK * CH / 64;    // whole-wave 1 KB pieces per K (or V) tile
  static_assert(NKPIECE == 2 || NKPIECE == 4 || NKPIECE == 8, "K/V tiles must split over the four waves");
  constexpr int NDB = D / 16;  // 16-wide feature blocks of O
  constexpr float kSumLimit = 0x1p64f;     // tile sum that forces a new reference maximum
  typedef typename DOp<D>::T QT;
  constexpr int QL = DOp<D>::kPerLane;

  // separate arrays per buffer: the compiler can then tell the in-flight
  // direct loads into one buffer from the reads of the other
  __shared__ __align__(16) uint16_t sK0[TK * KP], sK1[TK * KP];
  __shared__ __align__(16) uint16_t sV0[TK * KP], sV1[TK * KP];
  __shared__ __align__(16) float sM0[256], sM1[256];   // mask of the tile (first 64 floats)
  // bias tile: 128 query rows x 64 keys, 128-byte rows with swizzled 16-byte chunks;
  // wave w stages (and alone reads) rows 32w .. 32w + 31
  __shared__ __align__(16) uint16_t sB0[TQ * TK], sB1[TQ * TK];

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
  // register path (odd N): bias planes are only 2-byte aligned, so the descriptor starts
  // at the 4-byte boundary at or below the plane (bextra bytes earlier) and the rows are
  // read as aligned dwords and shifted into place
  const uint16_t* bplane = a.bias + ((int64_t)b * a.H + h) * N * N;
  const uint32_t bextra = (uint32_t)((uintptr_t)bplane & 3u);
  const __amdgpu_buffer_rsrc_t rB =
      make_rsrc((const char*)bplane - bextra, ((uint32_t)N * N * 2 + bextra + 3u) & ~3u);
  const __amdgpu_buffer_rsrc_t rM =
      make_rsrc(MASK ? (const void*)(a.mask + (int64_t)bo * N) : (const void*)a.q, MASK ? (uint32_t)N * 4 : 0u);

  // queries of this lane (rows past N read as zero and are never stored),
  // pre-multiplied by the scale and split into hi + lo bf16 terms
  int qrow[2];
  uint32_t boff[2];
  QT qhi[2], qlo[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    qrow[qb] = qt * TQ + 32 * w + 16 * qb + c;
    const uint32_t qo = (uint32_t)(qrow[qb] * D + g * QL) * 2;
    if constexpr (D == 64) {
      split_scaled(buf_ld16(rQ, qo), a.scale, qhi[qb].x[0], qlo[qb].x[0]);
      split_scaled(buf_ld16(rQ, qo + 16), a.scale, qhi[qb].x[1], qlo[qb].x[1]);
    } else if constexpr (D == 32) {
      split_scaled(buf_ld16(rQ, qo), a.scale, qhi[qb], qlo[qb]);
    } else {
      split_scaled(buf_ld8(rQ, qo), a.scale, qhi[qb], qlo[qb]);
    }
    boff[qb] = (uint32_t)qrow[qb] * N * 2;
  }

  // identity blocks (A operands of 16x16x32 products, one per half e of the 8 bias keys
  // a lane group holds): lane (g, c) holds row c, slots 8g..8g+7, and row c picks slot
  // 4e + (c mod 4) of group c / 4.  (A 16x16x16 product would need half the registers, but
  // gfx950 runs it as long as the 16x16x32 one and the compiler's wait states after it are
  // too short for a dependent read, so this file uses 16x16x32 products only.)
  u32x4 ident[2];
  {
    const int i = c & 3;
    const bool mine = (c >> 2) == g;
    const uint32_t one = (i & 1) ? 0x3F800000u : 0x3F80u;
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) ident[e][wd] = (mine && wd == 2 * e + (i >> 1)) ? one : 0u;
  }

  const int nkt = (N + TK - 1) / TK;
  const bool ragged = (N % TK) != 0;
  // a power-of-two scale (D = 16, 64 with the usual 1/sqrt(D)) makes every lo term exactly
  // zero: its products are skipped (D = 32, 64; D = 16 folds both terms into one product)
  const bool need_lo = (__float_as_uint(a.scale) & 0x7FFFFFu) != 0u;

  // Direct global->LDS loads of a tile, in whole-wave pieces (lane l of a piece fills
  // 16-byte slot l).  K and V tiles are unpadded, with row r stored at row position pr(r)
  // and its 16-byte chunks at positions chunk ^ sw(r) (the source address of each lane is
  // permuted, so the loads stay whole-wave): the K operand reads and the transposing V^T
  // reads then spread over the LDS banks.  With D = 32 each wave loads one K and one V piece, with D = 16 one
  // piece of K (waves 0, 1) or V (waves 2, 3), with D = 64 two pieces of each.  With a mask, wave 0 also loads the tile's
  // 64 mask values (lanes 0..15; the others read zeros past the end of the buffer).  With 16-byte aligned bias
  // rows (N % 8 == 0) each wave then loads its 32 bias rows of the tile (four pieces,
  // chunk position chunk ^ swb(row)); otherwise the bias goes through registers.
  // Tiles beyond N read zeros into the free buffer.  Per-lane offsets are fixed; a tile
  // only adds its key offset.  Everything a tile reads from LDS was requested one tile
  // earlier, and the only wait is vmcnt(0) before the barrier that ends each tile.
  constexpr uint32_t kOOB = 0xFFFFF000u;       // any offset past every buffer
  constexpr bool LDSIN = LD != 0;              // mask and bias through LDS (aligned rows)
  constexpr bool MLDS = MASK && LDSIN;
  // K / V tile layout: row position pr(r) and chunk XOR sw(r).  Per half-wave the K reads
  // touch 16 rows (bits 0-1 and 3-4 varying) at two chunks each and the transposing V^T reads
  // 8 rows (bits 0-1 and 3) at two chunks each.  D = 32 (64-byte rows, 8 rows per 512 bytes):
  // bit 2 of the position flips with bit 4 and the chunk XOR is 2 with bit 3, which puts both
  // on distinct 16-byte slots / 8-byte units.  D = 64 (128-byte rows): the chunk XOR alone
  // (bit 1 -> 2, bit 3 -> 5, bit 4 -> 4) does it.  An involution: pr(pr(r)) = r.
  auto pr = [](int r) {
    if constexpr (D == 32) return r ^ (((r >> 4) & 1) << 2);
    else return r;
  };
  auto sw = [](int r) {
    if constexpr (D == 64) return (((r >> 1) & 1) * 2) ^ (((r >> 3) & 1) * 5) ^ (((r >> 4) & 1) * 4);
    else if constexpr (D == 32) return ((r >> 3) & 1) * 2;
    else return (r >> 3) & (CH - 1);
  };
  // element offset of (row r, column col) in a K or V tile
  auto kv_at = [&](int r, int col) { return pr(r) * KP + (((col >> 3) ^ sw(r)) * 8) + (col & 7); };
  auto swb = [](int r) { return (r >> 1) & 7; };   // bias rows: 8 chunks of 8 keys
  // kv_off[i]: the lane's source offset in the wave's i-th piece (pieces w and w + 4
  // when D = 64)
  uint32_t kv_off[2], m_off, b_off[4];
  {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int piece = NKPIECE == 8 ? w + 4 * i : NKPIECE == 4 ? w : (w & 1);
      // slot (position row, position chunk) holds logical row pr(position row)
      const int row = pr(piece * (64 / CH) + lane / CH), pos = lane % CH;
      kv_off[i] = (uint32_t)(row * D + (pos ^ sw(row)) * 8) * 2;
    }
    if (LD == 4) {
      // 4-byte loads: one load fills two 128-byte bias rows 2i, 2i+1 of the wave; lane l
      // takes row 2i + (l >> 5) and dword l & 31 of it, whose chunk position XOR swb =
      // (l & 31) / 4 XOR (i & 7) names the keys: b_off[0] = the lane's row base, b_off[1]
      // = its dword's byte offset before the XOR
      m_off = MLDS ? (uint32_t)lane * 4 : kOOB;
      b_off[0] = (uint32_t)(qt * TQ + 32 * w + (lane >> 5)) * N * 2;
      b_off[1] = (uint32_t)(lane & 31) * 4;
      b_off[2] = b_off[3] = 0;
    } else {
      m_off = (MLDS && lane < TK / 4) ? (uint32_t)lane * 16 : kOOB;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rl = 8 * j + lane / 8, pos8 = lane % 8;   // row within the wave's 32
        const int q = qt * TQ + 32 * w + rl;
        b_off[j] = (uint32_t)q * N * 2 + (uint32_t)((pos8 ^ swb(rl)) * 16);
      }
    }
  }
  // descriptor words for the untracked direct loads (used when every input of the
  // loop comes through LDS); the tracked form otherwise
  const u32x4 wK = make_rsrc_words(a.k + slice * D, sbytes), wV = make_rsrc_words(a.v + slice * D, sbytes);
  const u32x4 wB = make_rsrc_words(a.bias + ((int64_t)b * a.H + h) * N * N, (uint32_t)N * N * 2);
  const u32x4 wM = make_rsrc_words(MASK ? (const void*)(a.mask + (int64_t)bo * N) : (const void*)a.q,
                                    MASK ? (uint32_t)N * 4 : 0u);
  auto ld2lds = [&](const __amdgpu_buffer_rsrc_t& r, const u32x4& rw, void* dst, uint32_t off) {
    if constexpr (LDSIN) dma16(rw, dst, off);
    else buf_to_lds16(r, dst, off);
  };
  auto load_kv = [&](int kt, uint16_t* dK, uint16_t* dV, float* dM, uint16_t* dB) {
    const bool real = kt < nkt;
    const uint32_t kvo = real ? (uint32_t)(kt * TK * D) * 2 + kv_off[0] : kOOB;
    if constexpr (NKPIECE == 8) {
      const uint32_t kvo1 = real ? (uint32_t)(kt * TK * D) * 2 + kv_off[1] : kOOB;
      ld2lds(rK, wK, dK + w * 512, kvo);
      ld2lds(rK, wK, dK + (w + 4) * 512, kvo1);
      ld2lds(rV, wV, dV + w * 512, kvo);
      ld2lds(rV, wV, dV + (w + 4) * 512, kvo1);
    } else if constexpr (NKPIECE == 4) {
      ld2lds(rK, wK, dK + w * 512, kvo);
      ld2lds(rV, wV, dV + w * 512, kvo);
    } else {
      if (w < 2) ld2lds(rK, wK, dK + (w & 1) * 512, kvo);
      else ld2lds(rV, wV, dV + (w & 1) * 512, kvo);
    }
    // the tile's 64 mask values: one wave, and only when there is a mask (these
    // loads are untracked, so the per-wave load count may differ)
    if constexpr (MLDS) {
      if (LD == 4) {
        // 64 mask values, one per lane; keys past N read past the extent as zeros
        if (w == 0) dma4(wM, dM, real ? (uint32_t)(kt * TK) * 4 + m_off : kOOB);
      } else {
        if (w == 0) dma16(wM, dM, real && m_off != kOOB ? (uint32_t)(kt * TK) * 4 + m_off : kOOB);
      }
    }
    if constexpr (LD == 4) {
      // keys past N (last tile only) must read as zero: pairs of keys are entirely in or
      // out (N even), and rows past N fall outside the plane's extent
      const int klim = N - kt * TK;       // keys of this tile inside N
      // the 16 offsets are formed here from opaque copies of the lane bases, so that the
      // compiler does not hoist them out of the loop into 16 more live registers
      uint32_t rowb = b_off[0], dwb = b_off[1];
      asm volatile("" : "+v"(rowb), "+v"(dwb));
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t x = dwb ^ (uint32_t)(16 * (i & 7));     // byte offset of the lane's keys
        const uint32_t off = rowb + (uint32_t)(2 * i) * N * 2 + (uint32_t)(kt * TK) * 2 + x;
        const bool ok = real && (klim >= TK || (int)(x >> 1) < klim);
        dma4(wB, dB + (32 * w + 2 * i) * TK, ok ? off : kOOB);
      }
    } else if constexpr (LDSIN) {
      const uint32_t bo = (uint32_t)(kt * TK) * 2;
#pragma unroll
      for (int j = 0; j < 4; ++j) dma16(wB, dB + (32 * w + 8 * j) * TK, real ? bo + b_off[j] : kOOB);
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
        // 8 keys from a 2-byte aligned address: five aligned dwords, shifted by 0 or 16 bits
        const uint32_t e0 = bextra + boff[qb] + (uint32_t)kk * 2;
        const uint32_t a0 = e0 & ~3u, sh = (e0 & 2u) << 3;
        uint32_t x[5];
#pragma unroll
        for (int p = 0; p < 5; ++p) x[p] = buf_ld4(rB, a0 + 4u * p);
        rb[qb][m] = u32x4{__builtin_amdgcn_alignbit(x[1], x[0], sh), __builtin_amdgcn_alignbit(x[2], x[1], sh),
                          __builtin_amdgcn_alignbit(x[3], x[2], sh), __builtin_amdgcn_alignbit(x[4], x[3], sh)};
      }
      if (MASK) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
#pragma unroll
          for (int i = 0; i < 4; ++i) rm[m][e][i] = __uint_as_float(buf_ld4(rM, (uint32_t)(kk + 4 * e + i) * 4));
        }
      }
    }
  };

  // D = 16, 32 with every tile in LDS: the lane's byte offsets of its tile reads, formed once.
  // Within a read kind the other reads differ from these by compile-time amounts (m: +32
  // rows; qb: +16 bias rows; e of the mask: +4 floats), so each read is one of these
  // registers plus the instruction's offset field; without them the compiler forms the
  // swizzled addresses again in every tile.
  constexpr bool HOIST = D != 64 && LDSIN;
  uint32_t rbo[2] = {0u, 0u}, kao[2] = {0u, 0u}, vao[2][NDB], rmo = 0u;
  if constexpr (HOIST) {
#pragma unroll
    for (int m = 0; m < 2; ++m) rbo[m] = (uint32_t)((32 * w + c) * TK + (((4 * m + g) ^ swb(c)) * 8)) * 2;
#pragma unroll
    for (int e = 0; e < 2; ++e) kao[e] = (uint32_t)kv_at(8 * (c >> 2) + 4 * e + (c & 3), g * QL) * 2;
    const int k = (lane & 15) >> 2;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi)
#pragma unroll
      for (int db = 0; db < NDB; ++db) vao[hi][db] = (uint32_t)kv_at(8 * g + k + 4 * hi, 16 * db + 4 * (lane & 3)) * 2;
    rmo = (uint32_t)(8 * g) * 4;
    asm volatile("" : "+v"(rbo[0]), "+v"(rbo[1]), "+v"(kao[0]), "+v"(kao[1]), "+v"(rmo));
#pragma unroll
    for (int hi = 0; hi < 2; ++hi)
#pragma unroll
      for (int db = 0; db < NDB; ++db) asm volatile("" : "+v"(vao[hi][db]));
  }
  auto at = [](const void* base, uint32_t off) { return (const uint16_t*)((const char*)base + off); };

  float mref[2] = {-INFINITY, -INFINITY};   // reference maximum (natural units)
  float lsum[2] = {0.f, 0.f};               // this lane's part of the row sum, relative to mref
  f32x4 oacc[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) oacc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // one key tile; TAIL = the last tile has keys past N (their scores become -inf);
  // BUF = which LDS buffer holds the tile
  auto tile = [&](int kt, auto tail_tag, auto buf_tag) {
    constexpr bool TAIL = decltype(tail_tag)::value;
    constexpr int BUF = decltype(buf_tag)::value;
    uint16_t* const tK = BUF ? sK1 : sK0;
    uint16_t* const tV = BUF ? sV1 : sV0;
    float* const tM = BUF ? sM1 : sM0;
    uint16_t* const tB = BUF ? sB1 : sB0;
    if constexpr (HOIST) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int m = 0; m < 2; ++m) rb[qb][m] = ld_shared<u32x4>(at(tB + 16 * qb * TK, rbo[m]));
    } else if constexpr (LDSIN) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int rl = 16 * qb + c, ch = 4 * m + g;
          rb[qb][m] = ld_shared<u32x4>(&tB[(32 * w + rl) * TK + ((ch ^ swb(rl)) * 8)]);
        }
    }
    if constexpr (MLDS) {
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          if constexpr (HOIST) rm[m][e] = *reinterpret_cast<const f32x4*>(at(tM + 32 * m + 4 * e, rmo));
          else rm[m][e] = *reinterpret_cast<const f32x4*>(&tM[32 * m + 8 * g + 4 * e]);
        }
    }

    // S^T blocks: rows = keys 32m + 8(r/4) + 4e + (r%4), so that lane group g
    // holds keys 32m + 8g + 4e + 0..3 (contiguous bias/mask, and the V^T slots).
    // bias + mask first (identity product), then K (scale Q)^T as lo and hi terms.
    f32x4 sacc[2][2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int e = 0; e < 2; ++e)
          sacc[qb][m][e] = mfma_k32(ident[e], rb[qb][m], MASK ? rm[m][e] : f32x4{0.f, 0.f, 0.f, 0.f});
    if constexpr (!LDSIN) {
      if (kt + 1 < nkt) load_bm(kt + 1);
    }

    QT ka[2][2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int kl = 32 * m + 8 * (c >> 2) + 4 * e + (c & 3);
        const int kc = (g * QL) / 8;   // 16-byte chunk of this lane's features
        if constexpr (D == 64) {       // two chunks, each at its own swizzled position
          ka[m][e].x[0] = ld_shared<u32x4>(&tK[kv_at(kl, 8 * kc)]);
          ka[m][e].x[1] = ld_shared<u32x4>(&tK[kv_at(kl, 8 * kc + 8)]);
        } else if constexpr (HOIST) {
          ka[m][e] = ld_shared<QT>(at(tK + 32 * m * KP, kao[e]));
        } else {
          ka[m][e] = ld_shared<QT>(&tK[kv_at(kl, g * QL)]);
        }
      }
    if constexpr (D == 16) {
      // one 16x16x32 product per block takes both terms: slots 8g..8g+3 hold the K
      // features against the hi terms, 8g+4..8g+7 the same features against the lo terms
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const u32x4 kk = u32x4{ka[m][e][0], ka[m][e][1], ka[m][e][0], ka[m][e][1]};
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            sacc[qb][m][e] = mfma_k32(kk, u32x4{qhi[qb][0], qhi[qb][1], qlo[qb][0], qlo[qb][1]}, sacc[qb][m][e]);
        }
    } else {
      if (need_lo) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) sacc[qb][m][e] = DOp<D>::mma(ka[m][e], qlo[qb], sacc[qb][m][e]);
      }
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) sacc[qb][m][e] = DOp<D>::mma(ka[m][e], qhi[qb], sacc[qb][m][e]);
    }

    if (TAIL) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int kx2 = kt * TK + 32 * m + 8 * g + 4 * e + i;
              sacc[qb][m][e][i] = kx2 < N ? sacc[qb][m][e][i] : -INFINITY;
            }
    }

    // V^T operands of the tile: contraction over the 32 keys of group m
    u32x4 va[2][NDB];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        // lane (k, a) of its group: rows r0 + k and r0 + 4 + k, columns 16 db + 4a .. +3
        if constexpr (HOIST) {
          const u32x2 lo = ds_read_tr(at(tV + 32 * m * KP, vao[0][db]));
          const u32x2 hi = ds_read_tr(at(tV + 32 * m * KP, vao[1][db]));
          va[m][db] = u32x4{lo[0], lo[1], hi[0], hi[1]};
        } else {
          const int k = (lane & 15) >> 2, a4 = 16 * db + 4 * (lane & 3);
          const int r0 = 32 * m + 8 * g + k, r1 = r0 + 4;
          va[m][db] = ds_read_tr8_at(tV, kv_at(r0, a4), kv_at(r1, a4));
        }
      }

#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      u32x4 pp[2];
      // probabilities relative to mref, packed to bf16, and their column sums
      auto probs = [&]() {
        const float nm = -mref[qb] * kLog2e;
        // four independent partial sums (by row i of the 4-row groups), combined in a fixed tree
        float ts[4];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          float p[2][4];
#pragma unroll
          for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              p[e][i] = __builtin_amdgcn_exp2f(fmaf(sacc[qb][m][e][i], kLog2e, nm));
              ts[i] = (m == 0 && e == 0) ? p[e][i] : ts[i] + p[e][i];
            }
          pp[m] = u32x4{pack_bf16(p[0][0], p[0][1]), pack_bf16(p[0][2], p[0][3]), pack_bf16(p[1][0], p[1][1]),
                        pack_bf16(p[1][2], p[1][3])};
        }
        return (ts[0] + ts[1]) + (ts[2] + ts[3]);
      };
      // new reference maximum: the tile's maximum (or the old one if larger)
      auto rebase = [&]() {
        float tmax = -INFINITY;
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
          for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, sacc[qb][m][e][i]);
        tmax = wave_max_groups(tmax);
        const float mnew = fmaxf(mref[qb], tmax);
        const float alpha = __builtin_amdgcn_exp2f((mref[qb] - mnew) * kLog2e);
        mref[qb] = mnew;
        lsum[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db][qb] *= alpha;
      };
      float ts;
      if (kt == 0) {
        rebase();
        ts = probs();
      } else {
        ts = probs();
        if (!__all(ts < kSumLimit)) {   // also taken for NaN
          rebase();
          ts = probs();
        }
      }
      lsum[qb] += ts;
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db][qb] = mfma_k32(va[m][db], pp[m], oacc[db][qb]);
    }

    // the next tile's direct loads (and register loads) were issued one tile ago
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    lds_barrier();
    load_kv(kt + 2, tK, tV, tM, tB);
  };

  load_kv(0, sK0, sV0, sM0, sB0);
  if constexpr (!LDSIN) load_bm(0);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  load_kv(1, sK1, sV1, sM1, sB1);

  using F = std::integral_constant<bool, false>;
  using T = std::integral_constant<bool, true>;
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  const int nfull = ragged ? nkt - 1 : nkt;
  int kt = 0;
  for (; kt + 2 <= nfull; kt += 2) {
    tile(kt, F{}, B0{});
    tile(kt + 1, F{}, B1{});
  }
  if (kt < nfull) tile(kt++, F{}, B0{});
  if (ragged) {
    if (kt & 1) tile(kt, T{}, B1{});
    else tile(kt, T{}, B0{});
  }

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

template <int D, bool MASK, int LD>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t s) {
  const int64_t nunit = (int64_t)a.B * a.N_o * a.H;
  const int64_t nqt = (a.N + kFwdQueryTile - 1) / kFwdQueryTile;
  const int64_t nblk = 8 * ((nunit + 7) / 8) * nqt;
  hipLaunchKernelGGL((fwd_kernel<D, MASK, LD>), dim3((unsigned)nblk), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, int D, hipStream_t s) {
  const bool mask = a.mask != nullptr;
  const int ld = bias_load_width(a.N);
#define TRI_FWD_CASE(DD, MM, LL) \
  if (D == DD && mask == MM && ld == LL) return launch_fwd_t<DD, MM, LL>(a, s);
  TRI_FWD_CASE(32, false, 16)
  TRI_FWD_CASE(32, true, 16)
  TRI_FWD_CASE(32, false, 4)
  TRI_FWD_CASE(32, true, 4)
  TRI_FWD_CASE(32, false, 0)
  TRI_FWD_CASE(32, true, 0)
  TRI_FWD_CASE(16, false, 16)
  TRI_FWD_CASE(16, true, 16)
  TRI_FWD_CASE(16, false, 4)
  TRI_FWD_CASE(16, true, 4)
  TRI_FWD_CASE(16, false, 0)
  TRI_FWD_CASE(16, true, 0)
  TRI_FWD_CASE(64, false, 16)
  TRI_FWD_CASE(64, true, 16)
  TRI_FWD_CASE(64, false, 4)
  TRI_FWD_CASE(64, true, 4)
  TRI_FWD_CASE(64, false, 0)
  TRI_FWD_CASE(64, true, 0)
#undef TRI_FWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace tri
