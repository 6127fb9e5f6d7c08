// Tile-level building blocks shared by the attention kernels (fused
// attention, differential attention, Evoformer gated attention).
//
// Layout conventions (one wave, 32 query rows; lane l = 32*hh + l32):
//  * S^T block = K_blk (32 keys x d) . Q^T (d x 32 queries), 32x32x16 bf16
//    MFMA.  Lane l holds query l32 and keys 8*(j/4) + 4*hh + j%4, j = 0..15,
//    of the 32-key block: one query per lane pair, so row reductions are
//    in-register plus one cross-half swap.
//  * O^T block = V^T (32 d x keys) . P^T (keys x 32 queries).  The P^T
//    operand of k-step t (16 keys) is registers j = 8*(t%2) .. +7 of S^T
//    block t/2 converted to bf16; the matching V^T operand is read from a
//    row-major V tile with two transposed LDS reads.
//  * Scores are in log2 units; the exponent reference m_ref is raised only
//    when a tile max exceeds it by more than 2^kLazyTau.
#pragma once

#include "av_device.hpp"

namespace av {

constexpr float kLazyTau = 8.f;
// Largest tile sum of exponentials accepted without taking the tile max
// (2^64: exponentials, their bf16 copies and the fp32 accumulators stay far
// from overflow).
constexpr float kOptBound = 18446744073709551616.f;

// S^T for key block kb of an LDS K tile (row pitch KP elements), over NSTEP
// k-steps of 16 starting at column c0.
template <int NSTEP, int KP>
__device__ __forceinline__ f32x16 qk_block(const bf16* Ks, int kb, int c0, const bf16x8* qreg, int l32, int hh) {
  f32x16 s = {};
  const bf16* krow = Ks + (kb * 32 + l32) * KP + c0 + hh * 8;
#pragma unroll
  for (int st = 0; st < NSTEP; ++st) s = mfma32(*(const bf16x8*)(krow + st * 16), qreg[st], s);
  return s;
}

// Row-major LDS tile read by transposed reads (V, or W of the projection
// GEMM): W elements per row, no padding.  A transposed read serves 32 lanes
// per pass from 4 consecutive rows (4*q .. 4*q+3) and 32 columns (64 bytes)
// of each; the LDS bank window is 256 bytes, so those 4 row pieces must land
// in 4 distinct 64-byte segments.  Rows of 128 or 256 bytes alone would
// collide, so the 64-byte segments of each row are XOR-swizzled by a function
// of (row mod 4): element column c of row r lives at c ^ (tr_swz<W>(r) * 32).
template <int W>
__device__ __forceinline__ constexpr int tr_swz(int row) {
  return W == 64 ? ((row >> 1) & 1) : W == 128 ? (row & 3) : 0;  // W = 32: rows already 64 bytes apart
}
// Element offset of the 8-element (16-byte) chunk starting at column c (c % 8 == 0).
template <int W>
__device__ __forceinline__ int tr_tile_off(int row, int c) {
  return row * W + (c ^ (tr_swz<W>(row) << 5));
}

// Per-lane parts of the transposed read: rows 4*hh + r/4 (+8), columns
// 16*g + 4*(r%4) of the 32-column block; the swizzle depends only on the
// lane, because every row this lane reads is congruent to 4*hh + r/4 mod 4.
template <int W>
struct TrLane {
  int row0, col0, xo;
  __device__ __forceinline__ explicit TrLane(int lane)
      : row0(4 * (lane >> 5) + ((lane & 15) >> 2)),
        col0(16 * ((lane >> 4) & 1) + 4 * (lane & 3)),
        xo(tr_swz<W>((lane & 15) >> 2) << 5) {}
};

// V^T operand (32 d-columns starting at dcol x 16 keys) of PV k-step t, from
// a swizzled row-major LDS V tile of W columns.
template <int W>
__device__ __forceinline__ bf16x8 vt_operand(const bf16* Vs, int t, int dcol, const TrLane<W>& vl) {
  const bf16* vp = Vs + ((t >> 1) * 32 + 16 * (t & 1) + vl.row0) * W + ((dcol + vl.col0) ^ vl.xo);
  const i16x4 lo = lds_read_tr16(vp);
  const i16x4 hi = lds_read_tr16(vp + 8 * W);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// In-place element mask of one S^T block: keep[off] decides, off = key offset
// of the register inside the 32-key block.
template <typename Keep>
__device__ __forceinline__ void mask_block(f32x16& s, Keep keep) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int off = 8 * (j >> 2) + (j & 3);
    s[j] = keep(off) ? s[j] : neg_inf();
  }
}

// Max over the registers of NB S^T blocks: four independent chains, each
// step folding two new values (one v_max3).
template <int NB>
__device__ __forceinline__ float block_max(const f32x16* s) {
  float mx[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) mx[c] = fmaxf(s[0][2 * c], s[0][2 * c + 1]);
#pragma unroll
  for (int kb = 0; kb < NB; ++kb)
#pragma unroll
    for (int j = (kb == 0 ? 8 : 0); j < 16; j += 2) {
      const int c = (j >> 1) & 3;
      mx[c] = fmaxf(fmaxf(mx[c], s[kb][j]), s[kb][j + 1]);
    }
  return fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
}

// Max of |x| over the registers of NB S^T blocks (abs is a free input
// modifier of v_max3).
template <int NB>
__device__ __forceinline__ float block_absmax(const f32x16* s) {
  float mx[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) mx[c] = fmaxf(fabsf(s[0][2 * c]), fabsf(s[0][2 * c + 1]));
#pragma unroll
  for (int kb = 0; kb < NB; ++kb)
#pragma unroll
    for (int j = (kb == 0 ? 8 : 0); j < 16; j += 2) {
      const int c = (j >> 1) & 3;
      mx[c] = fmaxf(fmaxf(mx[c], fabsf(s[kb][j])), fabsf(s[kb][j + 1]));
    }
  return fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
}

// Online-softmax state of one query row held by a lane pair.  The reference
// m_ref only has to keep the exponentials representable: the softmax is
// exp(x - m) / sum exp(x - m) for ANY common m.
struct RowState {
  float m_ref = neg_inf();  // exponent reference (log2 units), equal in lanes l and l^32
  float m_sub = 0.f;        // m_ref with -inf replaced by 0
  float thr = neg_inf();    // m_ref + kLazyTau: a tile max above it raises the reference
  float l = 0.f;            // this lane's share of the row sum, relative to m_ref

  // Raise the reference to the tile max where it is higher; rescale l and the
  // NO accumulators by the same factor.
  template <int NO>
  __device__ __forceinline__ void raise(float tile_max, f32x16* o) {
    const float m_new = fmaxf(m_ref, tile_max);
    const float m_new_sub = (m_new == neg_inf()) ? 0.f : m_new;
    const float alpha = exp2_fast(m_ref - m_new_sub);
    l *= alpha;
#pragma unroll
    for (int i = 0; i < NO; ++i) o[i] *= alpha;
    m_ref = m_new;
    m_sub = m_new_sub;
    thr = m_new + kLazyTau;
  }
  // Lazy variant: only when some lane's tile max exceeds m_ref by > 2^kLazyTau.
  template <int NO>
  __device__ __forceinline__ void update(float tile_max, f32x16* o) {
    if (any_lane(tile_max > thr)) raise<NO>(tile_max, o);
  }
};

// p = exp2(s * c - m_sub) (MODE 0), exp2(s - m_sub) (MODE 1) or exp2(s)
// (MODE 2) for the registers of NB S^T blocks, packed to bf16 P^T operands
// pb[2*NB]; returns this lane's sum of the bf16 values (EXACT = false: the
// normaliser then equals what the PV product consumes) or of the fp32 values
// (EXACT = true: one more add per two scores, and a log-sum-exp exact to fp32
// rounding).  The sum runs in four independent partial accumulators so the
// chain does not serialise.
template <int NB, int MODE, bool EXACT = false>
__device__ __forceinline__ float exp_pack_sum(const f32x16* s, float c, float m_sub, bf16x8* pb) {
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < NB; ++kb) {
#pragma unroll
    for (int j = 0; j < 16; j += 2) {
      float x0 = s[kb][j], x1 = s[kb][j + 1];
      if constexpr (MODE == 0) {
        x0 = fmaf(x0, c, -m_sub);
        x1 = fmaf(x1, c, -m_sub);
      } else if constexpr (MODE == 1) {
        x0 -= m_sub;
        x1 -= m_sub;
      }
      const float e0 = exp2_fast(x0), e1 = exp2_fast(x1);
      const bf16x2 pp = {(bf16)e0, (bf16)e1};
      if constexpr (EXACT) {
        acc[(j >> 1) & 3] += e0 + e1;
      } else {
        acc[(j >> 1) & 3] = add_bf16_pair(pp, acc[(j >> 1) & 3]);
      }
      pb[kb * 2 + (j >> 3)][j & 7] = pp[0];
      pb[kb * 2 + (j >> 3)][(j & 7) + 1] = pp[1];
    }
  }
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

}  // namespace av
