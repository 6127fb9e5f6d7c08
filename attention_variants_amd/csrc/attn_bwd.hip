// Attention backward for gfx950: dQ, dK, dV of attn_fwd's output.
//
// The pages name training as the other half of the workload their fused
// kernels serve (talk notes "Flashlight: PyTorch Compiler Extensions to
// Accelerate Attention Variants", "Background and motivation").  The
// arithmetic is the chain rule of the forward definition, recomputing P
// instead of storing it:
//   t = mod(scale q.k) (+ mask),  P = softmax(t)
//   dV = P^T dO,   dP = dO V^T,   dT = P (dP - Delta),  Delta = rowsum(P dP)
//   dS = dT mod'(scale q.k)   (softcap: 1 - tanh^2; none / ALiBi: 1)
//   dQ = scale dS K,   dK = scale dS^T Q
// Masks: the forward's five (none, causal, sliding window, PrefixLM,
// document), with the forward's analytic tile ranges on both sides: the
// query-owner launches walk only the key tiles a query tile can see, the
// key-owner launch only the query tiles that can see its keys.
// Three launches over the same forward-shaped and key-owner layouts:
//  1. row statistics: per query row, with the forward's lse only as an
//     exponent reference, l = sum exp(t - lse) and Delta = sum exp(t - lse) dP / l,
//     stored as a corrected reference (lse + ln l, log2 units) and Delta.
//     P recomputed against the corrected reference sums to one in fp32, so
//     neither the forward's bf16 row sum nor its bf16 output enters the
//     gradients (Delta from rowsum(dO O) with a bf16 O cancels badly where
//     attention concentrates).
//  2. dK and dV by workgroups that own a 128-key tile and stream the query
//     tiles of every query head of the KV head;
//  3. dQ by workgroups that own 128 query rows and stream the key tiles.
// P and dS enter the gradient products rounded to bf16, plus their rounding
// residue as a second bf16 operand in the blocks that hold large values.
// No atomics: every output element has one writer (deterministic).

#include <type_traits>

#include "attn_tile.hpp"
#include "av_kernels.hpp"

namespace av {
namespace {

constexpr int NT = 256;
constexpr int D = 64;

// Workgroup -> (tile, b * heads + head) through the document work order of
// attn_doc_order: entry blockIdx.x / heads is a (sequence, 128-row tile)
// pair, heaviest first, and the heads of one pair are consecutive blocks
// (with heads a multiple of 8 every XCD keeps the same heads throughout).
// Under the document mask a 128-key tile spans the same documents as the
// 128-row query tile at its position, so one order serves the key-owner
// launch too.  False for an entry outside B * nT (not an order of this
// shape): the workgroup then touches nothing.
__device__ __forceinline__ bool ordered_tile(const int* order, int heads, int B, int nT, int& tile, int& bh) {
  const int item = order[blockIdx.x / heads];
  if (item < 0 || item >= B * nT) return false;
  tile = item % nT;
  bh = (item / nT) * heads + blockIdx.x % heads;
  return true;
}

// Query rows per statistics workgroup: two 32-row blocks per wave; one under
// the document and sliding-window masks, whose short per-row key ranges
// favour more, smaller workgroups (the forward's tile there, and under the
// document mask the tile of its order).  Same box, S = 4096: sliding window
// 199 -> 185 us; unmasked, causal and PrefixLM within 1 % either way.
template <int MK>
constexpr int stats_bm() {
  return MK == MK_DOC || MK == MK_WINDOW ? 128 : 256;
}
constexpr int NDS = D / 16;   // k-steps over the head dimension
constexpr int NDB = D / 32;   // 32-wide blocks of the head dimension
constexpr int CPR = D / 8;    // 16-byte chunks per row
// A 32 x 32 block of P (or dS) whose largest magnitude exceeds this feeds its
// gradient product as a bf16 hi + lo pair, other blocks as bf16 alone.  A
// dropped residue is at most 2^-9 of its operand, so under 2^-12 in absolute
// terms; its sign follows the inputs, so over N products the sum grows like
// sqrt(N).  Concentrated attention (P near 1 over many queries, the case
// the pairs exist for) always takes the pair.
constexpr float kLoThresh = 0.125f;

// LDS tiles that the gradient kernels read both ways: as 16-byte row pieces
// (the A operand of S and dP) and transposed (the operand of dV^T, dK^T, dQ^T).
// Rows are 128 bytes (D = 64), half of the 256-byte bank window.  A row read
// serves 16 lanes per pass from 16 consecutive rows, so those 16 pieces need
// 16 distinct 16-byte slots; a transposed read serves 32 lanes from 4
// consecutive rows, whose 64-byte pieces need 4 distinct 64-byte segments.
// The 16-byte chunks of row r are XOR-swizzled by pi((r >> 1) mod 8) with
// pi(m) = 4 (m mod 2) + m / 2: a permutation (row reads conflict-free), and
// the two same-parity rows of every aligned group of 4 rows get different
// 64-byte halves (transposed reads conflict-free).  A swizzle of whole 64-byte
// segments serves only the transposed reads and costs the row reads four
// passes each.
static_assert(D == 64, "the dual-read swizzle is laid out for 128-byte rows");
__device__ __forceinline__ int dual_swz(int row) {
  const int m = (row >> 1) & 7;
  return ((m & 1) << 2) | (m >> 1);
}
// Element offset of the 8-element chunk starting at column c (c % 8 == 0).
__device__ __forceinline__ int dual_off(int row, int c) { return row * D + (c ^ (dual_swz(row) << 3)); }

// Per-lane parts of a transposed read of a dual tile: rows base + row0 and
// base + row0 + 8 (base a multiple of 16), columns dcol + col0 .. + 3; the two
// rows take different chunk swizzles, both per-lane constants.
struct DualLane {
  int row0, col0, xlo, xhi;
  __device__ __forceinline__ explicit DualLane(int lane)
      : row0(4 * (lane >> 5) + ((lane & 15) >> 2)),
        col0(16 * ((lane >> 4) & 1) + 4 * (lane & 3)),
        xlo(dual_swz(4 * (lane >> 5) + ((lane & 15) >> 2)) << 3),
        xhi(dual_swz(4 * (lane >> 5) + ((lane & 15) >> 2) + 8) << 3) {}
};

// Transposed operand (32 columns from dcol x 16 rows) of k-step t of a dual tile.
__device__ __forceinline__ bf16x8 dual_vt_operand(const bf16* tile, int t, int dcol, const DualLane& dl) {
  const bf16* rp = tile + ((t >> 1) * 32 + 16 * (t & 1) + dl.row0) * D;
  const i16x4 lo = lds_read_tr16(rp + ((dcol + dl.col0) ^ dl.xlo));
  const i16x4 hi = lds_read_tr16(rp + 8 * D + ((dcol + dl.col0) ^ dl.xhi));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Score pieces shared by both gradient kernels, for one element: raw q.k in
// `s`, query position qp, key position kp.  Returns p = exp(t - lse) (0 when
// masked) and writes the factor mod'(scale q.k) to `dmod`.
// POLY (softcap, a tile inside the cubic's range, bwd_poly_tile): the
// forward's cubic, t = s (p0 + p1 s^2) = cap2 tanh(k s), and mod' = 1 - (t /
// cap2)^2 from it; one exponential per element instead of two and a rcp.
template <int SM, bool POLY = false>
__device__ __forceinline__ float bwd_prob(const BwdArgs& a, float s, float l2, float slope2, float& dmod) {
  if constexpr ((SM == SM_SOFTCAP || SM == SM_SOFTCAP_FIXED) && POLY) {
    const float t = s * fmaf(s * s, a.sc_poly[1], a.sc_poly[0]);
    const float z = t * a.sc_inv_cap2;
    dmod = fmaf(-z, z, 1.f);
    return exp2_fast(t - l2);
  } else if constexpr (SM == SM_SOFTCAP || SM == SM_SOFTCAP_FIXED) {
    // t = cap2 - 2 cap2 u, u = 1 / (1 + 2^(s sc_k)); mod' = 1 - tanh^2 = 4 u (1 - u)
    const float cap2 = a.softcap * kLog2e;
    const float u = rcp_fast(1.f + exp2_fast(s * a.sc_k));
    dmod = 4.f * u * (1.f - u);
    return exp2_fast(fmaf(-2.f * cap2, u, cap2 - l2));
  } else {
    dmod = 1.f;
    return exp2_fast(fmaf(s, a.c, slope2 - l2));
  }
}

// Whether the softcap cubic serves the NB S fragments of a wave: every raw
// score within |raw| <= sc_poly_lim (wave-uniform; NaN fails the test).
template <int SM, int NB>
__device__ __forceinline__ bool bwd_poly_tile(const BwdArgs& a, const f32x16* s) {
  if constexpr (SM == SM_SOFTCAP || SM == SM_SOFTCAP_FIXED) {
    return !any_lane(!(block_absmax<NB>(s) <= a.sc_poly_lim));
  } else {
    return false;
  }
}

// Whether key kp is visible to query q under mask MK (the forward's
// predicates); qd and kd are the two rows' document ids (document mask).
template <int MK>
__device__ __forceinline__ bool bwd_visible(const BwdArgs& a, int q, int kp, int qd, int kd) {
  if constexpr (MK == MK_CAUSAL) return kp <= q;
  // (no short circuit: the callers' element loops stay free of branches)
  if constexpr (MK == MK_WINDOW) return (kp <= q) & (q - kp < a.window);
  if constexpr (MK == MK_PREFIX) return (kp < a.prefix) | (kp <= q);
  if constexpr (MK == MK_DOC) return qd == kd;
  return true;
}

// p where `ok`, else 0, with p computed on every lane first: a plain select
// lets the compiler move p's exponential into a branch per element.
__device__ __forceinline__ float keep_if(bool ok, float p) {
  asm volatile("" : "+v"(p));
  return ok ? p : 0.f;
}

// Whether every key n0..n1 of a tile is visible to every query qw..qwlast of
// a wave (the forward's full-tile classes); kdoc = the tile's key document ids.
template <int MK>
__device__ __forceinline__ bool bwd_tile_full(const BwdArgs& a, int n0, int n1, int qw, int qwlast, const int* kdoc,
                                              int qd_lo, int qd_hi) {
  bool full = n1 < a.Skv;
  if constexpr (MK == MK_CAUSAL) full &= n1 <= qw;
  if constexpr (MK == MK_WINDOW) full &= n1 <= qw && qwlast - n0 < a.window;
  if constexpr (MK == MK_PREFIX) full &= n1 < a.prefix || n1 <= qw;
  if constexpr (MK == MK_DOC) full &= kdoc[0] == qd_lo && kdoc[n1 - n0] == qd_lo && qd_lo == qd_hi;
  return full;
}

// ---------------------------------------------------------------------------
// dK, dV.  Workgroup = 128 keys of one (b, KV head); wave w owns keys
// k0 + 32 w .. +31, held in registers as the B operand of S = Q K^T and
// dP = dO V^T (lane = key).  Query tiles of 128 rows (four 32-row blocks) of
// every query head of the group are staged in LDS, row-major and swizzled,
// and read two ways: rows for the A operand of S and dP, transposed for the
// A operand of dV^T += dO^T P and dK^T += Q^T dS.
template <int SM, int MK>
__global__ __launch_bounds__(NT, 2) void attn_bwd_dkdv_kernel(const BwdArgs a) {
  constexpr int BQ = 128;
  constexpr int QCH = BQ * CPR / NT;  // 16-byte chunks per thread per tensor
  constexpr bool kDoc = MK == MK_DOC;
  __shared__ __attribute__((aligned(16))) bf16 Qs[2][BQ * D];
  __shared__ __attribute__((aligned(16))) bf16 Gs[2][BQ * D];  // dO
  __shared__ __attribute__((aligned(16))) float Ls[2][BQ];     // lse in log2 units (+inf past Sq)
  __shared__ __attribute__((aligned(16))) float Es[2][BQ];     // Delta
  __shared__ __attribute__((aligned(16))) int Dq[2][kDoc ? BQ : 1];  // document ids of the query rows

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hh = lane >> 5, l32 = lane & 31;
  const int nKT = (a.Skv + 127) / 128;
  int kt, bk;
  if constexpr (MK == MK_CAUSAL || MK == MK_PREFIX) {  // key tile 0 is reached by every query: heaviest first
    const TileIdx ti = weighted_tile(blockIdx.x, a.total, nKT);
    kt = ti.mt_lin;
    bk = ti.bh;
  } else if (MK == MK_DOC && a.doc_order != nullptr) {
    if (!ordered_tile(a.doc_order, a.Hkv, a.B, nKT, kt, bk)) return;
  } else {
    const int L = xcd_remap(blockIdx.x, a.total);
    kt = L % nKT;
    bk = L / nKT;
  }
  const int hk = bk % a.Hkv, b = bk / a.Hkv;
  const int k0 = kt * 128;
  const int kw0 = k0 + 32 * w;      // first key of this wave
  const int key = kw0 + l32;        // this lane's key (column of S, dP)

  const size_t kvoff = ((size_t)b * a.Hkv + hk) * (size_t)a.Skv * D;
  const auto krs = make_rsrc((const bf16*)a.k + kvoff, (uint32_t)a.Skv * D * 2);
  const auto vrs = make_rsrc((const bf16*)a.v + kvoff, (uint32_t)a.Skv * D * 2);
  bf16x8 kreg[NDS], vreg[NDS];
#pragma unroll
  for (int s = 0; s < NDS; ++s) {
    kreg[s] = __builtin_bit_cast(bf16x8, buf_load16(krs, (uint32_t)(key * D + s * 16 + hh * 8) * 2));
    vreg[s] = __builtin_bit_cast(bf16x8, buf_load16(vrs, (uint32_t)(key * D + s * 16 + hh * 8) * 2));
  }
  f32x16 dkT[NDB], dvT[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dkT[db] = dvT[db] = f32x16{};
  const DualLane tl(lane);
  const bool key_live = key < a.Skv;
  const int* docrow = kDoc ? a.doc + (size_t)b * a.Skv : nullptr;
  const int kdoc = kDoc ? docrow[min(key, a.Skv - 1)] : 0;
  const int kwlast = min(kw0 + 31, a.Skv - 1);  // last key of this wave
  int kd_lo = 0, kd_hi = 0;                     // document ids of the wave's first and last key
  if constexpr (kDoc) {
    kd_lo = __builtin_amdgcn_readfirstlane(docrow[min(kw0, a.Skv - 1)]);
    kd_hi = __builtin_amdgcn_readfirstlane(docrow[kwlast]);
  }

  // work items: (query head of the group, 64-row query tile), over the query
  // tiles that can see this workgroup's keys [k0, klast]
  const int nQT = (a.Sq + BQ - 1) / BQ;
  const int klast = min(k0 + 127, a.Skv - 1);
  int qt_lo = 0, qt_hi = nQT;
  if constexpr (MK == MK_CAUSAL) {
    qt_lo = k0 / BQ;
  } else if constexpr (MK == MK_WINDOW) {
    qt_lo = k0 / BQ;
    qt_hi = min(nQT, (klast + a.window - 1) / BQ + 1);
  } else if constexpr (MK == MK_PREFIX) {
    qt_lo = k0 < a.prefix ? 0 : k0 / BQ;
  } else if constexpr (MK == MK_DOC) {
    const int qstart = wave_lower_bound(docrow, a.Sq, docrow[k0]);
    const int qend = wave_upper_bound(docrow, a.Sq, docrow[klast]);
    qt_lo = qstart / BQ;
    qt_hi = min(nQT, (qend + BQ - 1) / BQ);
  }
  const int per_head = max(qt_hi - qt_lo, 0);
  const int n_items = a.g * per_head;

  i32x4 qr[QCH], gr[QCH];
  float lr = 0.f, er = 0.f;
  int dr = 0;
  auto gload = [&](int item) {
    const int hq = hk * a.g + item / per_head;
    const int qt = qt_lo + item % per_head;
    const size_t qoff = ((size_t)b * a.Hq + hq) * (size_t)a.Sq * D;
    const auto qrs = make_rsrc((const bf16*)a.q + qoff, (uint32_t)a.Sq * D * 2);
    const auto grs = make_rsrc((const bf16*)a.dout + qoff, (uint32_t)a.Sq * D * 2);
#pragma unroll
    for (int c = 0; c < QCH; ++c) {
      const int idx = tid + NT * c;
      const uint32_t off = (uint32_t)((qt * BQ + idx / CPR) * D + (idx % CPR) * 8) * 2;
      qr[c] = buf_load16(qrs, off);
      gr[c] = buf_load16(grs, off);
    }
    if (tid < BQ) {
      const int q = qt * BQ + tid;
      const size_t r = ((size_t)b * a.Hq + hq) * a.Sq + q;
      lr = q < a.Sq ? a.stats[2 * r] : __builtin_inff();
      er = q < a.Sq ? a.stats[2 * r + 1] : 0.f;
      if constexpr (kDoc) dr = q < a.Sq ? docrow[q] : -1;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int c = 0; c < QCH; ++c) {
      const int idx = tid + NT * c;
      *(i32x4*)&Qs[buf][dual_off(idx / CPR, (idx % CPR) * 8)] = qr[c];
      *(i32x4*)&Gs[buf][dual_off(idx / CPR, (idx % CPR) * 8)] = gr[c];
    }
    if (tid < BQ) {
      Ls[buf][tid] = lr;
      Es[buf][tid] = er;
      if constexpr (kDoc) Dq[buf][tid] = dr;
    }
  };

  if (n_items > 0) gload(0);
  for (int it = 0; it < n_items; ++it) {
    const int buf = it & 1;
    sstore(buf);
    __syncthreads();
    if (it + 1 < n_items) gload(it + 1);
    const int hq = hk * a.g + it / per_head;
    const int qt = qt_lo + it % per_head;
    const float slope2 =
        SM == SM_ALIBI ? uniform_f(kLog2e * exp2f(-a.alibi_max_bias * (float)(hq + 1) / (float)a.Hq)) : 0.f;
#pragma unroll
    for (int blk = 0; blk < BQ / 32; ++blk) {
      const int qb0 = qt * BQ + 32 * blk;  // first query of the block
      const int qblast = qb0 + 31;
      // skip the block when no key of the wave is visible to any of its queries
      bool skip = kw0 >= a.Skv || qb0 >= a.Sq;
      if constexpr (MK == MK_CAUSAL) {
        skip |= kw0 > qblast;
      } else if constexpr (MK == MK_WINDOW) {
        skip |= kw0 > qblast || qb0 - kwlast >= a.window;
      } else if constexpr (MK == MK_PREFIX) {
        skip |= kw0 >= a.prefix && kw0 > qblast;
      } else if constexpr (MK == MK_DOC) {
        const int qd_lo = Dq[buf][32 * blk], qd_hi = Dq[buf][32 * blk + 31];
        skip |= kd_hi < qd_lo || (kd_lo > qd_hi && qd_hi >= 0);
      }
      if (__builtin_amdgcn_readfirstlane((int)skip)) continue;
      // full block: every live key of the wave is visible to every query of
      // the block, so no element mask (keys past Skv are never stored, rows
      // past Sq have p = 0 from their +inf reference)
      bool full = true;
      if constexpr (MK == MK_CAUSAL) {
        full = kwlast <= qb0;
      } else if constexpr (MK == MK_WINDOW) {
        full = kwlast <= qb0 && qblast - kw0 < a.window;
      } else if constexpr (MK == MK_PREFIX) {
        full = kwlast < a.prefix || kwlast <= qb0;
      } else if constexpr (MK == MK_DOC) {
        full = kd_lo == kd_hi && Dq[buf][32 * blk] == kd_lo && Dq[buf][32 * blk + 31] == kd_lo;
      }
      full = __builtin_amdgcn_readfirstlane((int)full) != 0;
      // S = Q K^T, dP = dO V^T: lane = key, registers = queries qb0 + 8(j/4) + 4hh + j%4
      f32x16 sc = {}, dp = {};
#pragma unroll
      for (int s = 0; s < NDS; ++s) {
        const int off = dual_off(32 * blk + l32, s * 16 + hh * 8);
        sc = mfma32(*(const bf16x8*)&Qs[buf][off], kreg[s], sc);
        dp = mfma32(*(const bf16x8*)&Gs[buf][off], vreg[s], dp);
      }
      float pv[16], dsv[16], dmv[16];
      bf16x8 phi[2], dhi[2];
      float pmax = 0.f, dsmax = 0.f;
      auto probs = [&](auto poly) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 l4 = *(const f32x4*)&Ls[buf][32 * blk + 8 * g4 + 4 * hh];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = 4 * g4 + e;
            const int q = qb0 + 8 * g4 + 4 * hh + e;
            const float bias = SM == SM_ALIBI ? slope2 * (float)(key - q) : 0.f;
            pv[j] = bwd_prob<SM, decltype(poly)::value>(a, sc[j], l4[e], bias, dmv[j]);
          }
        }
      };
      if (bwd_poly_tile<SM, 1>(a, &sc)) {
        probs(std::true_type{});
      } else {
        probs(std::false_type{});
      }
      if (!full) {
        i32x4 qd4[4];  // document ids of the block's query rows, four per 16-byte LDS read
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) qd4[g4] = kDoc ? *(const i32x4*)&Dq[buf][32 * blk + 8 * g4 + 4 * hh] : i32x4{};
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int r = 8 * (j >> 2) + 4 * hh + (j & 3);
          pv[j] = keep_if(bwd_visible<MK>(a, qb0 + r, key, qd4[j >> 2][j & 3], kdoc), pv[j]);
        }
      }
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 e4 = *(const f32x4*)&Es[buf][32 * blk + 8 * g4 + 4 * hh];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int j = 4 * g4 + e;
          const float p = pv[j];
          const float ds = p * (dp[j] - e4[e]) * dmv[j];
          dsv[j] = ds;
          pmax = fmaxf(pmax, p);
          dsmax = fmaxf(dsmax, fabsf(ds));
          phi[j >> 3][j & 7] = (bf16)p;
          dhi[j >> 3][j & 7] = (bf16)ds;
        }
      }
      // dV^T += dO^T P, dK^T += Q^T dS (query k-steps in the register order),
      // with P and dS rounded to bf16 ...
#pragma unroll
      for (int d2 = 0; d2 < NDB; ++d2)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          dvT[d2] = mfma32(dual_vt_operand(Gs[buf], 2 * blk + tt, d2 * 32, tl), phi[tt], dvT[d2]);
          dkT[d2] = mfma32(dual_vt_operand(Qs[buf], 2 * blk + tt, d2 * 32, tl), dhi[tt], dkT[d2]);
        }
      // ... plus their rounding residues (the bf16 lo halves) where the block
      // holds a large value: where attention concentrates, the sums over
      // queries of nearly equal P (or dS) cancel the random signs of the
      // inputs, and one bf16 rounding would show in the result.  Below the
      // threshold the residue is under kLoThresh * 2^-9 per product.
      const bool lo_p = any_lane(pmax > kLoThresh), lo_ds = any_lane(dsmax > kLoThresh);
      if (lo_p) {
        bf16x8 plo[2];
#pragma unroll
        for (int j = 0; j < 16; ++j) plo[j >> 3][j & 7] = (bf16)(pv[j] - (float)phi[j >> 3][j & 7]);
#pragma unroll
        for (int d2 = 0; d2 < NDB; ++d2)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
            dvT[d2] = mfma32(dual_vt_operand(Gs[buf], 2 * blk + tt, d2 * 32, tl), plo[tt], dvT[d2]);
      }
      if (lo_ds) {
        bf16x8 dlo[2];
#pragma unroll
        for (int j = 0; j < 16; ++j) dlo[j >> 3][j & 7] = (bf16)(dsv[j] - (float)dhi[j >> 3][j & 7]);
#pragma unroll
        for (int d2 = 0; d2 < NDB; ++d2)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
            dkT[d2] = mfma32(dual_vt_operand(Qs[buf], 2 * blk + tt, d2 * 32, tl), dlo[tt], dkT[d2]);
      }
    }
  }

  // ---- dK = scale dK^T^T, dV: lane holds d = 32 d2 + 8(j/4) + 4hh + j%4 of key `key`
  if (!key_live) return;
  bf16* dkrow = (bf16*)a.dk + kvoff + (size_t)key * D;
  bf16* dvrow = (bf16*)a.dv + kvoff + (size_t)key * D;
#pragma unroll
  for (int d2 = 0; d2 < NDB; ++d2)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      bf16x4 vk, vv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vk[e] = (bf16)(dkT[d2][4 * g4 + e] * a.scale);
        vv[e] = (bf16)dvT[d2][4 * g4 + e];
      }
      *(bf16x4*)(dkrow + d2 * 32 + 8 * g4 + 4 * hh) = vk;
      *(bf16x4*)(dvrow + d2 * 32 + 8 * g4 + 4 * hh) = vv;
    }
}

// ---------------------------------------------------------------------------
// Row statistics (launch 1).  Workgroup = 256 query rows of one (b, query
// head), wave = 64 rows as two 32-row blocks in the forward's layout (128
// rows and one block per wave under the document and window masks, see
// stats_bm):
// S^T = K Q^T and dP^T = V dO^T with Q and dO in registers (lane = query),
// so each K and V fragment read from LDS feeds the MFMAs of both blocks.
// K and V are only read as rows here, so both tiles use the forward's padded
// row pitch.  With the forward's lse only as an exponent reference, the
// pass sums l = sum p and sum p dP per row, p = exp(t - lse).
template <int SM, int MK>
__global__ __launch_bounds__(NT, 2) void attn_bwd_stats_kernel(const BwdArgs a) {
  constexpr int BN = 64;
  constexpr int BM = stats_bm<MK>();
  constexpr int QB = BM / 128;
  constexpr int NCH = BN * CPR / NT;
  constexpr int KP = D + 8;
  constexpr bool kDoc = MK == MK_DOC;
  constexpr bool kWeighted = MK == MK_CAUSAL || MK == MK_PREFIX;
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][BN * KP];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][BN * KP];
  __shared__ __attribute__((aligned(16))) int Dk[2][kDoc ? BN : 1];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hh = lane >> 5, l32 = lane & 31;
  const int nM = (a.Sq + BM - 1) / BM;
  int mt_lin, bh;
  if constexpr (kWeighted) {
    const TileIdx ti = weighted_tile(blockIdx.x, gridDim.x, nM);
    mt_lin = ti.mt_lin;
    bh = ti.bh;
  } else if (kDoc && a.doc_order != nullptr) {
    if (!ordered_tile(a.doc_order, a.Hq, a.B, nM, mt_lin, bh)) return;
  } else {
    const int L = xcd_remap(blockIdx.x, gridDim.x);
    mt_lin = L % nM;
    bh = L / nM;
  }
  const int hq = bh % a.Hq, b = bh / a.Hq;
  const int hk = hq / a.g;
  const int mt = kWeighted ? nM - 1 - mt_lin : mt_lin;
  const int q0 = mt * BM;
  const int qw = q0 + 32 * QB * __builtin_amdgcn_readfirstlane(w);
  int qi[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) qi[qb] = qw + 32 * qb + l32;
  const size_t qoff = ((size_t)b * a.Hq + hq) * (size_t)a.Sq * D;
  const size_t kvoff = ((size_t)b * a.Hkv + hk) * (size_t)a.Skv * D;
  const auto qrs = make_rsrc((const bf16*)a.q + qoff, (uint32_t)a.Sq * D * 2);
  const auto grs = make_rsrc((const bf16*)a.dout + qoff, (uint32_t)a.Sq * D * 2);
  const auto krs = make_rsrc((const bf16*)a.k + kvoff, (uint32_t)a.Skv * D * 2);
  const auto vrs = make_rsrc((const bf16*)a.v + kvoff, (uint32_t)a.Skv * D * 2);
  // rows past Sq read as zero (buffer bounds) and are never stored
  bf16x8 qreg[QB][NDS], greg[QB][NDS];
  float l2[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
    for (int s = 0; s < NDS; ++s) {
      const uint32_t off = (uint32_t)(qi[qb] * D + s * 16 + hh * 8) * 2;
      qreg[qb][s] = __builtin_bit_cast(bf16x8, buf_load16(qrs, off));
      greg[qb][s] = __builtin_bit_cast(bf16x8, buf_load16(grs, off));
    }
    l2[qb] = qi[qb] < a.Sq ? a.lse[((size_t)b * a.Hq + hq) * a.Sq + qi[qb]] * kLog2e : __builtin_inff();
  }
  const float slope2 = SM == SM_ALIBI ? uniform_f(kLog2e * exp2f(-a.alibi_max_bias * (float)(hq + 1) / (float)a.Hq)) : 0.f;

  // the forward's analytic key range of the query tile [q0, qlast]
  const int nKV = (a.Skv + BN - 1) / BN;
  const int qlast = min(q0 + BM - 1, a.Sq - 1);
  const int qwlast = min(qw + 32 * QB - 1, a.Sq - 1);
  const int* docrow = kDoc ? a.doc + (size_t)b * a.Sq : nullptr;
  int n_lo = 0, n_hi = nKV;
  int qdoc[QB] = {};
  int qd_lo = 0, qd_hi = 0;
  if constexpr (MK == MK_CAUSAL) {
    n_hi = min(nKV, qlast / BN + 1);
  } else if constexpr (MK == MK_WINDOW) {
    n_lo = max(0, q0 - a.window + 1) / BN;
    n_hi = min(nKV, qlast / BN + 1);
  } else if constexpr (MK == MK_PREFIX) {
    n_hi = min(nKV, max(a.prefix - 1, qlast) / BN + 1);
  } else if constexpr (MK == MK_DOC) {
    const int kstart = wave_lower_bound(docrow, a.Skv, docrow[q0]);
    const int kend = wave_upper_bound(docrow, a.Skv, docrow[qlast]);
    n_lo = kstart / BN;
    n_hi = min(nKV, (kend + BN - 1) / BN);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) qdoc[qb] = docrow[min(qi[qb], a.Sq - 1)];
    qd_lo = __builtin_amdgcn_readfirstlane(docrow[min(qw, a.Sq - 1)]);
    qd_hi = __builtin_amdgcn_readfirstlane(docrow[max(qwlast, 0)]);
  }

  i32x4 kr[NCH], vr[NCH];
  int dr = 0;
  auto gload = [&](int nt) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int idx = tid + NT * c;
      const uint32_t off = (uint32_t)((nt * BN + idx / CPR) * D + (idx % CPR) * 8) * 2;
      kr[c] = buf_load16(krs, off);
      vr[c] = buf_load16(vrs, off);
    }
    if constexpr (kDoc) {
      if (tid < BN) {
        const int kp = nt * BN + tid;
        dr = kp < a.Skv ? docrow[kp] : 0x7fffffff;
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int idx = tid + NT * c;
      const int off = (idx / CPR) * KP + (idx % CPR) * 8;
      *(i32x4*)&Ks[buf][off] = kr[c];
      *(i32x4*)&Vs[buf][off] = vr[c];
    }
    if constexpr (kDoc) {
      if (tid < BN) Dk[buf][tid] = dr;
    }
  };

  float psum[QB] = {}, pdsum[QB] = {};  // this lane's half of each row
  if (n_lo < n_hi) gload(n_lo);
  for (int nt = n_lo; nt < n_hi; ++nt) {
    const int buf = (nt - n_lo) & 1;
    sstore(buf);
    __syncthreads();
    if (nt + 1 < n_hi) gload(nt + 1);
    const int n0 = nt * BN, n1 = n0 + BN - 1;
    // skip the tile when none of its keys is visible to this wave's queries
    bool skip = qw >= a.Sq;
    if constexpr (MK == MK_CAUSAL) {
      skip |= n0 > qwlast;
    } else if constexpr (MK == MK_WINDOW) {
      skip |= n0 > qwlast || qw - n1 >= a.window;
    } else if constexpr (MK == MK_PREFIX) {
      skip |= n0 >= a.prefix && n0 > qwlast;
    } else if constexpr (MK == MK_DOC) {
      skip |= Dk[buf][BN - 1] < qd_lo || Dk[buf][0] > qd_hi;
    }
    if (__builtin_amdgcn_readfirstlane((int)skip)) continue;
    const bool full = __builtin_amdgcn_readfirstlane((int)bwd_tile_full<MK>(a, n0, n1, qw, qwlast, Dk[buf], qd_lo, qd_hi)) != 0;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // S^T, dP^T of 32 keys: registers = keys n0 + 32 kb + 8(j/4) + 4hh + j%4
      f32x16 sc[QB], dp[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sc[qb] = dp[qb] = f32x16{};
      const bf16* krow = Ks[buf] + (kb * 32 + l32) * KP + hh * 8;
      const bf16* vrow = Vs[buf] + (kb * 32 + l32) * KP + hh * 8;
#pragma unroll
      for (int s = 0; s < NDS; ++s) {
        const bf16x8 kf = *(const bf16x8*)(krow + s * 16);
        const bf16x8 vf = *(const bf16x8*)(vrow + s * 16);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          sc[qb] = mfma32(kf, qreg[qb][s], sc[qb]);
          dp[qb] = mfma32(vf, greg[qb][s], dp[qb]);
        }
      }
      // the element mask only on tiles that are not full (two copies of the
      // accumulation, so that full tiles carry no mask registers)
      i32x4 kd4[4];  // document ids of this lane's keys, four per 16-byte LDS read
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) kd4[g4] = kDoc ? *(const i32x4*)&Dk[buf][kb * 32 + 8 * g4 + 4 * hh] : i32x4{};
      auto accumulate = [&](auto masked, auto poly) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int ko = kb * 32 + 8 * (j >> 2) + 4 * hh + (j & 3);
            const float bias = SM == SM_ALIBI ? slope2 * (float)(n0 + ko - qi[qb]) : 0.f;
            float dmod;
            float p = bwd_prob<SM, decltype(poly)::value>(a, sc[qb][j], l2[qb], bias, dmod);
            if constexpr (decltype(masked)::value) {
              p = keep_if((n0 + ko < a.Skv) & bwd_visible<MK>(a, qi[qb], n0 + ko, qdoc[qb], kd4[j >> 2][j & 3]), p);
            }
            psum[qb] += p;
            pdsum[qb] = fmaf(p, dp[qb][j], pdsum[qb]);
          }
      };
      const bool poly = bwd_poly_tile<SM, QB>(a, sc);
      if (full) {
        if (poly) {
          accumulate(std::false_type{}, std::true_type{});
        } else {
          accumulate(std::false_type{}, std::false_type{});
        }
      } else {
        if (poly) {
          accumulate(std::true_type{}, std::true_type{});
        } else {
          accumulate(std::true_type{}, std::false_type{});
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // one 32-key block of S and dP live at a time
    }
  }

  // corrected reference lse + log2(l) (log2 units) and Delta = sum p dP / l
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lsum = xhalf_sum(psum[qb]), dsum = xhalf_sum(pdsum[qb]);
    if (qi[qb] < a.Sq && hh == 0) {
      const size_t r = ((size_t)b * a.Hq + hq) * a.Sq + qi[qb];
      a.stats[2 * r] = lsum > 0.f ? l2[qb] + __log2f(lsum) : __builtin_inff();
      a.stats[2 * r + 1] = lsum > 0.f ? dsum / lsum : 0.f;
    }
  }
}

// ---------------------------------------------------------------------------
// dQ.  Workgroup = 128 query rows of one (b, query head), wave = 32 rows;
// the forward's layout: S^T = K Q^T and dP^T = V dO^T with Q, dO held in
// registers (lane = query), K and V tiles staged in LDS (swizzled), then
// dQ^T += K^T dS^T with K^T read transposed.
template <int SM, int MK>
__global__ __launch_bounds__(NT, 2) void attn_bwd_dq_kernel(const BwdArgs a) {
  constexpr int BN = 64;
  constexpr int NCH = BN * CPR / NT;
  constexpr bool kDoc = MK == MK_DOC;
  constexpr bool kWeighted = MK == MK_CAUSAL || MK == MK_PREFIX;  // later query tiles see more keys
  __shared__ __attribute__((aligned(16))) bf16 Ks[2][BN * D];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][BN * D];
  __shared__ __attribute__((aligned(16))) int Dk[2][kDoc ? BN : 1];  // document ids of the keys

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hh = lane >> 5, l32 = lane & 31;
  const int nM = (a.Sq + 127) / 128;
  int mt_lin, bh;
  if constexpr (kWeighted) {
    const TileIdx ti = weighted_tile(blockIdx.x, a.total_q, nM);
    mt_lin = ti.mt_lin;
    bh = ti.bh;
  } else if (kDoc && a.doc_order != nullptr) {
    if (!ordered_tile(a.doc_order, a.Hq, a.B, nM, mt_lin, bh)) return;
  } else {
    const int L = xcd_remap(blockIdx.x, a.total_q);
    mt_lin = L % nM;
    bh = L / nM;
  }
  const int hq = bh % a.Hq, b = bh / a.Hq;
  const int hk = hq / a.g;
  const int mt = kWeighted ? nM - 1 - mt_lin : mt_lin;  // heaviest query tiles first
  const int q0 = mt * 128;
  const int qw = q0 + 32 * __builtin_amdgcn_readfirstlane(w);
  const int q = qw + l32;
  const size_t qoff = ((size_t)b * a.Hq + hq) * (size_t)a.Sq * D;
  const size_t kvoff = ((size_t)b * a.Hkv + hk) * (size_t)a.Skv * D;
  const auto qrs = make_rsrc((const bf16*)a.q + qoff, (uint32_t)a.Sq * D * 2);
  const auto grs = make_rsrc((const bf16*)a.dout + qoff, (uint32_t)a.Sq * D * 2);
  const auto krs = make_rsrc((const bf16*)a.k + kvoff, (uint32_t)a.Skv * D * 2);
  const auto vrs = make_rsrc((const bf16*)a.v + kvoff, (uint32_t)a.Skv * D * 2);
  bf16x8 qreg[NDS], greg[NDS];
#pragma unroll
  for (int s = 0; s < NDS; ++s) {
    qreg[s] = __builtin_bit_cast(bf16x8, buf_load16(qrs, (uint32_t)(q * D + s * 16 + hh * 8) * 2));
    greg[s] = __builtin_bit_cast(bf16x8, buf_load16(grs, (uint32_t)(q * D + s * 16 + hh * 8) * 2));
  }
  const bool q_live = q < a.Sq;
  const size_t rrow = ((size_t)b * a.Hq + hq) * a.Sq + (q_live ? q : 0);
  // exponent reference (log2 units) and Delta from the statistics pass
  float l2 = __builtin_inff(), dl = 0.f;
  if (q_live) {
    l2 = a.stats[2 * rrow];
    dl = a.stats[2 * rrow + 1];
  }
  const float slope2 = SM == SM_ALIBI ? uniform_f(kLog2e * exp2f(-a.alibi_max_bias * (float)(hq + 1) / (float)a.Hq)) : 0.f;

  f32x16 dqT[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dqT[db] = f32x16{};
  const DualLane tl(lane);

  // the forward's analytic key range of the query tile [q0, qlast]
  const int nKV = (a.Skv + BN - 1) / BN;
  const int qlast = min(q0 + 127, a.Sq - 1);
  const int qwlast = min(qw + 31, a.Sq - 1);
  const int* docrow = kDoc ? a.doc + (size_t)b * a.Sq : nullptr;
  int n_lo = 0, n_hi = nKV;
  int qdoc = 0, qd_lo = 0, qd_hi = 0;
  if constexpr (MK == MK_CAUSAL) {
    n_hi = min(nKV, qlast / BN + 1);
  } else if constexpr (MK == MK_WINDOW) {
    n_lo = max(0, q0 - a.window + 1) / BN;
    n_hi = min(nKV, qlast / BN + 1);
  } else if constexpr (MK == MK_PREFIX) {
    n_hi = min(nKV, max(a.prefix - 1, qlast) / BN + 1);
  } else if constexpr (MK == MK_DOC) {
    const int kstart = wave_lower_bound(docrow, a.Skv, docrow[q0]);
    const int kend = wave_upper_bound(docrow, a.Skv, docrow[qlast]);
    n_lo = kstart / BN;
    n_hi = min(nKV, (kend + BN - 1) / BN);
    qdoc = docrow[min(q, a.Sq - 1)];
    qd_lo = __builtin_amdgcn_readfirstlane(docrow[min(qw, a.Sq - 1)]);
    qd_hi = __builtin_amdgcn_readfirstlane(docrow[max(qwlast, 0)]);
  }

  i32x4 kr[NCH], vr[NCH];
  int dr = 0;
  auto gload = [&](int nt) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int idx = tid + NT * c;
      const uint32_t off = (uint32_t)((nt * BN + idx / CPR) * D + (idx % CPR) * 8) * 2;
      kr[c] = buf_load16(krs, off);
      vr[c] = buf_load16(vrs, off);
    }
    if constexpr (kDoc) {
      if (tid < BN) {
        const int kp = nt * BN + tid;
        dr = kp < a.Skv ? docrow[kp] : 0x7fffffff;
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int idx = tid + NT * c;
      const int off = dual_off(idx / CPR, (idx % CPR) * 8);
      *(i32x4*)&Ks[buf][off] = kr[c];
      *(i32x4*)&Vs[buf][off] = vr[c];
    }
    if constexpr (kDoc) {
      if (tid < BN) Dk[buf][tid] = dr;
    }
  };

  if (n_lo < n_hi) gload(n_lo);
  for (int nt = n_lo; nt < n_hi; ++nt) {
    const int buf = (nt - n_lo) & 1;
    sstore(buf);
    __syncthreads();
    if (nt + 1 < n_hi) gload(nt + 1);
    const int n0 = nt * BN, n1 = n0 + BN - 1;
    // skip the tile when none of its keys is visible to this wave's queries
    bool skip = qw >= a.Sq;
    if constexpr (MK == MK_CAUSAL) {
      skip |= n0 > qwlast;
    } else if constexpr (MK == MK_WINDOW) {
      skip |= n0 > qwlast || qw - n1 >= a.window;
    } else if constexpr (MK == MK_PREFIX) {
      skip |= n0 >= a.prefix && n0 > qwlast;
    } else if constexpr (MK == MK_DOC) {
      skip |= Dk[buf][BN - 1] < qd_lo || Dk[buf][0] > qd_hi;
    }
    if (__builtin_amdgcn_readfirstlane((int)skip)) continue;
    const bool full = __builtin_amdgcn_readfirstlane((int)bwd_tile_full<MK>(a, n0, n1, qw, qwlast, Dk[buf], qd_lo, qd_hi)) != 0;
    // one 32-key half of the tile at a time (S, dP, dS and its dQ products),
    // so that only one half's scores are live
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // S^T, dP^T: lane = query, registers = keys n0 + 32 kb + 8(j/4) + 4hh + j%4
      f32x16 sc = {}, dp = {};
#pragma unroll
      for (int s = 0; s < NDS; ++s) {
        const int off = dual_off(kb * 32 + l32, s * 16 + hh * 8);
        sc = mfma32(*(const bf16x8*)&Ks[buf][off], qreg[s], sc);
        dp = mfma32(*(const bf16x8*)&Vs[buf][off], greg[s], dp);
      }
      float dsv[16], dmv[16];
      auto probs = [&](auto poly) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int kp = n0 + kb * 32 + 8 * (j >> 2) + 4 * hh + (j & 3);
          const float bias = SM == SM_ALIBI ? slope2 * (float)(kp - q) : 0.f;
          dsv[j] = bwd_prob<SM, decltype(poly)::value>(a, sc[j], l2, bias, dmv[j]);
        }
      };
      if (bwd_poly_tile<SM, 1>(a, &sc)) {
        probs(std::true_type{});
      } else {
        probs(std::false_type{});
      }
      if (!full) {
        i32x4 kd4[4];  // document ids of this lane's keys, four per 16-byte LDS read
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) kd4[g4] = kDoc ? *(const i32x4*)&Dk[buf][kb * 32 + 8 * g4 + 4 * hh] : i32x4{};
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int ko = kb * 32 + 8 * (j >> 2) + 4 * hh + (j & 3);
          dsv[j] = keep_if((n0 + ko < a.Skv) & bwd_visible<MK>(a, q, n0 + ko, qdoc, kd4[j >> 2][j & 3]), dsv[j]);
        }
      }
      bf16x8 dhi[2];
      float dsmax = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float ds = dsv[j] * (dp[j] - dl) * dmv[j];
        dsv[j] = ds;
        dsmax = fmaxf(dsmax, fabsf(ds));
        dhi[j >> 3][j & 7] = (bf16)ds;
      }
      // dQ^T += K^T dS^T over these 32 keys (k-steps 2 kb, 2 kb + 1) with dS
      // rounded to bf16, plus its rounding residue (the lo half) where the
      // block holds a large |dS|: the row of dS sums to zero, so the products
      // cancel (the threshold as in dK, dV)
#pragma unroll
      for (int d2 = 0; d2 < NDB; ++d2)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
          dqT[d2] = mfma32(dual_vt_operand(Ks[buf], 2 * kb + tt, d2 * 32, tl), dhi[tt], dqT[d2]);
      if (any_lane(dsmax > kLoThresh)) {
        bf16x8 dlo[2];
#pragma unroll
        for (int j = 0; j < 16; ++j) dlo[j >> 3][j & 7] = (bf16)(dsv[j] - (float)dhi[j >> 3][j & 7]);
#pragma unroll
        for (int d2 = 0; d2 < NDB; ++d2)
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
            dqT[d2] = mfma32(dual_vt_operand(Ks[buf], 2 * kb + tt, d2 * 32, tl), dlo[tt], dqT[d2]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  if (!q_live) return;
  bf16* dqrow = (bf16*)a.dq + qoff + (size_t)q * D;
#pragma unroll
  for (int d2 = 0; d2 < NDB; ++d2)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      bf16x4 vq;
#pragma unroll
      for (int e = 0; e < 4; ++e) vq[e] = (bf16)(dqT[d2][4 * g4 + e] * a.scale);
      *(bf16x4*)(dqrow + d2 * 32 + 8 * g4 + 4 * hh) = vq;
    }
}

__global__ __launch_bounds__(NT) void zero_fill_kernel(i32x4* p, size_t n16) {
  const size_t i = (size_t)blockIdx.x * NT + threadIdx.x;
  if (i < n16) p[i] = i32x4{0, 0, 0, 0};
}

template <int SM, int MK>
hipError_t launch_bwd2(const BwdArgs& a, hipStream_t stream) {
  constexpr int BMS = stats_bm<MK>();
  const int total_s = a.B * a.Hq * ((a.Sq + BMS - 1) / BMS);
  hipLaunchKernelGGL((attn_bwd_stats_kernel<SM, MK>), dim3(total_s), dim3(NT), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<SM, MK>), dim3(a.total), dim3(NT), 0, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_bwd_dq_kernel<SM, MK>), dim3(a.total_q), dim3(NT), 0, stream, a);
  return hipGetLastError();
}

template <int SM>
hipError_t launch_bwd1(const BwdArgs& a, int mask, hipStream_t stream) {
  switch (mask) {
    case MK_NONE: return launch_bwd2<SM, MK_NONE>(a, stream);
    case MK_CAUSAL: return launch_bwd2<SM, MK_CAUSAL>(a, stream);
    case MK_WINDOW: return launch_bwd2<SM, MK_WINDOW>(a, stream);
    case MK_PREFIX: return launch_bwd2<SM, MK_PREFIX>(a, stream);
    case MK_DOC: return launch_bwd2<SM, MK_DOC>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t stream) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)((n16 + NT - 1) / NT)), dim3(NT), 0, stream, (i32x4*)p, n16);
  return hipGetLastError();
}

hipError_t launch_attn_bwd(const BwdArgs& a, int score_mod, int mask, hipStream_t stream) {
  switch (score_mod) {
    case SM_NONE: return launch_bwd1<SM_NONE>(a, mask, stream);
    case SM_ALIBI: return launch_bwd1<SM_ALIBI>(a, mask, stream);
    case SM_SOFTCAP: return launch_bwd1<SM_SOFTCAP>(a, mask, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace av
