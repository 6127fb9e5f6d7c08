// Fused attention forward for gfx950: QK^T -> score modifier -> analytic
// mask -> online softmax -> PV in one kernel; the score matrix lives only
// in registers.
//
// The method is the one the Flashlight pages derive for their generated
// kernels (talk notes "Flashlight: PyTorch Compiler Extensions to Accelerate
// Attention Variants", section "Compiler design": 1. both contractions are
// reductions inside one kernel, 2. the stable softmax rewritten online with a
// running max and a running sum rescaled through exp(a - b) = exp(a)/exp(b),
// 3. the score tile is never written to global memory, 4. the head dimension
// is one whole tile and the multi-dimensional tile grid is linearised into one
// physical grid dimension).  The mapping onto CDNA4 is this file's own:
//
//  * One workgroup = 4 waves of one (batch, query head); each wave owns
//    32*QB query rows for the whole KV loop (QB = 2 blocks of 32 at D <= 64,
//    1 at D = 128).  Every K fragment and every transposed V fragment read
//    from LDS feeds the MFMAs of all QB blocks, which halves LDS traffic per
//    FLOP and gives each wave two independent softmax/MFMA chains.
//  * Scores are computed transposed, S^T = K Q^T, with the 32x32x16 bf16
//    MFMA.  In its output layout every lane holds 16 keys of ONE query
//    (lanes l and l^32 share the query), so the row max is an in-register
//    reduction plus one v_permlane32_swap, and the exponentiated tile feeds
//    the second MFMA (O^T = V^T P^T) straight from registers as its B
//    operand: no LDS round trip for P.
//  * K and V tiles sit row-major in LDS, double-buffered, with the next
//    tile's global loads in flight while the current one is computed.  K has
//    a padded pitch (conflict-free 16-byte reads); V is XOR-swizzled in
//    64-byte segments (conflict-free transposed reads, no padding).  The V^T
//    operand is read with gfx950's transposed LDS read, two per MFMA.
//  * Scores are carried in log2 units (scale * log2 e folded in); exp2 is the
//    hardware v_exp_f32; accumulation is fp32 (talk notes, "Implementation
//    details", precision item).
//  * The running max used as the exponent reference is only raised when a
//    tile's max exceeds it by more than 2^8 (then O and l are rescaled);
//    otherwise the exponentials stay below 256 and no rescale is paid.  The
//    result is the same softmax: every exponential and the sum share one
//    reference.  The row sum adds the bf16-rounded probabilities, exactly the
//    values the PV product consumes; calls that ask for the log-sum-exp add
//    the fp32 exponentials instead, so that it is exact to fp32 rounding.
//  * Masks are analytic: each workgroup computes the KV tile range that
//    holds any visible key (document masks: two 64-way wave searches over
//    the doc-id row), each wave classifies every tile as skipped, full (no
//    element test) or partial (element test), and only partial tiles pay for
//    the predicate.  No block mask is built or read.
//  * The linear grid is remapped so that each XCD receives a contiguous run
//    of tiles of the same (batch, head) and the K/V of that head stay in the
//    XCD's L2 (the pages' L2 swizzle, talk notes "Implementation details",
//    made XCD-aware); causal and PrefixLM grids start with the heaviest query
//    tiles, and under the document mask an optional order computed from the
//    document ids (doc_order.hip) does the same.

#include "attn_tile.hpp"
#include "av_kernels.hpp"

namespace av {
namespace {

constexpr int BN = 64;   // keys per KV tile
constexpr int NT = 256;  // threads per workgroup (4 waves)

// Waves per SIMD each instantiation's register budget is sized for: two
// with two query blocks per wave, D = 128 or a bias tile at D = 64 (the
// prefetched bias of the bias tensor or the Evoformer pair bias does not fit
// a third wave's budget), three otherwise.
template <int D, int SM, int MK, bool ONE>
constexpr int min_waves() {
  return (attn_qb(D, SM, MK) == 2 && !ONE) || D == 128 || ((SM == SM_TBIAS || SM == SM_BIAS) && D == 64) ? 2 : 3;
}

// EXACT: the row sums add the fp32 exponentials (calls that ask for lse), else
// their bf16 copies (see exp_pack_sum).
// ONE: one query block per wave where attn_qb picks two (attn_one_block).
template <int D, int SM, int MK, bool EXACT, bool ONE>
__global__ __launch_bounds__(NT, (min_waves<D, SM, MK, ONE>())) void attn_fwd_kernel(const AttnArgs a) {
  constexpr int QB = ONE ? 1 : attn_qb(D, SM, MK);  // 32-row query blocks per wave
  constexpr int BM = 4 * 32 * QB;                  // query rows per workgroup
  constexpr bool kBias = SM == SM_BIAS || SM == SM_TBIAS;  // a bias tile is read per KV tile
  constexpr int WQ = 32 * QB;        // query rows per wave
  constexpr int NKB = BN / 32;       // 32-key blocks per tile (S^T MFMA rows)
  constexpr int NDB = D / 32;        // 32-wide d blocks of O^T
  constexpr int NDS = D / 16;        // k-steps of the QK^T MFMA
  constexpr int NPS = BN / 16;       // k-steps of the PV MFMA
  constexpr int CPR = D / 8;         // 16-byte chunks per K/V row
  constexpr int NCH = BN * CPR / NT; // chunks per thread per tensor
  constexpr int KP = D + 8;          // K row pitch (elements): 16 rows hit 16 distinct 16-byte bank slots
  static_assert(NCH >= 1 && BN * CPR % NT == 0, "tile/thread mismatch");

  // LDS: the K/V double buffer during the key loop; before it the Q tile
  // and after it the O tile pass through the same bytes, so that Q is read
  // and O written as whole contiguous rows (row pitch KP).
  // (Q/O staging: all but the gated Evoformer forms, the document mask and
  // the sliding window, whose short rows or register budget gain nothing from
  // it; measured: sliding window 47.0 -> 46.3 us unstaged, S = 512 48.6 ->
  // 52.8 us unstaged)
  constexpr bool kStageQO = SM != SM_BIAS && SM != SM_GATE && MK != MK_DOC && MK != MK_WINDOW;
  constexpr int KV_BYTES = 2 * BN * KP * 2 + 2 * BN * D * 2;
  constexpr int QO_BYTES = BM * KP * 2;
  __shared__ __attribute__((aligned(16))) char lds_raw[(kStageQO && QO_BYTES > KV_BYTES) ? QO_BYTES : KV_BYTES];
  bf16 (*Ks)[BN * KP] = reinterpret_cast<bf16 (*)[BN * KP]>(lds_raw);
  bf16 (*Vs)[BN * D] = reinterpret_cast<bf16 (*)[BN * D]>(lds_raw + 2 * BN * KP * 2);  // swizzled for transposed reads
  bf16* QOs = reinterpret_cast<bf16*>(lds_raw);
  __shared__ __attribute__((aligned(16))) int Ds[2][MK == MK_DOC ? BN : 1];
  // Bias tile (BM query rows x BN keys) staged through LDS at D <= 64: loaded
  // with the K/V tile as coalesced 16-byte row chunks, double-buffered, row
  // pitch BN + 4 elements (136 bytes: the 32 query rows that one 8-byte-per-
  // lane read touches fall in 32 distinct bank pairs).  At D = 128 the two
  // buffers would halve the resident workgroups; there each lane loads its
  // own bias from memory one tile ahead.
  constexpr bool kBiasLds = kBias && D <= 64;
  constexpr int BP = BN + 4;
  constexpr int BCH = BM * (BN / 8) / NT;  // 16-byte bias chunks per thread per tile
  static_assert(!kBiasLds || (QB == 1 && BCH >= 1 && BM * (BN / 8) % NT == 0), "bias tile/thread mismatch");
  static_assert(SM != SM_BIAS || kBiasLds, "the pair bias enters the MFMA from the staged tile");
  __shared__ __attribute__((aligned(16))) bf16 Bs[kBiasLds ? 2 : 1][kBiasLds ? BM * BP : 1];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hh = lane >> 5, l32 = lane & 31;

  // ---- logical tile of this workgroup
  int mt_lin, bh;
  if constexpr (MK == MK_CAUSAL || MK == MK_PREFIX) {
    const TileIdx ti = weighted_tile(blockIdx.x, a.total, a.nM);
    mt_lin = ti.mt_lin;
    bh = ti.bh;
  } else {
    int L = -1;
    if constexpr (MK == MK_DOC) {
      if (a.doc_order != nullptr) {
        // heaviest-first order of the (b, query tile) pairs; the query heads
        // of one pair are consecutive blocks, so with Hq a multiple of 8 every
        // XCD keeps the same heads (and their keys in its L2) throughout
        static_assert(BM == kDocTileM && BN == kDocTileN, "document order tile sizes");
        const int item = a.doc_order[blockIdx.x / a.Hq];
        if (item < 0 || item >= a.B * a.nM) return;  // not an order of this shape: touch nothing
        L = ((item / a.nM) * a.Hq + blockIdx.x % a.Hq) * a.nM + item % a.nM;
      }
    }
    if (L >= 0) {
      mt_lin = L % a.nM;
      bh = L / a.nM;
    } else {
      L = xcd_remap(blockIdx.x, a.total);
      if (SM == SM_TBIAS && a.bias_bs == 0) {
        // bias shared over the batch: the batch entries of one (head, query
        // tile) are consecutive blocks, so they run together on one XCD and
        // read each bias row from its L2 instead of once per batch entry
        const int r = L / a.B;
        mt_lin = r % a.nM;
        bh = (L % a.B) * a.Hq + r / a.nM;
      } else {
        mt_lin = L % a.nM;
        bh = L / a.nM;
      }
    }
  }
  // Evoformer (pair bias shared over the batch): heads outermost, so one XCD's
  // run of tiles covers few heads and their bias stays in its L2.
  const int hq = (SM == SM_BIAS) ? bh / a.B : bh % a.Hq;
  const int b = (SM == SM_BIAS) ? bh % a.B : bh / a.Hq;
  const int hk = hq / a.g;
  const int mt = (MK == MK_CAUSAL || MK == MK_PREFIX) ? (a.nM - 1 - mt_lin) : mt_lin;
  const int q0 = mt * BM;
  const int qw = q0 + WQ * __builtin_amdgcn_readfirstlane(w);  // first query row of this wave
  int qi[QB];                                                  // this lane's query row per block
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) qi[qb] = qw + 32 * qb + l32;
  const int qlast = min(q0 + BM, a.Sq) - 1;
  const bool wave_live = qw < a.Sq;
  const int qwlast = min(qw + WQ - 1, a.Sq - 1);

  const size_t qoff = ((size_t)b * a.Hq + hq) * (size_t)a.Sq * D;
  const size_t kvoff = ((size_t)b * a.Hkv + hk) * (size_t)a.Skv * D;
  const auto qrs = make_rsrc((const bf16*)a.q + qoff, (uint32_t)a.Sq * D * 2);
  const auto krs = make_rsrc((const bf16*)a.k + kvoff, (uint32_t)a.Skv * D * 2);
  const auto vrs = make_rsrc((const bf16*)a.v + kvoff, (uint32_t)a.Skv * D * 2);
  const int* docrow = (MK == MK_DOC) ? a.doc + (size_t)b * a.Sq : nullptr;

  // ---- analytic KV tile range [n_lo, n_hi) of the workgroup
  const int nKV = (a.Skv + BN - 1) / BN;
  int n_lo = 0, n_hi = nKV;
  int dq[QB] = {};
  int dqw = 0, dqwlast = 0;
  if constexpr (MK == MK_CAUSAL) {
    n_hi = min(nKV, qlast / BN + 1);
  } else if constexpr (MK == MK_WINDOW) {
    n_lo = max(0, q0 - a.window + 1) / BN;
    n_hi = min(nKV, qlast / BN + 1);
  } else if constexpr (MK == MK_PREFIX) {
    n_hi = min(nKV, max(a.prefix - 1, qlast) / BN + 1);
  } else if constexpr (MK == MK_DOC) {
    const int dfirst = docrow[q0], dlast = docrow[qlast];
    const int kstart = wave_lower_bound(docrow, a.Skv, dfirst);
    const int kend = wave_upper_bound(docrow, a.Skv, dlast);
    n_lo = kstart / BN;
    n_hi = min(nKV, (kend + BN - 1) / BN);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) dq[qb] = docrow[min(qi[qb], a.Sq - 1)];
    dqw = __builtin_amdgcn_readfirstlane(docrow[min(qw, a.Sq - 1)]);
    dqwlast = __builtin_amdgcn_readfirstlane(docrow[max(qwlast, 0)]);
  }

  // ---- Q^T operands in registers: lane holds query qi[qb], 8 consecutive d per k-step
  // rows q0 .. q0+BM-1 of this (b, hq) slice are contiguous: 16-byte chunks,
  // consecutive threads on consecutive chunks, through LDS into the operands
  constexpr int QCH = BM * CPR / NT;  // Q chunks per thread
  static_assert(BM * CPR % NT == 0, "Q tile/thread mismatch");
  bf16x8 qreg[QB][NDS];
  if constexpr (!kStageQO) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int s = 0; s < NDS; ++s)
        qreg[qb][s] = __builtin_bit_cast(bf16x8, buf_load16(qrs, (uint32_t)(qi[qb] * D + s * 16 + hh * 8) * 2));
  } else {
    i32x4 qst[QCH];
#pragma unroll
    for (int c = 0; c < QCH; ++c) {
      const int idx = tid + NT * c;
      qst[c] = buf_load16(qrs, (uint32_t)((q0 + idx / CPR) * D + (idx % CPR) * 8) * 2);
    }
#pragma unroll
    for (int c = 0; c < QCH; ++c) {
      const int idx = tid + NT * c;
      *(i32x4*)&QOs[(idx / CPR) * KP + (idx % CPR) * 8] = qst[c];
    }
    __syncthreads();
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int s = 0; s < NDS; ++s)
        qreg[qb][s] = *(const bf16x8*)&QOs[(qi[qb] - q0) * KP + s * 16 + hh * 8];
    __syncthreads();  // the key loop reuses these bytes
  }
  // Fixed-reference softcap without lse: the key loop's S holds x = beta * raw
  // (q scaled once, rounded to bf16; that rounding moves the log-sum-exp by
  // about 1.5e-3, so calls that ask for lse keep the unscaled q)
  constexpr bool kScaledQ = SM == SM_SOFTCAP_FIXED && !EXACT;
  if constexpr (kScaledQ) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int s = 0; s < NDS; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e) qreg[qb][s][e] = (bf16)((float)qreg[qb][s][e] * a.sc_x[1]);
  }

  f32x16 o[QB][NDB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[qb][db] = f32x16{};
  RowState st[QB];
  const TrLane<D> vl(lane);

  // Evoformer gate pre-activations of this lane's output channels, loaded
  // up front so that their latency hides behind the KV loop
  constexpr bool kGated = SM == SM_BIAS || SM == SM_GATE;
  bf16x4 gate[QB][kGated ? NDB * 4 : 1];
  if constexpr (kGated) {
    const auto grs = make_rsrc((const bf16*)a.gate + qoff, (uint32_t)a.Sq * D * 2);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const auto w2 = __builtin_amdgcn_raw_buffer_load_b64(
              grs, (uint32_t)(qi[qb] * D + db * 32 + 8 * g4 + 4 * hh) * 2, 0, 0);
          gate[qb][db * 4 + g4] = __builtin_bit_cast(bf16x4, w2);
        }
  }

  // ALiBi, log2 units: bias(kb, j) = slope * (kj - qi) with kj = n0 + 4*hh + 32*kb + 8*(j/4) + j%4
  //   = [slope * (n0 + 4*hh - qi + j%4)]  (4 per-lane values per tile and block)
  //   + [slope * (32*kb + 8*(j/4))]       (wave-uniform, one SGPR each)
  float alibi_slope2 = 0.f;
  float alibi_u[NKB * 4];
  if constexpr (SM == SM_ALIBI) {
    alibi_slope2 = uniform_f(kLog2e * exp2f(-a.alibi_max_bias * (float)(hq + 1) / (float)a.Hq));
#pragma unroll
    for (int g = 0; g < NKB * 4; ++g) alibi_u[g] = uniform_f(alibi_slope2 * (float)(8 * g));
  }
  // bias slice of (b, hq) (Evoformer pair bias or bias tensor): 4 keys (8 bytes) per load
  const auto brs = make_rsrc(kBias ? (const bf16*)a.bias + (size_t)b * a.bias_bs + (size_t)hq * a.bias_hs : nullptr,
                             kBias ? (uint32_t)a.Sq * a.Skv * 2 : 0u);
  // softcap in log2 units: cap*log2e*tanh(raw*scale/cap) = cap2 - 2*cap2 / (1 + 2^(raw*sc_k))
  // = cap2 - 1 / fma(E, invK, invK) with E = 2^(raw*sc_k), invK = 1/(2*cap2): one exp2,
  // one fma, one rcp.  The fixed-reference form keeps t itself (reference 0:
  // every exponential lies in [2^-cap2, 2^cap2]), in x = beta * raw without lse
  const float cap2 = a.softcap * kLog2e;
  const float sc_k = 2.f * a.scale * kLog2e / a.softcap / (kScaledQ ? a.sc_x[1] : 1.f);
  const float invK = 0.5f / cap2;
  auto softcap_t = [&](float raw) {
    const float r = rcp_fast(fmaf(exp2_fast(raw * sc_k), invK, invK));
    return cap2 - r;
  };
  if constexpr (SM == SM_SOFTCAP_FIXED) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) st[qb].m_ref = 0.f;  // the scores hold t - m_ref already
  }
  // Fixed-reference softcap on a tile whose scores all lie in |raw * scale /
  // cap| <= 0.25: cap*tanh is an odd cubic there (tanh(x) = x (c0 + c1 x^2)
  // within 6.4e-5 relative), t = raw (p0 + p1 raw^2); with q scaled by beta,
  // beta^3 = -p1, it is t = x (A - x^2): one FMA and one multiply instead of
  // exp2 + fma + rcp.
  auto softcap_poly = [&](float x) {
    if constexpr (kScaledQ) {
      return x * fmaf(-x, x, a.sc_x[0]);
    } else {
      return x * fmaf(x * x, a.sc_poly[1], a.sc_poly[0]);
    }
  };
  const float sc_lim = kScaledQ ? a.sc_x_lim : a.sc_poly_lim;

  i32x4 kr[NCH], vr[NCH];
  i32x4 br[kBiasLds ? BCH : 1];
  // 16-byte bias loads need 16-byte aligned rows: Skv a multiple of 8 and an
  // aligned slice base (the ABI guarantees 8 bytes)
  const bool bias_rows16 = kBiasLds && a.Skv % 8 == 0 &&
                           (reinterpret_cast<uintptr_t>((const bf16*)a.bias + (size_t)b * a.bias_bs +
                                                        (size_t)hq * a.bias_hs) & 15) == 0;
  int dr = 0;
  auto gload = [&](int nt) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int idx = tid + NT * c;
      const int row = idx / CPR, col = idx % CPR;
      const uint32_t off = (uint32_t)((nt * BN + row) * D + col * 8) * 2;
      kr[c] = buf_load16(krs, off);
      vr[c] = buf_load16(vrs, off);
    }
    if constexpr (kBiasLds) {
      // rows q0 + row, keys nt*BN + 8*col ..; rows past Sq read as zero (buffer
      // bounds), keys past Skv belong to partial tiles, whose mask drops them
#pragma unroll
      for (int c = 0; c < BCH; ++c) {
        const int idx = tid + NT * c;
        const int row = idx / (BN / 8), col = idx % (BN / 8);
        const uint32_t off = (uint32_t)((q0 + row) * a.Skv + nt * BN + col * 8) * 2;
        if (bias_rows16) {
          br[c] = buf_load16(brs, off);
        } else {  // rows not 16-byte aligned: 16-bit loads
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t x0 = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(brs, off + 4 * e, 0, 0);
            const uint32_t x1 = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(brs, off + 4 * e + 2, 0, 0);
            br[c][e] = (int)(x0 | (x1 << 16));
          }
        }
      }
    }
    if constexpr (MK == MK_DOC) {
      if (tid < BN) {
        const int key = nt * BN + tid;
        dr = key < a.Skv ? docrow[key] : 0x7fffffff;
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int idx = tid + NT * c;
      const int row = idx / CPR, col = idx % CPR;
      *(i32x4*)&Ks[buf][row * KP + col * 8] = kr[c];
      *(i32x4*)&Vs[buf][tr_tile_off<D>(row, col * 8)] = vr[c];
    }
    if constexpr (kBiasLds) {
#pragma unroll
      for (int c = 0; c < BCH; ++c) {
        const int idx = tid + NT * c;
        const int row = idx / (BN / 8), col = idx % (BN / 8);
        bf16* dst = &Bs[buf][row * BP + col * 8];  // 8-byte aligned (the pitch is 136 bytes)
        *(i32x2*)dst = i32x2{br[c][0], br[c][1]};
        *(i32x2*)(dst + 4) = i32x2{br[c][2], br[c][3]};
      }
    }
    if constexpr (MK == MK_DOC) {
      if (tid < BN) Ds[buf][tid] = dr;
    }
  };

  // bias of this lane's (query, key) elements: keys n0 + 4*hh + 32*kb +
  // 8*g + 0..3, loaded one tile ahead of its use
  i32x4 braw[QB][kBiasLds ? 1 : NKB * 2];
  auto bias_load = [&](int n0) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const uint32_t rowoff = (uint32_t)(qi[qb] * a.Skv + n0 + 4 * hh) * 2;
      if (a.Skv % 4 == 0) {
#pragma unroll
        for (int g = 0; g < NKB * 4; g += 2) {
          const auto lo = __builtin_amdgcn_raw_buffer_load_b64(brs, rowoff + g * 16, 0, 0);
          const auto hi = __builtin_amdgcn_raw_buffer_load_b64(brs, rowoff + g * 16 + 16, 0, 0);
          braw[qb][g >> 1] = i32x4{(int)lo[0], (int)lo[1], (int)hi[0], (int)hi[1]};
        }
      } else {  // rows not 8-byte aligned: 16-bit loads
#pragma unroll
        for (int g = 0; g < NKB * 4; ++g) {
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const uint32_t o0 = rowoff + g * 16 + h2 * 4;
            const uint32_t x0 = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(brs, o0, 0, 0);
            const uint32_t x1 = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(brs, o0 + 2, 0, 0);
            braw[qb][g >> 1][(g & 1) * 2 + h2] = (int)(x0 | (x1 << 16));
          }
        }
      }
    }
  };
  // exponent argument scale: scores of vanilla attention are raw q.k, biased
  // scores are q.k*scale + bias (natural units); the other modifiers produce log2 units
  const float cexp = kBias ? kLog2e : a.c;

  // S^T = K Q^T of LDS tile buf for every query block; with the Evoformer
  // pair bias (q already scaled) the accumulators start at the bias instead
  // of zero, so the MFMA adds it
  auto qk = [&](f32x16 (&s)[QB][NKB], int buf, const i32x2* bq) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if constexpr (SM == SM_BIAS) {
#pragma unroll
          for (int j = 0; j < 16; ++j) {  // bf16 -> fp32 is a 16-bit shift
            const int wd = bq[kb * 4 + (j >> 2)][(j & 3) >> 1];
            s[qb][kb][j] = __builtin_bit_cast(float, (j & 1) ? (wd & (int)0xffff0000) : (wd << 16));
          }
        } else {
          s[qb][kb] = f32x16{};
        }
      }
      const bf16* krow = Ks[buf] + (kb * 32 + l32) * KP + hh * 8;
#pragma unroll
      for (int st_ = 0; st_ < NDS; ++st_) {
        const bf16x8 kf = *(const bf16x8*)(krow + st_ * 16);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mfma32(kf, qreg[qb][st_], s[qb][kb]);
      }
    }
  };

  // One KV tile for this wave.  Only the element mask depends on the tile
  // class, and it edits the score registers in place, so the MFMA
  // accumulators flow through a single path (no copies at a merge point).
  auto tile = [&](bool full, int buf, int n0) {
    const int kbase = n0 + 4 * hh;

    // ---- S^T = K Q^T : s[qb][kb] holds keys kb*32 + 8*(j/4) + 4*hh + j%4 of query qi[qb];
    //      each K fragment read from LDS feeds the MFMAs of every query block
    // staged bias of this lane's elements: row qi - q0, keys 32*kb + 8*g + 4*hh + 0..3
    i32x2 bq[kBiasLds ? NKB * 4 : 1];
    if constexpr (kBiasLds) {
      const bf16* brow = Bs[buf] + (qi[0] - q0) * BP + 4 * hh;
#pragma unroll
      for (int g = 0; g < NKB * 4; ++g) bq[g] = *(const i32x2*)(brow + 8 * g);
    }
    f32x16 s[QB][NKB];
    qk(s, buf, bq);

    // ---- fixed-reference softcap: the polynomial form in place; a tile with
    //      a raw score outside its range (wave-uniform, rare) recomputes
    //      S^T from the K tile still in LDS and takes the exact exp2/rcp form
    if constexpr (SM == SM_SOFTCAP_FIXED) {
      float amax = 0.f;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) amax = fmaxf(amax, block_absmax<NKB>(s[qb]));
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j) s[qb][kb][j] = softcap_poly(s[qb][kb][j]);
      if (any_lane(amax > sc_lim)) {
        qk(s, buf, bq);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int j = 0; j < 16; ++j) s[qb][kb][j] = softcap_t(s[qb][kb][j]);
      }
    }

#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      // ---- score modifier: ALiBi and softcap in log2 units, bias in natural
      //      units (q.k*scale + bias); vanilla keeps the raw q.k, its scale folded into exp2
      if constexpr (SM != SM_NONE && SM != SM_GATE && SM != SM_SOFTCAP_FIXED && SM != SM_BIAS) {
        // ALiBi goes straight to the exponent argument, relative to the
        // current reference: s*c + slope*(key - query) - m_sub
        float ab[4];
        if constexpr (SM == SM_ALIBI) {
#pragma unroll
          for (int c = 0; c < 4; ++c) ab[c] = fmaf(alibi_slope2, (float)(kbase - qi[qb] + c), -st[qb].m_sub);
        }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            if constexpr (SM == SM_ALIBI) {
              s[qb][kb][j] = fmaf(s[qb][kb][j], a.c, ab[j & 3] + alibi_u[kb * 4 + (j >> 2)]);
            } else if constexpr (SM == SM_SOFTCAP) {
              s[qb][kb][j] = softcap_t(s[qb][kb][j]);
            } else {  // bias: bf16 -> fp32 is a 16-bit shift
              const int wd = kBiasLds ? bq[kb * 4 + (j >> 2)][(j & 3) >> 1]
                                      : braw[qb][(kb * 4 + (j >> 2)) >> 1][((j >> 2) & 1) * 2 + ((j & 3) >> 1)];
              const float bv = __builtin_bit_cast(float, (j & 1) ? (wd & (int)0xffff0000) : (wd << 16));
              s[qb][kb][j] = fmaf(s[qb][kb][j], a.scale, bv);
            }
          }
      }
      // ---- element mask, partial tiles only (wave-uniform branch).  The
      //      limits pass through an empty asm so that the compares are not
      //      hoisted out of the branch into every tile.
      if (!full) {
        // the visible key offsets of this lane's row form one range
        // (wlo, hi] (the document mask adds its id test): hi = the last key
        // before Skv, capped at the row's own position for causal masks and
        // at max(prefix - 1, own position) for PrefixLM
        const int rel = qi[qb] - kbase;
        int hi = a.Skv - kbase - 1, wlo = rel - a.window;
        if constexpr (MK == MK_CAUSAL || MK == MK_WINDOW) hi = min(hi, rel);
        if constexpr (MK == MK_PREFIX) hi = min(hi, max(a.prefix - kbase - 1, rel));
        asm volatile("" : "+v"(hi), "+v"(wlo));
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int off = kb * 32 + 8 * (j >> 2) + (j & 3);
            bool ok = off <= hi;
            if constexpr (MK == MK_WINDOW) {
              ok = ok && (off > wlo);
            } else if constexpr (MK == MK_DOC) {
              // the document ids of this lane's four keys (one 16-byte LDS
              // read), and no short circuit: a branch and a read per score otherwise
              const i32x4 d4 = *(const i32x4*)&Ds[buf][kb * 32 + 8 * (j >> 2) + 4 * hh];
              ok = ok & (d4[j & 3] == dq[qb]);
            }
            s[qb][kb][j] = ok ? s[qb][kb][j] : neg_inf();
            if ((j & 3) == 3) __builtin_amdgcn_sched_barrier(0);  // bounds the live compare masks
          }
        }
      }
    }

    // ---- exponent reference and p = exp2(t - m_ref) -> bf16 P^T operands,
    //      with the row sum of the bf16 values
    constexpr bool kOptimistic = SM == SM_NONE || kBias || SM == SM_GATE;
    constexpr int MODE = kOptimistic ? 0 : (SM == SM_SOFTCAP_FIXED || SM == SM_ALIBI) ? 2 : 1;
    bf16x8 pb[QB][NPS];
    // Fixed-reference softcap and the bias tensor: the wave raises its issue
    // priority over its exponentials (its longest VALU stretch), so that
    // stretch is not starved by the other wave of the SIMD (measured: softcap
    // 5-6 % faster unmasked at S = 1k-16k, bias tensor 4 %; the same region
    // made vanilla, causal, ALiBi-causal and Evoformer kernels slower)
    constexpr bool kPrioExp = SM == SM_SOFTCAP_FIXED || SM == SM_TBIAS;
    if constexpr (kPrioExp) __builtin_amdgcn_s_setprio(1);
    if constexpr (kOptimistic) {
      // Optimistic: exponentiate against the current reference and keep the
      // result unless some exponential exceeds 2^64 (then the tile sum does)
      // or the row has no reference yet.  The reference is only ever a
      // previous tile max, so the row's largest exponential stays >= 1; the
      // max is taken only on the rare tiles that fail the check.
      float tsum[QB];
      bool redo = false;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        tsum[qb] = exp_pack_sum<NKB, MODE, EXACT>(s[qb], cexp, st[qb].m_sub, pb[qb]);
        redo |= (tsum[qb] > kOptBound) || (st[qb].m_ref == neg_inf());
      }
      if (any_lane(redo)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const float rmax = xhalf_max(block_max<NKB>(s[qb]));
          st[qb].template raise<NDB>(rmax * cexp, o[qb]);
          tsum[qb] = exp_pack_sum<NKB, MODE, EXACT>(s[qb], cexp, st[qb].m_sub, pb[qb]);
        }
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) st[qb].l += tsum[qb];
    } else {
      // ALiBi scores can climb along the row, so the tile max is tracked
      // with the lazy rescale (one wave-uniform decision for all blocks; each
      // lane tests its own half of the row, the raise uses the whole row).
      // ALiBi scores already hold the exponent argument relative to the
      // reference, so the test is against kLazyTau and a raise shifts them.
      // A softcap with a small cap has bounded scores: its reference sits at
      // the cap and no max is taken.
      if constexpr (SM == SM_ALIBI) {
        float hmax[QB];
        bool grow = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          hmax[qb] = block_max<NKB>(s[qb]);
          grow |= (hmax[qb] > kLazyTau) || (st[qb].m_ref == neg_inf());
        }
        if (any_lane(grow)) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const float old_sub = st[qb].m_sub;
            st[qb].template raise<NDB>(old_sub + xhalf_max(hmax[qb]), o[qb]);
            const float shift = st[qb].m_sub - old_sub;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
              for (int j = 0; j < 16; ++j) s[qb][kb][j] -= shift;
          }
        }
      } else if constexpr (SM != SM_SOFTCAP_FIXED) {
        float hmax[QB];
        bool grow = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          hmax[qb] = block_max<NKB>(s[qb]);
          grow |= hmax[qb] > st[qb].thr;
        }
        if (any_lane(grow)) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) st[qb].template raise<NDB>(xhalf_max(hmax[qb]), o[qb]);
        }
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) st[qb].l += exp_pack_sum<NKB, MODE, EXACT>(s[qb], a.c, st[qb].m_sub, pb[qb]);
    }

    if constexpr (kPrioExp) __builtin_amdgcn_s_setprio(0);
    // ---- O^T += V^T P^T; each transposed V fragment feeds every query block
    // all V^T operands of the tile are read before the first MFMA (the
    // scheduler would otherwise keep two in flight and wait on LDS eight times)
    bf16x8 vfa[NDB][NPS];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int t = 0; t < NPS; ++t) vfa[db][t] = vt_operand<D>(Vs[buf], t, db * 32, vl);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int t = 0; t < NPS; ++t) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) o[qb][db] = mfma32(vfa[db][t], pb[qb][t], o[qb][db]);
      }
  };

  // Key tile order.  ALiBi walks the keys from last to first: its term grows
  // with the key index (by up to ~65 log2 units per tile on the steepest
  // heads), so in ascending order most tiles would raise the exponent
  // reference and rescale O; descending, the first tile holds the row's
  // largest term and later tiles rarely raise it.
  constexpr bool kDescending = SM == SM_ALIBI;
  auto tile_at = [&](int it) { return kDescending ? n_hi - 1 - (it - n_lo) : it; };

  if (n_lo < n_hi) gload(tile_at(n_lo));
  if constexpr (kBias && !kBiasLds) {
    if (n_lo < n_hi) bias_load(tile_at(n_lo) * BN);
  }

  for (int it = n_lo; it < n_hi; ++it) {
    const int nt = tile_at(it);
    const int buf = (it - n_lo) & 1;
    sstore(buf);
    __syncthreads();
    if (it + 1 < n_hi) gload(tile_at(it + 1));

    const int n0 = nt * BN, n1 = n0 + BN - 1;
    // ---- per-wave tile class: skip / full / partial (wave-uniform)
    bool skip = !wave_live;
    bool full = n1 < a.Skv;
    if constexpr (MK == MK_CAUSAL) {
      skip |= n0 > qwlast;
      full &= n1 <= qw;
    } else if constexpr (MK == MK_WINDOW) {
      skip |= (n0 > qwlast) || (qw - n1 >= a.window);
      full &= (n1 <= qw) && (qwlast - n0 < a.window);
    } else if constexpr (MK == MK_PREFIX) {
      skip |= (n0 >= a.prefix) && (n0 > qwlast);
      full &= (n1 < a.prefix) || (n1 <= qw);
    } else if constexpr (MK == MK_DOC) {
      const int d0 = Ds[buf][0], d1 = Ds[buf][BN - 1];
      skip |= (d1 < dqw) || (d0 > dqwlast);
      full &= (d0 == dqw) && (d1 == dqwlast) && (dqw == dqwlast);
    }
    if (!__builtin_amdgcn_readfirstlane((int)skip)) tile(__builtin_amdgcn_readfirstlane((int)full) != 0, buf, n0);
    // the bias is loaded one tile ahead, also after a tile this wave skips,
    // so that every processed tile finds its own bias in braw
    if constexpr (kBias && !kBiasLds) {
      if (it + 1 < n_hi) bias_load(tile_at(it + 1) * BN);
    }
  }

  // ---- epilogue: O / l, bf16 store (staged through LDS), optional LSE.
  // The lane-derived values come from an opaque copy of the thread id: the
  // compiler would otherwise keep the prologue's copies (the Q row offsets
  // in LDS, the lane id) alive across the key loop, and spill them.
  if constexpr (kStageQO) __syncthreads();  // every wave is done with the K/V tiles
  int tid_e = tid;
  asm volatile("" : "+v"(tid_e));
  const int hh_e = (tid_e >> 5) & 1, l32_e = tid_e & 31;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = xhalf_sum(st[qb].l);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const int q = qw + 32 * qb + l32_e;
    if (q >= a.Sq) continue;
    if constexpr (kGated) {
      // Evoformer: out[token, hq*D + d] = sigmoid(gate[b, hq, q, d]) * O[d] / l with
      // token = (b, q) row-wise (b sequence, q residue) and (q, b) column-wise
      // (b residue column, q sequence)
      const size_t tok = SM == SM_BIAS ? (size_t)b * a.Sq + q : (size_t)q * a.B + b;
      bf16* orow = (bf16*)a.o + tok * (size_t)(a.Hq * D) + (size_t)hq * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d0 = db * 32 + 8 * g4 + 4 * hh_e;
          const bf16x4 gv = gate[qb][db * 4 + g4];
          bf16x4 val;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float sig = rcp_fast(1.f + exp2_fast(-(float)gv[e] * kLog2e));
            val[e] = (bf16)(o[qb][db][g4 * 4 + e] * inv * sig);
          }
          *(bf16x4*)(orow + d0) = val;
        }
      }
    } else {
      bf16* orow = kStageQO ? QOs + (q - q0) * KP : (bf16*)a.o + qoff + (size_t)q * D;  // staged: written out below
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          bf16x4 val;
#pragma unroll
          for (int e = 0; e < 4; ++e) val[e] = (bf16)(o[qb][db][g4 * 4 + e] * inv);
          *(bf16x4*)(orow + db * 32 + 8 * g4 + 4 * hh_e) = val;
        }
      }
      if (a.lse != nullptr && hh_e == 0) {
        a.lse[((size_t)b * a.Hq + hq) * a.Sq + q] =
            l_tot > 0.f ? (st[qb].m_ref + __log2f(l_tot)) * kLn2 : neg_inf();
      }
    }
  }
  if constexpr (kStageQO) {
    // O tile: rows q0 .. q0+BM-1 of the (b, hq) slice, contiguous in memory,
    // at the offsets of the Q tile load (recomputed from the opaque thread id)
    __syncthreads();
    bf16* obase = (bf16*)a.o + qoff;
#pragma unroll
    for (int c = 0; c < QCH; ++c) {
      const int idx = tid_e + NT * c;
      const int row = idx / CPR, col = idx % CPR;
      if (q0 + row < a.Sq) *(i32x4*)(obase + (size_t)(q0 + row) * D + col * 8) = *(const i32x4*)&QOs[row * KP + col * 8];
    }
  }
}

template <int D, int SM, int MK, bool EXACT = false, bool ONE = false>
hipError_t launch_one(const AttnArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((attn_fwd_kernel<D, SM, MK, EXACT, ONE>), dim3(a.total), dim3(NT), 0, stream, a);
  return hipGetLastError();
}

template <int D, int SM, bool EXACT>
hipError_t launch_mask_x(const AttnArgs& a, int mask, hipStream_t stream) {
  switch (mask) {
    case MK_NONE: return launch_one<D, SM, MK_NONE, EXACT>(a, stream);
    case MK_CAUSAL:
      if constexpr (attn_qb(D, SM, MK_CAUSAL) == 2) {
        if (a.one_block) return launch_one<D, SM, MK_CAUSAL, EXACT, true>(a, stream);
      }
      return launch_one<D, SM, MK_CAUSAL, EXACT>(a, stream);
    case MK_WINDOW: return launch_one<D, SM, MK_WINDOW, EXACT>(a, stream);
    case MK_PREFIX:
      if constexpr (attn_qb(D, SM, MK_PREFIX) == 2) {
        if (a.one_block) return launch_one<D, SM, MK_PREFIX, EXACT, true>(a, stream);
      }
      return launch_one<D, SM, MK_PREFIX, EXACT>(a, stream);
    case MK_DOC: return launch_one<D, SM, MK_DOC, EXACT>(a, stream);
  }
  return hipErrorInvalidValue;
}

// calls that ask for lse take the exact-sum instantiations
template <int D, int SM>
hipError_t launch_mask(const AttnArgs& a, int mask, hipStream_t stream) {
  return a.lse != nullptr ? launch_mask_x<D, SM, true>(a, mask, stream) : launch_mask_x<D, SM, false>(a, mask, stream);
}

template <int D>
hipError_t launch_sm(const AttnArgs& a, int sm, int mask, hipStream_t stream) {
  switch (sm) {
    case SM_NONE: return launch_mask<D, SM_NONE>(a, mask, stream);
    case SM_ALIBI: return launch_mask<D, SM_ALIBI>(a, mask, stream);
    case SM_SOFTCAP:
      return a.fixed_ref ? launch_mask<D, SM_SOFTCAP_FIXED>(a, mask, stream) : launch_mask<D, SM_SOFTCAP>(a, mask, stream);
    case SM_TBIAS: return launch_mask<D, SM_TBIAS>(a, mask, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_evo_attention(const AttnArgs& a, int D, int col, hipStream_t stream) {
  if (D == 64) return col ? launch_one<64, SM_GATE, MK_NONE>(a, stream) : launch_one<64, SM_BIAS, MK_NONE>(a, stream);
  return col ? launch_one<32, SM_GATE, MK_NONE>(a, stream) : launch_one<32, SM_BIAS, MK_NONE>(a, stream);
}

hipError_t launch_attn_fwd(const AttnArgs& a, int D, int score_mod, int mask, hipStream_t stream) {
  switch (D) {
    case 32: return launch_sm<32>(a, score_mod, mask, stream);
    case 64: return launch_sm<64>(a, score_mod, mask, stream);
    case 128: return launch_sm<128>(a, score_mod, mask, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace av
