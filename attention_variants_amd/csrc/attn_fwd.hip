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
//  * One workgroup = 4 waves = 128 query rows of one (batch, query head);
//    each wave owns 32 rows for the whole KV loop.
//  * Scores are computed transposed, S^T = K Q^T, with the 32x32x16 bf16
//    MFMA.  In its output layout every lane holds 16 keys of ONE query
//    (lanes l and l^32 share the query), so the row max is an in-register
//    reduction plus one v_permlane32_swap, and the exponentiated tile feeds
//    the second MFMA (O^T = V^T P^T) straight from registers as its B
//    operand: no LDS round trip for P.
//  * K and V tiles sit row-major in LDS (padded pitches, conflict-free for
//    the read patterns below), double-buffered, with the next tile's global
//    loads in flight while the current one is computed.  The V^T operand is
//    read with gfx950's transposed LDS read, two per MFMA.
//  * Scores are carried in log2 units (scale * log2 e folded in); exp2 is the
//    hardware v_exp_f32; accumulation is fp32 (talk notes, "Implementation
//    details", precision item).
//  * The running max used as the exponent reference is only raised when a
//    tile's max exceeds it by more than 2^8 (then O and l are rescaled);
//    otherwise the exponentials stay below 256 and no rescale is paid.  The
//    result is the same softmax: every exponential and the sum share one
//    reference.  The row sum adds the bf16-rounded probabilities, exactly the
//    values the PV product consumes.
//  * Masks are analytic: each workgroup computes the KV tile range that
//    holds any visible key (document masks: two 64-way wave searches over
//    the doc-id row), each wave classifies every tile as skipped, full (no
//    element test) or partial (element test), and only partial tiles pay for
//    the predicate.  No block mask is built or read.
//  * The linear grid is remapped so that each XCD receives a contiguous run
//    of tiles of the same (batch, head) and the K/V of that head stay in the
//    XCD's L2 (the pages' L2 swizzle, talk notes "Implementation details",
//    made XCD-aware); causal and PrefixLM grids start with the heaviest query
//    tiles.

#include "av_device.hpp"
#include "av_kernels.hpp"

namespace av {
namespace {

constexpr int BM = kAttnBM;  // query rows per workgroup
constexpr int BN = 64;       // keys per KV tile
constexpr int NT = 256;      // threads per workgroup
constexpr float kTau = 8.f;  // lazy-rescale threshold, log2 units

// Waves per SIMD each instantiation's register budget is sized for.  Four
// (<= 128 VGPRs; the LDS of four 38 KB workgroups also fits a CU) where the
// code fits without spilling, else three (<= 168 VGPRs); two at D = 128.
template <int D, int SM, int MK>
constexpr int min_waves() {
  if (D <= 32) return 4;
  if (D == 64) return (SM == SM_NONE && (MK == MK_NONE || MK == MK_CAUSAL || MK == MK_WINDOW)) ? 4 : 3;
  return 2;
}

template <int D, int SM, int MK>
__global__ __launch_bounds__(NT, (min_waves<D, SM, MK>())) void attn_fwd_kernel(const AttnArgs a) {
  constexpr int NKB = BN / 32;       // 32-key blocks per tile (S^T MFMA rows)
  constexpr int NDB = D / 32;        // 32-wide d blocks of O^T
  constexpr int NDS = D / 16;        // k-steps of the QK^T MFMA
  constexpr int NPS = BN / 16;       // k-steps of the PV MFMA
  constexpr int CPR = D / 8;         // 16-byte chunks per K/V row
  constexpr int NCH = BN * CPR / NT; // chunks per thread per tensor
  constexpr int KP = D + 8;          // K row pitch (elements): 8 rows hit 8 distinct 16-byte bank groups
  constexpr int VP = D + 16;         // V row pitch: 4 rows hit 4 distinct 32-byte bank groups
  static_assert(NCH >= 1 && BN * CPR % NT == 0, "tile/thread mismatch");

  __shared__ __attribute__((aligned(16))) bf16 Ks[2][BN * KP];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][BN * VP];
  __shared__ __attribute__((aligned(16))) int Ds[2][MK == MK_DOC ? BN : 1];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hh = lane >> 5, l32 = lane & 31;

  // ---- logical tile of this workgroup
  const int L = xcd_remap(blockIdx.x, a.total);
  const int mt_lin = L % a.nM;
  const int bh = L / a.nM;
  const int hq = bh % a.Hq, b = bh / a.Hq;
  const int hk = hq / a.g;
  const int mt = (MK == MK_CAUSAL || MK == MK_PREFIX) ? (a.nM - 1 - mt_lin) : mt_lin;
  const int q0 = mt * BM;
  const int qw = q0 + 32 * __builtin_amdgcn_readfirstlane(w);  // first query row of this wave
  const int qi = qw + l32;                                       // this lane's query row
  const int qlast = min(q0 + BM, a.Sq) - 1;
  const bool wave_live = qw < a.Sq;
  const int qwlast = min(qw + 31, a.Sq - 1);

  const size_t qoff = ((size_t)b * a.Hq + hq) * (size_t)a.Sq * D;
  const size_t kvoff = ((size_t)b * a.Hkv + hk) * (size_t)a.Skv * D;
  const auto qrs = make_rsrc((const bf16*)a.q + qoff, (uint32_t)a.Sq * D * 2);
  const auto krs = make_rsrc((const bf16*)a.k + kvoff, (uint32_t)a.Skv * D * 2);
  const auto vrs = make_rsrc((const bf16*)a.v + kvoff, (uint32_t)a.Skv * D * 2);
  const int* docrow = (MK == MK_DOC) ? a.doc + (size_t)b * a.Sq : nullptr;

  // ---- analytic KV tile range [n_lo, n_hi) of the workgroup
  const int nKV = (a.Skv + BN - 1) / BN;
  int n_lo = 0, n_hi = nKV;
  int dq = 0, dqw = 0, dqwlast = 0;
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
    dq = docrow[min(qi, a.Sq - 1)];
    dqw = __builtin_amdgcn_readfirstlane(docrow[min(qw, a.Sq - 1)]);
    dqwlast = __builtin_amdgcn_readfirstlane(docrow[max(qwlast, 0)]);
  }

  // ---- Q^T operands in registers: lane holds query qi, 8 consecutive d per k-step
  bf16x8 qreg[NDS];
#pragma unroll
  for (int s = 0; s < NDS; ++s) {
    const uint32_t off = (uint32_t)(qi * D + s * 16 + hh * 8) * 2;
    qreg[s] = __builtin_bit_cast(bf16x8, buf_load16(qrs, off));
  }

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
  float m_ref = neg_inf();  // exponent reference (log2 units), identical in lanes l and l^32
  float m_sub = 0.f;        // m_ref with -inf replaced by 0 (the value subtracted in exp2)
  float l_run = 0.f;        // sum of this lane's bf16 probabilities, relative to m_ref

  // score-modifier constants
  // ALiBi, log2 units: bias(kb, j) = slope * (kj - qi) with kj = n0 + 4*hh + 32*kb + 8*(j/4) + j%4
  //   = [slope * (n0 + 4*hh - qi + j%4)]  (4 per-lane values per tile)
  //   + [slope * (32*kb + 8*(j/4))]       (wave-uniform, one SGPR each)
  float alibi_slope2 = 0.f;
  float alibi_u[NKB * 4];
  if constexpr (SM == SM_ALIBI) {
    alibi_slope2 = uniform_f(kLog2e * exp2f(-a.alibi_max_bias * (float)(hq + 1) / (float)a.Hq));
#pragma unroll
    for (int g = 0; g < NKB * 4; ++g) alibi_u[g] = uniform_f(alibi_slope2 * (float)(8 * g));
  }
  const float cap2 = a.softcap * kLog2e;  // softcap in log2 units
  const float sc_k = 2.f * a.scale * kLog2e / a.softcap;
  // cap * log2e * tanh(raw * scale / cap) from exp2 and rcp
  auto softcap_t = [&](float raw) { return fmaf(-2.f * cap2, rcp_fast(1.f + exp2_fast(raw * sc_k)), cap2); };

  i32x4 kr[NCH], vr[NCH];
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
      *(i32x4*)&Vs[buf][row * VP + col * 8] = vr[c];
    }
    if constexpr (MK == MK_DOC) {
      if (tid < BN) Ds[buf][tid] = dr;
    }
  };

  // per-lane parts of the transposed V read: rows 4*hh + r/4 (+8), columns 16*g + 4*(r%4)
  const int r16 = lane & 15;
  const int v_row0 = 4 * hh + (r16 >> 2);
  const int v_col0 = 16 * ((lane >> 4) & 1) + 4 * (r16 & 3);

  // One KV tile for this wave.  Only the element mask depends on the tile
  // class, and it edits the score registers in place, so the MFMA
  // accumulators flow through a single path (no copies at a merge point).
  auto tile = [&](bool full, int buf, int n0) {
    // ---- S^T = K Q^T : s[kb] holds keys kb*32 + 8*(j/4) + 4*hh + j%4 of query qi
    f32x16 s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      s[kb] = f32x16{};
      const bf16* krow = &Ks[buf][(kb * 32 + l32) * KP + hh * 8];
#pragma unroll
      for (int st = 0; st < NDS; ++st) s[kb] = mfma32(*(const bf16x8*)(krow + st * 16), qreg[st], s[kb]);
    }

    // ---- score modifier (log2 units except vanilla, whose scale is folded into exp2)
    const int kbase = n0 + 4 * hh;
    if constexpr (SM != SM_NONE) {
      float ab[4];
      if constexpr (SM == SM_ALIBI) {
#pragma unroll
        for (int c = 0; c < 4; ++c) ab[c] = alibi_slope2 * (float)(kbase - qi + c);
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          if constexpr (SM == SM_ALIBI) s[kb][j] = fmaf(s[kb][j], a.c, ab[j & 3] + alibi_u[kb * 4 + (j >> 2)]);
          else s[kb][j] = softcap_t(s[kb][j]);
        }
    }
    // ---- element mask, partial tiles only (wave-uniform branch)
    if (!full) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int off = kb * 32 + 8 * (j >> 2) + (j & 3);
          bool ok = off < a.Skv - kbase;
          if constexpr (MK == MK_CAUSAL) {
            ok = ok && (off <= qi - kbase);
          } else if constexpr (MK == MK_WINDOW) {
            const int rel = qi - kbase;
            ok = ok && (off <= rel) && (off > rel - a.window);
          } else if constexpr (MK == MK_PREFIX) {
            ok = ok && ((off < a.prefix - kbase) || (off <= qi - kbase));
          } else if constexpr (MK == MK_DOC) {
            ok = ok && (Ds[buf][off + 4 * hh] == dq);
          }
          s[kb][j] = ok ? s[kb][j] : neg_inf();
        }
      }
    }
    // ---- tile row max: four independent v_max3 chains, then the lane pair
    float mx[4] = {neg_inf(), neg_inf(), neg_inf(), neg_inf()};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int j = 0; j < 16; j += 2) mx[(j >> 1) & 3] = fmaxf(mx[(j >> 1) & 3], fmaxf(s[kb][j], s[kb][j + 1]));
    const float lmax = fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
    float tile_max;  // log2 units, shared by lanes l and l^32
    if constexpr (SM == SM_NONE) {
      tile_max = xhalf_max(lmax) * a.c;
    } else {
      tile_max = xhalf_max(lmax);
    }

    // ---- lazy rescale: raise the reference only when the max grew by > 2^kTau
    if (any_lane(tile_max > m_ref + kTau)) {
      const float m_new = fmaxf(m_ref, tile_max);
      const float m_new_sub = (m_new == neg_inf()) ? 0.f : m_new;
      const float alpha = exp2_fast(m_ref - m_new_sub);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) o[db] *= alpha;
      m_ref = m_new;
      m_sub = m_new_sub;
    }

    // ---- p = exp2(t - m_ref) -> bf16 P^T operands; row sum of the bf16 values
    bf16x8 pb[NPS];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int j = 0; j < 16; j += 2) {
        float p0, p1;
        if constexpr (SM == SM_NONE) {
          p0 = exp2_fast(fmaf(s[kb][j], a.c, -m_sub));
          p1 = exp2_fast(fmaf(s[kb][j + 1], a.c, -m_sub));
        } else {
          p0 = exp2_fast(s[kb][j] - m_sub);
          p1 = exp2_fast(s[kb][j + 1] - m_sub);
        }
        const bf16x2 pp = {(bf16)p0, (bf16)p1};
        l_run = add_bf16_pair(pp, l_run);
        pb[kb * 2 + (j >> 3)][j & 7] = pp[0];
        pb[kb * 2 + (j >> 3)][(j & 7) + 1] = pp[1];
      }
    }

    // ---- O^T += V^T P^T, V^T operand via two transposed LDS reads per MFMA
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int t = 0; t < NPS; ++t) {
        const bf16* vp = &Vs[buf][((t >> 1) * 32 + 16 * (t & 1) + v_row0) * VP + db * 32 + v_col0];
        const i16x4 lo = lds_read_tr16(vp);
        const i16x4 hi = lds_read_tr16(vp + 8 * VP);
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[db] = mfma32(vf, pb[t], o[db]);
      }
    }
  };

  if (n_lo < n_hi) gload(n_lo);

  for (int nt = n_lo; nt < n_hi; ++nt) {
    const int buf = (nt - n_lo) & 1;
    sstore(buf);
    __syncthreads();
    if (nt + 1 < n_hi) gload(nt + 1);

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
    if (__builtin_amdgcn_readfirstlane((int)skip)) continue;
    tile(__builtin_amdgcn_readfirstlane((int)full) != 0, buf, n0);
  }

  // ---- epilogue: O / l, bf16 store, optional LSE
  const float l_tot = xhalf_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qi < a.Sq) {
    bf16* orow = (bf16*)a.o + qoff + (size_t)qi * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 val;
#pragma unroll
        for (int e = 0; e < 4; ++e) val[e] = (bf16)(o[db][g4 * 4 + e] * inv);
        *(bf16x4*)(orow + db * 32 + 8 * g4 + 4 * hh) = val;
      }
    }
    if (a.lse != nullptr && hh == 0) {
      a.lse[((size_t)b * a.Hq + hq) * a.Sq + qi] = l_tot > 0.f ? (m_ref + __log2f(l_tot)) * kLn2 : neg_inf();
    }
  }
}

template <int D, int SM, int MK>
hipError_t launch_one(const AttnArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((attn_fwd_kernel<D, SM, MK>), dim3(a.total), dim3(NT), 0, stream, a);
  return hipGetLastError();
}

template <int D, int SM>
hipError_t launch_mask(const AttnArgs& a, int mask, hipStream_t stream) {
  switch (mask) {
    case MK_NONE: return launch_one<D, SM, MK_NONE>(a, stream);
    case MK_CAUSAL: return launch_one<D, SM, MK_CAUSAL>(a, stream);
    case MK_WINDOW: return launch_one<D, SM, MK_WINDOW>(a, stream);
    case MK_PREFIX: return launch_one<D, SM, MK_PREFIX>(a, stream);
    case MK_DOC: return launch_one<D, SM, MK_DOC>(a, stream);
  }
  return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_sm(const AttnArgs& a, int sm, int mask, hipStream_t stream) {
  switch (sm) {
    case SM_NONE: return launch_mask<D, SM_NONE>(a, mask, stream);
    case SM_ALIBI: return launch_mask<D, SM_ALIBI>(a, mask, stream);
    case SM_SOFTCAP: return launch_mask<D, SM_SOFTCAP>(a, mask, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attn_fwd(const AttnArgs& a, int D, int score_mod, int mask, hipStream_t stream) {
  switch (D) {
    case 32: return launch_sm<32>(a, score_mod, mask, stream);
    case 64: return launch_sm<64>(a, score_mod, mask, stream);
    case 128: return launch_sm<128>(a, score_mod, mask, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace av
