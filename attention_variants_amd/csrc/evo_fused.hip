// Evoformer gated self-attention in one kernel, gfx950: row-wise with pair
// bias, and column-wise (no bias).
//
// The operation is the one evoformer.hip computes in two launches (talk
// notes "Flashlight: PyTorch Compiler Extensions to Accelerate Attention
// Variants", "Evaluation: complex attention variants"; reading: per MSA
// sequence s and head h, q, k, v, g = m Wq, m Wk, m Wv, m Wg and
// out[s, i, h*dh + e] = sigmoid(g_i[e]) * softmax_j(scale q_i.k_j + bias[h, i, j]) v_j[e];
// column-wise the same over the sequences of one residue column, without
// the bias).  The text below says "residues" for the tokens of one
// attention problem; column-wise they are the sequences of the column.
// Here the projections never leave the chip, as the pages' fusion does for
// this variant (talk notes, "Compiler design" 3: the intermediate is not
// written to global memory):
//
//  * One workgroup = one (sequence, head), column-wise one (residue column,
//    head).  Its NW waves own the 32-residue blocks w, w + NW, ... of the
//    sequence.
//  * Phase A: K and V of every residue, C^T = W^T m^T with the head's
//    [Wk | Wv] slice staged in LDS (read transposed as the MFMA A operand;
//    in two halves of the channels where LDS is short, see FusedCfg) and
//    the m rows loaded straight from memory as the B operand; the
//    results go to LDS, K with its columns in the order the QK^T operands
//    want (so no register shuffle is needed), V swizzled for transposed reads.
//  * Phase B: q (softmax scale folded in before the one bf16 rounding) and
//    the gate pre-activations of the wave's own residues, with [Wq | Wg] in
//    the same LDS bytes, kept in registers: q already in the B-operand
//    layout of S^T = K Q^T, g in the layout of the O^T accumulator.
//  * Phase C: each wave runs the fused attention of its 32-row blocks over
//    all residues with K and V resident in LDS, so the waves never meet: no
//    barrier in the key loop.  Row-wise, the pair bias of a 32 x 64 tile is
//    loaded as coalesced 16-byte row chunks into a wave-private LDS slot,
//    two tiles ahead, and read back as the initial value of the QK^T
//    accumulators; column-wise the accumulators start at zero.
//  * Sequences (columns) outermost in the grid, heads innermost, remapped so
//    that one XCD runs the heads of a few sequences side by side: each m row
//    comes from HBM once and then from that XCD's L2.
// Instantiated for Cm = 256, dh in {32, 64} and up to 256 residues (row-wise
// N_res a multiple of 8, for the 16-byte bias rows): K and V of the whole
// sequence in LDS and at most two residue blocks per wave, whose m operand
// stays in registers through both projection phases (see evo_fused_fits for
// the measured limit).

#include <type_traits>

#include "attn_tile.hpp"
#include "av_kernels.hpp"

namespace av {
namespace {

constexpr int FCM = 256;  // channels of m (Cm) of this form
constexpr int FBN = 64;   // keys per attention tile
constexpr int FBP = FBN + 4;  // bias slot pitch: 8-byte reads of 32 rows hit 32 distinct bank pairs

// K tile: rows of DH elements in 16-byte chunks; chunk c of row r is stored
// at chunk c ^ swz(r) so that the 16 lanes of one ds_read_b128 pass (16
// consecutive rows, one chunk each) cover 16 distinct 16-byte bank groups.
template <int DH>
__device__ __forceinline__ int k_chunk(int row, int c) {
  constexpr int CPR = DH / 8;         // chunks per row
  constexpr int RPW = 16 / CPR;       // rows per 256-byte bank window
  return row * DH + 8 * (c ^ ((row / RPW) % CPR));
}

// WS: the W slice of a projection phase is staged in WS parts of FCM / WS
// rows (channels of m), the next part's loads in flight during the current
// part's MFMAs.
template <int DH, int NW, int LMAX, int WS>
struct FusedCfg {
  static constexpr int NT = NW * 64;
  static constexpr int MT = (LMAX / 32 + NW - 1) / NW;    // 32-residue blocks per wave
  static constexpr int NCB = 2 * DH / 32;                 // 32-channel blocks of one projection pair
  static constexpr int W_ELEMS = FCM / WS * 2 * DH;       // one part of the [Wk | Wv] or [Wq | Wg] slice
  static constexpr int SLOT_ELEMS = 32 * FBP;             // one wave's bias slot
  static constexpr int U_ELEMS = W_ELEMS > NW * SLOT_ELEMS ? W_ELEMS : NW * SLOT_ELEMS;
  static constexpr int LDS_BYTES = (2 * LMAX * DH + U_ELEMS) * 2;
  // waves per SIMD the registers are sized for: three where the LDS holds
  // three four-wave workgroups per CU (160 KB), else two
  static constexpr int OCC = NW == 4 && 3 * LDS_BYTES <= 160 * 1024 ? 3 : 2;
};

// LDS-only workgroup barrier (the global stores of earlier phases need not
// complete before the next phase starts).
__device__ __forceinline__ void lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Two waves per SIMD (four-wave workgroups two per CU, eight-wave workgroups
// one per CU), three for the small-LDS four-wave forms.
template <int DH, int NW, int LMAX, int WS, bool COL>
__global__ __launch_bounds__(NW * 64, (FusedCfg<DH, NW, LMAX, WS>::OCC)) void evo_fused_row_kernel(const EvoArgs a) {
  using C = FusedCfg<DH, NW, LMAX, WS>;
  constexpr int NT = C::NT, MT = C::MT, NCB = C::NCB;
  constexpr int NDB = DH / 32;   // d-blocks of O^T
  constexpr int NDS = DH / 16;   // QK^T k-steps
  constexpr int NKB = FBN / 32;  // 32-key blocks per tile
  constexpr int NPS = FBN / 16;  // PV k-steps
  constexpr int WW = 2 * DH;     // W slice width (two projections)
  __shared__ __attribute__((aligned(16))) bf16 Ks[LMAX * DH];
  __shared__ __attribute__((aligned(16))) bf16 Vs[LMAX * DH];
  __shared__ __attribute__((aligned(16))) bf16 Us[C::U_ELEMS];  // W slice (phases A, B), bias slots (C)

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so the per-wave guards are scalar
  const int hh = lane >> 5, l32 = lane & 31;
  // The workgroup's attention runs over Nr tokens: row-wise the residues of
  // sequence `s` (m rows s * Nr .. + Nr - 1), column-wise the sequences of
  // residue column `s` (m rows s, s + Nr, ...; no pair bias).
  const int total = (COL ? a.Nr : a.Ns) * a.H;
  const int L = xcd_remap(blockIdx.x, total);
  const int s = L / a.H, h = L % a.H;
  const int Nr = COL ? a.Ns : a.Nr, HD = a.H * DH;
  const size_t tok_stride = COL ? (size_t)a.Nr * FCM : (size_t)FCM;  // elements between the tokens' m rows
  const int nTB = (Nr + 31) / 32;
  const int nKT = (Nr + FBN - 1) / FBN;  // 64-key tiles of the attention
  // this wave's token blocks: w, w + NW, ...
  const int nmine = w < nTB ? (nTB - 1 - w) / NW + 1 : 0;

  // m rows of these tokens; rows past Nr read as zero (buffer bounds)
  const uint32_t m_bytes = (uint32_t)(((size_t)(Nr - 1) * tok_stride + FCM) * 2);
  const auto mrs = make_rsrc((const bf16*)a.m + (COL ? (size_t)s * FCM : (size_t)s * Nr * FCM), m_bytes);
  uint32_t mrow[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int r = (w + NW * i) * 32 + l32;
    mrow[i] = (i < nmine && r < Nr) ? (uint32_t)((size_t)r * tok_stride * 2) + hh * 16 : m_bytes;
  }
  // W^T operand of projection k-step t (32 channels from dcol x 16 rows of
  // m's channels): lane (channel l32, half hh) needs rows 16 t + 8 hh + 0..7,
  // in order, to pair with the m operand; lane r of each 16-lane group points
  // at row 16 t + 8 hh + r/4 (and + 4), columns 16 g + 4 (r%4) of the block
  // (rows congruent to r/4 mod 4: the swizzle is a per-lane constant)
  const TrLane<WW> wl(lane);
  const int w_row0 = 8 * hh + ((lane & 15) >> 2);
  auto w_operand = [&](int t, int dcol) {
    const bf16* wp = Us + (16 * t + w_row0) * WW + ((dcol + wl.col0) ^ wl.xo);
    const i16x4 lo = lds_read_tr16(wp);
    const i16x4 hi = lds_read_tr16(wp + 4 * WW);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // The head's slice of two projections, [Wa | Wb] = [FCM x 2 DH], in WS
  // parts of FCM / WS rows: load_w brings part `part` into registers,
  // store_w writes it to LDS row-major, swizzled for transposed reads.
  constexpr int WR = FCM / WS;      // rows of one part
  constexpr int CH = WR * DH / 8;   // 16-byte chunks of one matrix's part
  static_assert(CH % NT == 0, "W slice / thread mismatch");
  using WRegs = i32x4[2][CH / NT];
  auto load_w = [&](const void* wa, const void* wb, int part, WRegs& t) {
    // one pass per matrix: a per-lane choice between the two buffer
    // descriptors would make the descriptor divergent (a loop per load)
    const auto ars = make_rsrc(wa, (uint32_t)FCM * HD * 2);
    const auto brs = make_rsrc(wb, (uint32_t)FCM * HD * 2);
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int c = 0; c < CH / NT; ++c) {
        const int idx = tid + NT * c;
        const int row = part * WR + idx / (DH / 8), col = (idx % (DH / 8)) * 8;
        t[m][c] = buf_load16(m == 0 ? ars : brs, (uint32_t)(row * HD + h * DH + col) * 2);
      }
  };
  auto store_w = [&](const WRegs& t) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int c = 0; c < CH / NT; ++c) {
        const int idx = tid + NT * c;
        const int row = idx / (DH / 8), col = (idx % (DH / 8)) * 8;
        *(i32x4*)&Us[tr_tile_off<WW>(row, m * DH + col)] = t[m][c];
      }
  };

  // The m operand of every k-step of this wave's residue blocks, loaded once
  // (up front, so that the latency overlaps the first W staging) and used by
  // both projection phases: lane (residue l32, half hh) of k-step t holds
  // m[r][16 t + 8 hh .. + 7].
  constexpr int NST = FCM / 16;
  bf16x8 mall[MT][NST];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < NST; ++t) mall[i][t] = __builtin_bit_cast(bf16x8, buf_load16(mrs, mrow[i] + t * 32));

  // C^T = [Wa | Wb]^T m^T for this wave's residue blocks: acc[cb][i] is the
  // 32 x 32 tile of channel block cb (cb < NCB / 2: Wa) and residue block i.
  // The W part in LDS covers the k-steps part * NST / WS ..
  auto project_part = [&](f32x16 (&acc)[NCB][MT], auto part) {
    constexpr int T0 = decltype(part)::value * (NST / WS);
    auto run = [&](auto all) {
#pragma unroll
      for (int t = 0; t < NST / WS; ++t) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
          const bf16x8 wf = w_operand(t, 32 * cb);
#pragma unroll
          for (int i = 0; i < MT; ++i)
            if (decltype(all)::value || i < nmine) acc[cb][i] = mfma32(wf, mall[i][T0 + t], acc[cb][i]);
        }
      }
    };
    // the usual case (every wave owns MT blocks) without a branch per MFMA
    if (nmine == MT) {
      run(std::true_type{});
    } else {
      run(std::false_type{});
    }
  };
  // One projection phase: stage part 0 (the loads of part 1 go out behind
  // it), project, and with two parts stage and project the second.
  auto project = [&](const void* wa, const void* wb, f32x16 (&acc)[NCB][MT]) {
    static_assert(WS == 1 || WS == 2, "one or two W parts");
    WRegs wt;
    load_w(wa, wb, 0, wt);
    store_w(wt);
    if constexpr (WS == 2) load_w(wa, wb, 1, wt);
    lds_sync();
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int i = 0; i < MT; ++i) acc[cb][i] = f32x16{};
    project_part(acc, std::integral_constant<int, 0>{});
    if constexpr (WS == 2) {
      lds_sync();  // every wave is done with part 0
      store_w(wt);
      lds_sync();
      project_part(acc, std::integral_constant<int, 1>{});
    }
  };

  // ---- phase A: K and V of every residue into LDS
  {
    f32x16 acc[NCB][MT];
    project(a.w[1], a.w[2], acc);
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      if (i >= nmine) continue;
      const int r = (w + NW * i) * 32 + l32;  // residue of this lane (rows past Nr hold zeros)
#pragma unroll
      for (int cb = 0; cb < NCB / 2; ++cb) {
        // K: channels 32 cb + 8 (j/4) + 4 hh + j%4 of residue r; registers
        // j = 0..7 and 8..15 become the 16-byte chunks 4 cb + hh and
        // 4 cb + 2 + hh of the row (the operand order of the QK^T k-steps)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          bf16x8 v8;
#pragma unroll
          for (int e = 0; e < 8; ++e) v8[e] = (bf16)acc[cb][i][8 * half + e];
          *(bf16x8*)&Ks[k_chunk<DH>(r, 4 * cb + 2 * half + hh)] = v8;
        }
        // V: natural channel order, swizzled for the transposed PV reads
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          bf16x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = (bf16)acc[NCB / 2 + cb][i][4 * g4 + e];
          *(bf16x4*)&Vs[tr_tile_off<DH>(r, 32 * cb + 8 * g4 + 4 * hh)] = v4;
        }
      }
    }
  }
  // V rows from the last residue block to the end of the last 64-key tile
  // enter the PV product with p = 0: they must hold zeros, not stale bytes
  for (int idx = tid; idx < (nKT * FBN - nTB * 32) * (DH / 8); idx += NT) {
    const int row = nTB * 32 + idx / (DH / 8), col = (idx % (DH / 8)) * 8;
    *(i32x4*)&Vs[tr_tile_off<DH>(row, col)] = i32x4{0, 0, 0, 0};
  }
  lds_sync();  // K, V complete; the W slice bytes are free

  // ---- phase B: q (scaled) and the gate of this wave's residues, in registers
  bf16x8 qreg[MT][NDS];
  bf16x4 gate[MT][NDB * 4];
  {
    f32x16 acc[NCB][MT];
    project(a.w[0], a.w[3], acc);
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int cb = 0; cb < NDB; ++cb) {
#pragma unroll
        for (int half = 0; half < 2; ++half)
#pragma unroll
          for (int e = 0; e < 8; ++e) qreg[i][2 * cb + half][e] = (bf16)(acc[cb][i][8 * half + e] * a.scale);
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
          for (int e = 0; e < 4; ++e) gate[i][cb * 4 + g4][e] = (bf16)acc[NDB + cb][i][4 * g4 + e];
      }
  }
  lds_sync();  // every wave is done with the W slice: its bytes become the bias slots

  // ---- phase C: attention of this wave's 32-row blocks over all residues.
  // The pair-bias tiles of the wave's (block, key tile) sequence stream through
  // two register buffers, two tiles ahead, across block boundaries.
  bf16* slot = Us + w * C::SLOT_ELEMS;
  const auto brs = make_rsrc(COL ? nullptr : (const bf16*)a.bias + (size_t)h * Nr * Nr, COL ? 0u : (uint32_t)Nr * Nr * 2);
  const TrLane<DH> vl(lane);
  const int nflat = nmine * nKT;
  // bias rows q0 .. q0+31, keys n0 .. n0+63 of flat tile f: lane loads row
  // q0 + lane/8 + 8c, keys n0 + 8 (lane%8) .. +7 (rows past Nr read as zero;
  // keys past Nr are masked)
  auto bload = [&](int f, i32x4 (&dst)[4]) {
    const int bi = f / nKT, kt = f - bi * nKT;
    const int q0 = (w + NW * bi) * 32, n0 = kt * FBN;
#pragma unroll
    for (int c = 0; c < 4; ++c)
      dst[c] = buf_load16(brs, (uint32_t)((q0 + (lane >> 3) + 8 * c) * Nr + n0 + 8 * (lane & 7)) * 2);
  };
  i32x4 br0[4], br1[4];
  if constexpr (!COL) {
    if (nflat > 0) bload(0, br0);
    if (nflat > 1) bload(1, br1);
  }
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    if (i >= nmine) break;
    if (!COL && i > 0 && (nKT & 1)) {  // the flat tile parity flips at this block
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const i32x4 t = br0[c];
        br0[c] = br1[c];
        br1[c] = t;
      }
    }
    const int q0 = (w + NW * i) * 32;
    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
    RowState st;
    auto step = [&](int kt, i32x4 (&bcur)[4]) {
      const int n0 = kt * FBN;
      if constexpr (!COL) {
        // stage this tile's bias (wave-private slot; the wave's LDS accesses
        // execute in order, so no barrier), then fetch the tile two ahead
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          bf16* dst = slot + ((lane >> 3) + 8 * c) * FBP + 8 * (lane & 7);
          *(i32x2*)dst = i32x2{bcur[c][0], bcur[c][1]};
          *(i32x2*)(dst + 4) = i32x2{bcur[c][2], bcur[c][3]};
        }
        const int f = i * nKT + kt;
        if (f + 2 < nflat) bload(f + 2, bcur);
      }
      // S^T = K Q^T (+ bias: row-wise the accumulators start at the bias)
      f32x16 sc[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        if constexpr (COL) {
          sc[kb] = f32x16{};
        } else {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const i32x2 b2 = *(const i32x2*)(slot + l32 * FBP + 32 * kb + 8 * g + 4 * hh);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int wd = b2[e >> 1];
              sc[kb][4 * g + e] = __builtin_bit_cast(float, (e & 1) ? (wd & (int)0xffff0000) : (wd << 16));
            }
          }
        }
        const int key = n0 + 32 * kb + l32;
#pragma unroll
        for (int st_ = 0; st_ < NDS; ++st_) {
          const bf16x8 kf = *(const bf16x8*)&Ks[k_chunk<DH>(key, 2 * st_ + hh)];
          sc[kb] = mfma32(kf, qreg[i][st_], sc[kb]);
        }
      }
      // keys past Nr (ragged last tile): -inf
      if (n0 + FBN > Nr) {
        const int lim = Nr - n0 - 4 * hh;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
          mask_block(sc[kb], [&](int off) { return 32 * kb + off < lim; });
      }
      // online softmax, optimistic exponent reference (as the fused attention kernel)
      bf16x8 pb[NPS];
      float tsum = exp_pack_sum<NKB, 0>(sc, kLog2e, st.m_sub, pb);
      if (any_lane(tsum > kOptBound || st.m_ref == neg_inf())) {
        st.template raise<NDB>(xhalf_max(block_max<NKB>(sc)) * kLog2e, o);
        tsum = exp_pack_sum<NKB, 0>(sc, kLog2e, st.m_sub, pb);
      }
      st.l += tsum;
      // O^T += V^T P^T
      bf16x8 vfa[NDB][NPS];
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int t = 0; t < NPS; ++t) vfa[db][t] = vt_operand<DH>(Vs + (size_t)n0 * DH, t, 32 * db, vl);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int t = 0; t < NPS; ++t) o[db] = mfma32(vfa[db][t], pb[t], o[db]);
    };
#pragma unroll 1
    for (int kt = 0; kt < nKT; kt += 2) {
      step(kt, br0);
      if (kt + 1 < nKT) step(kt + 1, br1);
    }
    // epilogue: out[token, h*DH + d] = sigmoid(g) * O / l (token (s, q)
    // row-wise, (q, s) column-wise)
    const int q = q0 + l32;
    const float l_tot = xhalf_sum(st.l);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (q < Nr) {
      const size_t tok = COL ? (size_t)q * a.Nr + s : (size_t)s * Nr + q;
      bf16* orow = (bf16*)a.out + tok * HD + (size_t)h * DH;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const bf16x4 gv = gate[i][db * 4 + g4];
          bf16x4 val;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float sig = rcp_fast(1.f + exp2_fast(-(float)gv[e] * kLog2e));
            val[e] = (bf16)(o[db][g4 * 4 + e] * inv * sig);
          }
          *(bf16x4*)(orow + 32 * db + 8 * g4 + 4 * hh) = val;
        }
    }
  }
}

template <int DH, int NW, int LMAX, int WS, bool COL>
hipError_t launch_fused(const EvoArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((evo_fused_row_kernel<DH, NW, LMAX, WS, COL>), dim3((COL ? a.Nr : a.Ns) * a.H), dim3(NW * 64),
                     0, stream, a);
  return hipGetLastError();
}

}  // namespace

// Row-wise, up to 256 residues: same-box timings at 128 sequences, against
// the two launches, 52.7 vs 58.6 us (8 x 32) and 43.3 vs 56.4 us (4 x 64).
// At 384 residues (eight waves, one workgroup per CU) the single launch
// measured 96.9 against 91.1 us: its serial phases no longer overlap another
// workgroup's, so longer sequences keep the two launches.  Column-wise over
// 128 sequences (the 128-token forms), against the two launches at 256 / 384
// / 768 residues: 36.8 / 51.7 / 94.0 vs 52.7 / 68.0 / 138.0 us (8 x 32) and
// 32.7 / 45.7 / 84.6 vs 51.4 / 67.0 / 137.0 us (4 x 64; with the W slice in
// one part, 96 KB of LDS and one workgroup per CU, 45.3 / 65.8 / 126.5 us).
// Over 256 sequences (the 256-token forms) at 256 residues: 75.9 vs 94.6 us
// (8 x 32) and 77.7 vs 93.8 us (4 x 64).
bool evo_fused_fits(const EvoArgs& a) {
  if (a.Cm != FCM || (a.dh != 32 && a.dh != 64)) return false;
  if (a.col) return a.Ns <= 256 && (size_t)a.Ns * a.Nr * FCM * 2 < (1ull << 31);
  return a.Nr % 8 == 0 && a.Nr <= 256;
}

hipError_t launch_evo_fused(const EvoArgs& a, hipStream_t stream) {
  if (a.col) {
    // four waves and the LDS of 128 tokens: 48 KB at dh 32 (three workgroups
    // per CU), 64 KB at dh 64 with the W slice in two parts (two per CU)
    if (a.Ns <= 128) {
      if (a.dh == 64) return launch_fused<64, 4, 128, 2, true>(a, stream);
      return launch_fused<32, 4, 128, 1, true>(a, stream);
    }
    if (a.dh == 64) return launch_fused<64, 8, 256, 1, true>(a, stream);
    return launch_fused<32, 4, 256, 1, true>(a, stream);
  }
  if (a.dh == 64) return launch_fused<64, 8, 256, 1, false>(a, stream);
  return launch_fused<32, 4, 256, 1, false>(a, stream);
}

}  // namespace av
