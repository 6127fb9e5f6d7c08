// Differential attention forward for gfx950, fused in one kernel.
//
// The pages name differential attention as one of the variants that static
// templates cannot express and that Flashlight fuses (talk notes "Flashlight:
// PyTorch Compiler Extensions to Accelerate Attention Variants", sections
// "Background and motivation" and "Evaluation: complex attention variants")
// but do not define it.  The reading implemented: Q and K rows hold two
// halves of width Dh (64 for the 16 heads x 128 shape, 32 for 32 heads x 64);
// each half yields its own softmax with scale 1/sqrt(Dh) (causal when asked);
// out = (P1 - lambda * P2) V with V of width Dv.
//
// Kernel shape: the fused attention kernel's skeleton with two score tiles
// and two online-softmax states per query row.  One workgroup = 4 waves =
// 128 query rows; each KV tile (32 keys) is loaded once into LDS and serves
// both branches; each V^T operand read from LDS feeds both PV products.  The
// two output accumulators (32 rows x Dv fp32 per wave each) are combined in
// the epilogue: out = O1 / l1 - lambda * O2 / l2.
//
// Full head form (HEAD): the DiffTransformer head around that core, as the
// published Differential Transformer defines it (Ye et al., 2024; the pages
// name DiffTransformer under related work, talk notes "Related work").  The
// kernel derives lambda = exp(lq1.lk1) - exp(lq2.lk2) + lambda_init from the
// four Dh-wide parameter vectors (one lane per component, a wave-wide sum),
// keeps A = O1/l1 - lambda O2/l2 in fp32, and stores
// (1 - lambda_init) * gamma * A / sqrt(mean(A^2) + eps) per row: each query
// row's Dv values sit in one lane pair, so the row's sum of squares is an
// in-register sum plus one cross-half swap, and nothing leaves the kernel
// before the normalised bf16 row.

#include "attn_tile.hpp"
#include "av_kernels.hpp"

namespace av {
namespace {

constexpr int BM = kAttnBM;
constexpr int BN = 32;   // keys per KV tile (register budget: two score tiles, two accumulators)
constexpr int NT = 256;

// DH: width of one Q/K half (32 or 64); DV: width of V and of the output
template <int DH, int DV, bool HEAD>
__global__ __launch_bounds__(NT, 2) void diff_attn_fwd_kernel(const DiffArgs a) {
  constexpr int DQ = 2 * DH;
  constexpr int NDS = DH / 16;          // QK^T k-steps per branch
  constexpr int NDB = DV / 32;          // O^T d-blocks per branch
  constexpr int NPS = BN / 16;          // PV k-steps
  constexpr int KP = DQ + 8;
  constexpr int KCPR = DQ / 8, VCPR = DV / 8;
  constexpr int KCH = BN * KCPR / NT, VCH = BN * VCPR / NT;
  static_assert(KCH >= 1 && VCH >= 1, "tile/thread mismatch");

  __shared__ __attribute__((aligned(16))) bf16 Ks[2][BN * KP];
  __shared__ __attribute__((aligned(16))) bf16 Vs[2][BN * DV];  // swizzled for transposed reads

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hh = lane >> 5, l32 = lane & 31;

  int mt_lin, bh;
  if (a.causal) {
    const TileIdx ti = weighted_tile(blockIdx.x, a.total, a.nM);
    mt_lin = ti.mt_lin;
    bh = ti.bh;
  } else {
    const int L = xcd_remap(blockIdx.x, a.total);
    mt_lin = L % a.nM;
    bh = L / a.nM;
  }
  const int mt = a.causal ? (a.nM - 1 - mt_lin) : mt_lin;
  const int S = a.S;
  const int q0 = mt * BM;
  const int qw = q0 + 32 * __builtin_amdgcn_readfirstlane(w);
  const int qi = qw + l32;
  const int qlast = min(q0 + BM, S) - 1;
  const bool wave_live = qw < S;
  const int qwlast = min(qw + 31, S - 1);

  const size_t qkoff = (size_t)bh * S * DQ;
  const size_t voff = (size_t)bh * S * DV;
  const auto qrs = make_rsrc((const bf16*)a.q + qkoff, (uint32_t)S * DQ * 2);
  const auto krs = make_rsrc((const bf16*)a.k + qkoff, (uint32_t)S * DQ * 2);
  const auto vrs = make_rsrc((const bf16*)a.v + voff, (uint32_t)S * DV * 2);

  const int nKV = (S + BN - 1) / BN;
  const int n_hi = a.causal ? min(nKV, qlast / BN + 1) : nKV;

  // Q^T operands of both halves: qreg[0..3] half 1, qreg[4..7] half 2
  bf16x8 qreg[2 * NDS];
#pragma unroll
  for (int s = 0; s < 2 * NDS; ++s)
    qreg[s] = __builtin_bit_cast(bf16x8, buf_load16(qrs, (uint32_t)(qi * DQ + s * 16 + hh * 8) * 2));

  f32x16 o1[NDB], o2[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) o1[i] = o2[i] = f32x16{};
  RowState st1, st2;
  const TrLane<DV> vl(lane);

  i32x4 kr[KCH], vr[VCH];
  auto gload = [&](int nt) {
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int idx = tid + NT * c, row = idx / KCPR, col = idx % KCPR;
      kr[c] = buf_load16(krs, (uint32_t)((nt * BN + row) * DQ + col * 8) * 2);
    }
#pragma unroll
    for (int c = 0; c < VCH; ++c) {
      const int idx = tid + NT * c, row = idx / VCPR, col = idx % VCPR;
      vr[c] = buf_load16(vrs, (uint32_t)((nt * BN + row) * DV + col * 8) * 2);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int idx = tid + NT * c, row = idx / KCPR, col = idx % KCPR;
      *(i32x4*)&Ks[buf][row * KP + col * 8] = kr[c];
    }
#pragma unroll
    for (int c = 0; c < VCH; ++c) {
      const int idx = tid + NT * c, row = idx / VCPR, col = idx % VCPR;
      *(i32x4*)&Vs[buf][tr_tile_off<DV>(row, col * 8)] = vr[c];
    }
  };

  if (n_hi > 0) gload(0);
  for (int nt = 0; nt < n_hi; ++nt) {
    const int buf = nt & 1;
    sstore(buf);
    __syncthreads();
    if (nt + 1 < n_hi) gload(nt + 1);

    const int n0 = nt * BN, n1 = n0 + BN - 1;
    bool skip = !wave_live;
    bool full = n1 < S;
    if (a.causal) {
      skip |= n0 > qwlast;
      full &= n1 <= qw;
    }
    if (__builtin_amdgcn_readfirstlane((int)skip)) continue;

    f32x16 s1 = qk_block<NDS, KP>(Ks[buf], 0, 0, qreg, l32, hh);
    f32x16 s2 = qk_block<NDS, KP>(Ks[buf], 0, DH, qreg + NDS, l32, hh);
    if (!__builtin_amdgcn_readfirstlane((int)full)) {
      const int kbase = n0 + 4 * hh;
      const int lim = S - kbase, rel = qi - kbase;
      const bool causal = a.causal;
      auto keep = [&](int off) { return off < lim && (!causal || off <= rel); };
      mask_block(s1, keep);
      mask_block(s2, keep);
    }
    st1.update<NDB>(xhalf_max(block_max<1>(&s1)) * a.c, o1);
    st2.update<NDB>(xhalf_max(block_max<1>(&s2)) * a.c, o2);
    bf16x8 pb1[NPS], pb2[NPS];
    st1.l += exp_pack_sum<1, 0>(&s1, a.c, st1.m_sub, pb1);
    st2.l += exp_pack_sum<1, 0>(&s2, a.c, st2.m_sub, pb2);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int t = 0; t < NPS; ++t) {
        const bf16x8 vf = vt_operand<DV>(Vs[buf], t, db * 32, vl);
        o1[db] = mfma32(vf, pb1[t], o1[db]);
        o2[db] = mfma32(vf, pb2[t], o2[db]);
      }
    }
  }

  // A = O1 / l1 - lambda * O2 / l2 (fp32, in place in o1)
  float lam = a.lambda;
  if constexpr (HEAD) {
    const float d1 = wave_sum(lane < DH ? a.lam_q1[lane] * a.lam_k1[lane] : 0.f);
    const float d2 = wave_sum(lane < DH ? a.lam_q2[lane] * a.lam_k2[lane] : 0.f);
    lam = expf(d1) - expf(d2) + a.lambda_init;
  }
  const float l1 = xhalf_sum(st1.l), l2 = xhalf_sum(st2.l);
  const float inv1 = l1 > 0.f ? 1.f / l1 : 0.f;
  const float inv2 = l2 > 0.f ? lam / l2 : 0.f;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) o1[db][j] = fmaf(o1[db][j], inv1, -o2[db][j] * inv2);
  // head form: (1 - lambda_init) / sqrt(mean(A^2) + eps) over the row's DV values
  float post = 1.f;
  if constexpr (HEAD) {
    float ss = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 16; ++j) ss = fmaf(o1[db][j], o1[db][j], ss);
    ss = xhalf_sum(ss);
    post = (1.f - a.lambda_init) * rsqrtf(ss * (1.f / DV) + a.eps);
  }
  if (qi < S) {
    bf16* orow = (bf16*)a.o + voff + (size_t)qi * DV;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int col = db * 32 + 8 * g4 + 4 * hh;
        bf16x4 val;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float y = o1[db][g4 * 4 + e];
          if constexpr (HEAD) y *= post * (a.gamma != nullptr ? a.gamma[col + e] : 1.f);
          val[e] = (bf16)y;
        }
        *(bf16x4*)(orow + col) = val;
      }
    }
  }
}

template <int DH>
hipError_t launch_diff_dh(const DiffArgs& a, int Dv, hipStream_t stream) {
  const bool head = a.lam_q1 != nullptr;
  if (Dv == 64 && !head)
    hipLaunchKernelGGL((diff_attn_fwd_kernel<DH, 64, false>), dim3(a.total), dim3(NT), 0, stream, a);
  else if (Dv == 64)
    hipLaunchKernelGGL((diff_attn_fwd_kernel<DH, 64, true>), dim3(a.total), dim3(NT), 0, stream, a);
  else if (Dv == 128 && !head)
    hipLaunchKernelGGL((diff_attn_fwd_kernel<DH, 128, false>), dim3(a.total), dim3(NT), 0, stream, a);
  else if (Dv == 128)
    hipLaunchKernelGGL((diff_attn_fwd_kernel<DH, 128, true>), dim3(a.total), dim3(NT), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

hipError_t launch_diff_attn_fwd(const DiffArgs& a, int Dh, int Dv, hipStream_t stream) {
  switch (Dh) {
    case 32: return launch_diff_dh<32>(a, Dv, stream);
    case 64: return launch_diff_dh<64>(a, Dv, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace av
