// Evoformer row-wise gated self-attention with pair bias, gfx950.
//
// The pages name this variant among those Flashlight fuses and templates
// cannot express (talk notes "Flashlight: PyTorch Compiler Extensions to
// Accelerate Attention Variants", "Evaluation: complex attention variants"
// and the AlphaFold2 end-to-end section: 8 heads x 32) but print no formula.
// Reading implemented, per MSA sequence s and head h:
//   q, k, v, g = m Wq, m Wk, m Wv, m Wg
//   out[s, i, h*dh + e] = sigmoid(g[s, i, h*dh + e]) * softmax_j(q_i.k_j * scale + bias[h, i, j]) v_j[e]
//
// Two launches:
//  1. evo_proj_kernel: the four projections as one bf16 MFMA GEMM with fp32
//     accumulation (the pages' precision rule), M = Ns*Nr tokens, N = 4*H*dh
//     channels, K = Cm.  It computes C^T = W^T m^T so that each lane ends up
//     holding 4 consecutive channels of one token; results are rounded to
//     bf16 and scattered head-major into the workspace as four planes
//     [Ns, H, Nr, dh] (scale*q, k, v, g).  The softmax scale is applied to q
//     in fp32 before its one bf16 rounding, so the attention kernel's raw
//     scores are already scaled and the pair bias becomes the initial
//     accumulator of the QK^T MFMA.
//  2. the fused attention kernel at D = dh (32 or 64) with the pair bias as score
//     modifier and the sigmoid gate + token-major store as epilogue; each
//     (sequence, head, 128-residue tile) is one workgroup, sequences vary
//     fastest within a head so bias[h] stays resident in L2.
//
// The column-wise form (attention over the sequences of each residue column,
// no pair bias) runs the same two launches where it does not take the
// one-kernel path (more than 256 sequences, or Cm other than 256): the GEMM
// orders tokens column-major and writes planes [Nr, H, Ns, dh], and the
// attention kernel takes one (residue, head) per problem with the gated
// epilogue only.

#include "attn_tile.hpp"
#include "av_kernels.hpp"

namespace av {
namespace {

constexpr int GK = 64;   // K chunk staged in LDS
constexpr int MP = GK + 8;   // m tile pitch: 8 rows -> 8 distinct 16-byte bank groups

// Row-major W tile of GN (128 or 256) columns read by transposed LDS reads: a
// read serves 4 consecutive rows x 64 bytes, which must fall in distinct
// 64-byte segments of the 256-byte bank window, so the 64-byte segments of
// row r are XOR-permuted by r mod 4.
__device__ __forceinline__ int w_swz(int row) { return row & 3; }
template <int GN>
__device__ __forceinline__ int w_off(int row, int c) { return row * GN + (c ^ (w_swz(row) << 5)); }

// GM tokens x GN channels per workgroup of NT threads; each wave computes 64
// channels x (GM / WM) tokens.  The 256 x 256 form (8 waves) reads half the
// operand bytes per FLOP of the 128 x 128 form (with K = Cm = 256 the MFMAs
// are a small part of the time) but holds one workgroup per CU.
// DH: head width (32 or 64), which sets how the C tile splits into the
// head-major planes.
template <int GM, int GN, int NT, int DH>
__global__ __launch_bounds__(NT, NT == 256 ? 2 : 1) void evo_proj_kernel(const EvoArgs a) {
  constexpr int NW = NT / 64;
  constexpr int WN = GN / 64;            // waves along the channels
  constexpr int WM = NW / WN;            // waves along the tokens
  constexpr int MB = GM / WM / 32;       // 32-token MFMA blocks per wave
  constexpr int MCH = GM * GK / 8 / NT;  // 16-byte m chunks per thread and K chunk
  constexpr int WCH = GK * GN / 8 / NT;  // 16-byte W chunks per thread and K chunk
  static_assert(WN * WM == NW && MB >= 1 && MCH >= 1 && WCH >= 1, "tile/thread mismatch");
  constexpr int M_ELEMS = GM * MP, W_ELEMS = GK * GN;
  constexpr int CP = GN + 8;             // epilogue C tile pitch
  constexpr int LDS_ELEMS = 2 * (M_ELEMS + W_ELEMS) > GM * CP ? 2 * (M_ELEMS + W_ELEMS) : GM * CP;
  __shared__ __attribute__((aligned(16))) bf16 lds[LDS_ELEMS];
  bf16* const Ms0 = lds;
  bf16* const Ws0 = lds + 2 * M_ELEMS;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hh = lane >> 5, l32 = lane & 31;
  const int HD = a.H * a.dh;            // channels per projection
  const int N = 4 * HD;
  const int M = a.Ns * a.Nr;
  const int ntiles = N / GN;
  const int total = ((M + GM - 1) / GM) * ntiles;
  const int L = xcd_remap(blockIdx.x, total);
  const int mt = L / ntiles, nt = L % ntiles;  // the channel tiles of one token tile are neighbours
  const int n0 = nt * GN;
  const int p = n0 / HD;                       // projection of this tile (GN divides HD)
  const int c0 = n0 % HD;
  const int wn = w % WN, wm = w / WN;          // wave: 64 channels x GM / WM tokens

  // Token order: row-wise, token t = (sequence, residue) in MSA order; column-
  // wise, t = residue * Ns + sequence, so that the tokens of one attention
  // problem (one residue column) are consecutive.  Linner is the attention
  // length, the inner factor of t.
  const int Linner = a.col ? a.Ns : a.Nr;
  const uint32_t m_bytes = (uint32_t)M * a.Cm * 2;
  const auto mrs = make_rsrc(a.m, m_bytes);
  const bf16* wbase = (const bf16*)a.w[p];
  const auto wrs = make_rsrc(wbase, (uint32_t)a.Cm * HD * 2);

  // byte offset of the m row of each token this thread stages (past the end:
  // tokens beyond M, read as zeros)
  uint32_t mrow_off[MCH];
#pragma unroll
  for (int c = 0; c < MCH; ++c) {
    const int t = mt * GM + ((tid + NT * c) >> 3);
    const int row = a.col ? (t % a.Ns) * a.Nr + t / a.Ns : t;
    mrow_off[c] = t < M ? (uint32_t)row * a.Cm * 2 : m_bytes;
  }

  i32x4 mr[MCH], wr[WCH];
  auto gload = [&](int kc) {
#pragma unroll
    for (int c = 0; c < MCH; ++c) {
      const int idx = tid + NT * c;
      mr[c] = buf_load16(mrs, mrow_off[c] + (uint32_t)(kc * GK + (idx & 7) * 8) * 2);
    }
#pragma unroll
    for (int c = 0; c < WCH; ++c) {
      const int idx = tid + NT * c;
      const int wrow = idx / (GN / 8), wcol = idx % (GN / 8);
      wr[c] = buf_load16(wrs, (uint32_t)((kc * GK + wrow) * HD + c0 + wcol * 8) * 2);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int c = 0; c < MCH; ++c) {
      const int idx = tid + NT * c;
      *(i32x4*)&Ms0[buf * M_ELEMS + (idx >> 3) * MP + (idx & 7) * 8] = mr[c];
    }
#pragma unroll
    for (int c = 0; c < WCH; ++c) {
      const int idx = tid + NT * c;
      *(i32x4*)&Ws0[buf * W_ELEMS + w_off<GN>(idx / (GN / 8), (idx % (GN / 8)) * 8)] = wr[c];
    }
  };

  // W^T operand by transposed reads: lane (channel n, half hh) needs W[k0 + 8*hh + 0..7][n];
  // lane r of each 16-lane group points at row k0 + 8*hh + r/4 (+4), columns 16*g + 4*(r%4).
  // Those rows are congruent to r/4 mod 4, so the tile swizzle is a per-lane constant.
  const int wr_row = 8 * hh + ((lane & 15) >> 2);
  const int wr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int wr_xo = w_swz((lane & 15) >> 2) << 5;

  f32x16 acc[2][MB];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j) acc[i][j] = f32x16{};

  const int nkc = a.Cm / GK;
  gload(0);
  for (int kc = 0; kc < nkc; ++kc) {
    const int buf = kc & 1;
    sstore(buf);
    __syncthreads();
    if (kc + 1 < nkc) gload(kc + 1);
    const bf16* Ms = Ms0 + buf * M_ELEMS;
    const bf16* Ws = Ws0 + buf * W_ELEMS;
#pragma unroll
    for (int ks = 0; ks < GK / 16; ++ks) {
      bf16x8 wa[2], mb[MB];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const bf16* wp = &Ws[(ks * 16 + wr_row) * GN + ((wn * 64 + nb * 32 + wr_col) ^ wr_xo)];
        const i16x4 lo = lds_read_tr16(wp);
        const i16x4 hi = lds_read_tr16(wp + 4 * GN);
        wa[nb] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
#pragma unroll
      for (int mb2 = 0; mb2 < MB; ++mb2)
        mb[mb2] = *(const bf16x8*)&Ms[(wm * MB * 32 + mb2 * 32 + l32) * MP + ks * 16 + hh * 8];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb2 = 0; mb2 < MB; ++mb2) acc[nb][mb2] = mfma32(wa[nb], mb[mb2], acc[nb][mb2]);
    }
  }

  // Epilogue through LDS: the GM x GN bf16 C tile is staged token-major (row
  // pitch CP keeps rows 16-byte aligned; the 32 tokens of one 8-byte write
  // spread over the banks with at most 2-way conflicts), then written out as
  // 16-byte chunks.  In the head-major planes the DH channels of one head are
  // 2*DH contiguous bytes per token, so consecutive tokens of one head form one
  // contiguous run.
  __syncthreads();  // every wave is done with the staging tiles
  bf16* Cs = lds;
  const float os = p == 0 ? a.scale : 1.f;  // q plane: softmax scale folded in
#pragma unroll
  for (int mb2 = 0; mb2 < MB; ++mb2) {
    const int tl = wm * MB * 32 + mb2 * 32 + l32;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 val;
#pragma unroll
        for (int q = 0; q < 4; ++q) val[q] = (bf16)(acc[nb][mb2][g4 * 4 + q] * os);
        *(bf16x4*)&Cs[tl * CP + wn * 64 + nb * 32 + 8 * g4 + 4 * hh] = val;
      }
    }
  }
  __syncthreads();
  const size_t plane = (size_t)a.Ns * a.H * a.Nr * a.dh;
  bf16* out = (bf16*)a.ws + (size_t)p * plane;
  constexpr int CPT = DH / 8;            // 16-byte chunks per token and head
  constexpr int HPT = GN / DH;           // heads per channel tile
  constexpr int NCHUNK = GM * HPT * CPT / NT;
  static_assert(GM * HPT * CPT % NT == 0, "chunk/thread mismatch");
  const int h0 = c0 / DH;
#pragma unroll
  for (int k = 0; k < NCHUNK; ++k) {
    const int id = tid + NT * k;
    const int hl = id / (GM * CPT);
    const int rem = id % (GM * CPT);
    const int tl = rem / CPT, e8 = rem % CPT;
    const int tok = mt * GM + tl;
    if (tok >= M) continue;
    const int outer = tok / Linner, inner = tok % Linner;
    const i32x4 v = *(const i32x4*)&Cs[tl * CP + hl * DH + e8 * 8];
    *(i32x4*)(out + (((size_t)outer * a.H + h0 + hl) * Linner + inner) * a.dh + e8 * 8) = v;
  }
}

// Persistent form for Cm = 256: one workgroup per CU keeps a 256 x 128 W
// tile (one projection's 128 channels) resident and streams 128-token tiles
// of m past it, the next tile's loads in flight in registers during the
// current tile's MFMAs.  W passes through LDS once; each wave then holds the
// W^T operands of its 64 channels for the whole K in registers (128 VGPRs),
// so the per-tile LDS traffic is the m tile and the C tile only.  A workgroup's life is then many token tiles instead
// of four 64-wide K chunks.  Block b runs on XCD b % 8; the 32 blocks of an
// XCD are the Nt channel tiles of 32 / Nt token streams, so the channel tiles
// of one token tile run side by side on one XCD and read its m rows from
// that XCD's L2.
// Workgroup barrier ordering LDS accesses only.  __syncthreads() also waits
// for the workgroup's outstanding global stores, which would hold every token
// tile of the persistent loop behind the previous tile's output writes.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

constexpr int PP_K = 256;            // Cm of this form
constexpr int PP_MP = PP_K + 8;      // m tile pitch: 16 consecutive rows -> 16 distinct 16-byte bank groups
constexpr int PP_BLOCKS = 256;       // 8 XCDs x 32 CUs
template <int DH>
__global__ __launch_bounds__(512, 1) void evo_proj_persistent_kernel(const EvoArgs a) {
  constexpr int NT = 512, GM = 128, GN = 128, WN = GN / 64, MB = 1;
  constexpr int MCH = GM * PP_K / 8 / NT;  // 16-byte m chunks per thread per token tile
  constexpr int WCH = PP_K * GN / 8 / NT;  // 16-byte W chunks per thread
  constexpr int CP = GN + 8;               // C tile pitch
  static_assert(MCH * NT * 8 == GM * PP_K && WCH * NT * 8 == PP_K * GN, "tile/thread mismatch");
  static_assert(GM * CP <= GM * PP_MP, "the C tile reuses the m tile's bytes");
  __shared__ __attribute__((aligned(16))) bf16 Ws[PP_K * GN];
  __shared__ __attribute__((aligned(16))) bf16 Ms[GM * PP_MP];
  bf16* const Cs = Ms;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hh = lane >> 5, l32 = lane & 31;
  const int HD = a.H * a.dh, N = 4 * HD, M = a.Ns * a.Nr;
  const int Nt = N / GN;                   // channel tiles; the launcher checks that Nt divides 32
  const int Mt = (M + GM - 1) / GM;
  const int spx = 32 / Nt;                 // token streams per XCD
  const int x = blockIdx.x % 8, r = blockIdx.x / 8;
  const int nt = r % Nt;
  const int streams = 8 * spx;
  const int stream = x * spx + r / Nt;
  const int n0 = nt * GN, p = n0 / HD, c0 = n0 % HD;
  const int wn = w % WN, wm = w / WN;
  const int Linner = a.col ? a.Ns : a.Nr;  // token order as in evo_proj_kernel
  const uint32_t m_bytes = (uint32_t)M * a.Cm * 2;
  const auto mrs = make_rsrc(a.m, m_bytes);
  const auto wrs = make_rsrc(a.w[p], (uint32_t)a.Cm * HD * 2);

  // resident W tile (stored before the first barrier of the loop)
#pragma unroll
  for (int c = 0; c < WCH; ++c) {
    const int idx = tid + NT * c;
    const int wrow = idx / (GN / 8), wcol = idx % (GN / 8);
    const i32x4 v = buf_load16(wrs, (uint32_t)(wrow * HD + c0 + wcol * 8) * 2);
    *(i32x4*)&Ws[w_off<GN>(wrow, wcol * 8)] = v;
  }

  i32x4 mr[MCH];
  auto mload = [&](int mt) {
#pragma unroll
    for (int c = 0; c < MCH; ++c) {
      const int idx = tid + NT * c;
      const int tl = idx / (PP_K / 8), kc = idx % (PP_K / 8);
      const int t = mt * GM + tl;
      const int row = a.col ? (t % a.Ns) * a.Nr + t / a.Ns : t;
      const uint32_t off = t < M ? (uint32_t)row * a.Cm * 2 + kc * 16 : m_bytes;  // past M: zeros
      mr[c] = buf_load16(mrs, off);
    }
  };

  const int wr_row = 8 * hh + ((lane & 15) >> 2);
  const int wr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int wr_xo = w_swz((lane & 15) >> 2) << 5;
  const float os = p == 0 ? a.scale : 1.f;  // q plane: softmax scale folded in
  const size_t plane = (size_t)a.Ns * a.H * a.Nr * a.dh;
  const auto ors = make_rsrc((bf16*)a.ws + (size_t)p * plane, (uint32_t)(plane * 2));
  const int h0 = c0 / DH;

  if (stream < Mt) mload(stream);
  lds_barrier();  // W is stored
  bf16x8 wa[PP_K / 16][2];
#pragma unroll
  for (int ks = 0; ks < PP_K / 16; ++ks)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const bf16* wp = &Ws[(ks * 16 + wr_row) * GN + ((wn * 64 + nb * 32 + wr_col) ^ wr_xo)];
      const i16x4 lo = lds_read_tr16(wp);
      const i16x4 hi = lds_read_tr16(wp + 4 * GN);
      wa[ks][nb] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  for (int mt = stream; mt < Mt; mt += streams) {
    lds_barrier();  // the previous tile's C staging is consumed
#pragma unroll
    for (int c = 0; c < MCH; ++c) {
      const int idx = tid + NT * c;
      *(i32x4*)&Ms[(idx / (PP_K / 8)) * PP_MP + (idx % (PP_K / 8)) * 8] = mr[c];
    }
    lds_barrier();
    if (mt + streams < Mt) mload(mt + streams);

    f32x16 acc[2][MB];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) acc[nb][0] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < PP_K / 16; ++ks) {
      const bf16x8 mb = *(const bf16x8*)&Ms[(wm * 32 + l32) * PP_MP + ks * 16 + hh * 8];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[nb][0] = mfma32(wa[ks][nb], mb, acc[nb][0]);
    }
    lds_barrier();  // every wave is done with the m tile
    {
      const int tl = wm * 32 + l32;
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          bf16x4 val;
#pragma unroll
          for (int q = 0; q < 4; ++q) val[q] = (bf16)(acc[nb][0][g4 * 4 + q] * os);
          *(bf16x4*)&Cs[tl * CP + wn * 64 + nb * 32 + 8 * g4 + 4 * hh] = val;
        }
      }
    }
    lds_barrier();
    constexpr int CPT = DH / 8;   // 16-byte chunks per token and head
    constexpr int HPT = GN / DH;  // heads per channel tile
    constexpr int NCHUNK = GM * HPT * CPT / NT;
    static_assert(GM * HPT * CPT % NT == 0, "chunk/thread mismatch");
#pragma unroll
    for (int k = 0; k < NCHUNK; ++k) {
      const int id = tid + NT * k;
      const int hl = id / (GM * CPT);
      const int rem = id % (GM * CPT);
      const int tl = rem / CPT, e8 = rem % CPT;
      // tokens past M land past the plane and the buffer store drops them:
      // every tile issues the same four stores, so the next tile's wait for
      // its prefetched m rows can leave these stores in flight
      const int tok = mt * GM + tl;
      const int outer = tok / Linner, inner = tok % Linner;
      const i32x4 v = *(const i32x4*)&Cs[tl * CP + hl * DH + e8 * 8];
      __builtin_amdgcn_raw_buffer_store_b128(
          v, ors, (uint32_t)((((outer * a.H + h0 + hl) * Linner + inner) * a.dh + e8 * 8) * 2), 0, 0);
    }
  }
}

template <int DH>
hipError_t launch_evo_proj(const EvoArgs& a, hipStream_t stream) {
  const int M = a.Ns * a.Nr, HD = a.H * a.dh, N = 4 * HD;
  // The 256 x 256 tile (one workgroup per CU) pays once its grid fills the
  // 256 CUs at least four times over (N_res = 768 at 128 sequences: -5 %);
  // smaller grids keep the 128 x 128 tile at two workgroups per CU.
  const long long big_tiles = (long long)((M + 255) / 256) * (N / 256);
  if (a.Cm == PP_K && N % 128 == 0 && 32 % (N / 128) == 0) {
    hipLaunchKernelGGL((evo_proj_persistent_kernel<DH>), dim3(PP_BLOCKS), dim3(512), 0, stream, a);
  } else if (HD % 256 == 0 && big_tiles >= 4 * 256) {
    hipLaunchKernelGGL((evo_proj_kernel<256, 256, 512, DH>), dim3(((M + 255) / 256) * (N / 256)), dim3(512), 0,
                       stream, a);
  } else {
    hipLaunchKernelGGL((evo_proj_kernel<128, 128, 256, DH>), dim3(((M + 127) / 128) * (N / 128)), dim3(256), 0,
                       stream, a);
  }
  return hipGetLastError();
}

}  // namespace

size_t evo_workspace_bytes(int Ns, int Nr, int H, int dh) { return (size_t)4 * Ns * Nr * H * dh * 2; }

hipError_t launch_evoformer(const EvoArgs& a, hipStream_t stream) {
  if (evo_fused_fits(a)) return launch_evo_fused(a, stream);
  hipError_t e = a.dh == 64 ? launch_evo_proj<64>(a, stream) : launch_evo_proj<32>(a, stream);
  if (e != hipSuccess) return e;

  // attention problems: row-wise, one per (sequence, head) over the residues;
  // column-wise, one per (residue, head) over the sequences
  const int nB = a.col ? a.Nr : a.Ns;
  const int L = a.col ? a.Ns : a.Nr;
  const size_t plane = (size_t)a.Ns * a.H * a.Nr * a.dh;
  const bf16* ws = (const bf16*)a.ws;
  AttnArgs t{};
  t.q = ws;
  t.k = ws + plane;
  t.v = ws + 2 * plane;
  t.gate = ws + 3 * plane;
  t.o = a.out;
  t.lse = nullptr;
  t.doc = nullptr;
  t.bias = a.col ? nullptr : a.bias;
  t.bias_bs = 0;                         // the pair bias is shared by every sequence
  t.bias_hs = (long long)L * L;
  t.B = nB;
  t.Hq = t.Hkv = a.H;
  t.Sq = t.Skv = L;
  t.g = 1;
  const int bm = attn_bm(a.dh, a.col ? SM_GATE : SM_BIAS, MK_NONE);
  t.nM = (L + bm - 1) / bm;
  t.total = nB * a.H * t.nM;
  t.c = kLog2e;  // q arrives scaled
  t.scale = 1.f;
  t.softcap = 1.f;
  return launch_evo_attention(t, a.dh, a.col, stream);
}

}  // namespace av
