// Decoding / short-query attention forward for gfx950 (split-KV).
//
// The pages' serving workload runs causal and softcapped LLaMA-3.2-1B
// variants under vLLM (talk notes "Flashlight: PyTorch Compiler Extensions to
// Accelerate Attention Variants", end-to-end section, LLaMA-3.2-1B on the
// Mooncake trace); after prefill, every step attends a few new queries to a
// long key/value cache.  Reading implemented: the Sq queries of a sequence
// are the last Sq positions of its Skv keys (absolute position
// Skv - Sq + q), which is where the causal mask and the ALiBi distances are
// measured from.  The arithmetic per score is the prefill kernel's (same
// score modifiers, same exponent-reference schemes, fp32 accumulation); the
// row sums add the fp32 exponentials (this kernel is bound by memory, so the
// exact log-sum-exp costs nothing).
//
// Mapping onto CDNA4 (memory-bound: every K/V byte is read once, the
// matrix work is small):
//  * One workgroup = one (batch, KV head, key split).  All g = Hq/Hkv query
//    heads of the KV head and all Sq queries share one 32-row MFMA block
//    (g*Sq <= 32 rows), so each K/V byte is read once per KV head.
//  * The 4 waves take the split's 64-key tiles round-robin and never meet
//    inside the key loop (no barrier): K goes from memory straight into the
//    MFMA A-operand registers of S^T = K Q^T, V is staged row-major in a
//    wave-private LDS slot and read transposed for O^T = V^T P^T.
//  * At the end the 4 waves merge (m, l, O) through LDS.  With one split the
//    result is final; with several, each split writes its partial state to
//    the workspace and a second kernel merges the splits (the same rescale as
//    the online softmax), one workgroup per output row.

#include <algorithm>
#include <mutex>

#include "attn_tile.hpp"
#include "av_kernels.hpp"

namespace av {
namespace {

constexpr int NT = 256;
constexpr int BN = 64;   // keys per tile
constexpr int ROWS = 32; // query rows per workgroup (one MFMA block)
#ifndef AV_DECODE_TARGET_WG
#define AV_DECODE_TARGET_WG 512
#endif
#ifndef AV_DECODE_MIN_TILES
#define AV_DECODE_MIN_TILES 4
#endif
constexpr int kDecodeTargetWG = AV_DECODE_TARGET_WG;
constexpr int kDecodeMinTiles = AV_DECODE_MIN_TILES;
static_assert((size_t)2 * kDecodeTargetWG * 32 * (64 + 2) * 4 <= kDecodeScratchBytes,
              "the allocation-free decode scratch must hold the partials of every plan");

// (the paged form holds 64-bit row addresses: two waves per SIMD instead of three)
template <int D, int SM, bool CAUSAL, bool PAGED>
__global__ __launch_bounds__(NT, (PAGED ? 2 : 3)) void attn_decode_kernel(const DecodeArgs a) {
  constexpr int NKB = BN / 32, NDB = D / 32, NDS = D / 16, NPS = BN / 16;
  constexpr int VCH = BN * D / 8 / 64;  // 16-byte V chunks per lane per tile
  __shared__ __attribute__((aligned(16))) bf16 Vs[4][BN * D];  // one slot per wave, swizzled
  __shared__ float Ms[4][ROWS], Ls[4][ROWS];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int hh = lane >> 5, l32 = lane & 31;
  const int L = xcd_remap(blockIdx.x, a.total);
  const int split = L % a.NS;
  const int bk = L / a.NS;
  const int hk = bk % a.Hkv, b = bk / a.Hkv;

  // ---- this lane's query row: r -> (head hk*g + r/Sq, query r%Sq)
  const int R = a.g * a.Sq;
  const int r = l32;
  const bool row_live = r < R;
  const int hq = hk * a.g + (row_live ? r / a.Sq : 0);
  const int qq = row_live ? r % a.Sq : 0;
  // key count of this sequence (paged: its own length, at most the table's reach)
  const int Skv = PAGED ? min(max(a.seq_lens[b], 0), a.max_pages * a.page_size) : a.Skv;
  const int pos = Skv - a.Sq + qq;  // absolute position of the query
  const auto qrs = make_rsrc((const bf16*)a.q + (((size_t)b * a.Hq + hq) * a.Sq + qq) * D,
                             row_live ? (uint32_t)D * 2 : 0u);
  bf16x8 qreg[NDS];
#pragma unroll
  for (int s = 0; s < NDS; ++s) qreg[s] = __builtin_bit_cast(bf16x8, buf_load16(qrs, (uint32_t)(s * 16 + hh * 8) * 2));

  const size_t kvoff = PAGED ? 0 : ((size_t)b * a.Hkv + hk) * (size_t)a.Skv * D;
  const auto krs = make_rsrc((const bf16*)a.k + kvoff, PAGED ? 0u : (uint32_t)a.Skv * D * 2);
  const auto vrs = make_rsrc((const bf16*)a.v + kvoff, PAGED ? 0u : (uint32_t)a.Skv * D * 2);
  // Paged cache [num_pages, Hkv, page_size, D]: the pages of one 64-key tile
  // (64 / page_size of them) are looked up once per tile, lane i holding the
  // tile's i-th page; rows past the sequence reuse its last page (masked) and
  // page ids are clamped into the cache, so a bad table cannot fault.
  const int* bt_row = PAGED ? a.block_table + (size_t)b * a.max_pages : nullptr;
  const int last_pidx = PAGED ? max(Skv - 1, 0) / a.page_size : 0;
  auto tile_page = [&](int n0) {
    if constexpr (PAGED) {
      const int np = BN / a.page_size;
      const int pidx = min(n0 / a.page_size + lane % np, last_pidx);
      return min(max(bt_row[pidx], 0), a.num_pages - 1);
    } else {
      return 0;
    }
  };
  // element offset of key row n0 + row (paged: via the tile's page ids)
  auto key_off = [&](int pg, int n0, int row) -> size_t {
    if constexpr (PAGED) {
      const int page = __shfl(pg, row / a.page_size);
      return (((size_t)page * a.Hkv + hk) * a.page_size + row % a.page_size) * D;
    } else {
      return (size_t)(n0 + row) * D;
    }
  };

  const int nKV = (Skv + BN - 1) / BN;
  const int t_lo = split * a.tps, t_hi = min(nKV, t_lo + a.tps);

  f32x16 o[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
  RowState st;
  const TrLane<D> vl(lane);
  bf16* Vw = Vs[w];

  const float cap2 = a.softcap * kLog2e;
  const float sc_k = 2.f * a.scale * kLog2e / a.softcap;
  const float invK = 0.5f / cap2;
  if constexpr (SM == SM_SOFTCAP_FIXED) st.m_ref = cap2;
  // per-row ALiBi slope (log2 units); rows of one workgroup span several heads
  const float slope2 = SM == SM_ALIBI ? kLog2e * exp2f(-a.alibi_max_bias * (float)(hq + 1) / (float)a.Hq) : 0.f;

  // ALiBi walks the split's tiles from last to first (its term grows with the
  // key index; descending, later tiles seldom raise the exponent reference)
  for (int i = w; i < t_hi - t_lo; i += 4) {
    const int t = SM == SM_ALIBI ? t_hi - 1 - i : t_lo + i;
    const int n0 = t * BN;
    const int pg = tile_page(n0);
    // ---- V tile -> registers -> this wave's LDS slot (row-major, swizzled)
    i32x4 vr[VCH];
#pragma unroll
    for (int c = 0; c < VCH; ++c) {
      const int idx = lane + 64 * c;
      const int row = idx / (D / 8), col = idx % (D / 8);
      if constexpr (PAGED) {
        vr[c] = *(const i32x4*)((const bf16*)a.v + key_off(pg, n0, row) + col * 8);
      } else {
        vr[c] = buf_load16(vrs, (uint32_t)((n0 + row) * D + col * 8) * 2);
      }
    }
    // ---- K fragments straight into the A operand: key kb*32 + l32, d = st*16 + 8*hh .. +7
    bf16x8 kf[NKB][NDS];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const size_t koff = key_off(pg, n0, kb * 32 + l32);
#pragma unroll
      for (int s = 0; s < NDS; ++s) {
        if constexpr (PAGED) {
          kf[kb][s] = *(const bf16x8*)((const bf16*)a.k + koff + s * 16 + hh * 8);
        } else {
          kf[kb][s] = __builtin_bit_cast(bf16x8, buf_load16(krs, (uint32_t)((n0 + kb * 32 + l32) * D + s * 16 + hh * 8) * 2));
        }
      }
    }
#pragma unroll
    for (int c = 0; c < VCH; ++c) {
      const int idx = lane + 64 * c;
      const int row = idx / (D / 8), col = idx % (D / 8);
      *(i32x4*)&Vw[tr_tile_off<D>(row, col * 8)] = vr[c];
    }

    // ---- S^T = K Q^T: lane holds keys n0 + kb*32 + 8*(j/4) + 4*hh + j%4 of row r
    f32x16 s[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      s[kb] = f32x16{};
#pragma unroll
      for (int st_ = 0; st_ < NDS; ++st_) s[kb] = mfma32(kf[kb][st_], qreg[st_], s[kb]);
    }
    const int kbase = n0 + 4 * hh;
    // ---- score modifier
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int off = kb * 32 + 8 * (j >> 2) + (j & 3);
        if constexpr (SM == SM_ALIBI) {
          s[kb][j] = fmaf(s[kb][j], a.c, slope2 * (float)(kbase + off - pos));
        } else if constexpr (SM == SM_SOFTCAP || SM == SM_SOFTCAP_FIXED) {
          const float rr = rcp_fast(fmaf(exp2_fast(s[kb][j] * sc_k), invK, invK));
          s[kb][j] = SM == SM_SOFTCAP_FIXED ? -rr : cap2 - rr;
        }
      }
    // ---- mask: keys past the end, and (causal) keys after the query's position
    const bool full = (n0 + BN <= Skv) && (!CAUSAL || n0 + BN - 1 <= Skv - a.Sq);
    if (!full) {
      int lim = Skv - kbase, rel = pos - kbase;
      asm volatile("" : "+v"(lim), "+v"(rel));
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int off = kb * 32 + 8 * (j >> 2) + (j & 3);
          const bool ok = (off < lim) && (!CAUSAL || off <= rel);
          s[kb][j] = ok ? s[kb][j] : neg_inf();
          if ((j & 3) == 3) __builtin_amdgcn_sched_barrier(0);
        }
    }
    // ---- exponent reference and exponentials (the prefill kernel's schemes)
    bf16x8 pb[NPS];
    if constexpr (SM == SM_NONE) {
      float tsum = exp_pack_sum<NKB, 0, true>(s, a.c, st.m_sub, pb);
      if (any_lane(tsum > kOptBound || st.m_ref == neg_inf())) {
        st.template raise<NDB>(xhalf_max(block_max<NKB>(s)) * a.c, o);
        tsum = exp_pack_sum<NKB, 0, true>(s, a.c, st.m_sub, pb);
      }
      st.l += tsum;
    } else if constexpr (SM == SM_SOFTCAP_FIXED) {
      st.l += exp_pack_sum<NKB, 2, true>(s, a.c, st.m_sub, pb);
    } else {  // ALiBi, softcap with a large cap: lazy rescale on the tile max
      const float hmax = block_max<NKB>(s);
      if (any_lane(hmax > st.thr)) st.template raise<NDB>(xhalf_max(hmax), o);
      st.l += exp_pack_sum<NKB, 1, true>(s, a.c, st.m_sub, pb);
    }
    // ---- O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int tt = 0; tt < NPS; ++tt) o[db] = mfma32(vt_operand<D>(Vw, tt, db * 32, vl), pb[tt], o[db]);
  }

  // ---- merge the 4 waves: m, l per row, then O through the (now free) V slots
  const float l_row = xhalf_sum(st.l);
  __syncthreads();
  if (hh == 0) {
    Ms[w][r] = st.m_ref;
    Ls[w][r] = l_row;
  }
  float* Os = (float*)&Vs[0][0];  // [4 waves][ROWS][D] fp32 = 4 * 32 * D * 4 bytes
  static_assert(4 * ROWS * D * 4 <= (int)sizeof(Vs), "merge buffer does not fit");
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int d = db * 32 + 8 * (j >> 2) + 4 * hh + (j & 3);
      Os[(w * ROWS + r) * D + d] = o[db][j];
    }
  __syncthreads();
  // each thread merges ROWS*D/NT elements: row rr, columns dd .. dd+EPT-1
  constexpr int EPT = ROWS * D / NT;
  const int rr = tid / (D / EPT);
  const int dd = (tid % (D / EPT)) * EPT;
  float mw[4], M = neg_inf();
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) {
    mw[ww] = Ms[ww][rr];
    M = fmaxf(M, mw[ww]);
  }
  const float Msub = M == neg_inf() ? 0.f : M;
  float f[4], Lsum = 0.f;
#pragma unroll
  for (int ww = 0; ww < 4; ++ww) {
    f[ww] = exp2_fast(mw[ww] - Msub);
    Lsum = fmaf(Ls[ww][rr], f[ww], Lsum);
  }
  float acc[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    float x = 0.f;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) x = fmaf(Os[(ww * ROWS + rr) * D + dd + e], f[ww], x);
    acc[e] = x;
  }
  if (rr >= R) return;
  const int ohq = hk * a.g + rr / a.Sq, oq = rr % a.Sq;
  const size_t orow = ((size_t)b * a.Hq + ohq) * a.Sq + oq;
  if (a.NS == 1) {
    const float inv = Lsum > 0.f ? 1.f / Lsum : 0.f;
#pragma unroll
    for (int e = 0; e < EPT; e += 4) {
      bf16x4 val;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) val[q4] = (bf16)(acc[e + q4] * inv);
      *(bf16x4*)((bf16*)a.o + orow * D + dd + e) = val;
    }
    if (a.lse != nullptr && dd == 0) a.lse[orow] = Lsum > 0.f ? (M + __log2f(Lsum)) * kLn2 : neg_inf();
  } else {
    // partial state of this split: O relative to 2^M, and (M, L)
    const size_t unit = ((size_t)bk * a.NS + split) * ROWS + rr;
#pragma unroll
    for (int e = 0; e < EPT; e += 4)
      *(f32x4*)(a.ws_o + unit * D + dd + e) = f32x4{acc[e], acc[e + 1], acc[e + 2], acc[e + 3]};
    if (dd == 0) {
      a.ws_ml[unit * 2] = M;
      a.ws_ml[unit * 2 + 1] = Lsum;
    }
  }
}

// Merge of the key splits: one workgroup per output row (batch, KV head,
// packed row); lane = column (D = 64), the 4 waves take the splits
// round-robin and meet in LDS.
template <int D>
__global__ __launch_bounds__(NT) void attn_decode_combine(const DecodeArgs a) {
  static_assert(D == 64, "one lane per column");
  __shared__ float red[4][D + 2];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int R = a.g * a.Sq;
  const int rr = blockIdx.x % R;
  const int bk = blockIdx.x / R;
  const float* ml = a.ws_ml + ((size_t)bk * a.NS * ROWS + rr) * 2;  // split s at ml[s * ROWS * 2]
  const float* os = a.ws_o + ((size_t)bk * a.NS * ROWS + rr) * D;   // split s at os[s * ROWS * D]
  // pass 1: the common reference M = max over the splits
  float M = neg_inf();
  for (int s = tid; s < a.NS; s += NT) M = fmaxf(M, ml[(size_t)s * ROWS * 2]);
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  if (lane == 0) red[w][0] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red[0][0], red[1][0]), fmaxf(red[2][0], red[3][0]));
  const float Msub = M == neg_inf() ? 0.f : M;
  __syncthreads();
  // pass 2: rescaled sums of this wave's splits
  float acc = 0.f, lsum = 0.f;
#pragma unroll 4
  for (int s = w; s < a.NS; s += 4) {
    const float f = exp2_fast(ml[(size_t)s * ROWS * 2] - Msub);
    lsum = fmaf(ml[(size_t)s * ROWS * 2 + 1], f, lsum);
    acc = fmaf(os[(size_t)s * ROWS * D + lane], f, acc);
  }
  red[w][lane] = acc;
  if (lane == 0) red[w][D] = lsum;
  __syncthreads();
  if (w != 0) return;
  const float L = red[0][D] + red[1][D] + red[2][D] + red[3][D];
  const float x = red[0][lane] + red[1][lane] + red[2][lane] + red[3][lane];
  const int hk = bk % a.Hkv, b = bk / a.Hkv;
  const int ohq = hk * a.g + rr / a.Sq, oq = rr % a.Sq;
  const size_t orow = ((size_t)b * a.Hq + ohq) * a.Sq + oq;
  const float inv = L > 0.f ? 1.f / L : 0.f;
  ((bf16*)a.o)[orow * D + lane] = (bf16)(x * inv);
  if (a.lse != nullptr && lane == 0) a.lse[orow] = L > 0.f ? (M + __log2f(L)) * kLn2 : neg_inf();
}

template <int D, int SM, bool CAUSAL>
hipError_t launch_dec(const DecodeArgs& a, hipStream_t stream) {
  if (a.block_table != nullptr) {
    hipLaunchKernelGGL((attn_decode_kernel<D, SM, CAUSAL, true>), dim3(a.total), dim3(NT), 0, stream, a);
  } else {
    hipLaunchKernelGGL((attn_decode_kernel<D, SM, CAUSAL, false>), dim3(a.total), dim3(NT), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.NS == 1) return e;
  const long long rows = (long long)a.B * a.Hkv * a.g * a.Sq;
  hipLaunchKernelGGL((attn_decode_combine<D>), dim3((unsigned)rows), dim3(NT), 0, stream, a);
  return hipGetLastError();
}

template <int SM>
hipError_t launch_dec_mask(const DecodeArgs& a, int causal, hipStream_t stream) {
  return causal ? launch_dec<64, SM, true>(a, stream) : launch_dec<64, SM, false>(a, stream);
}

}  // namespace

DecodePlan decode_plan(int B, int Hkv, int Skv) {
  DecodePlan p{};
  const int nKV = (Skv + 63) / 64;
  const int units = B * Hkv;
  // enough workgroups to fill the chip (kDecodeTargetWG), and at least
  // kDecodeMinTiles 64-key tiles in every split
  int ns = (kDecodeTargetWG + units - 1) / units;
  ns = std::min(ns, std::max(1, nKV / kDecodeMinTiles));
  ns = std::max(ns, 1);
  p.tps = nKV == 0 ? 1 : (nKV + ns - 1) / ns;
  p.NS = nKV == 0 ? 1 : (nKV + p.tps - 1) / p.tps;
  return p;
}

size_t decode_workspace_bytes(int B, int Hkv, int Skv, int D) {
  const DecodePlan p = decode_plan(B, Hkv, Skv);
  if (p.NS == 1) return 0;
  return (size_t)B * Hkv * p.NS * 32 * ((size_t)D + 2) * 4;
}

// Split-KV partials of the allocation-free decode entry point, one copy per
// GPU, held until the process ends.  The plan splits the keys only while
// B * Hkv < kDecodeTargetWG, and then into at most ceil(target / (B * Hkv))
// splits, so B * Hkv * NS < 2 * kDecodeTargetWG: the partial state of any
// plan at D = 64 fits kDecodeScratchBytes (8.25 MiB at the default target).
// Every call overwrites the rows it later reads, so nothing needs clearing;
// calls that overlap on one GPU share these bytes and race.
__device__ __align__(256) char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    // the host-side name of the array is a stand-in, not a device address:
    // this device's copy lives at the address the runtime reports
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_attn_decode(const DecodeArgs& a, int score_mod, int causal, hipStream_t stream) {
  switch (score_mod) {
    case SM_NONE: return launch_dec_mask<SM_NONE>(a, causal, stream);
    case SM_ALIBI: return launch_dec_mask<SM_ALIBI>(a, causal, stream);
    case SM_SOFTCAP:
      return a.fixed_ref ? launch_dec_mask<SM_SOFTCAP_FIXED>(a, causal, stream)
                         : launch_dec_mask<SM_SOFTCAP>(a, causal, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace av
