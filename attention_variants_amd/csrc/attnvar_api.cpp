// C ABI of the attention-variant library: host-side validation, derived
// launch parameters, dispatch.  Nothing here touches the GPU until every
// argument has been checked, so every error path is testable without one.

#include <math.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "../../include/attnvar.h"
#include "av_kernels.hpp"

namespace {

constexpr double kLog2e = 1.4426950408889634;
constexpr uint64_t kMaxSliceBytes = (1ull << 31) - 1;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? AV_OK : AV_ERR_HIP; }

// Shared validation and launch of the differential forms; `a` arrives with
// the form's own fields (lambda, or the head parameters) already set.
int diff_launch(av::DiffArgs& a, const void* q, const void* k, const void* v, void* out, int B, int H, int S,
                int Dh, int Dv, float scale, int causal, hipStream_t stream) {
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return AV_ERR_NULL;
  if (B <= 0 || H <= 0 || S < 0 || Dh <= 0 || Dv <= 0) return AV_ERR_SHAPE;
  if ((Dh != 32 && Dh != 64) || (Dv != 64 && Dv != 128)) return AV_ERR_UNSUPPORTED;
  if (!(isfinite(scale) && scale >= 0.f)) return AV_ERR_PARAM;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return AV_ERR_ALIGN;
  if ((uint64_t)(S + av::kAttnBM) * 2 * Dh * 2 > kMaxSliceBytes) return AV_ERR_TOO_LARGE;
  if ((uint64_t)(S + av::kAttnBM) * Dv * 2 > kMaxSliceBytes) return AV_ERR_TOO_LARGE;
  const int64_t nM = ((int64_t)S + av::kAttnBM - 1) / av::kAttnBM;
  const int64_t total = (int64_t)B * H * nM;
  if (total > INT32_MAX) return AV_ERR_TOO_LARGE;
  if (total == 0) return AV_OK;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = out;
  a.B = B;
  a.H = H;
  a.S = S;
  a.nM = (int)nM;
  a.total = (int)total;
  const double sc = scale > 0.f ? (double)scale : 1.0 / sqrt((double)Dh);
  a.c = (float)(sc * kLog2e);
  a.causal = causal != 0;
  return hip_status(av::launch_diff_attn_fwd(a, Dh, Dv, stream));
}

}  // namespace

// tanh(x) ~= x (c0 + c1 x^2) on |x| <= 0.25, max relative error 6.4e-5: the
// minimax (equal-ripple) fit of tanh(x)/x there.  In the exponent that is at
// most 6.4e-5 * cap*log2(e) * tanh(0.25) <= 7.5e-4 for every cap with
// 2 * cap * log2(e) <= 96, below a third of the 2^-9 rounding of the bf16
// probabilities.  Scores of N(0,1)-scaled attention stay inside the range
// except on a few tiles per thousand, which take the exact form.  In raw
// units (x = k raw, k = scale / cap) and log2 units:
// cap*log2(e) * tanh(k raw) = raw * sum_i (cap*log2(e) * c_i * k^(2i+1)) raw^(2i).
static void softcap_cubic(double scale, double cap, float (&poly)[2], float& lim) {
  constexpr double c[2] = {0.9999366663950144, -0.3251848147732782};
  constexpr double kPolyX = 0.25;
  const double k = scale / cap;
  const double cap2 = cap * kLog2e;
  double kp = k;
  for (int i = 0; i < 2; ++i, kp *= k * k) poly[i] = (float)(cap2 * c[i] * kp);
  lim = (float)(kPolyX / k);
}

extern "C" {

int av_abi_version(void) { return AV_ABI_VERSION; }

const char* av_status_string(int status) {
  switch (status) {
    case AV_OK: return "AV_OK: success";
    case AV_ERR_NULL: return "AV_ERR_NULL: a required pointer is NULL";
    case AV_ERR_SHAPE: return "AV_ERR_SHAPE: inconsistent sizes";
    case AV_ERR_UNSUPPORTED: return "AV_ERR_UNSUPPORTED: head dim or enum value not implemented";
    case AV_ERR_ALIGN: return "AV_ERR_ALIGN: pointer misaligned";
    case AV_ERR_WORKSPACE: return "AV_ERR_WORKSPACE: workspace missing or too small";
    case AV_ERR_HIP: return "AV_ERR_HIP: the HIP runtime refused the launch";
    case AV_ERR_PARAM: return "AV_ERR_PARAM: scalar parameter out of range";
    case AV_ERR_TOO_LARGE: return "AV_ERR_TOO_LARGE: size exceeds 32-bit kernel addressing";
  }
  return "unknown av_status";
}

int attn_doc_order_len(int B, int S) {
  if (B <= 0 || S < 0) return AV_ERR_SHAPE;
  const int64_t n = (int64_t)B * (((int64_t)S + av::kDocTileM - 1) / av::kDocTileM);
  return n > av::kDocOrderMax ? AV_ERR_TOO_LARGE : (int)n;
}

int attn_doc_order(const int32_t* doc_id, int B, int S, int32_t* order, int order_len, hipStream_t stream) {
  const int n = attn_doc_order_len(B, S);
  if (n < 0) return n;
  if (n == 0) return AV_OK;
  if (doc_id == nullptr || order == nullptr) return AV_ERR_NULL;
  if (!aligned(doc_id, 4) || !aligned(order, 4)) return AV_ERR_ALIGN;
  if (order_len < n) return AV_ERR_WORKSPACE;
  return hip_status(av::launch_doc_order(doc_id, B, S, order, stream));
}

// The document work order of av_variant, as attn_fwd and attn_bwd read it:
// the kernels read entry blockIdx.x / heads < B * ceil(Sq / 128), so the
// order must be the one attn_doc_order writes for this B and Sq.
static int check_doc_order(const av_variant* var, int B, int Sq) {
  if (var->doc_order == nullptr) return AV_OK;
  if (var->mask != AV_MASK_DOCUMENT) return AV_ERR_PARAM;
  if (!aligned(var->doc_order, 4)) return AV_ERR_ALIGN;
  const int n = attn_doc_order_len(B, Sq);
  if (n < 0) return n;
  return var->doc_order_len == n ? AV_OK : AV_ERR_PARAM;
}

int attn_fwd(const av_variant* var, const void* q, const void* k, const void* v, void* out, float* lse, int B,
             int Hq, int Hkv, int Sq, int Skv, int D, hipStream_t stream) {
  if (var == nullptr) return AV_ERR_NULL;
  // Empty tensors may come with NULL data pointers: only sizes > 0 need memory.
  if ((Sq > 0 && (q == nullptr || out == nullptr)) || (Skv > 0 && (k == nullptr || v == nullptr)))
    return AV_ERR_NULL;
  if (var->score_mod < AV_SCORE_NONE || var->score_mod > AV_SCORE_BIAS) return AV_ERR_UNSUPPORTED;
  if (var->mask < AV_MASK_NONE || var->mask > AV_MASK_DOCUMENT) return AV_ERR_UNSUPPORTED;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq < 0 || Skv < 0 || D <= 0) return AV_ERR_SHAPE;
  if (Hq % Hkv != 0) return AV_ERR_SHAPE;
  if (var->kv_group != 0 && var->kv_group != Hq / Hkv) return AV_ERR_SHAPE;
  if (var->mask != AV_MASK_NONE && Sq != Skv) return AV_ERR_SHAPE;
  if (D != 32 && D != 64 && D != 128) return AV_ERR_UNSUPPORTED;
  if (var->mask == AV_MASK_DOCUMENT && var->doc_id == nullptr) return AV_ERR_NULL;
  const bool tbias = var->score_mod == AV_SCORE_BIAS;
  if (tbias && Sq > 0 && Skv > 0 && var->bias == nullptr) return AV_ERR_NULL;
  if (tbias && (var->bias_batch_stride < 0 || var->bias_head_stride < 0)) return AV_ERR_PARAM;
  if (!(isfinite(var->scale) && var->scale >= 0.f)) return AV_ERR_PARAM;
  if (var->score_mod == AV_SCORE_SOFTCAP && !(isfinite(var->softcap) && var->softcap > 0.f)) return AV_ERR_PARAM;
  if (var->score_mod == AV_SCORE_ALIBI && !isfinite(var->alibi_max_bias)) return AV_ERR_PARAM;
  if (var->mask == AV_MASK_SLIDING_WINDOW && var->window < 1) return AV_ERR_PARAM;
  if (var->mask == AV_MASK_PREFIX_LM && (var->prefix_len < 0 || var->prefix_len > Sq)) return AV_ERR_PARAM;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return AV_ERR_ALIGN;
  if (lse != nullptr && !aligned(lse, 4)) return AV_ERR_ALIGN;
  if (var->mask == AV_MASK_DOCUMENT && !aligned(var->doc_id, 4)) return AV_ERR_ALIGN;
  if (const int rc = check_doc_order(var, B, Sq); rc != AV_OK) return rc;
  // bias rows are read 8 bytes at a time when Skv % 4 == 0: every slice must
  // then start on an 8-byte boundary
  if (tbias && (!aligned(var->bias, 8) ||
                (Skv % 4 == 0 && (var->bias_batch_stride % 4 != 0 || var->bias_head_stride % 4 != 0))))
    return AV_ERR_ALIGN;
  // Per-slice byte offsets are 32-bit inside the kernel; query rows of a
  // ragged last tile may index up to BM-1 rows past Sq.
  if ((uint64_t)(Sq + av::kAttnBMMax) * D * 2 > kMaxSliceBytes) return AV_ERR_TOO_LARGE;
  if ((uint64_t)(Skv + 64) * D * 2 > kMaxSliceBytes) return AV_ERR_TOO_LARGE;
  if (tbias && (uint64_t)(Sq + av::kAttnBMMax) * (Skv + 64) * 2 > kMaxSliceBytes) return AV_ERR_TOO_LARGE;
  const int sm = tbias ? av::SM_TBIAS : var->score_mod;
  const bool one_block = av::attn_one_block(D, sm, var->mask, Sq);
  const int bm = one_block ? 128 : av::attn_bm(D, sm, var->mask);
  const int64_t nM = ((int64_t)Sq + bm - 1) / bm;
  const int64_t total = (int64_t)B * Hq * nM;
  if (total > INT32_MAX) return AV_ERR_TOO_LARGE;
  if (total == 0) return AV_OK;

  av::AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = out;
  a.lse = lse;
  a.doc = var->doc_id;
  a.doc_order = var->mask == AV_MASK_DOCUMENT ? var->doc_order : nullptr;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Sq = Sq;
  a.Skv = Skv;
  a.g = Hq / Hkv;
  a.nM = (int)nM;
  a.total = (int)total;
  a.one_block = one_block;
  const double scale = var->scale > 0.f ? (double)var->scale : 1.0 / sqrt((double)D);
  a.scale = (float)scale;
  a.c = (float)(scale * kLog2e);
  a.alibi_max_bias = var->alibi_max_bias;
  a.softcap = var->score_mod == AV_SCORE_SOFTCAP ? var->softcap : 1.f;
  a.window = var->window;
  a.prefix = var->prefix_len;
  // softcapped scores lie in [-cap, cap]: with the reference at +cap every
  // exponential is in [2^(-2 cap log2 e), 1], far from fp32 underflow when <= 96
  a.fixed_ref = var->score_mod == AV_SCORE_SOFTCAP && 2.0 * var->softcap * kLog2e <= 96.0;
  if (a.fixed_ref) {
    // raw (p0 + p1 raw^2) with p1 < 0 is x (A - x^2) in x = beta raw, beta^3 =
    // -p1, A = p0 / beta: without lse the kernel scales q by beta
    softcap_cubic(scale, var->softcap, a.sc_poly, a.sc_poly_lim);
    const double beta = cbrt(-(double)a.sc_poly[1]);
    a.sc_x[0] = (float)(a.sc_poly[0] / beta);
    a.sc_x[1] = (float)beta;
    a.sc_x_lim = (float)(a.sc_poly_lim * beta);
  }
  if (tbias) {
    a.bias = var->bias;
    a.bias_bs = var->bias_batch_stride;
    a.bias_hs = var->bias_head_stride;
  }
  return hip_status(av::launch_attn_fwd(a, D, sm, var->mask, stream));
}

size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Skv, int D) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 0 || Skv < 0 || D <= 0) return 0;
  return av::decode_workspace_bytes(B, Hkv, Skv, D);
}

}  // extern "C"

namespace {

// Validation and argument block of the dense decode forms; `need` receives
// the split-KV partials' byte count (0 when the plan does not split).
int decode_prepare(const av_variant* var, const void* q, const void* k, const void* v, void* out, float* lse, int B,
                   int Hq, int Hkv, int Sq, int Skv, int D, av::DecodeArgs& a, size_t& need) {
  need = 0;
  if (var == nullptr) return AV_ERR_NULL;
  if ((Sq > 0 && (q == nullptr || out == nullptr)) || (Skv > 0 && (k == nullptr || v == nullptr)))
    return AV_ERR_NULL;
  if (var->score_mod < AV_SCORE_NONE || var->score_mod > AV_SCORE_SOFTCAP) return AV_ERR_UNSUPPORTED;
  if (var->mask != AV_MASK_NONE && var->mask != AV_MASK_CAUSAL) return AV_ERR_UNSUPPORTED;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq < 0 || Skv < 0 || D <= 0) return AV_ERR_SHAPE;
  if (Hq % Hkv != 0) return AV_ERR_SHAPE;
  if (var->kv_group != 0 && var->kv_group != Hq / Hkv) return AV_ERR_SHAPE;
  if (var->mask == AV_MASK_CAUSAL && Skv < Sq) return AV_ERR_SHAPE;
  if (D != 64) return AV_ERR_UNSUPPORTED;
  if ((int64_t)(Hq / Hkv) * Sq > 32) return AV_ERR_UNSUPPORTED;
  if (!(isfinite(var->scale) && var->scale >= 0.f)) return AV_ERR_PARAM;
  if (var->score_mod == AV_SCORE_SOFTCAP && !(isfinite(var->softcap) && var->softcap > 0.f)) return AV_ERR_PARAM;
  if (var->score_mod == AV_SCORE_ALIBI && !isfinite(var->alibi_max_bias)) return AV_ERR_PARAM;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return AV_ERR_ALIGN;
  if (lse != nullptr && !aligned(lse, 4)) return AV_ERR_ALIGN;
  if ((uint64_t)(Skv + 64) * D * 2 > kMaxSliceBytes) return AV_ERR_TOO_LARGE;
  if (Sq == 0) return AV_OK;
  const av::DecodePlan plan = av::decode_plan(B, Hkv, Skv);
  const int64_t total = (int64_t)B * Hkv * plan.NS;
  if (total > INT32_MAX || (int64_t)B * Hkv * 32 > INT32_MAX) return AV_ERR_TOO_LARGE;
  need = av::decode_workspace_bytes(B, Hkv, Skv, D);

  a = av::DecodeArgs{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = out;
  a.lse = lse;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Sq = Sq;
  a.Skv = Skv;
  a.g = Hq / Hkv;
  a.NS = plan.NS;
  a.tps = plan.tps;
  a.total = (int)total;
  const double scale = var->scale > 0.f ? (double)var->scale : 1.0 / sqrt((double)D);
  a.scale = (float)scale;
  a.c = (float)(scale * kLog2e);
  a.alibi_max_bias = var->alibi_max_bias;
  a.softcap = var->score_mod == AV_SCORE_SOFTCAP ? var->softcap : 1.f;
  a.fixed_ref = var->score_mod == AV_SCORE_SOFTCAP && 2.0 * var->softcap * kLog2e <= 96.0;
  return AV_OK;
}

// partial O [B*Hkv, NS, 32, D] fp32, then (m, l) [B*Hkv, NS, 32, 2] fp32
void decode_set_workspace(av::DecodeArgs& a, void* ws, size_t need, int D) {
  a.ws_o = need > 0 ? (float*)ws : nullptr;
  a.ws_ml = need > 0 ? (float*)ws + (size_t)a.B * a.Hkv * a.NS * 32 * D : nullptr;
}

}  // namespace

extern "C" {

int attn_decode_fwd(const av_variant* var, const void* q, const void* k, const void* v, void* out, float* lse,
                    void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int Sq, int Skv, int D,
                    hipStream_t stream) {
  av::DecodeArgs a{};
  size_t need = 0;
  const int rc = decode_prepare(var, q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, a, need);
  if (rc != AV_OK || Sq == 0) return rc;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return AV_ERR_WORKSPACE;
  if (need > 0 && !aligned(workspace, 16)) return AV_ERR_ALIGN;
  decode_set_workspace(a, workspace, need, D);
  return hip_status(av::launch_attn_decode(a, var->score_mod, var->mask == AV_MASK_CAUSAL, stream));
}

int attn_decode_fwd_noalloc(const av_variant* var, const void* q, const void* k, const void* v, void* out,
                            float* lse, int B, int Hq, int Hkv, int Sq, int Skv, int D, hipStream_t stream) {
  av::DecodeArgs a{};
  size_t need = 0;
  const int rc = decode_prepare(var, q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, a, need);
  if (rc != AV_OK || Sq == 0) return rc;
  if (need > av::kDecodeScratchBytes) return AV_ERR_TOO_LARGE;
  void* ws = nullptr;
  if (need > 0 && av::decode_scratch(&ws) != hipSuccess) return AV_ERR_HIP;
  decode_set_workspace(a, ws, need, D);
  return hip_status(av::launch_attn_decode(a, var->score_mod, var->mask == AV_MASK_CAUSAL, stream));
}

size_t attn_decode_paged_workspace_bytes(int B, int Hq, int Hkv, int Sq, int D, int page_size, int max_pages) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 0 || D <= 0 || page_size <= 0 || max_pages <= 0) return 0;
  if ((int64_t)max_pages * page_size > INT32_MAX - 64) return 0;
  return av::decode_workspace_bytes(B, Hkv, max_pages * page_size, D);
}

int attn_decode_paged_fwd(const av_variant* var, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_table, const int32_t* seq_lens, void* out, float* lse,
                          void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int Sq, int D,
                          int page_size, int max_pages, int num_pages, hipStream_t stream) {
  if (var == nullptr) return AV_ERR_NULL;
  if (Sq > 0 && (q == nullptr || out == nullptr || k_cache == nullptr || v_cache == nullptr ||
                 block_table == nullptr || seq_lens == nullptr))
    return AV_ERR_NULL;
  if (var->score_mod < AV_SCORE_NONE || var->score_mod > AV_SCORE_SOFTCAP) return AV_ERR_UNSUPPORTED;
  if (var->mask != AV_MASK_NONE && var->mask != AV_MASK_CAUSAL) return AV_ERR_UNSUPPORTED;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq < 0 || D <= 0 || max_pages <= 0 || num_pages <= 0) return AV_ERR_SHAPE;
  if (Hq % Hkv != 0) return AV_ERR_SHAPE;
  if (var->kv_group != 0 && var->kv_group != Hq / Hkv) return AV_ERR_SHAPE;
  if (page_size != 16 && page_size != 32 && page_size != 64) return AV_ERR_UNSUPPORTED;
  if (D != 64) return AV_ERR_UNSUPPORTED;
  if ((int64_t)(Hq / Hkv) * Sq > 32) return AV_ERR_UNSUPPORTED;
  if (!(isfinite(var->scale) && var->scale >= 0.f)) return AV_ERR_PARAM;
  if (var->score_mod == AV_SCORE_SOFTCAP && !(isfinite(var->softcap) && var->softcap > 0.f)) return AV_ERR_PARAM;
  if (var->score_mod == AV_SCORE_ALIBI && !isfinite(var->alibi_max_bias)) return AV_ERR_PARAM;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16)) return AV_ERR_ALIGN;
  if (!aligned(block_table, 4) || !aligned(seq_lens, 4)) return AV_ERR_ALIGN;
  if (lse != nullptr && !aligned(lse, 4)) return AV_ERR_ALIGN;
  if ((int64_t)max_pages * page_size > INT32_MAX - 64) return AV_ERR_TOO_LARGE;
  if (Sq == 0) return AV_OK;
  const int Skv_max = max_pages * page_size;
  const av::DecodePlan plan = av::decode_plan(B, Hkv, Skv_max);
  const int64_t total = (int64_t)B * Hkv * plan.NS;
  if (total > INT32_MAX || (int64_t)B * Hkv * 32 > INT32_MAX) return AV_ERR_TOO_LARGE;
  const size_t need = av::decode_workspace_bytes(B, Hkv, Skv_max, D);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return AV_ERR_WORKSPACE;
  if (need > 0 && !aligned(workspace, 16)) return AV_ERR_ALIGN;

  av::DecodeArgs a{};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.o = out;
  a.lse = lse;
  a.ws_o = need > 0 ? (float*)workspace : nullptr;
  a.ws_ml = need > 0 ? (float*)workspace + (size_t)B * Hkv * plan.NS * 32 * D : nullptr;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Sq = Sq;
  a.Skv = Skv_max;
  a.g = Hq / Hkv;
  a.NS = plan.NS;
  a.tps = plan.tps;
  a.total = (int)total;
  const double scale = var->scale > 0.f ? (double)var->scale : 1.0 / sqrt((double)D);
  a.scale = (float)scale;
  a.c = (float)(scale * kLog2e);
  a.alibi_max_bias = var->alibi_max_bias;
  a.softcap = var->score_mod == AV_SCORE_SOFTCAP ? var->softcap : 1.f;
  a.fixed_ref = var->score_mod == AV_SCORE_SOFTCAP && 2.0 * var->softcap * kLog2e <= 96.0;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.page_size = page_size;
  a.max_pages = max_pages;
  a.num_pages = num_pages;
  return hip_status(av::launch_attn_decode(a, var->score_mod, var->mask == AV_MASK_CAUSAL, stream));
}

size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Skv, int D) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 0 || Skv < 0 || D <= 0) return 0;
  return (size_t)B * Hq * Sq * 8;
}

int attn_bwd(const av_variant* var, const void* q, const void* k, const void* v, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B,
             int Hq, int Hkv, int Sq, int Skv, int D, hipStream_t stream) {
  if (var == nullptr) return AV_ERR_NULL;
  if ((Sq > 0 && (q == nullptr || dout == nullptr || lse == nullptr || dq == nullptr)) ||
      (Skv > 0 && (k == nullptr || v == nullptr || dk == nullptr || dv == nullptr)))
    return AV_ERR_NULL;
  if (var->score_mod < AV_SCORE_NONE || var->score_mod > AV_SCORE_SOFTCAP) return AV_ERR_UNSUPPORTED;
  if (var->mask < AV_MASK_NONE || var->mask > AV_MASK_DOCUMENT) return AV_ERR_UNSUPPORTED;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq < 0 || Skv < 0 || D <= 0) return AV_ERR_SHAPE;
  if (Hq % Hkv != 0) return AV_ERR_SHAPE;
  if (var->kv_group != 0 && var->kv_group != Hq / Hkv) return AV_ERR_SHAPE;
  if (var->mask != AV_MASK_NONE && Sq != Skv) return AV_ERR_SHAPE;
  if (D != 64) return AV_ERR_UNSUPPORTED;
  if (var->mask == AV_MASK_DOCUMENT && Sq > 0 && var->doc_id == nullptr) return AV_ERR_NULL;
  if (!(isfinite(var->scale) && var->scale >= 0.f)) return AV_ERR_PARAM;
  if (var->score_mod == AV_SCORE_SOFTCAP && !(isfinite(var->softcap) && var->softcap > 0.f)) return AV_ERR_PARAM;
  if (var->score_mod == AV_SCORE_ALIBI && !isfinite(var->alibi_max_bias)) return AV_ERR_PARAM;
  if (var->mask == AV_MASK_SLIDING_WINDOW && var->window < 1) return AV_ERR_PARAM;
  if (var->mask == AV_MASK_PREFIX_LM && (var->prefix_len < 0 || var->prefix_len > Sq)) return AV_ERR_PARAM;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(dout, 16) ||
      !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4))
    return AV_ERR_ALIGN;
  if (var->mask == AV_MASK_DOCUMENT && !aligned(var->doc_id, 4)) return AV_ERR_ALIGN;
  if (const int rc = check_doc_order(var, B, Sq); rc != AV_OK) return rc;
  if ((uint64_t)(Sq + 256) * D * 2 > kMaxSliceBytes || (uint64_t)(Skv + 128) * D * 2 > kMaxSliceBytes)
    return AV_ERR_TOO_LARGE;
  const int64_t total = (int64_t)B * Hkv * ((Skv + 127) / 128);
  const int64_t total_q = (int64_t)B * Hq * ((Sq + 127) / 128);
  if (total > INT32_MAX || total_q > INT32_MAX || (int64_t)B * Hq * Sq > INT32_MAX) return AV_ERR_TOO_LARGE;
  if (Sq == 0) {
    // no query: every key gets a zero gradient
    if (Skv > 0) {
      const size_t n = (size_t)B * Hkv * Skv * D * 2;
      if (av::launch_zero_fill(dk, n, stream) != hipSuccess || av::launch_zero_fill(dv, n, stream) != hipSuccess)
        return AV_ERR_HIP;
    }
    return AV_OK;
  }
  if (Skv == 0) {
    // no key (mask none only: a mask needs Sq == Skv): the output is the
    // constant zero row, so every query gets a zero gradient
    return hip_status(av::launch_zero_fill(dq, (size_t)B * Hq * Sq * D * 2, stream));
  }
  const size_t need = (size_t)B * Hq * Sq * 8;
  if (workspace == nullptr || workspace_bytes < need) return AV_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return AV_ERR_ALIGN;

  av::BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.stats = (float*)workspace;
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Sq = Sq;
  a.Skv = Skv;
  a.g = Hq / Hkv;
  a.total = (int)total;
  a.total_q = (int)total_q;
  const double scale = var->scale > 0.f ? (double)var->scale : 1.0 / sqrt((double)D);
  a.scale = (float)scale;
  a.c = (float)(scale * kLog2e);
  a.softcap = var->score_mod == AV_SCORE_SOFTCAP ? var->softcap : 1.f;
  a.sc_k = (float)(2.0 * scale * kLog2e / a.softcap);
  a.sc_inv_cap2 = (float)(1.0 / (a.softcap * kLog2e));
  a.sc_poly_lim = -1.f;
  if (var->score_mod == AV_SCORE_SOFTCAP && 2.0 * var->softcap * kLog2e <= 96.0)
    softcap_cubic(scale, var->softcap, a.sc_poly, a.sc_poly_lim);
  a.alibi_max_bias = var->alibi_max_bias;
  a.window = var->window;
  a.prefix = var->prefix_len;
  a.doc = var->mask == AV_MASK_DOCUMENT ? var->doc_id : nullptr;
  a.doc_order = var->mask == AV_MASK_DOCUMENT ? var->doc_order : nullptr;
  return hip_status(av::launch_attn_bwd(a, var->score_mod, var->mask, stream));
}

int diff_attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int H, int S, int Dh, int Dv,
                  float lambda, float scale, int causal, hipStream_t stream) {
  if (!isfinite(lambda)) return AV_ERR_PARAM;
  av::DiffArgs a{};
  a.lambda = lambda;
  return diff_launch(a, q, k, v, out, B, H, S, Dh, Dv, scale, causal, stream);
}

int diff_head_fwd(const void* q, const void* k, const void* v, const float* lambda_q1, const float* lambda_k1,
                  const float* lambda_q2, const float* lambda_k2, const float* gamma, void* out, int B, int H, int S,
                  int Dh, int Dv, float lambda_init, float eps, float scale, int causal, hipStream_t stream) {
  if (lambda_q1 == nullptr || lambda_k1 == nullptr || lambda_q2 == nullptr || lambda_k2 == nullptr)
    return AV_ERR_NULL;
  if (!isfinite(lambda_init) || !(isfinite(eps) && eps > 0.f)) return AV_ERR_PARAM;
  if (!aligned(lambda_q1, 4) || !aligned(lambda_k1, 4) || !aligned(lambda_q2, 4) || !aligned(lambda_k2, 4) ||
      (gamma != nullptr && !aligned(gamma, 4)))
    return AV_ERR_ALIGN;
  av::DiffArgs a{};
  a.lam_q1 = lambda_q1;
  a.lam_k1 = lambda_k1;
  a.lam_q2 = lambda_q2;
  a.lam_k2 = lambda_k2;
  a.gamma = gamma;
  a.lambda_init = lambda_init;
  a.eps = eps;
  return diff_launch(a, q, k, v, out, B, H, S, Dh, Dv, scale, causal, stream);
}

size_t evoformer_workspace_bytes(int Ns, int Nr, int H, int dh) {
  if (Ns <= 0 || Nr <= 0 || H <= 0 || dh <= 0) return 0;
  return av::evo_workspace_bytes(Ns, Nr, H, dh);
}

}  // extern "C"

namespace {

// Shared validation and launch of both Evoformer forms (bias == nullptr and
// col == 1 for the column-wise form).
int evoformer_launch(const void* m, const void* wq, const void* wk, const void* wv, const void* wg, const void* bias,
                     void* out, void* workspace, size_t workspace_bytes, int Ns, int Nr, int Cm, int H, int dh,
                     float scale, int col, hipStream_t stream) {
  if (m == nullptr || wq == nullptr || wk == nullptr || wv == nullptr || wg == nullptr || out == nullptr ||
      (!col && bias == nullptr))
    return AV_ERR_NULL;
  if (Ns <= 0 || Nr <= 0 || Cm <= 0 || H <= 0 || dh <= 0) return AV_ERR_SHAPE;
  if ((dh != 32 && dh != 64) || Cm % 64 != 0 || (H * dh) % 128 != 0) return AV_ERR_UNSUPPORTED;
  if (!(isfinite(scale) && scale >= 0.f)) return AV_ERR_PARAM;
  if (!aligned(m, 16) || !aligned(wq, 16) || !aligned(wk, 16) || !aligned(wv, 16) || !aligned(wg, 16) ||
      (!col && !aligned(bias, 16)) || !aligned(out, 16))
    return AV_ERR_ALIGN;
  if ((uint64_t)Ns * Nr * Cm * 2 > kMaxSliceBytes || (uint64_t)Ns * Nr * H * dh * 2 > kMaxSliceBytes ||
      (!col && (uint64_t)H * Nr * Nr * 2 > kMaxSliceBytes))
    return AV_ERR_TOO_LARGE;
  const size_t need = av::evo_workspace_bytes(Ns, Nr, H, dh);
  if (workspace == nullptr || workspace_bytes < need) return AV_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return AV_ERR_ALIGN;
  av::EvoArgs a{};
  a.m = m;
  a.w[0] = wq;
  a.w[1] = wk;
  a.w[2] = wv;
  a.w[3] = wg;
  a.bias = col ? nullptr : bias;
  a.out = out;
  a.ws = workspace;
  a.Ns = Ns;
  a.Nr = Nr;
  a.Cm = Cm;
  a.H = H;
  a.dh = dh;
  a.col = col;
  a.scale = scale > 0.f ? scale : (float)(1.0 / sqrt((double)dh));
  return hip_status(av::launch_evoformer(a, stream));
}

}  // namespace

extern "C" {

int evoformer_gated_attn_fwd(const void* m, const void* wq, const void* wk, const void* wv, const void* wg,
                             const void* bias, void* out, void* workspace, size_t workspace_bytes, int Ns, int Nr,
                             int Cm, int H, int dh, float scale, hipStream_t stream) {
  return evoformer_launch(m, wq, wk, wv, wg, bias, out, workspace, workspace_bytes, Ns, Nr, Cm, H, dh, scale, 0,
                          stream);
}

int evoformer_col_gated_attn_fwd(const void* m, const void* wq, const void* wk, const void* wv, const void* wg,
                                 void* out, void* workspace, size_t workspace_bytes, int Ns, int Nr, int Cm, int H,
                                 int dh, float scale, hipStream_t stream) {
  return evoformer_launch(m, wq, wk, wv, wg, nullptr, out, workspace, workspace_bytes, Ns, Nr, Cm, H, dh, scale, 1,
                          stream);
}

}  // extern "C"
