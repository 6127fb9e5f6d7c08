// Launch-side declarations shared by the C ABI (attnvar_api.cpp) and the
// kernel translation units.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace av {

// Internal score modifiers: SM_BIAS = Evoformer pair bias added to the score
// of queries that arrive already scaled (the projection folds the softmax
// scale into q), with the sigmoid-gate epilogue and a token-major [B, Sq, Hq*D]
// output (row-wise form); SM_GATE = no modifier, sigmoid-gate epilogue and a
// token-major [Sq, B, Hq*D] output (column-wise form: problem b is residue
// column b, query q is sequence q); SM_SOFTCAP_FIXED = softcap whose exponent
// reference is fixed at the cap (chosen by the launcher when fixed_ref is set);
// SM_TBIAS = additive bias tensor read per (batch, head) through strides, the
// plain epilogue and [B, Hq, Sq, D] output (the public AV_SCORE_BIAS).
enum ScoreMod : int {
  SM_NONE = 0, SM_ALIBI = 1, SM_SOFTCAP = 2, SM_BIAS = 3, SM_SOFTCAP_FIXED = 4, SM_GATE = 5, SM_TBIAS = 6
};
enum MaskKind : int { MK_NONE = 0, MK_CAUSAL = 1, MK_WINDOW = 2, MK_PREFIX = 3, MK_DOC = 4 };

// Kernel argument block of the fused attention forward (passed by value).
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;        // nullable
  const int* doc;    // MK_DOC only
  const int* doc_order;  // MK_DOC, nullable: (b * nM + query tile) in visiting order
  const void* bias;  // SM_BIAS / SM_TBIAS: bf16, rows of Skv; (b, hq) slice at b * bias_bs + hq * bias_hs
  const void* gate;  // SM_BIAS: [B, Hq, Sq, D] bf16 gate pre-activations (same layout as q)
  int B, Hq, Hkv, Sq, Skv;
  int g;             // Hq / Hkv
  int nM;            // query tiles per (b, head)
  int total;         // B * Hq * nM
  float c;           // scale * log2(e): scores are carried in log2 units
  float scale;
  float alibi_max_bias;
  float softcap;
  int window;
  int prefix;
  int fixed_ref;     // softcap with 2 * cap * log2(e) <= 96: exponent reference fixed at the cap
  long long bias_bs, bias_hs;  // bias element strides of batch and head (0 = shared)
  // fixed-reference softcap: t = cap*log2(e)*tanh(scale*raw/cap) = raw * P(raw^2) with
  // the linear P below, valid while |raw| <= sc_poly_lim (raw = unscaled q.k); without
  // lse the kernel scales q by beta = sc_x[1] and in x = beta * raw t = x * (sc_x[0] - x^2),
  // valid while |x| <= sc_x_lim
  float sc_poly[2];
  float sc_poly_lim;
  float sc_x[2];
  float sc_x_lim;
  int one_block;     // causal / PrefixLM rows run one 32-row block per wave (attn_one_block)
};

// Query rows per workgroup: the differential kernel uses 4 waves x 32 rows;
// the fused attention kernel uses 4 waves x 32*QB rows, QB = query blocks per
// wave: 2 at D = 64, so every K/V fragment read from LDS feeds two MFMAs;
// 1 at D = 128 (two blocks do not fit the register file), at D = 32 (the
// Evoformer shapes: short rows, where more and smaller workgroups hide the
// load latency better), for the sliding window and document masks, whose
// short per-row key ranges favour more, smaller workgroups, and for the bias
// tensor and the Evoformer forms (their staged bias tile or gate
// pre-activations take the registers of a second block).
constexpr int kAttnBM = 128;
constexpr int attn_qb(int D, int sm, int mask) {
  return (D == 64 && mask != MK_WINDOW && mask != MK_DOC && sm != SM_TBIAS && sm != SM_BIAS && sm != SM_GATE) ? 2
                                                                                                             : 1;
}
constexpr int attn_bm(int D, int sm, int mask) { return 4 * 32 * attn_qb(D, sm, mask); }
// Causal and PrefixLM over at most kShortRows queries take one query block
// per wave too (128-row workgroups): their key loops are short, so more and
// smaller workgroups win.  Same box, 16 heads, B * S = 16384: S = 512
// 43.3 -> 41.0 us (GQA 16/2: 41.4 -> 36.0 us), S = 1024 2-5 % faster; from
// S = 2048 on two blocks per wave are 2.5-4 % faster.
constexpr int kShortRows = 1024;
constexpr bool attn_one_block(int D, int sm, int mask, int Sq) {
  return attn_qb(D, sm, mask) == 2 && (mask == MK_CAUSAL || mask == MK_PREFIX) && Sq <= kShortRows;
}
constexpr int kAttnBMMax = 256;

// Work order of the document mask: query tiles of kDocTileM rows (the
// fused kernel's tile under that mask at every D and score modifier), key
// tiles of kDocTileN, at most kDocOrderMax query tiles per order.
constexpr int kDocTileM = attn_bm(64, SM_NONE, MK_DOC);
constexpr int kDocTileN = 64;
constexpr int kDocOrderMax = 16384;
static_assert(attn_bm(32, SM_NONE, MK_DOC) == kDocTileM && attn_bm(128, SM_NONE, MK_DOC) == kDocTileM &&
                  attn_bm(64, SM_TBIAS, MK_DOC) == kDocTileM,
              "one query tile height under the document mask");
hipError_t launch_doc_order(const int* doc, int B, int S, int* order, hipStream_t stream);

hipError_t launch_attn_fwd(const AttnArgs& a, int D, int score_mod, int mask, hipStream_t stream);
// Evoformer gated attention over the projected workspace (D = head width, 32
// or 64): row-wise (SM_BIAS) or column-wise (SM_GATE).
hipError_t launch_evo_attention(const AttnArgs& a, int D, int col, hipStream_t stream);

// Decoding / short-query attention (split-KV): the Sq queries are the last
// Sq positions of the keys; one workgroup per (batch, KV head, key split)
// holds the g*Sq <= 32 query rows of the KV head's query heads.
struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;        // nullable
  float* ws_o;       // [B*Hkv, NS, 32, D] partial O of each split (NS > 1)
  float* ws_ml;      // [B*Hkv, NS, 32, 2] (max, sum) of each split
  int B, Hq, Hkv, Sq, Skv;
  int g;             // Hq / Hkv
  int NS, tps;       // key splits, 64-key tiles per split
  int total;         // B * Hkv * NS
  float c, scale, alibi_max_bias, softcap;
  int fixed_ref;
  // paged cache (block_table != nullptr): k, v are [num_pages, Hkv, page_size, D];
  // Skv is then max_pages * page_size, the plan's bound on every sequence
  const int* block_table;  // [B, max_pages]
  const int* seq_lens;     // [B]
  int page_size, max_pages, num_pages;
};
struct DecodePlan {
  int NS, tps;
};
DecodePlan decode_plan(int B, int Hkv, int Skv);
size_t decode_workspace_bytes(int B, int Hkv, int Skv, int D);
// Bound of decode_workspace_bytes over every plan at D = 64 (the plan splits
// only while B * Hkv < 512 and keeps B * Hkv * NS < 1024), and the per-device
// address of the static array of that size that the allocation-free decode
// entry point uses in place of a caller workspace (looked up once per device,
// on the current device).
constexpr size_t kDecodeScratchBytes = (size_t)1024 * 32 * (64 + 2) * 4;
hipError_t decode_scratch(void** ptr);
hipError_t launch_attn_decode(const DecodeArgs& a, int score_mod, int causal, hipStream_t stream);

// Attention backward (D = 64; the forward's five masks).
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* lse;   // forward log-sum-exp, natural log, [B, Hq, Sq]
  void* dq;
  void* dk;
  void* dv;
  float* stats;       // workspace [B, Hq, Sq, 2]: corrected reference (log2 units), Delta
  int B, Hq, Hkv, Sq, Skv, g;
  int total;          // dK/dV workgroups: B * Hkv * ceil(Skv / 128)
  int total_q;        // dQ workgroups: B * Hq * ceil(Sq / 128)
  float c;            // scale * log2(e)
  float scale;
  float sc_k;         // softcap: 2 * scale * log2(e) / cap
  float alibi_max_bias;
  float softcap;
  int window;         // MK_WINDOW
  int prefix;         // MK_PREFIX
  const int* doc;     // MK_DOC: [B, S] document ids
  const int* doc_order;  // MK_DOC, optional: heaviest-first order of the 128-row tiles (attn_doc_order)
  // softcap on a tile whose raw scores all satisfy |raw| <= sc_poly_lim (the
  // forward's cubic): cap*log2(e)*tanh(scale*raw/cap) = raw*(sc_poly[0] +
  // sc_poly[1]*raw^2); sc_poly_lim < 0 keeps every tile on the exact form
  float sc_poly[2];
  float sc_poly_lim;
  float sc_inv_cap2;  // 1 / (cap*log2(e))
};
hipError_t launch_attn_bwd(const BwdArgs& a, int score_mod, int mask, hipStream_t stream);
// Zero `bytes` (a multiple of 16, 16-byte aligned) with a kernel (no memset
// node, so the call can sit in a captured graph).
hipError_t launch_zero_fill(void* p, size_t bytes, hipStream_t stream);

struct DiffArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  int B, H, S;
  int nM, total;
  float c;        // scale * log2(e)
  float lambda;
  int causal;
  // full head form (lam_q1 != nullptr): lambda = exp(lq1.lk1) - exp(lq2.lk2)
  // + lambda_init computed in the kernel from four fp32 [Dh] vectors, then
  // the per-row RMS norm with the fp32 [Dv] weight gamma (nullable = ones)
  // and the (1 - lambda_init) factor
  const float* lam_q1;
  const float* lam_k1;
  const float* lam_q2;
  const float* lam_k2;
  const float* gamma;
  float lambda_init, eps;
};
hipError_t launch_diff_attn_fwd(const DiffArgs& a, int Dh, int Dv, hipStream_t stream);

struct EvoArgs {
  const void* m;
  const void* w[4];  // wq, wk, wv, wg  [Cm, H*dh]
  const void* bias;  // [H, Nr, Nr]
  void* out;         // [Ns, Nr, H*dh]
  void* ws;          // 4 planes (q, k, v, g) bf16: [Ns, H, Nr, dh] row-wise, [Nr, H, Ns, dh] column-wise
  int Ns, Nr, Cm, H, dh;
  int col;           // 0: row-wise (pair bias), 1: column-wise (no bias)
  float scale;       // softmax scale, applied to q in the projection epilogue
};
size_t evo_workspace_bytes(int Ns, int Nr, int H, int dh);
hipError_t launch_evoformer(const EvoArgs& a, hipStream_t stream);
// Both forms in one launch (projections kept on chip, no workspace traffic)
// for the shapes whose K and V fit one workgroup's LDS.
bool evo_fused_fits(const EvoArgs& a);
hipError_t launch_evo_fused(const EvoArgs& a, hipStream_t stream);

}  // namespace av
