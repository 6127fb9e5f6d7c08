/*
 * attnvar.h -- C ABI of the MI355X (gfx950) fused attention-variant library.
 *
 * The operations are the fused attention forward passes that the Flashlight
 * pages describe ("Flashlight: PyTorch Compiler Extensions to Accelerate
 * Attention Variants", MLSys 2026 talk notes, sections "Compiler design"
 * 1-4 and "Evaluation"; Spanish summary "Resumen Tecnico: FLASHLIGHT",
 * section "Metodologia"): QK^T, a per-element score modifier, a mask, a
 * softmax computed online with a running max and running sum, and PV, in
 * one kernel without writing the score matrix to memory.
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer.  Memory is allocated and
 *     owned by the caller; the library allocates nothing and frees nothing.
 *   - Element type is bfloat16 (bf16) for every tensor unless stated;
 *     products accumulate in fp32 (talk notes, "Implementation details",
 *     precision item: fp16/bf16 inputs compute in fp32).
 *   - Tensors are dense, contiguous, row-major, in the shapes given.
 *     Tensor pointers must be 16-byte aligned; float and int32 pointers
 *     4-byte aligned.
 *   - Calls are asynchronous on `stream` (0 = the null stream).  The library
 *     never synchronises.  Device faults surface at the caller's next sync.
 *   - Every argument is validated on the host before anything is launched.
 *     On error nothing is launched and nothing is written.
 *   - Return value: AV_OK (0) or a negative av_status.  No C++ exception
 *     crosses this boundary.  av_status_string() names a status.
 *   - Calls on different streams may run concurrently; they share no state.
 */
#ifndef ATTNVAR_H
#define ATTNVAR_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  AV_OK = 0,
  AV_ERR_NULL = -1,        /* a required pointer is NULL */
  AV_ERR_SHAPE = -2,       /* sizes inconsistent (Hq % Hkv, Sq != Skv with a mask, negative sizes, ...) */
  AV_ERR_UNSUPPORTED = -3, /* head dim or enum value this library does not implement */
  AV_ERR_ALIGN = -4,       /* pointer misaligned */
  AV_ERR_WORKSPACE = -5,   /* workspace missing or too small */
  AV_ERR_HIP = -6,         /* the HIP runtime refused the launch */
  AV_ERR_PARAM = -7,       /* a scalar parameter is out of range (window < 1, softcap <= 0, ...) */
  AV_ERR_TOO_LARGE = -8    /* a size exceeds the 32-bit addressing the kernels use */
} av_status;

/* Per-element score modifiers (talk notes, "Evaluation: FlexAttention-
 * supported variants").  Applied to the scaled score s = scale * q.k:
 *   AV_SCORE_ALIBI:   s + slope_h * (j - i),  slope_h = 2^(-alibi_max_bias * (h+1) / Hq)
 *                     for 0-based query head h, query row i, key row j.
 *   AV_SCORE_SOFTCAP: softcap * tanh(s / softcap).
 *   AV_SCORE_BIAS:    s + bias(b, h, i, j), read from a tensor: the
 *                     data-dependent modifier (the talk notes' abstract sets
 *                     Flashlight apart by data-dependent formulations; the
 *                     Evoformer pair bias is one).  attn_fwd only. */
typedef enum { AV_SCORE_NONE = 0, AV_SCORE_ALIBI = 1, AV_SCORE_SOFTCAP = 2, AV_SCORE_BIAS = 3 } av_score_mod;

/* Masks (same section).  Key j is visible to query i when:
 *   AV_MASK_NONE:           always
 *   AV_MASK_CAUSAL:         j <= i
 *   AV_MASK_SLIDING_WINDOW: 0 <= i - j < window      (window keys, self included)
 *   AV_MASK_PREFIX_LM:      j < prefix_len  or  j <= i
 *   AV_MASK_DOCUMENT:       doc_id[b, i] == doc_id[b, j]   (not causal)
 * A query row with no visible key yields an all-zero output row and
 * lse = -inf.  Every mask other than AV_MASK_NONE needs Sq == Skv. */
typedef enum {
  AV_MASK_NONE = 0,
  AV_MASK_CAUSAL = 1,
  AV_MASK_SLIDING_WINDOW = 2,
  AV_MASK_PREFIX_LM = 3,
  AV_MASK_DOCUMENT = 4
} av_mask;

/* Variant descriptor: {score_mod, mask, params, kv_group}. */
typedef struct {
  int32_t score_mod;      /* av_score_mod */
  int32_t mask;           /* av_mask */
  float scale;            /* multiplies q.k; 0 selects 1/sqrt(D); must be finite and >= 0 */
  float softcap;          /* AV_SCORE_SOFTCAP: cap > 0 */
  float alibi_max_bias;   /* AV_SCORE_ALIBI: 8 gives slopes 2^(-8(h+1)/Hq); finite */
  int32_t window;         /* AV_MASK_SLIDING_WINDOW: >= 1 */
  int32_t prefix_len;     /* AV_MASK_PREFIX_LM: 0 <= prefix_len <= S */
  const int32_t* doc_id;  /* AV_MASK_DOCUMENT: device [B, S] int32, values in [0, INT32_MAX),
                             non-decreasing along each row (a precondition the host cannot
                             check: rows that break it give unspecified output) */
  int32_t kv_group;       /* Hq / Hkv (1 = MHA); 0 = derive from Hq and Hkv */
  /* AV_SCORE_BIAS: device bf16; element (b, h, i, j) is
   *   bias[b * bias_batch_stride + h * bias_head_stride + i * Skv + j]
   * (strides in elements, >= 0; 0 shares one slice over every batch or
   * query head).  8-byte aligned; when Skv % 4 == 0 both strides must be
   * multiples of 4.  (Sq + 256) * (Skv + 64) * 2 bytes must stay below 2 GiB. */
  const void* bias;
  int64_t bias_batch_stride;
  int64_t bias_head_stride;
  /* AV_MASK_DOCUMENT, optional (NULL = natural order): device int32 order of
   * the query tiles written by attn_doc_order for the same doc_id, B and S.
   * It changes only the order in which attn_fwd and attn_bwd visit their
   * work, never a result bit.  Non-NULL with any other mask is
   * AV_ERR_PARAM; 4-byte aligned.  Read by attn_fwd and attn_bwd. */
  const int32_t* doc_order;
  /* Entries the doc_order buffer holds.  attn_fwd and attn_bwd read exactly
   * n = attn_doc_order_len(B, Sq) of them; doc_order_len != n is
   * AV_ERR_PARAM (an order built for another shape), and a shape for which
   * attn_doc_order_len fails is that function's error.  Ignored when
   * doc_order is NULL. */
  int32_t doc_order_len;
} av_variant;

/* Fused attention forward, MHA and GQA.
 *   q   [B, Hq,  Sq,  D]    k [B, Hkv, Skv, D]    v [B, Hkv, Skv, D]
 *   out [B, Hq,  Sq,  D]    written (bf16, round-to-nearest-even from fp32)
 *   lse [B, Hq,  Sq]  fp32  natural-log sum-exp of the modified, masked
 *                           scores per row; may be NULL (not written).  When
 *                           it is requested the row sums add the fp32
 *                           exponentials (lse exact to fp32 rounding, one more
 *                           add per two scores); without it they add the
 *                           bf16-rounded probabilities that the PV product
 *                           consumes.  Either sum normalises out.
 * Query head h reads key/value head h / (Hq / Hkv).  D in {32, 64, 128}.
 * Sq == 0 launches nothing; Skv == 0 writes zero rows and lse = -inf.
 * Pointers of empty tensors may be NULL (q/out when Sq == 0, k/v when Skv == 0).
 * Each (b, Hkv head) slice of K and V, and each (b, Hq head) slice of Q
 * and out, must be smaller than 2 GiB. */
int attn_fwd(const av_variant* variant, const void* q, const void* k, const void* v, void* out,
             float* lse, int B, int Hq, int Hkv, int Sq, int Skv, int D, hipStream_t stream);

/* Work order of attn_fwd under the document mask (one of the masked variants
 * of talk notes, "Evaluation: FlexAttention-supported variants"; like
 * FlexAttention's block_mask in "Comparison with FlexAttention", it is built
 * once from the mask's data and reused across calls, but it skips nothing:
 * the key ranges stay analytic).  A query
 * tile there attends to the keys of its own documents, so its run time
 * follows the document lengths; visiting the heaviest tiles first shortens
 * the tail that heavy tiles starting late would leave.  attn_doc_order
 * writes the n = attn_doc_order_len(B, S) query tiles (b * ceil(S/128) + t
 * for 128-row tile t of sequence b) sorted by the number of 64-key tiles
 * their documents span, largest first, ties by ascending index.  The order
 * depends only on doc_id: compute it once per document layout and pass it
 * as av_variant.doc_order to every attn_fwd and attn_bwd call (layer, head count, score
 * modifier, D) over that layout.
 *   doc_id [B, S] int32 device, non-decreasing rows (as av_variant.doc_id)
 *   order  [order_len] int32 device, caller-owned, 4-byte aligned; the
 *          first n entries are written
 * attn_doc_order_len returns n, or AV_ERR_SHAPE (B <= 0, S < 0) or
 * AV_ERR_TOO_LARGE (n > 16384, i.e. more than 2^21 tokens).  attn_doc_order
 * returns those errors, AV_ERR_NULL, AV_ERR_ALIGN, AV_ERR_WORKSPACE when
 * order_len < n; n == 0 launches nothing. */
int attn_doc_order_len(int B, int S);
int attn_doc_order(const int32_t* doc_id, int B, int S, int32_t* order, int order_len, hipStream_t stream);

/* Decoding / short-query attention forward (split over the keys).  The
 * pages' serving workload decodes causal and softcapped LLaMA-3.2-1B variants
 * under vLLM (talk notes, end-to-end section); the operation is attn_fwd's,
 * with the queries placed at the end of the keys: query q of a sequence has
 * absolute position Skv - Sq + q, which the causal mask and the ALiBi
 * distance use.
 *   q [B, Hq, Sq, D]   k, v [B, Hkv, Skv, D]   out [B, Hq, Sq, D]
 *   lse [B, Hq, Sq] fp32, nullable (natural log, as attn_fwd)
 * Supported: D = 64; (Hq/Hkv) * Sq <= 32 (all queries of one KV head fit one
 * 32-row block); mask none or causal (causal needs Skv >= Sq); score
 * modifiers none, ALiBi and softcap.  `workspace` (device, caller-owned, 16-byte aligned) must hold
 * attn_decode_workspace_bytes(B, Hq, Hkv, Sq, Skv, D) bytes; when that is 0
 * it may be NULL.  Skv == 0 writes zero rows and lse = -inf. */
size_t attn_decode_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Skv, int D);
int attn_decode_fwd(const av_variant* variant, const void* q, const void* k, const void* v, void* out, float* lse,
                    void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int Sq, int Skv, int D,
                    hipStream_t stream);

/* attn_decode_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same operation, arguments, limits, kernels and results, with no
 * workspace argument.  The split-KV partials go to a static device array of
 * 8650752 bytes (8.25 MiB) that every GPU the library runs on holds until
 * the process ends; the call itself allocates nothing.  Every plan of the supported shapes fits (the keys are split only
 * while B * Hkv < 512, into fewer than 1024 (b, KV head, split) units of
 * 32 x 66 fp32 values); a plan that would not returns AV_ERR_TOO_LARGE.  The
 * call runs on the current device (the stream must belong to it); the first
 * call on a device looks the array's address up there (AV_ERR_HIP if that
 * fails).  All calls on one GPU share the array: calls that can overlap on
 * one GPU (different streams, or graphs replayed concurrently) race and
 * must be ordered by the caller. */
int attn_decode_fwd_noalloc(const av_variant* variant, const void* q, const void* k, const void* v, void* out,
                            float* lse, int B, int Hq, int Hkv, int Sq, int Skv, int D, hipStream_t stream);

/* Decoding against a paged key/value cache (the vLLM-style serving layout of
 * the pages' end-to-end workload; same operation and limits as
 * attn_decode_fwd, with per-sequence key counts):
 *   k_cache, v_cache [num_pages, Hkv, page_size, D]
 *   block_table [B, max_pages] int32: key j of sequence b is in page
 *     block_table[b, j / page_size], slot j % page_size
 *   seq_lens [B] int32: keys of sequence b (<= max_pages * page_size; the Sq
 *     queries are its last Sq positions)
 * Device data are not read on the host: seq_lens is clamped to
 * [0, max_pages * page_size] and page ids to [0, num_pages) in the kernel, so
 * a bad table gives wrong rows, never an out-of-bounds access.  A sequence
 * shorter than Sq under the causal mask gets zero rows (lse = -inf) for its
 * queries that precede every key.  Supported page_size: 16, 32, 64.
 * `workspace` as attn_decode_fwd, sized by attn_decode_paged_workspace_bytes. */
size_t attn_decode_paged_workspace_bytes(int B, int Hq, int Hkv, int Sq, int D, int page_size, int max_pages);
int attn_decode_paged_fwd(const av_variant* variant, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_table, const int32_t* seq_lens, void* out, float* lse,
                          void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int Sq, int D,
                          int page_size, int max_pages, int num_pages, hipStream_t stream);

/* Attention backward: gradients of attn_fwd's output (the pages name
 * training as the other half of the workload, talk notes "Background and
 * motivation").  With t = mod(scale q.k) masked and P = softmax(t):
 *   dV = P^T dO,  dP = dO V^T,  dT = P (dP - rowsum(P dP)),
 *   dS = dT mod'(scale q.k)  (softcap: 1 - tanh^2(scale q.k / cap); else 1),
 *   dQ = scale dS K,  dK = scale dS^T Q   (dK, dV summed over the query heads
 *   of a KV head).
 * Inputs: q, k, v as given to attn_fwd, attn_fwd's `lse` (natural log,
 * [B, Hq, Sq], required: it serves as the exponent reference; a first pass
 * renormalises P in fp32, so its bf16 rounding does not reach the gradients)
 * and dout [B, Hq, Sq, D].  Outputs dq [B, Hq, Sq, D], dk, dv
 * [B, Hkv, Skv, D], bf16 (fp32 accumulation).  `workspace` (device,
 * caller-owned, 16-byte aligned) holds attn_bwd_workspace_bytes(...) bytes.
 * Supported: D = 64; every mask of attn_fwd with its parameters in the
 * variant (window, prefix_len, doc_id; a mask needs Sq == Skv); every score
 * modifier but AV_SCORE_BIAS.  Sq > 0 with Skv == 0 writes a zero dq.
 * Under the document mask the variant's doc_order (as for attn_fwd) orders
 * the three launches heaviest first: a 128-key tile there spans the same
 * documents as the 128-row query tile at its position.
 * Deterministic (no atomics). */
size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Skv, int D);
int attn_bwd(const av_variant* variant, const void* q, const void* k, const void* v, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int B,
             int Hq, int Hkv, int Sq, int Skv, int D, hipStream_t stream);

/* Differential attention forward (talk notes, "Background and motivation"
 * and "Evaluation: complex attention variants"; the pages name the variant
 * without a formula; the reading implemented is):
 *   q, k [B, H, S, 2*Dh]: two halves q1 = q[..., :Dh], q2 = q[..., Dh:]
 *   v    [B, H, S, Dv],  out [B, H, S, Dv]
 *   out = (softmax(scale * q1 k1^T + M) - lambda * softmax(scale * q2 k2^T + M)) v
 * M is the causal mask when `causal` != 0, else nothing.  scale = 0 selects
 * 1/sqrt(Dh).  Supported: Dh in {32, 64}, Dv in {64, 128} (the talk notes'
 * "16 heads x 128" shape read as Dh = 64, Dv = 128; "32 heads x 64" as
 * Dh = 32, Dv = 64). */
int diff_attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int H, int S, int Dh,
                  int Dv, float lambda, float scale, int causal, hipStream_t stream);

/* Full differential-attention head (DiffTransformer, which the talk notes
 * name under "Related work"; the pages benchmark only the attention core
 * above).  The head follows the published Differential Transformer (Ye et
 * al., 2024: differential attention and its multi-head form):
 *   lambda = exp(lambda_q1 . lambda_k1) - exp(lambda_q2 . lambda_k2) + lambda_init
 *   A      = the diff_attn_fwd result with that lambda, kept in fp32
 *   out[b, h, i, e] = (1 - lambda_init) * gamma[e] * A[i, e] / sqrt(mean_e' A[i, e']^2 + eps)
 * i.e. RMSNorm over the Dv channels of each row (per head), then the
 * (1 - lambda_init) factor.  The published depth schedule is
 * lambda_init = 0.8 - 0.6 exp(-0.3 (l - 1)) for 1-based layer l; the caller
 * passes the value.  lambda_q1 .. lambda_k2: device fp32 [Dh] each; gamma:
 * device fp32 [Dv] or NULL (all ones); all 4-byte aligned, caller-owned.
 * The kernel computes lambda on the device, so the parameters may change
 * between calls without a host round trip.  q, k, v, out, shapes, scale,
 * causal and support as diff_attn_fwd.  eps must be finite and > 0. */
int diff_head_fwd(const void* q, const void* k, const void* v, const float* lambda_q1, const float* lambda_k1,
                  const float* lambda_q2, const float* lambda_k2, const float* gamma, void* out, int B, int H, int S,
                  int Dh, int Dv, float lambda_init, float eps, float scale, int causal, hipStream_t stream);

/* Evoformer row-wise gated self-attention with pair bias (talk notes,
 * "Evaluation: complex attention variants" and the AlphaFold2 end-to-end
 * section; no formula on the pages; the reading implemented is, per MSA
 * sequence s, head h, residue rows i, j):
 *   q, k, v, g = m Wq, m Wk, m Wv, m Wg                 (no bias, no LayerNorm)
 *   out[s, i, h*dh + e] = sigmoid(g[s, i, h*dh + e])
 *                         * sum_j softmax_j(scale * q_i.k_j + bias[h, i, j]) v_j[e]
 *   m    [Ns, Nr, Cm]      w* [Cm, H*dh] each      bias [H, Nr, Nr]
 *   out  [Ns, Nr, H*dh]
 * The projections are computed into `workspace` (bf16, owned by the caller,
 * at least evoformer_workspace_bytes(...) bytes, 256-byte aligned) by one
 * kernel, then consumed by the attention kernel; the q plane holds scale*q
 * (the softmax scale applied before the bf16 rounding).  With Cm = 256 and
 * Nr <= 256, Nr a multiple of 8, one kernel keeps the projections on chip
 * and leaves the workspace untouched (it is still required).  scale = 0 selects
 * 1/sqrt(dh).  Supported: dh in {32, 64} (the AlphaFold2 8 heads x 32 and the talk
 * notes' kernel-benchmark 4 heads x 64), Cm a multiple of 64, H*dh a multiple
 * of 128. */
size_t evoformer_workspace_bytes(int Ns, int Nr, int H, int dh);
int evoformer_gated_attn_fwd(const void* m, const void* wq, const void* wk, const void* wv, const void* wg,
                             const void* bias, void* out, void* workspace, size_t workspace_bytes, int Ns,
                             int Nr, int Cm, int H, int dh, float scale, hipStream_t stream);

/* Evoformer column-wise gated self-attention (the sibling the pages name with
 * the row-wise form: talk notes "Background and motivation" and "Evaluation:
 * complex attention variants"; no formula on the pages; the reading
 * implemented is, per residue column r, head h, sequences s, t):
 *   q, k, v, g = m Wq, m Wk, m Wv, m Wg                 (the same projections)
 *   out[s, r, h*dh + e] = sigmoid(g[s, r, h*dh + e])
 *                         * sum_t softmax_t(scale * q[s, r].k[t, r]) v[t, r][e]
 *   m    [Ns, Nr, Cm]      w* [Cm, H*dh] each      (no pair bias)
 *   out  [Ns, Nr, H*dh]
 * Workspace, scale, supported shapes and errors as evoformer_gated_attn_fwd;
 * the workspace size is the same (evoformer_workspace_bytes).  With Cm = 256
 * and Ns <= 256, one kernel keeps the projections on chip and leaves the
 * workspace untouched (it is still required). */
int evoformer_col_gated_attn_fwd(const void* m, const void* wq, const void* wk, const void* wv, const void* wg,
                                 void* out, void* workspace, size_t workspace_bytes, int Ns, int Nr, int Cm, int H,
                                 int dh, float scale, hipStream_t stream);

/* Human-readable name of a status code (static storage; never NULL). */
const char* av_status_string(int status);

/* ABI version of this header; bumped when a signature or struct changes. */
#define AV_ABI_VERSION 4
int av_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTNVAR_H */
