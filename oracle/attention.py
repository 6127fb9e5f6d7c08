"""Plain fp64 CPU oracle for the attention variants.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import this module.  The GPU path
(``attention_variants_amd``) never imports it, and it imports nothing from
the GPU path: the two share only the seeded generators in ``workloads``.

What it computes is the plain definition of each variant, in float64, with a
two-pass stable softmax and explicit boolean mask matrices -- no tiling, no
online rescaling, no fusion.  The Flashlight pages describe kernels that reach
exactly this result over the reals (talk notes "Flashlight: PyTorch Compiler
Extensions to Accelerate Attention Variants", section "Compiler design",
2. Algebraic transformation and 3. Dimension demotion: softmax(Q K^T / sqrt(d_k))
computed by one fused kernel), and warn that the online form is not bitwise
equal to the two-pass form in floating point (section "Comparison with
FlexAttention", precision item).  Every reading of a point the pages leave
open is stated where it is used; the same list is kept with the design notes.

Inputs are float64 arrays (the bf16 values widened exactly).  Shapes:
  q [B, Hq, Sq, D], k [B, Hkv, Skv, D], v [B, Hkv, Skv, Dv]
  out [B, Hq, R, Dv] with R = number of computed query rows, lse [B, Hq, R].
"""

from __future__ import annotations

import math

import numpy as np

SCORE_MODS = ("none", "alibi", "softcap")
DATA_SCORE_MODS = ("bias",)  # modifiers that read a tensor besides Q and K
MASKS = ("none", "causal", "sliding_window", "prefix_lm", "document")


# --------------------------------------------------------------------------
# Step 1: scores.  S = scale * Q K^T (talk notes, "Compiler design",
# 3. Dimension demotion, which names softmax(Q K^T / sqrt(d_k)); the scale
# reading is 1/sqrt(D)).
# --------------------------------------------------------------------------
def raw_scores(q_rows: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """``scale * q_rows @ k^T`` in float64.  q_rows [R, D], k [Skv, D] -> [R, Skv]."""
    return scale * (q_rows @ k.T)


# --------------------------------------------------------------------------
# Step 2: score modifiers (talk notes, section "Evaluation: FlexAttention-
# supported variants", which lists ALiBi and tanh soft-capping as per-element
# score modifiers; the notes' background section describes score_mod as an
# element-wise transform of the score).  The additive bias tensor is the
# data-dependent modifier: the notes' abstract sets Flashlight apart by its
# support of data-dependent attention formulations, of which a score term read
# from a tensor (the Evoformer's pair bias) is the plainest.
# --------------------------------------------------------------------------
def alibi_slope(h: int, Hq: int, max_bias: float = 8.0) -> float:
    """Slope of 0-based query head ``h``: 2^(-max_bias * (h+1) / Hq).

    Reading: the geometric ALiBi sequence 2^(-8 h'/H) with h' = 1..H.
    """
    return 2.0 ** (-max_bias * (h + 1) / Hq)


def apply_score_mod(s, score_mod, rows, cols, *, slope=0.0, softcap=20.0, bias=None):
    """Element-wise score modifier on the *scaled* score.

    alibi:   s + slope * (j - i)        (reading: linear in signed distance,
                                         also for j > i when no mask is set)
    softcap: cap * tanh(s / cap)
    bias:    s + bias[i, j]             (a data-dependent modifier: the value
                                         comes from a tensor; ``bias`` holds the
                                         rows of this (batch, head), [R, Skv])
    """
    if score_mod == "none":
        return s
    if score_mod == "bias":
        return s + np.asarray(bias, dtype=np.float64)
    if score_mod == "alibi":
        return s + slope * (cols[None, :].astype(np.float64) - rows[:, None].astype(np.float64))
    if score_mod == "softcap":
        return softcap * np.tanh(s / softcap)
    raise ValueError(f"unknown score_mod {score_mod!r}")


# --------------------------------------------------------------------------
# Step 3: explicit boolean masks (the seven variants of the talk notes,
# section "Evaluation: FlexAttention-supported variants").  Readings:
#   causal          j <= i
#   sliding_window  0 <= i - j < window        (window keys, self included)
#   prefix_lm       j < prefix_len  or  j <= i
#   document        doc[i] == doc[j]           (not causal)
# --------------------------------------------------------------------------
def allowed_matrix(mask, rows, Skv, *, window=256, prefix_len=0, doc_row=None):
    i = rows[:, None].astype(np.int64)
    j = np.arange(Skv, dtype=np.int64)[None, :]
    if mask == "none":
        return np.ones((len(rows), Skv), dtype=bool)
    if mask == "causal":
        return j <= i
    if mask == "sliding_window":
        d = i - j
        return (d >= 0) & (d < window)
    if mask == "prefix_lm":
        return (j < prefix_len) | (j <= i)
    if mask == "document":
        doc_row = np.asarray(doc_row)
        return doc_row[rows][:, None] == doc_row[None, :]
    raise ValueError(f"unknown mask {mask!r}")


# --------------------------------------------------------------------------
# Step 4: two-pass stable softmax over the allowed entries (Spanish summary
# "Resumen Tecnico: FLASHLIGHT", section "Metodologia", item 3, and talk notes
# "Compiler design", 2. Algebraic transformation: pass one takes the row max,
# pass two sums exp(x - max)).  A row with no allowed entry gives p = 0 and
# lse = -inf (reading; no such row occurs in the benchmark shapes).
# --------------------------------------------------------------------------
def softmax_two_pass(s: np.ndarray, allowed: np.ndarray):
    """Return (p, lse) for scores ``s`` [R, N] restricted to ``allowed``."""
    t = np.where(allowed, s, -np.inf)
    has = allowed.any(axis=1)
    m = np.where(has, t.max(axis=1, initial=-np.inf), 0.0)  # pass 1: row max
    e = np.where(allowed, np.exp(t - m[:, None]), 0.0)  # pass 2: exp(x - max)
    l = e.sum(axis=1)
    p = e / np.where(l > 0, l, 1.0)[:, None]
    lse = np.where(has, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return p, lse


def _head_probs(qh, kh, rows, *, scale, score_mod, mask, slope, softcap, window, prefix_len, doc_row,
                q_offset=0, bias_rows=None):
    s = raw_scores(qh[rows], kh, scale)
    pos = rows + q_offset  # absolute position of each query row
    s = apply_score_mod(s, score_mod, pos, np.arange(kh.shape[0]), slope=slope, softcap=softcap, bias=bias_rows)
    a = allowed_matrix(mask, pos, kh.shape[0], window=window, prefix_len=prefix_len, doc_row=doc_row)
    return softmax_two_pass(s, a)


def attention(
    q,
    k,
    v,
    *,
    score_mod: str = "none",
    mask: str = "none",
    scale: float | None = None,
    softcap: float = 20.0,
    alibi_max_bias: float = 8.0,
    window: int = 256,
    prefix_len: int = 0,
    doc_id=None,
    rows=None,
    row_block: int = 1024,
    q_offset: int = 0,
    bias=None,
):
    """out = softmax(mask(score_mod(scale * Q K^T))) V, per (batch, query head).

    ``score_mod="bias"`` adds ``bias[b', h', i, j]`` (shape [Bb, Hb, Sq, Skv]
    with Bb in {1, B} and Hb in {1, Hq}; a size-1 axis is shared by every
    batch or head) to the scaled score before the mask.

    GQA reading: query head ``hq`` reads key/value head ``hq // (Hq // Hkv)``
    (contiguous groups).  ``rows`` restricts the computation to a subset of
    query rows (each row is independent, so a sampled row is exact).
    ``q_offset`` is the absolute position of query row 0 (ALiBi distances and
    masks use row + q_offset).  Decoding reading: the Sq queries are the last
    Sq positions of the Skv keys, q_offset = Skv - Sq; with a mask the queries
    must end at the last key.
    Returns ``(out, lse)``; ``lse`` is natural-log ``m + ln l`` of the scores
    after score_mod and mask.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Sq, D = q.shape
    _, Hkv, Skv, _ = k.shape
    Dv = v.shape[-1]
    if score_mod not in SCORE_MODS + DATA_SCORE_MODS:
        raise ValueError(score_mod)
    if score_mod == "bias":
        bias = np.asarray(bias, dtype=np.float64)
        if bias.ndim != 4 or bias.shape[0] not in (1, B) or bias.shape[1] not in (1, Hq) \
                or bias.shape[2:] != (Sq, Skv):
            raise ValueError("bias must be [1 or B, 1 or Hq, Sq, Skv]")
    if mask not in MASKS:
        raise ValueError(mask)
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if mask != "none" and Sq + q_offset != Skv:
        raise ValueError("masks need the queries to end at the last key (Sq + q_offset == Skv)")
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    rows = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    R = len(rows)
    out = np.zeros((B, Hq, R, Dv))
    lse = np.zeros((B, Hq, R))
    for b in range(B):
        doc_row = None if doc_id is None else np.asarray(doc_id)[b]
        for hq in range(Hq):
            hk = hq // g
            slope = alibi_slope(hq, Hq, alibi_max_bias)
            for r0 in range(0, R, row_block):
                rr = rows[r0 : r0 + row_block]
                br = None
                if score_mod == "bias":
                    br = bias[b if bias.shape[0] > 1 else 0, hq if bias.shape[1] > 1 else 0][rr]
                p, l_ = _head_probs(
                    q[b, hq], k[b, hk], rr,
                    scale=scale, score_mod=score_mod, mask=mask, slope=slope,
                    softcap=softcap, window=window, prefix_len=prefix_len, doc_row=doc_row,
                    q_offset=q_offset, bias_rows=br,
                )
                out[b, hq, r0 : r0 + len(rr)] = p @ v[b, hk]
                lse[b, hq, r0 : r0 + len(rr)] = l_
    return out, lse


def paged_decode_attention(q, k_cache, v_cache, block_table, seq_lens, *, page_size: int,
                           score_mod: str = "none", mask: str = "none", scale: float | None = None,
                           softcap: float = 20.0, alibi_max_bias: float = 8.0):
    """Decoding against a paged key/value cache.

    The pages' serving workload runs under vLLM (talk notes, end-to-end
    section), whose key/value cache is paged.  Reading: sequence b holds
    seq_lens[b] keys; key j lives in page block_table[b, j // page_size], slot
    j % page_size, of a cache laid out [num_pages, Hkv, page_size, D]; its Sq
    queries are its last Sq positions.  Gather each sequence's keys, then the
    plain definition (``attention`` with q_offset = seq_lens[b] - Sq).

    q [B, Hq, Sq, D] -> (out [B, Hq, Sq, D], lse [B, Hq, Sq]).
    """
    q = np.asarray(q, dtype=np.float64)
    kc = np.asarray(k_cache, dtype=np.float64)
    vc = np.asarray(v_cache, dtype=np.float64)
    block_table = np.asarray(block_table)
    B, Hq, Sq, D = q.shape
    out = np.zeros((B, Hq, Sq, vc.shape[-1]))
    lse = np.zeros((B, Hq, Sq))
    for b in range(B):
        n = int(seq_lens[b])
        j = np.arange(n)
        pages = block_table[b, j // page_size]
        kb = kc[pages, :, j % page_size].transpose(1, 0, 2)[None]  # [1, Hkv, n, D]
        vb = vc[pages, :, j % page_size].transpose(1, 0, 2)[None]
        o, l_ = attention(q[b:b + 1], kb, vb, score_mod=score_mod, mask=mask, scale=scale, softcap=softcap,
                          alibi_max_bias=alibi_max_bias, q_offset=n - Sq)
        out[b], lse[b] = o[0], l_[0]
    return out, lse


def attention_backward(q, k, v, dout, *, score_mod: str = "none", mask: str = "none", scale: float | None = None,
                       softcap: float = 20.0, alibi_max_bias: float = 8.0, window: int = 256, prefix_len: int = 0,
                       doc_id=None):
    """Gradients of ``attention`` (output only, not lse) for an upstream dout.

    The pages name training as the extension of their method (talk notes,
    "Background and motivation": attention is a bottleneck of training and
    inference).  This is the chain rule of the plain definition, in float64:
      t = mod(scale * q k^T), masked entries -inf;  p = softmax(t);  o = p v
      dv = p^T dout                     (summed over the query heads of a KV head)
      dp = dout v^T;  dt = p * (dp - rowsum(dp * p))
      ds = dt * mod'(scale * q k^T)     (softcap: 1 - tanh(s/cap)^2; ALiBi and none: 1)
      dq = scale * ds k;  dk = scale * ds^T q   (dk summed like dv)
    Returns (dq [B,Hq,Sq,D], dk [B,Hkv,Skv,D], dv [B,Hkv,Skv,Dv]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    B, Hq, Sq, D = q.shape
    _, Hkv, Skv, _ = k.shape
    if mask != "none" and Sq != Skv:
        raise ValueError("masks need Sq == Skv")
    g = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    rows = np.arange(Sq)
    cols = np.arange(Skv)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        doc_row = None if doc_id is None else np.asarray(doc_id)[b]
        for hq in range(Hq):
            hk = hq // g
            s = raw_scores(q[b, hq], k[b, hk], scale)
            slope = alibi_slope(hq, Hq, alibi_max_bias)
            t = apply_score_mod(s, score_mod, rows, cols, slope=slope, softcap=softcap)
            a = allowed_matrix(mask, rows, Skv, window=window, prefix_len=prefix_len, doc_row=doc_row)
            p, _ = softmax_two_pass(t, a)
            dv[b, hk] += p.T @ dout[b, hq]
            dp = dout[b, hq] @ v[b, hk].T
            dt = p * (dp - np.sum(dp * p, axis=1, keepdims=True))
            if score_mod == "softcap":
                dt = dt * (1.0 - np.tanh(s / softcap) ** 2)
            dq[b, hq] = scale * (dt @ k[b, hk])
            dk[b, hk] += scale * (dt.T @ q[b, hq])
    return dq, dk, dv


# --------------------------------------------------------------------------
# Differential attention.  The pages name it among the variants that
# templates cannot express (talk notes, "Background and motivation" and
# "Evaluation: complex attention variants"; 32 heads x 64 and 16 heads x 128)
# but do not define it.  Reading used here: Q and K hold two halves of width
# Dh; each half gives its own causal softmax with scale 1/sqrt(Dh); the
# output is (P1 - lambda * P2) V with a constant lambda (0.8 in the benchmark
# shape), V of width Dv shared by both halves.  No group norm, no
# (1 - lambda_init) factor, no learned lambda re-parameterisation.
# --------------------------------------------------------------------------
def diff_attention(q, k, v, *, lam: float = 0.8, scale: float | None = None,
                   causal: bool = True, rows=None, row_block: int = 1024):
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, S, D2 = q.shape
    if D2 % 2:
        raise ValueError("Q/K width must be even (two halves)")
    Dh = D2 // 2
    Dv = v.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(Dh)
    rows = np.arange(S) if rows is None else np.asarray(rows, dtype=np.int64)
    mask = "causal" if causal else "none"
    out = np.zeros((B, H, len(rows), Dv))
    for b in range(B):
        for h in range(H):
            for r0 in range(0, len(rows), row_block):
                rr = rows[r0 : r0 + row_block]
                kw = dict(scale=scale, score_mod="none", mask=mask, slope=0.0, softcap=1.0,
                          window=0, prefix_len=0, doc_row=None)
                p1, _ = _head_probs(q[b, h, :, :Dh], k[b, h, :, :Dh], rr, **kw)
                p2, _ = _head_probs(q[b, h, :, Dh:], k[b, h, :, Dh:], rr, **kw)
                out[b, h, r0 : r0 + len(rr)] = (p1 - lam * p2) @ v[b, h]
    return out


# --------------------------------------------------------------------------
# The full differential-attention head.  The pages name DiffTransformer among
# the flexible attention models that motivate the work (talk notes, "Related
# work") and benchmark only its attention core.  The head around that core is
# taken from the published Differential Transformer (Ye et al., 2024, the
# sections on differential attention and on its multi-head form):
#   lambda         = exp(lq1 . lk1) - exp(lq2 . lk2) + lambda_init
#   A              = (softmax(s Q1 K1^T) - lambda softmax(s Q2 K2^T)) V
#   y[i, e]        = (1 - lambda_init) * gamma[e] * A[i, e] / sqrt(mean_e' A[i, e']^2 + eps)
#   lambda_init(l) = 0.8 - 0.6 exp(-0.3 (l - 1)),   l = 1-based layer index
# The per-head normalisation is RMSNorm over the Dv channels of each row with
# a per-channel weight gamma (ones when absent).  The output projection over
# the concatenated heads is a plain GEMM and not part of the head.
# --------------------------------------------------------------------------
def diff_lambda_init(layer: int) -> float:
    return 0.8 - 0.6 * math.exp(-0.3 * (layer - 1))


def diff_lambda(lq1, lk1, lq2, lk2, lambda_init: float) -> float:
    d1 = float(np.dot(np.asarray(lq1, dtype=np.float64), np.asarray(lk1, dtype=np.float64)))
    d2 = float(np.dot(np.asarray(lq2, dtype=np.float64), np.asarray(lk2, dtype=np.float64)))
    return math.exp(d1) - math.exp(d2) + lambda_init


def diff_head(q, k, v, lq1, lk1, lq2, lk2, *, lambda_init: float, gamma=None, eps: float = 1e-5,
              scale: float | None = None, causal: bool = True, rows=None):
    lam = diff_lambda(lq1, lk1, lq2, lk2, lambda_init)
    a = diff_attention(q, k, v, lam=lam, scale=scale, causal=causal, rows=rows)
    Dv = a.shape[-1]
    g = np.ones(Dv) if gamma is None else np.asarray(gamma, dtype=np.float64)
    rms = np.sqrt(np.mean(a * a, axis=-1, keepdims=True) + eps)
    return (1.0 - lambda_init) * g * (a / rms)


# --------------------------------------------------------------------------
# Evoformer row-wise gated self-attention with pair bias.  The pages name it
# (talk notes, "Background and motivation", "Evaluation: complex attention
# variants", and the AlphaFold2 end-to-end section: 8 heads x 32) without a
# formula.  Reading used here, per MSA sequence s and head h:
#   q, k, v, g = m Wq, m Wk, m Wv, m Wg          (no bias terms, no LayerNorm)
#   o_i = sum_j softmax_j(q_i . k_j * scale + bias[h, i, j]) v_j
#   out[s, i, h*dh + e] = sigmoid(g[s, i, h*dh + e]) * o_i[e]
# "Row-wise" = attention across residues within one sequence; the pair bias
# is shared by all sequences.  No output projection.
# --------------------------------------------------------------------------
def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def evoformer_projections(m, wq, wk, wv, wg):
    m = np.asarray(m, dtype=np.float64)
    return tuple(m @ np.asarray(w, dtype=np.float64) for w in (wq, wk, wv, wg))


def evoformer_row_gated_attention(m, wq, wk, wv, wg, bias, *, H: int, dh: int,
                                  scale: float | None = None, rows=None, seqs=None):
    """m [Ns, Nr, Cm], w* [Cm, H*dh], bias [H, Nr, Nr] -> out [len(seqs), len(rows), H*dh]."""
    m = np.asarray(m, dtype=np.float64)
    bias = np.asarray(bias, dtype=np.float64)
    Ns, Nr, _ = m.shape
    if scale is None:
        scale = 1.0 / math.sqrt(dh)
    rows = np.arange(Nr) if rows is None else np.asarray(rows, dtype=np.int64)
    seqs = np.arange(Ns) if seqs is None else np.asarray(seqs, dtype=np.int64)
    ms = m[seqs]
    q, k, v, g = evoformer_projections(ms, wq, wk, wv, wg)
    out = np.zeros((len(seqs), len(rows), H * dh))
    everything = np.ones((len(rows), Nr), dtype=bool)
    for si in range(len(seqs)):
        for h in range(H):
            c = slice(h * dh, (h + 1) * dh)
            s = raw_scores(q[si, rows, c], k[si, :, c], scale) + bias[h][rows]
            p, _ = softmax_two_pass(s, everything)
            out[si, :, c] = sigmoid(g[si, rows, c]) * (p @ v[si, :, c])
    return out


def evoformer_col_gated_attention(m, wq, wk, wv, wg, *, H: int, dh: int,
                                  scale: float | None = None, cols=None, seqs=None):
    """Column-wise gated self-attention of the Evoformer MSA stack.

    The pages name the row- and column-wise gated self-attention of
    AlphaFold2's Evoformer together (talk notes "Flashlight: PyTorch Compiler
    Extensions to Accelerate Attention Variants", background and the
    complex-variant evaluation) and give no formula.  Reading: the same four
    projections of the MSA representation as the row-wise form; for every
    residue column r and head h, softmax attention over the N_seq sequences
    of that column (no pair bias), gated by sigmoid(m Wg), channels head-major.

    m [Ns, Nr, Cm], w* [Cm, H*dh] -> out [len(seqs), len(cols), H*dh].
    """
    m = np.asarray(m, dtype=np.float64)
    Ns, Nr, _ = m.shape
    if scale is None:
        scale = 1.0 / math.sqrt(dh)
    cols = np.arange(Nr) if cols is None else np.asarray(cols, dtype=np.int64)
    seqs = np.arange(Ns) if seqs is None else np.asarray(seqs, dtype=np.int64)
    mc = m[:, cols]                                   # every sequence of the chosen columns
    q, k, v, g = evoformer_projections(mc, wq, wk, wv, wg)
    out = np.zeros((len(seqs), len(cols), H * dh))
    everything = np.ones((len(seqs), Ns), dtype=bool)
    for ci in range(len(cols)):
        for h in range(H):
            c = slice(h * dh, (h + 1) * dh)
            s = raw_scores(q[seqs, ci, c], k[:, ci, c], scale)
            p, _ = softmax_two_pass(s, everything)
            out[:, ci, c] = sigmoid(g[seqs, ci, c]) * (p @ v[:, ci, c])
    return out

