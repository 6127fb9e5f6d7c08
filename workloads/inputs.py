"""Seeded input generators (no attention arithmetic lives here).

Every tensor is drawn in float32 from ``numpy.random.default_rng(seed)``,
then rounded to bfloat16 with round-to-nearest-even.  The result is returned
as raw ``uint16`` bit patterns so that the fp64 oracle and the GPU consume
exactly the same values: the oracle widens the bits to float64 (exact), the
GPU receives the bits as ``torch.bfloat16``.

Shapes and value distributions follow the synthetic shape sweeps described
on the Flashlight talk notes ("Flashlight: PyTorch Compiler Extensions to
Accelerate Attention Variants", section "Evaluation: FlexAttention-supported
variants"): 16 heads (or 16 query / 2 key-value heads), head dim 64, sequence
lengths 512..16k with the batch chosen so that every shape holds 16k tokens.
The pages print no value distribution; standard normal inputs are this
package's choice.
"""

from __future__ import annotations

import numpy as np

# Fixed seeds, one per tensor role.  The pages give none; these are ours and
# are recorded with every result.
SEEDS = {
    "q": 1,
    "k": 2,
    "v": 3,
    "doc": 4,
    "m": 11,
    "wq": 12,
    "wk": 13,
    "wv": 14,
    "wg": 15,
    "bias": 16,
}


def bf16_bits_from_f32(x) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    bias = ((u >> 16) & 1) + 0x7FFF
    r = ((u + bias) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r = np.where(nan, np.uint16(0x7FC0), r)
    return r


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Widen bfloat16 bit patterns to float64 (exact)."""
    return bf16_bits_to_f32(bits).astype(np.float64)


def normal_bf16(seed: int, shape, std: float = 1.0) -> np.ndarray:
    """``std * N(0,1)`` drawn in float32 from ``seed``, rounded to bf16 bits."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=tuple(shape), dtype=np.float32)
    if std != 1.0:
        x = (x * np.float32(std)).astype(np.float32)
    return bf16_bits_from_f32(x)


def doc_lengths(seed: int, B: int, S: int, lo: int = 64, hi: int | None = None):
    """Per batch row, split ``S`` tokens into documents of seeded random length.

    Lengths are uniform integers in ``[lo, hi]`` (inclusive; ``hi`` defaults to
    ``S // 2``); the last document is cut to fill the remainder, so it may be
    shorter than ``lo``.  One generator is consumed row after row.
    """
    if hi is None:
        hi = S // 2
    hi = max(hi, lo)
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(B):
        lens = []
        pos = 0
        while pos < S:
            L = int(rng.integers(lo, hi, endpoint=True))
            L = min(L, S - pos)
            lens.append(L)
            pos += L
        out.append(lens)
    return out


def doc_ids(seed: int, B: int, S: int, lo: int = 64, hi: int | None = None) -> np.ndarray:
    """``[B, S]`` int32 document index per token (non-decreasing along each row)."""
    ids = np.zeros((B, S), dtype=np.int32)
    for b, lens in enumerate(doc_lengths(seed, B, S, lo, hi)):
        ids[b] = np.repeat(np.arange(len(lens), dtype=np.int32), lens)
    return ids


def attention_inputs(B, Hq, Hkv, Sq, Skv, D, Dv=None, seeds=(1, 2, 3)):
    """Q ``[B,Hq,Sq,D]``, K ``[B,Hkv,Skv,D]``, V ``[B,Hkv,Skv,Dv]`` as bf16 bits, N(0,1)."""
    Dv = D if Dv is None else Dv
    sq, sk, sv = seeds
    return {
        "q": normal_bf16(sq, (B, Hq, Sq, D)),
        "k": normal_bf16(sk, (B, Hkv, Skv, D)),
        "v": normal_bf16(sv, (B, Hkv, Skv, Dv)),
    }


def diff_inputs(B, H, S, Dh=64, Dv=128, seeds=(1, 2, 3)):
    """Differential attention inputs: Q, K ``[B,H,S,2*Dh]`` (two halves), V ``[B,H,S,Dv]``."""
    sq, sk, sv = seeds
    return {
        "q": normal_bf16(sq, (B, H, S, 2 * Dh)),
        "k": normal_bf16(sk, (B, H, S, 2 * Dh)),
        "v": normal_bf16(sv, (B, H, S, Dv)),
    }


def diff_head_params(Dh=64, Dv=128, seed=17):
    """Parameters of a differential-attention head, float32: the four lambda
    vectors ``[Dh]`` ~ N(0, 0.1^2) (the published initialisation) and a
    per-channel norm weight ``gamma [Dv]`` ~ N(1, 0.1^2) (ones at
    initialisation; drawn here so that every channel's weight matters)."""
    rng = np.random.default_rng(seed)
    out = {n: (0.1 * rng.standard_normal(Dh)).astype(np.float32) for n in ("lq1", "lk1", "lq2", "lk2")}
    out["gamma"] = (1.0 + 0.1 * rng.standard_normal(Dv)).astype(np.float32)
    return out


def evoformer_inputs(Ns, Nr, Cm=256, H=8, dh=32, seeds=None):
    """MSA activations ``m [Ns,Nr,Cm]`` ~ N(0,1); four projection weights
    ``[Cm, H*dh]`` ~ N(0, 1/Cm) (variance 1/Cm); pair bias ``[H,Nr,Nr]`` ~ N(0,1)."""
    s = dict(SEEDS)
    if seeds:
        s.update(seeds)
    wstd = 1.0 / np.sqrt(Cm)
    return {
        "m": normal_bf16(s["m"], (Ns, Nr, Cm)),
        "wq": normal_bf16(s["wq"], (Cm, H * dh), wstd),
        "wk": normal_bf16(s["wk"], (Cm, H * dh), wstd),
        "wv": normal_bf16(s["wv"], (Cm, H * dh), wstd),
        "wg": normal_bf16(s["wg"], (Cm, H * dh), wstd),
        "bias": normal_bf16(s["bias"], (H, Nr, Nr)),
    }
