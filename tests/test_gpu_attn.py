"""GPU parity of ``attn_fwd`` against the fp64 oracle (called through the C ABI).

Small shapes are checked on every row; the benchmark shapes (16k tokens,
16 heads, D = 64) are checked on sampled rows, which is exact because rows
are independent.  Gate: |gpu - oracle| <= 1e-2 + 1e-2 |oracle| elementwise;
LSE within 1e-3 (absolute) + 1e-5 (relative): calls that ask for lse sum the
fp32 exponentials.  Closed-form cases use far tighter bounds.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import inputs as wi

from .gpu_util import (assert_close, assert_rms_rel, canary_empty, canary_intact, f64, sample_rows,
                       sample_rows_at_least, to_dev)

pytestmark = pytest.mark.gpu

SCORE_MODS = ("none", "alibi", "softcap")
LSE_ATOL = 1e-3  # the row sums add fp32 exponentials when lse is requested
MASKS = ("none", "causal", "sliding_window", "prefix_lm", "document")


def _params(mask, S, seed_doc=4, doc_lo=64):
    kw = {}
    if mask == "sliding_window":
        kw["window"] = 256 if S >= 1024 else max(1, S // 3)
    if mask == "prefix_lm":
        kw["prefix_len"] = S // 4
    if mask == "document":
        lo = doc_lo if S >= 256 else 4
        kw["doc_id"] = wi.doc_ids(seed_doc, 1, S, lo=lo)  # replaced per batch below
    return kw


def _run(av, B, Hq, Hkv, S, D, score_mod, mask, rows=None, seed=(1, 2, 3), Skv=None, check_lse=True,
         canary=True, softcap=20.0, batch=None, rms_check=False):
    """GPU on the whole shape; the oracle on `rows` (default all) of every
    batch entry, or of batch entry `batch` only (batch entries are independent)."""
    Skv = S if Skv is None else Skv
    x = wi.attention_inputs(B, Hq, Hkv, S, Skv, D, seeds=seed)
    kw = _params(mask, S)
    if mask == "document":
        kw["doc_id"] = wi.doc_ids(4, B, S, lo=64 if S >= 256 else 4)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    dev_kw = dict(kw)
    if "doc_id" in dev_kw:
        dev_kw["doc_id"] = torch.from_numpy(dev_kw["doc_id"]).cuda()
    out, big = canary_empty((B, Hq, S, D), torch.bfloat16)
    lse, bigl = canary_empty((B, Hq, S), torch.float32)
    av.attn_fwd(q, k, v, score_mod=score_mod, mask=mask, softcap=softcap, out=out, lse=lse, **dev_kw)
    torch.cuda.synchronize()
    if canary:
        assert canary_intact(big, out.numel()), "write past the end of out"
        assert canary_intact(bigl, lse.numel()), "write past the end of lse"
    got = out.float().cpu().numpy()
    got_lse = lse.cpu().numpy()
    bs = slice(None) if batch is None else slice(batch, batch + 1)
    okw = dict(kw)
    if "doc_id" in okw:
        okw["doc_id"] = okw["doc_id"][bs]
    ref, ref_lse = oracle.attention(f64(x["q"][bs]), f64(x["k"][bs]), f64(x["v"][bs]), score_mod=score_mod,
                                    mask=mask, softcap=softcap, rows=rows, **okw)
    got, got_lse = got[bs], got_lse[bs]
    if rows is not None:
        got, got_lse = got[:, :, rows], got_lse[:, :, rows]
    what = f"{score_mod}/{mask} B{B} Hq{Hq} Hkv{Hkv} S{S} Skv{Skv} D{D}"
    err = assert_close(got, ref, what)
    if check_lse:
        assert_close(got_lse, ref_lse, what + " lse", atol=LSE_ATOL, rtol=1e-5)
    if rms_check:
        assert_rms_rel(got, ref, what)
    return err, out


@pytest.mark.parametrize("score_mod", SCORE_MODS)
@pytest.mark.parametrize("mask", MASKS)
def test_small_all_rows(gpu_lib, score_mod, mask):
    for (B, Hq, Hkv, S, D) in ((1, 2, 2, 128, 64), (2, 4, 2, 100, 64), (1, 4, 1, 300, 64), (1, 2, 2, 17, 64)):
        _run(gpu_lib, B, Hq, Hkv, S, D, score_mod, mask)


@pytest.mark.parametrize("D", [32, 128])
@pytest.mark.parametrize("mask", ["none", "causal", "document"])
def test_other_head_dims(gpu_lib, D, mask):
    _run(gpu_lib, 2, 4, 2, 129, D, "softcap", mask)
    _run(gpu_lib, 1, 2, 2, 200, D, "alibi", mask)


def test_tiny_config(gpu_lib):
    """Vanilla, B=1, H=2, S=128, D=64, scale 1/8."""
    err, _ = _run(gpu_lib, 1, 2, 2, 128, 64, "none", "none")
    assert err < 5e-3


@pytest.mark.parametrize("S", [1, 2, 31, 63, 64, 65, 127, 129, 255, 257])
def test_ragged_lengths(gpu_lib, S):
    for mask in ("none", "causal", "sliding_window"):
        _run(gpu_lib, 1, 2, 1, S, 64, "none", mask)


def test_cross_attention_lengths(gpu_lib):
    for Sq, Skv in ((1, 300), (100, 7), (129, 1000), (64, 65)):
        _run(gpu_lib, 1, 2, 2, Sq, 64, "softcap", "none", Skv=Skv)


def test_empty_kv_gives_zero_rows(gpu_lib):
    q = torch.zeros(1, 2, 5, 64, dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros(1, 2, 0, 64, dtype=torch.bfloat16, device="cuda")
    out, lse = gpu_lib.attn_fwd(q, kv, kv, return_lse=True)
    torch.cuda.synchronize()
    assert torch.all(out == 0).item()
    assert torch.all(torch.isneginf(lse)).item()


def test_closed_forms_on_gpu(gpu_lib):
    """Exact answers: uniform scores give the mean of V over the visible set;
    causal row 0 is V[0]; a window of 1 and one-token documents give V."""
    B, H, S, D = 1, 2, 200, 64
    x = wi.attention_inputs(B, H, H, S, S, D)
    k, v = to_dev(x["k"]), to_dev(x["v"])
    q0 = torch.zeros(B, H, S, D, dtype=torch.bfloat16, device="cuda")
    vv = f64(x["v"])
    out = gpu_lib.attn_fwd(q0, k, v, mask="causal").float().cpu().numpy()
    ref = np.cumsum(vv, axis=2) / np.arange(1, S + 1)[None, None, :, None]
    assert np.all(np.abs(out - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)  # bf16 output rounding only
    q = to_dev(x["q"])
    out = gpu_lib.attn_fwd(q, k, v, mask="causal")
    assert torch.equal(out[:, :, 0], v[:, :, 0])
    out = gpu_lib.attn_fwd(q, k, v, mask="sliding_window", window=1)
    assert torch.equal(out, v)
    doc = torch.arange(S, dtype=torch.int32, device="cuda")[None]
    out = gpu_lib.attn_fwd(q, k, v, mask="document", doc_id=doc)
    assert torch.equal(out, v)
    out = gpu_lib.attn_fwd(q0, k, v, mask="none").float().cpu().numpy()
    ref = np.broadcast_to(vv.mean(axis=2, keepdims=True), out.shape)
    assert np.all(np.abs(out - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)


def test_reductions_on_gpu(gpu_lib):
    """GQA equals MHA on repeated K/V (bitwise); softcap with a huge cap equals vanilla."""
    B, Hq, Hkv, S, D = 2, 8, 2, 300, 64
    x = wi.attention_inputs(B, Hq, Hkv, S, S, D)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    for mask in ("none", "causal", "prefix_lm"):
        a = gpu_lib.attn_fwd(q, k, v, mask=mask, prefix_len=75)
        b = gpu_lib.attn_fwd(q, k.repeat_interleave(4, dim=1).contiguous(), v.repeat_interleave(4, dim=1).contiguous(),
                             mask=mask, prefix_len=75)
        assert torch.equal(a, b), mask
    a = gpu_lib.attn_fwd(q, k, v).float()
    c = gpu_lib.attn_fwd(q, k, v, score_mod="softcap", softcap=1e3).float()
    assert (a - c).abs().max().item() < 2e-2


def _ramp_inputs(B, H, S, D, q_val, k_step, descending=False):
    """q = q_val everywhere; key j = (j * k_step) in every column (bf16-rounded),
    so raw scores grow (or shrink) linearly along the row; V random."""
    x = wi.attention_inputs(B, H, H, S, S, D)
    j = np.arange(S, dtype=np.float32)
    if descending:
        j = j[::-1].copy()
    krow = wi.bf16_bits_from_f32(j * np.float32(k_step))
    k = np.broadcast_to(krow[None, None, :, None], (B, H, S, D)).copy()
    q = np.broadcast_to(wi.bf16_bits_from_f32(np.float32(q_val)), (B, H, S, D)).copy()
    return q, k, x["v"]


@pytest.mark.parametrize("descending", [False, True])
@pytest.mark.parametrize("score_mod", SCORE_MODS)
def test_rising_and_falling_scores(gpu_lib, score_mod, descending):
    """Scores that climb by ~185 (log2 units) per 64-key tile force the
    exponent reference up on every tile (without the raise the exponentials
    would overflow); falling scores keep the first tile's reference."""
    B, H, S, D = 1, 2, 300, 64
    q, k, v = _ramp_inputs(B, H, S, D, 8.0, 1.0 / 32, descending)
    for mask in ("none", "causal"):
        out, lse = gpu_lib.attn_fwd(to_dev(q), to_dev(k), to_dev(v), score_mod=score_mod, mask=mask, return_lse=True)
        torch.cuda.synchronize()
        ref, ref_lse = oracle.attention(f64(q), f64(k), f64(v), score_mod=score_mod, mask=mask)
        what = f"ramp {score_mod}/{mask} desc={descending}"
        assert_close(out.float().cpu().numpy(), ref, what)
        assert_close(lse.cpu().numpy(), ref_lse, what + " lse", atol=LSE_ATOL, rtol=1e-5)


def test_deterministic(gpu_lib):
    B, H, S, D = 2, 4, 1000, 64
    x = wi.attention_inputs(B, H, H, S, S, D)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    doc = torch.from_numpy(wi.doc_ids(4, B, S)).cuda()
    for sm, mk in (("alibi", "causal"), ("softcap", "document"), ("none", "none")):
        r = [gpu_lib.attn_fwd(q, k, v, score_mod=sm, mask=mk, doc_id=doc if mk == "document" else None)
             for _ in range(3)]
        assert torch.equal(r[0], r[1]) and torch.equal(r[1], r[2])


# ------------------------------------------------------------- benchmark shapes
BENCH_VARIANTS = ([(sm, "none", 16) for sm in SCORE_MODS]
                  + [("none", mk, hkv) for mk in MASKS[1:] for hkv in (16, 2)])


@pytest.mark.parametrize("S", [512, 1024, 2048])
@pytest.mark.parametrize("score_mod,mask,Hkv", BENCH_VARIANTS)
def test_benchmark_shapes_all_rows(gpu_lib, S, score_mod, mask, Hkv):
    """The benchmark shapes up to S = 2k (16k tokens, 16 query heads): every
    row of every head, for the last batch entry (entries are independent)."""
    B = 16384 // S
    _run(gpu_lib, B, 16, Hkv, S, 64, score_mod, mask, batch=B - 1, rms_check=True)


@pytest.mark.parametrize("score_mod", SCORE_MODS)
def test_score_mod_sweep_S4096(gpu_lib, score_mod):
    S = 4096
    rows = sample_rows_at_least(S, 512, seed=1)
    _run(gpu_lib, 16384 // S, 16, 16, S, 64, score_mod, "none", rows=rows, rms_check=True)


def _must_rows(S, B, mask):
    """Rows every sampled check includes beyond the tile edges: the PrefixLM
    prefix edge, the sliding window's first full row, every document edge."""
    must = [S // 4 - 1, S // 4, S // 4 + 1]
    if mask == "sliding_window":
        must += [255, 256, 257]
    if mask == "document":
        for b_lens in wi.doc_lengths(4, B, S):
            must += list(np.cumsum(b_lens)[:-1]) + list(np.cumsum(b_lens)[:-1] - 1)
    return must


@pytest.mark.parametrize("mask", MASKS[1:])
@pytest.mark.parametrize("Hkv", [16, 2])
def test_mask_sweep_S4096(gpu_lib, mask, Hkv):
    S = 4096
    B = 16384 // S
    rows = sample_rows_at_least(S, 512, seed=2, must=_must_rows(S, B, mask))
    _run(gpu_lib, B, 16, Hkv, S, 64, "none", mask, rows=rows, rms_check=True)


@pytest.mark.parametrize("score_mod,mask,Hkv", BENCH_VARIANTS)
def test_benchmark_shapes_S8192(gpu_lib, score_mod, mask, Hkv):
    """S = 8k, B = 2 (16k tokens, 16 query heads): at least 512 sampled rows
    per head of both batch entries, tile, prefix and document edges included."""
    S = 8192
    B = 16384 // S
    rows = sample_rows_at_least(S, 512, tiles=(128,), seed=6, must=_must_rows(S, B, mask))
    _run(gpu_lib, B, 16, Hkv, S, 64, score_mod, mask, rows=rows, rms_check=True)


@pytest.mark.parametrize("mask,Hkv", [("causal", 16), ("causal", 2), ("sliding_window", 16), ("sliding_window", 2),
                                      ("prefix_lm", 16), ("prefix_lm", 2), ("document", 16)])
def test_masks_S16384(gpu_lib, mask, Hkv):
    """The masked benchmark variants at S = 16k, B = 1 not covered by the
    sweep-extremes test, sampled as at S = 8k."""
    S = 16384
    rows = sample_rows_at_least(S, 512, tiles=(128,), seed=7, must=_must_rows(S, 1, mask))
    _run(gpu_lib, 1, 16, Hkv, S, 64, "none", mask, rows=rows, rms_check=True)


@pytest.mark.parametrize("S", [512, 16384])
def test_sweep_extremes(gpu_lib, S):
    rows = sample_rows_at_least(S, 512, tiles=(128,), seed=3)
    for sm, mk in (("softcap", "none"), ("alibi", "causal"), ("none", "document")):
        _run(gpu_lib, 16384 // S, 16, 16 if mk != "document" else 2, S, 64, sm, mk, rows=rows, rms_check=True)


@pytest.mark.parametrize("score_mod", SCORE_MODS)
def test_score_mod_S16384_rms(gpu_lib, score_mod):
    """S = 16k, where outputs have rms ~ 0.013: at least 512 rows per head,
    elementwise gate plus the rms-relative diagnostic."""
    S = 16384
    rows = sample_rows_at_least(S, 512, tiles=(128,), seed=4)
    _run(gpu_lib, 1, 16, 16, S, 64, score_mod, "none", rows=rows, rms_check=True)


@pytest.mark.parametrize("qmul", [0.25, 1.0, 4.0, 16.0])
@pytest.mark.parametrize("D,mask", [(64, "none"), (64, "causal"), (32, "document"), (128, "prefix_lm")])
def test_softcap_score_ranges(gpu_lib, qmul, D, mask):
    """Softcap (cap 20, fixed reference) with Q scaled by a power of two: small
    scores (every tile on the polynomial form), scores that reach past 0.25 cap
    in some tiles (mixed forms), and scores far into saturation (exact form)."""
    B, H, S = 2, 4, 300
    x = wi.attention_inputs(B, H, H, S, S, D, seeds=(31, 32, 33))
    qb = wi.bf16_bits_from_f32(wi.bf16_bits_to_f32(x["q"]) * np.float32(qmul))
    kw = _params(mask, S)
    if mask == "document":
        kw["doc_id"] = wi.doc_ids(4, B, S, lo=4)
    dev_kw = dict(kw)
    if "doc_id" in dev_kw:
        dev_kw["doc_id"] = torch.from_numpy(dev_kw["doc_id"]).cuda()
    q, k, v = to_dev(qb), to_dev(x["k"]), to_dev(x["v"])
    out, lse = gpu_lib.attn_fwd(q, k, v, score_mod="softcap", mask=mask, return_lse=True, **dev_kw)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attention(f64(qb), f64(x["k"]), f64(x["v"]), score_mod="softcap", mask=mask, **kw)
    what = f"softcap q*{qmul} D{D} {mask}"
    assert_close(out.float().cpu().numpy(), ref, what)
    assert_close(lse.cpu().numpy(), ref_lse, what + " lse", atol=LSE_ATOL, rtol=1e-5)
