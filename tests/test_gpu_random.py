"""Seeded random parity sweep against the fp64 oracle, through the C ABI: the
forward, the backward, dense and paged decode, differential attention and the
two Evoformer forms.

Each case draws its own shape and parameters from a fixed generator: head
dimension, batch, query and KV heads, ragged and cross lengths, score modifier,
mask, softmax scale, softcap, ALiBi maximum bias, bias-tensor broadcast, window,
prefix and document lengths, page size and per-sequence cache lengths, lambda,
MSA channels, heads and residues.  The sweep is the same on every run and a
failure names its case.  Every output row is compared.  Gates as in the
fixed-shape tests: |gpu - oracle| <= 1e-2 + 1e-2 |oracle|; LSE within 1e-3 +
1e-5 relative.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import inputs as wi

from .gpu_util import assert_close, canary_empty, canary_intact, f64, to_dev

pytestmark = pytest.mark.gpu

SCORE_MODS = ("none", "alibi", "softcap")
MASKS = ("none", "causal", "sliding_window", "prefix_lm", "document")


def _doc_ids(rng, B, S):
    """Non-decreasing document ids per row (the layout the kernels require):
    lengths uniform in [lo, hi], the last one filling the row."""
    lo = int(rng.integers(1, max(2, S // 3) + 1))
    hi = int(rng.integers(lo, max(lo, S) + 1))
    return wi.doc_ids(int(rng.integers(0, 1 << 16)), B, S, lo=lo, hi=hi)


def _mask_params(rng, mask, B, S):
    kw = {}
    if mask == "sliding_window":
        kw["window"] = int(rng.integers(1, S + 2))
    elif mask == "prefix_lm":
        kw["prefix_len"] = int(rng.integers(0, S + 1))
    elif mask == "document":
        kw["doc_id"] = _doc_ids(rng, B, S)
    return kw


def _mod_params(rng, score_mod, D):
    kw = {"scale": float(rng.choice([0.0, 0.5 / np.sqrt(D), 2.0 / np.sqrt(D)]))}
    if score_mod == "softcap":
        kw["softcap"] = float(rng.choice([5.0, 20.0, 50.0, 400.0]))
    if score_mod == "alibi":
        kw["alibi_max_bias"] = float(rng.choice([2.0, 8.0, 16.0]))
    return kw


def _fwd_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        D = int(rng.choice([32, 64, 64, 128]))
        B = int(rng.integers(1, 4))
        Hkv = int(rng.choice([1, 2, 4]))
        Hq = Hkv * int(rng.choice([1, 2, 4]))
        mask = str(rng.choice(MASKS))
        S = int(rng.integers(1, 400))
        Skv = S if mask != "none" or rng.random() < 0.5 else int(rng.integers(1, 600))
        score_mod = str(rng.choice(SCORE_MODS + ("bias",)))
        kw = _mod_params(rng, score_mod, D)
        if score_mod == "bias":  # broadcast over batch and/or heads
            kw["bias_shape"] = (int(rng.choice([1, B])), int(rng.choice([1, Hq])), S, Skv)
        kw.update(_mask_params(rng, mask, B, S))
        cases.append((i, D, B, Hq, Hkv, S, Skv, score_mod, mask, kw, bool(rng.random() < 0.5)))
    return cases


def _case_id(c):
    i, D, B, Hq, Hkv, S, Skv, score_mod, mask, kw = c[:10]
    return f"{i}-{score_mod}-{mask}-D{D}-B{B}-H{Hq}x{Hkv}-S{S}x{Skv}"


def _dev_kw(kw):
    out = dict(kw)
    if "doc_id" in out:
        out["doc_id"] = torch.from_numpy(out["doc_id"]).cuda()
    return out


def _describe(score_mod, mask, B, Hq, Hkv, S, Skv, D, kw):
    shown = {k: v for k, v in kw.items() if k not in ("doc_id", "bias")}
    if "doc_id" in kw:
        shown["docs"] = [int(r.max()) + 1 for r in kw["doc_id"]]
    return f"{score_mod}/{mask} B{B} Hq{Hq} Hkv{Hkv} S{S} Skv{Skv} D{D} {shown}"


FWD_CASES = _fwd_cases(128, 20261203)


@pytest.mark.parametrize("case", FWD_CASES, ids=[_case_id(c) for c in FWD_CASES])
def test_forward_random(gpu_lib, case):
    i, D, B, Hq, Hkv, S, Skv, score_mod, mask, kw, want_lse = case
    x = wi.attention_inputs(B, Hq, Hkv, S, Skv, D, seeds=(100 + i, 200 + i, 300 + i))
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    kw = dict(kw)
    if "bias_shape" in kw:
        kw["bias"] = wi.normal_bf16(1100 + i, kw.pop("bias_shape"), 2.0)
    what = _describe(score_mod, mask, B, Hq, Hkv, S, Skv, D, kw)
    print(what, flush=True)
    dkw = _dev_kw(kw)
    if "bias" in dkw:
        dkw["bias"] = to_dev(dkw["bias"])
    out, big = canary_empty((B, Hq, S, D), torch.bfloat16)
    lse = None
    if want_lse:
        lse, bigl = canary_empty((B, Hq, S), torch.float32)
    gpu_lib.attn_fwd(q, k, v, score_mod=score_mod, mask=mask, out=out, lse=lse, **dkw)
    torch.cuda.synchronize()
    assert canary_intact(big, out.numel()), "write past the end of out: " + what
    okw = dict(kw)
    if okw.get("scale") == 0.0:
        okw["scale"] = None
    if "bias" in okw:
        okw["bias"] = f64(okw["bias"])
    ref, ref_lse = oracle.attention(f64(x["q"]), f64(x["k"]), f64(x["v"]), score_mod=score_mod, mask=mask, **okw)
    assert_close(out.float().cpu().numpy(), ref, what)
    if want_lse:
        assert canary_intact(bigl, lse.numel()), "write past the end of lse: " + what
        assert_close(lse.cpu().numpy(), ref_lse, what + " lse", atol=1e-3, rtol=1e-5)


def _bwd_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        B = int(rng.integers(1, 3))
        Hkv = int(rng.choice([1, 2]))
        Hq = Hkv * int(rng.choice([1, 2, 4]))
        S = int(rng.integers(1, 260))
        score_mod = str(rng.choice(SCORE_MODS))
        mask = str(rng.choice(MASKS))
        kw = _mod_params(rng, score_mod, 64)
        kw.update(_mask_params(rng, mask, B, S))
        cases.append((i, 64, B, Hq, Hkv, S, S, score_mod, mask, kw))
    return cases


BWD_CASES = _bwd_cases(48, 20261204)


@pytest.mark.parametrize("case", BWD_CASES, ids=[_case_id(c) for c in BWD_CASES])
def test_backward_random(gpu_lib, case):
    i, D, B, Hq, Hkv, S, _, score_mod, mask, kw = case
    x = wi.attention_inputs(B, Hq, Hkv, S, S, D, seeds=(400 + i, 500 + i, 600 + i))
    g = wi.normal_bf16(700 + i, (B, Hq, S, D), 1.0)
    q, k, v, dout = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(g)
    what = "bwd " + _describe(score_mod, mask, B, Hq, Hkv, S, S, D, kw)
    print(what, flush=True)
    dkw = _dev_kw(kw)
    _, lse = gpu_lib.attn_fwd(q, k, v, score_mod=score_mod, mask=mask, return_lse=True, **dkw)
    dq, dk, dv = gpu_lib.attn_bwd(q, k, v, dout, lse, score_mod=score_mod, mask=mask, **dkw)
    torch.cuda.synchronize()
    okw = dict(kw)
    if okw.get("scale") == 0.0:
        okw["scale"] = None
    rq, rk, rv = oracle.attention_backward(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(g), score_mod=score_mod,
                                           mask=mask, **okw)
    assert_close(dq.float().cpu().numpy(), rq, what + " dq")
    assert_close(dk.float().cpu().numpy(), rk, what + " dk")
    assert_close(dv.float().cpu().numpy(), rv, what + " dv")


def _dec_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        B = int(rng.integers(1, 5))
        Hkv = int(rng.choice([1, 2, 8]))
        g = int(rng.choice([1, 2, 4, 8]))
        Sq = int(rng.integers(1, 32 // g + 1))
        Skv = int(rng.integers(Sq, 3000))
        score_mod = str(rng.choice(SCORE_MODS))
        mask = str(rng.choice(["none", "causal"]))
        kw = _mod_params(rng, score_mod, 64)
        cases.append((i, 64, B, Hkv * g, Hkv, Sq, Skv, score_mod, mask, kw))
    return cases


DEC_CASES = _dec_cases(32, 20261205)


@pytest.mark.parametrize("case", DEC_CASES, ids=[_case_id(c) for c in DEC_CASES])
def test_decode_random(gpu_lib, case):
    i, D, B, Hq, Hkv, Sq, Skv, score_mod, mask, kw = case
    x = wi.attention_inputs(B, Hq, Hkv, Sq, Skv, D, seeds=(800 + i, 900 + i, 1000 + i))
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    what = "decode " + _describe(score_mod, mask, B, Hq, Hkv, Sq, Skv, D, kw)
    print(what, flush=True)
    out, big = canary_empty((B, Hq, Sq, D), torch.bfloat16)
    lse, bigl = canary_empty((B, Hq, Sq), torch.float32)
    gpu_lib.attn_decode_fwd(q, k, v, score_mod=score_mod, mask=mask, out=out, lse=lse, **kw)
    torch.cuda.synchronize()
    assert canary_intact(big, out.numel()), "write past the end of out: " + what
    assert canary_intact(bigl, lse.numel()), "write past the end of lse: " + what
    okw = dict(kw)
    if okw.get("scale") == 0.0:
        okw["scale"] = None
    ref, ref_lse = oracle.attention(f64(x["q"]), f64(x["k"]), f64(x["v"]), score_mod=score_mod, mask=mask,
                                    q_offset=Skv - Sq, **okw)
    assert_close(out.float().cpu().numpy(), ref, what)
    assert_close(lse.cpu().numpy(), ref_lse, what + " lse", atol=1e-3, rtol=1e-5)


def _paged_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        B = int(rng.integers(1, 6))
        Hkv = int(rng.choice([1, 2, 8]))
        g = int(rng.choice([1, 2, 4]))
        Sq = int(rng.integers(1, 32 // g + 1))
        ps = int(rng.choice([16, 32, 64]))
        lens = [int(x) for x in rng.integers(Sq, 2500, size=B)]
        score_mod = str(rng.choice(SCORE_MODS))
        mask = str(rng.choice(["none", "causal"]))
        kw = _mod_params(rng, score_mod, 64)
        cases.append((i, 64, B, Hkv * g, Hkv, Sq, ps, score_mod, mask, kw, lens))
    return cases


PAGED_CASES = _paged_cases(24, 20261206)


@pytest.mark.parametrize("case", PAGED_CASES,
                         ids=[f"{c[0]}-{c[7]}-{c[8]}-B{c[2]}-H{c[3]}x{c[4]}-Sq{c[5]}-ps{c[6]}" for c in PAGED_CASES])
def test_paged_decode_random(gpu_lib, case):
    """Pages handed out in a shuffled order; unused block-table entries hold -1."""
    i, D, B, Hq, Hkv, Sq, ps, score_mod, mask, kw, lens = case
    rng = np.random.default_rng(1200 + i)
    maxp = max((n + ps - 1) // ps for n in lens) + int(rng.integers(0, 3))
    npages = sum((n + ps - 1) // ps for n in lens) + int(rng.integers(0, 4))
    x = wi.attention_inputs(npages, Hkv, Hkv, ps, ps, D, seeds=(1300 + i, 1400 + i, 1500 + i))
    kc, vc = x["k"], x["v"]
    q = wi.attention_inputs(B, Hq, Hkv, Sq, 1, D, seeds=(1600 + i, 1700 + i, 1800 + i))["q"]
    order = rng.permutation(npages)
    bt = np.full((B, maxp), -1, dtype=np.int32)
    nxt = 0
    for b, n in enumerate(lens):
        for p_ in range((n + ps - 1) // ps):
            bt[b, p_] = order[nxt]
            nxt += 1
    sl = np.asarray(lens, dtype=np.int32)
    what = (f"paged {score_mod}/{mask} B{B} Hq{Hq} Hkv{Hkv} Sq{Sq} ps{ps} pages{npages} table{maxp} "
            f"lens{lens} {kw}")
    print(what, flush=True)
    out, big = canary_empty((B, Hq, Sq, D), torch.bfloat16)
    lse, bigl = canary_empty((B, Hq, Sq), torch.float32)
    gpu_lib.attn_decode_paged_fwd(to_dev(q), to_dev(kc), to_dev(vc), torch.from_numpy(bt).cuda(),
                                  torch.from_numpy(sl).cuda(), score_mod=score_mod, mask=mask, out=out, lse=lse,
                                  **kw)
    torch.cuda.synchronize()
    assert canary_intact(big, out.numel()), "write past the end of out: " + what
    assert canary_intact(bigl, lse.numel()), "write past the end of lse: " + what
    okw = dict(kw)
    if okw.get("scale") == 0.0:
        okw["scale"] = None
    ref, ref_lse = oracle.paged_decode_attention(f64(q), f64(kc), f64(vc), np.where(bt < 0, 0, bt), sl,
                                                 page_size=ps, score_mod=score_mod, mask=mask, **okw)
    assert_close(out.float().cpu().numpy(), ref, what)
    assert_close(lse.cpu().numpy(), ref_lse, what + " lse", atol=1e-3, rtol=1e-5)


def _diff_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        B = int(rng.integers(1, 4))
        H = int(rng.integers(1, 7))
        S = int(rng.integers(1, 400))
        Dh, Dv = [(64, 128), (64, 64), (32, 64), (32, 128)][int(rng.integers(0, 4))]
        lam = float(np.round(rng.uniform(-0.5, 1.5), 3))
        causal = bool(rng.random() < 0.7)
        scale = float(rng.choice([0.0, 0.5 / np.sqrt(Dh)]))
        cases.append((i, B, H, S, Dh, Dv, lam, causal, scale))
    return cases


DIFF_CASES = _diff_cases(24, 20261207)


@pytest.mark.parametrize("case", DIFF_CASES,
                         ids=[f"{c[0]}-B{c[1]}-H{c[2]}-S{c[3]}-Dh{c[4]}-Dv{c[5]}" for c in DIFF_CASES])
def test_diff_random(gpu_lib, case):
    i, B, H, S, Dh, Dv, lam, causal, scale = case
    x = wi.diff_inputs(B, H, S, Dh, Dv, seeds=(1900 + i, 2000 + i, 2100 + i))
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    what = f"diff B{B} H{H} S{S} Dh{Dh} Dv{Dv} lam{lam} causal{causal} scale{scale}"
    print(what, flush=True)
    out, big = canary_empty((B, H, S, Dv), torch.bfloat16)
    gpu_lib.diff_attn_fwd(q, k, v, lam=lam, scale=scale, causal=causal, out=out)
    torch.cuda.synchronize()
    assert canary_intact(big, out.numel()), "write past the end of out: " + what
    ref = oracle.diff_attention(f64(x["q"]), f64(x["k"]), f64(x["v"]), lam=lam, causal=causal,
                                scale=None if scale == 0.0 else scale)
    assert_close(out.float().cpu().numpy(), ref, what)


def _evo_cases(n, seed, fused_share, ns_range):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dh = int(rng.choice([32, 64]))
        H = int(rng.choice([4, 8, 12, 16] if dh == 32 else [2, 4, 6, 8]))
        if rng.random() < fused_share:  # the one-launch row-wise form: Cm 256, N_res <= 256, a multiple of 8
            Cm, Nr = 256, 8 * int(rng.integers(1, 33))
        else:
            Cm, Nr = int(rng.choice([64, 128, 256, 320])), int(rng.integers(1, 300))
        Ns = int(rng.integers(*ns_range))
        cases.append((i, Ns, Nr, Cm, H, dh))
    return cases


EVO_CASES = _evo_cases(24, 20261208, 0.5, (1, 10))
# Column-wise attention runs over the Ns sequences of a residue column.  With
# only a few of them the bf16 rounding of the projected q and k (the MFMA
# operands) alone moves the output past the gate where it nearly cancels: exact
# fp64 attention over bf16-rounded projections reaches 0.96, 1.16 and 1.06 of
# the gate at Ns = 2, 6 and 8 (Nr 240-267, Cm 64-128).  The pages' shape has
# Ns = 128; the sweep draws Ns from 16 up.
EVO_COL_CASES = _evo_cases(16, 20261209, 0.0, (16, 49))


def _evo_inputs(i, Ns, Nr, Cm, H, dh):
    return wi.evoformer_inputs(Ns, Nr, Cm, H, dh, seeds={"m": 2200 + i, "wq": 2300 + i, "wk": 2400 + i,
                                                         "wv": 2500 + i, "wg": 2600 + i, "bias": 2700 + i})


@pytest.mark.parametrize("case", EVO_CASES, ids=[f"{c[0]}-Ns{c[1]}-Nr{c[2]}-Cm{c[3]}-H{c[4]}x{c[5]}" for c in EVO_CASES])
def test_evoformer_row_random(gpu_lib, case):
    i, Ns, Nr, Cm, H, dh = case
    x = _evo_inputs(i, Ns, Nr, Cm, H, dh)
    t = {n: to_dev(x[n]) for n in x}
    what = f"evoformer row Ns{Ns} Nr{Nr} Cm{Cm} H{H} dh{dh}"
    print(what, flush=True)
    out, big = canary_empty((Ns, Nr, H * dh), torch.bfloat16)
    gpu_lib.evoformer_gated_attn_fwd(t["m"], t["wq"], t["wk"], t["wv"], t["wg"], t["bias"], H=H, dh=dh, out=out)
    torch.cuda.synchronize()
    assert canary_intact(big, out.numel()), "write past the end of out: " + what
    ref = oracle.evoformer_row_gated_attention(f64(x["m"]), f64(x["wq"]), f64(x["wk"]), f64(x["wv"]), f64(x["wg"]),
                                               f64(x["bias"]), H=H, dh=dh)
    assert_close(out.float().cpu().numpy(), ref, what)


@pytest.mark.parametrize("case", EVO_COL_CASES,
                         ids=[f"{c[0]}-Ns{c[1]}-Nr{c[2]}-Cm{c[3]}-H{c[4]}x{c[5]}" for c in EVO_COL_CASES])
def test_evoformer_col_random(gpu_lib, case):
    i, Ns, Nr, Cm, H, dh = case
    x = _evo_inputs(100 + i, Ns, Nr, Cm, H, dh)
    t = {n: to_dev(x[n]) for n in x}
    what = f"evoformer col Ns{Ns} Nr{Nr} Cm{Cm} H{H} dh{dh}"
    print(what, flush=True)
    out, big = canary_empty((Ns, Nr, H * dh), torch.bfloat16)
    gpu_lib.evoformer_col_gated_attn_fwd(t["m"], t["wq"], t["wk"], t["wv"], t["wg"], H=H, dh=dh, out=out)
    torch.cuda.synchronize()
    assert canary_intact(big, out.numel()), "write past the end of out: " + what
    ref = oracle.evoformer_col_gated_attention(f64(x["m"]), f64(x["wq"]), f64(x["wk"]), f64(x["wv"]), f64(x["wg"]),
                                               H=H, dh=dh)
    assert_close(out.float().cpu().numpy(), ref, what)
