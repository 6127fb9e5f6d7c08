"""GPU parity of ``attn_bwd`` (dq, dk, dv of attn_fwd's output) against the
fp64 backward oracle, through the C ABI.

The GPU takes its own forward's log-sum-exp only as an exponent reference
and renormalises P in fp32 (a first pass computes the row sums and
Delta = rowsum(P dP)); P and dS are rounded to bf16 as MFMA operands.  The gate is the
forward's: |gpu - oracle| <= 1e-2 + 1e-2 |oracle| on every element.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import inputs as wi

from .gpu_util import assert_close, f64, to_dev

pytestmark = pytest.mark.gpu


MASKS = ("none", "causal", "sliding_window", "prefix_lm", "document")


def _mask_kw(mask, B, S):
    """The mask parameters of the forward tests: window 256 from S = 1k (S / 3
    below), prefix S / 4, seeded document lengths (uniform 64..S/2, 4..S/2
    below S = 256); returns (oracle kwargs, device kwargs)."""
    kw = {}
    if mask == "sliding_window":
        kw["window"] = 256 if S >= 1024 else max(1, S // 3)
    if mask == "prefix_lm":
        kw["prefix_len"] = S // 4
    dev_kw = dict(kw)
    if mask == "document":
        kw["doc_id"] = wi.doc_ids(4, B, S, lo=64 if S >= 256 else 4)
        dev_kw["doc_id"] = torch.from_numpy(kw["doc_id"]).cuda()
    return kw, dev_kw


def _run(av, B, Hq, Hkv, S, score_mod, mask, seed=(21, 22, 23), dseed=24, qmul=1.0):
    """qmul (a power of two, exact in bf16) scales q on both sides."""
    D = 64
    x = wi.attention_inputs(B, Hq, Hkv, S, S, D, seeds=seed)
    g = wi.normal_bf16(dseed, (B, Hq, S, D), 1.0)
    q, k, v, dout = to_dev(x["q"]) * qmul, to_dev(x["k"]), to_dev(x["v"]), to_dev(g)
    okw, dkw = _mask_kw(mask, B, S)
    kw = dict(score_mod=score_mod, mask=mask, softcap=20.0)
    out, lse = av.attn_fwd(q, k, v, return_lse=True, **kw, **dkw)
    dq, dk, dv = av.attn_bwd(q, k, v, dout, lse, **kw, **dkw)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_backward(f64(x["q"]) * qmul, f64(x["k"]), f64(x["v"]), f64(g), **kw, **okw)
    what = f"bwd {score_mod}/{mask} B{B} Hq{Hq} Hkv{Hkv} S{S} qmul {qmul}"
    e = [assert_close(dq.float().cpu().numpy(), rq, what + " dq"),
         assert_close(dk.float().cpu().numpy(), rk, what + " dk"),
         assert_close(dv.float().cpu().numpy(), rv, what + " dv")]
    return e, (dq, dk, dv)


@pytest.mark.parametrize("score_mod", ["none", "alibi", "softcap"])
@pytest.mark.parametrize("mask", MASKS)
def test_bwd_parity(gpu_lib, score_mod, mask):
    for (B, Hq, Hkv, S) in ((1, 4, 2, 128), (2, 2, 2, 300), (1, 2, 1, 65), (1, 2, 2, 1), (1, 8, 2, 200)):
        _run(gpu_lib, B, Hq, Hkv, S, score_mod, mask)


def test_bwd_longer(gpu_lib):
    _run(gpu_lib, 2, 8, 2, 1024, "softcap", "causal")
    _run(gpu_lib, 1, 4, 4, 777, "none", "none")


@pytest.mark.parametrize("qmul", [2.0, 4.0])
@pytest.mark.parametrize("mask", ["none", "causal"])
def test_bwd_softcap_tiles_outside_the_cubic(gpu_lib, qmul, mask):
    """Softcap (cap 20, scale 1/8) keeps the cubic for tiles whose raw scores stay
    within |q.k| <= 0.25 cap / scale = 40 and takes the exact tanh form on the
    others.  With q doubled (raw score sd 16) the two forms alternate from tile
    to tile; with q times 4 (sd 32) almost every tile is exact."""
    _run(gpu_lib, 1, 4, 2, 640, "softcap", mask, qmul=qmul)
    _run(gpu_lib, 2, 2, 2, 129, "softcap", mask, qmul=qmul)


@pytest.mark.parametrize("mask", ["sliding_window", "prefix_lm", "document"])
def test_bwd_longer_masks(gpu_lib, mask):
    """S = 1000 and 1024 (window 256, several 128-key tiles per document), MHA and GQA."""
    _run(gpu_lib, 2, 4, 2, 1024, "softcap", mask)
    _run(gpu_lib, 1, 4, 4, 1000, "alibi", mask)


def test_bwd_deterministic(gpu_lib):
    x = wi.attention_inputs(1, 8, 2, 513, 513, 64)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    dout = to_dev(wi.normal_bf16(5, (1, 8, 513, 64), 1.0))
    out, lse = gpu_lib.attn_fwd(q, k, v, mask="causal", return_lse=True)
    r = [gpu_lib.attn_bwd(q, k, v, dout, lse, mask="causal") for _ in range(3)]
    for i in range(3):
        assert torch.equal(r[0][i], r[1][i]) and torch.equal(r[1][i], r[2][i])


@pytest.mark.parametrize("score_mod,mask", [("none", "none"), ("softcap", "causal"), ("none", "sliding_window"),
                                            ("alibi", "prefix_lm"), ("softcap", "document")])
def test_bwd_benchmark_shape(gpu_lib, score_mod, mask):
    """The benchmark shape (B = 4, H = 16, S = 4096): the GPU computes every
    head; the oracle checks the first two heads of the last batch entry (heads
    and batch entries are independent for these score modifiers)."""
    B, H, S, D = 4, 16, 4096, 64
    x = wi.attention_inputs(B, H, H, S, S, D)
    g = wi.normal_bf16(5, (B, H, S, D), 1.0)
    q, k, v, dout = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(g)
    okw, dkw = _mask_kw(mask, B, S)
    kw = dict(score_mod=score_mod, mask=mask, softcap=20.0)
    out, lse = gpu_lib.attn_fwd(q, k, v, return_lse=True, **kw, **dkw)
    dq, dk, dv = gpu_lib.attn_bwd(q, k, v, dout, lse, **kw, **dkw)
    torch.cuda.synchronize()
    sl = (slice(B - 1, B), slice(0, 2))
    if "doc_id" in okw:
        okw["doc_id"] = okw["doc_id"][B - 1:B]
    # the oracle sees heads 0-1 as a 2-head problem: ALiBi slopes 2^(-8(h+1)/16)
    # are 2^(-mb(h+1)/2) with mb = 8 * 2 / 16
    okw["alibi_max_bias"] = 8.0 * 2 / H
    rq, rk, rv = oracle.attention_backward(f64(x["q"][sl]), f64(x["k"][sl]), f64(x["v"][sl]), f64(g[sl]), **kw,
                                           **okw)
    what = f"bwd {score_mod}/{mask} B{B} H{H} S{S} (batch {B - 1}, heads 0-1)"
    assert_close(dq[sl].float().cpu().numpy(), rq, what + " dq")
    assert_close(dk[sl].float().cpu().numpy(), rk, what + " dk")
    assert_close(dv[sl].float().cpu().numpy(), rv, what + " dv")


def test_bwd_no_keys_gives_zero_dq(gpu_lib):
    """Skv = 0: the output is the constant zero row, so dq is zero (and nothing else is written)."""
    q = torch.randn(1, 2, 5, 64, device="cuda").to(torch.bfloat16)
    kv = torch.zeros(1, 2, 0, 64, dtype=torch.bfloat16, device="cuda")
    out, lse = gpu_lib.attn_fwd(q, kv, kv, return_lse=True)
    dq = torch.full_like(q, 3.0)
    dq, dk, dv = gpu_lib.attn_bwd(q, kv, kv, torch.ones_like(q), lse, dq=dq)
    torch.cuda.synchronize()
    assert torch.all(dq == 0).item()
    assert dk.numel() == 0 and dv.numel() == 0


@pytest.mark.parametrize("score_mod", ["none", "alibi", "softcap"])
@pytest.mark.parametrize("B, Hq, Hkv, S", [(2, 4, 2, 1000), (4, 16, 16, 4096), (1, 8, 8, 16384)])
def test_bwd_document_order_changes_no_bit(gpu_lib, score_mod, B, Hq, Hkv, S):
    """The heaviest-first work order of attn_doc_order reorders the three
    backward launches only: dq, dk and dv equal the natural order's bit for
    bit (each element keeps its one writer and its arithmetic)."""
    D = 64
    x = wi.attention_inputs(B, Hq, Hkv, S, S, D, seeds=(31, 32, 33))
    g = wi.normal_bf16(34, (B, Hq, S, D), 1.0)
    q, k, v, dout = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(g)
    doc = torch.from_numpy(wi.doc_ids(4, B, S)).cuda()
    order = gpu_lib.attn_doc_order(doc)
    kw = dict(score_mod=score_mod, mask="document", doc_id=doc, softcap=20.0)
    out, lse = gpu_lib.attn_fwd(q, k, v, return_lse=True, **kw)
    natural = gpu_lib.attn_bwd(q, k, v, dout, lse, **kw)
    ordered = gpu_lib.attn_bwd(q, k, v, dout, lse, doc_order=order, **kw)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), natural, ordered):
        assert torch.equal(a, b), f"{name} differs under the order ({score_mod}, B{B} S{S})"


def test_bwd_document_order_parity(gpu_lib):
    """The ordered backward against the oracle (GQA, several documents per
    128-row tile and documents over several tiles)."""
    B, Hq, Hkv, S, D = 2, 4, 2, 1000, 64
    x = wi.attention_inputs(B, Hq, Hkv, S, S, D, seeds=(41, 42, 43))
    g = wi.normal_bf16(44, (B, Hq, S, D), 1.0)
    q, k, v, dout = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(g)
    doc_np = wi.doc_ids(4, B, S)
    doc = torch.from_numpy(doc_np).cuda()
    kw = dict(score_mod="softcap", mask="document", softcap=20.0)
    out, lse = gpu_lib.attn_fwd(q, k, v, return_lse=True, doc_id=doc, **kw)
    dq, dk, dv = gpu_lib.attn_bwd(q, k, v, dout, lse, doc_id=doc, doc_order=gpu_lib.attn_doc_order(doc), **kw)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.attention_backward(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(g), doc_id=doc_np, **kw)
    what = f"bwd softcap/document ordered B{B} Hq{Hq} Hkv{Hkv} S{S}"
    assert_close(dq.float().cpu().numpy(), rq, what + " dq")
    assert_close(dk.float().cpu().numpy(), rk, what + " dk")
    assert_close(dv.float().cpu().numpy(), rv, what + " dv")
