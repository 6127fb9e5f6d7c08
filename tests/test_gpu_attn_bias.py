"""GPU parity of ``attn_fwd`` with the bias-tensor score modifier (a
data-dependent score term) against the fp64 oracle, through the C ABI.

The bias is bf16 N(0, 2^2), shaped [Bb, Hb, Sq, Skv] with the batch and head
axes either full or shared (stride 0).  Every mask, D in {32, 64, 128}, MHA
and GQA, ragged tails, odd key counts (16-bit bias reads); the benchmark
shape on sampled rows.  Gate: |gpu - oracle| <= 1e-2 + 1e-2 |oracle|; LSE
within 1e-3 + 1e-5 |lse| (fp32 summands, as for attn_fwd).
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import inputs as wi

from .gpu_util import assert_close, canary_empty, canary_intact, f64, sample_rows, to_dev

pytestmark = pytest.mark.gpu

LSE_ATOL = 1e-3
MASKS = ("none", "causal", "sliding_window", "prefix_lm", "document")
BSHAPES = ("full", "batch_shared", "head_shared", "shared")


def _bias_shape(bshape, B, Hq, Sq, Skv):
    Bb = 1 if bshape in ("batch_shared", "shared") else B
    Hb = 1 if bshape in ("head_shared", "shared") else Hq
    return (Bb, Hb, Sq, Skv)


def _run(av, B, Hq, Hkv, S, D, mask, bshape, rows=None, Skv=None, bias_seed=18):
    Skv = S if Skv is None else Skv
    x = wi.attention_inputs(B, Hq, Hkv, S, Skv, D)
    bb = wi.normal_bf16(bias_seed, _bias_shape(bshape, B, Hq, S, Skv), 2.0)
    kw = {}
    if mask == "sliding_window":
        kw["window"] = 256 if S >= 1024 else max(1, S // 3)
    if mask == "prefix_lm":
        kw["prefix_len"] = S // 4
    if mask == "document":
        kw["doc_id"] = wi.doc_ids(4, B, S, lo=64 if S >= 256 else 4)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    dev_kw = dict(kw)
    if "doc_id" in dev_kw:
        dev_kw["doc_id"] = torch.from_numpy(dev_kw["doc_id"]).cuda()
    out, big = canary_empty((B, Hq, S, D), torch.bfloat16)
    lse, bigl = canary_empty((B, Hq, S), torch.float32)
    av.attn_fwd(q, k, v, score_mod="bias", mask=mask, bias=to_dev(bb), out=out, lse=lse, **dev_kw)
    torch.cuda.synchronize()
    assert canary_intact(big, out.numel()), "write past the end of out"
    assert canary_intact(bigl, lse.numel()), "write past the end of lse"
    ref, ref_lse = oracle.attention(f64(x["q"]), f64(x["k"]), f64(x["v"]), score_mod="bias", mask=mask,
                                    bias=f64(bb), rows=rows, **kw)
    got, got_lse = out.float().cpu().numpy(), lse.cpu().numpy()
    if rows is not None:
        got, got_lse = got[:, :, rows], got_lse[:, :, rows]
    what = f"bias({bshape})/{mask} B{B} Hq{Hq} Hkv{Hkv} S{S} Skv{Skv} D{D}"
    assert_close(got, ref, what)
    assert_close(got_lse, ref_lse, what + " lse", atol=LSE_ATOL, rtol=1e-5)
    return out


@pytest.mark.parametrize("mask", MASKS)
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("S", [1, 37, 130, 300])
def test_masks_all_rows(gpu_lib, mask, D, S):
    _run(gpu_lib, 2, 4, 2, S, D, mask, "full")


@pytest.mark.parametrize("bshape", BSHAPES)
@pytest.mark.parametrize("S", [64, 257])
def test_broadcast_forms(gpu_lib, bshape, S):
    _run(gpu_lib, 2, 4, 4, S, 64, "causal", bshape)
    _run(gpu_lib, 2, 4, 1, S, 64, "none", bshape)


def test_cross_attention_odd_keys(gpu_lib):
    """Sq != Skv with an odd key count: 16-bit bias reads, ragged key tail."""
    for Skv in (1, 63, 65, 191, 333):
        _run(gpu_lib, 1, 2, 2, 100, 64, "none", "full", Skv=Skv)


def test_alibi_as_a_tensor(gpu_lib):
    """The ALiBi slopes written out as a bias equal the ALiBi modifier up to
    the bias's bf16 rounding (distances up to 96 keys keep it within 2^-8 relative)."""
    B, H, S, D = 1, 4, 96, 64
    x = wi.attention_inputs(B, H, H, S, S, D)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    al = np.stack([oracle.alibi_slope(h, H, 8.0) * (j - i) for h in range(H)])[None].astype(np.float32)
    bias = torch.from_numpy(al).to(torch.bfloat16).cuda()
    a = gpu_lib.attn_fwd(q, k, v, score_mod="bias", mask="causal", bias=bias).float()
    b = gpu_lib.attn_fwd(q, k, v, score_mod="alibi", mask="causal").float()
    assert (a - b).abs().max().item() < 3e-2


def test_zero_bias_equals_plain(gpu_lib):
    B, H, S, D = 2, 4, 200, 64
    x = wi.attention_inputs(B, H, H, S, S, D)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    z = torch.zeros((1, 1, S, S), dtype=torch.bfloat16, device="cuda")
    for mask in ("none", "causal"):
        a = gpu_lib.attn_fwd(q, k, v, score_mod="bias", mask=mask, bias=z).float()
        b = gpu_lib.attn_fwd(q, k, v, mask=mask).float()
        assert (a - b).abs().max().item() < 1e-2


def test_deterministic(gpu_lib):
    B, H, S, D = 2, 4, 500, 64
    x = wi.attention_inputs(B, H, H, S, S, D)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    bias = to_dev(wi.normal_bf16(19, (B, H, S, S), 2.0))
    r = [gpu_lib.attn_fwd(q, k, v, score_mod="bias", mask="causal", bias=bias) for _ in range(3)]
    assert torch.equal(r[0], r[1]) and torch.equal(r[1], r[2])


@pytest.mark.parametrize("mask", ["none", "causal", "document"])
def test_benchmark_shape_sampled(gpu_lib, mask):
    """16k tokens (B = 4, S = 4096), 16 heads, one bias shared by batch and heads."""
    S = 4096
    rows = sample_rows(S, tiles=(128,), extra=24, seed=8)[::2]
    _run(gpu_lib, 4, 16, 16, S, 64, mask, "shared", rows=rows)


def test_full_bias_larger(gpu_lib):
    _run(gpu_lib, 2, 4, 4, 1024, 64, "causal", "full", rows=sample_rows(1024, tiles=(128,), extra=16, seed=9))


def test_bias_base_8_byte_aligned(gpu_lib):
    """A bias whose storage starts 8 bytes past a 16-byte boundary (the ABI
    asks for 8-byte alignment), with Skv a multiple of 8: every (b, h) slice
    then starts at 8 mod 16, where the staged bias tile must read its rows
    with narrower loads than its 16-byte row chunks."""
    B, H, S, D = 2, 4, 136, 64
    x = wi.attention_inputs(B, H, H, S, S, D)
    bb = wi.normal_bf16(18, (B, H, S, S), 2.0)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    store = torch.zeros(bb.size + 4, dtype=torch.bfloat16, device="cuda")
    bias = store[4:].view(B, H, S, S)
    bias.copy_(to_dev(bb))
    assert bias.data_ptr() % 16 == 8
    for mask in ("none", "causal"):
        out = gpu_lib.attn_fwd(q, k, v, score_mod="bias", mask=mask, bias=bias)
        torch.cuda.synchronize()
        ref, _ = oracle.attention(f64(x["q"]), f64(x["k"]), f64(x["v"]), score_mod="bias", mask=mask, bias=f64(bb))
        assert_close(out.float().cpu().numpy(), ref, f"bias at 8 mod 16 bytes, {mask}")
