"""GPU parity of ``attn_decode_fwd`` (decoding: the Sq queries are the last Sq
positions of the Skv keys) against the fp64 oracle with q_offset = Skv - Sq,
through the C ABI.  Every query row is checked (Sq is small).

Gate: |gpu - oracle| <= 1e-2 + 1e-2 |oracle|; LSE within 1e-3 (the row sums
add the fp32 exponentials).
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import inputs as wi

from .gpu_util import assert_close, canary_empty, canary_intact, f64, to_dev

pytestmark = pytest.mark.gpu

LSE_ATOL = 1e-3
SHAPES = [  # B, Hq, Hkv, Sq, Skv
    (1, 32, 8, 1, 4096),     # one sequence: keys split over many workgroups
    (3, 32, 8, 2, 1000),
    (2, 16, 16, 1, 300),
    (1, 8, 1, 4, 129),
    (4, 4, 2, 8, 63),
    (2, 32, 8, 1, 1),
    (128, 32, 8, 1, 256),    # many sequences: one split
]


def _run(av, B, Hq, Hkv, Sq, Skv, score_mod, mask, seed=(5, 6, 7)):
    D = 64
    xq = wi.attention_inputs(B, Hq, Hkv, Sq, Skv, D, seeds=seed)
    q, k, v = (to_dev(xq[n]) for n in ("q", "k", "v"))
    out, big = canary_empty((B, Hq, Sq, D), torch.bfloat16)
    lse, bigl = canary_empty((B, Hq, Sq), torch.float32)
    av.attn_decode_fwd(q, k, v, score_mod=score_mod, mask=mask, out=out, lse=lse)
    torch.cuda.synchronize()
    assert canary_intact(big, out.numel()), "write past the end of out"
    assert canary_intact(bigl, lse.numel()), "write past the end of lse"
    ref, ref_lse = oracle.attention(f64(xq["q"]), f64(xq["k"]), f64(xq["v"]), score_mod=score_mod, mask=mask,
                                    q_offset=Skv - Sq)
    what = f"decode {score_mod}/{mask} B{B} Hq{Hq} Hkv{Hkv} Sq{Sq} Skv{Skv}"
    assert_close(out.float().cpu().numpy(), ref, what)
    assert_close(lse.cpu().numpy(), ref_lse, what + " lse", atol=LSE_ATOL, rtol=1e-5)
    return out


@pytest.mark.parametrize("score_mod", ["none", "alibi", "softcap"])
@pytest.mark.parametrize("mask", ["none", "causal"])
def test_decode_parity(gpu_lib, score_mod, mask):
    for shape in SHAPES:
        _run(gpu_lib, *shape, score_mod, mask)


def test_decode_long_cache(gpu_lib):
    _run(gpu_lib, 1, 32, 8, 1, 16384, "softcap", "causal")
    _run(gpu_lib, 2, 32, 8, 4, 8191, "none", "causal")


def test_decode_equals_prefill_when_queries_fill_the_keys(gpu_lib):
    """Sq == Skv puts the queries at positions 0..S-1, which is attn_fwd's causal form."""
    B, Hq, Hkv, S, D = 2, 8, 4, 16, 64
    x = wi.attention_inputs(B, Hq, Hkv, S, S, D)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    for sm in ("none", "alibi", "softcap"):
        a = gpu_lib.attn_decode_fwd(q, k, v, score_mod=sm, mask="causal").float()
        b = gpu_lib.attn_fwd(q, k, v, score_mod=sm, mask="causal").float()
        assert (a - b).abs().max().item() < 2e-2, sm


def test_decode_empty_cache(gpu_lib):
    q = torch.zeros(2, 8, 1, 64, dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros(2, 2, 0, 64, dtype=torch.bfloat16, device="cuda")
    out, lse = gpu_lib.attn_decode_fwd(q, kv, kv, return_lse=True)
    torch.cuda.synchronize()
    assert torch.all(out == 0).item()
    assert torch.all(torch.isneginf(lse)).item()


def test_decode_deterministic(gpu_lib):
    x = wi.attention_inputs(1, 32, 8, 1, 5000, 64)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    r = [gpu_lib.attn_decode_fwd(q, k, v, score_mod="softcap", mask="causal") for _ in range(3)]
    assert torch.equal(r[0], r[1]) and torch.equal(r[1], r[2])
