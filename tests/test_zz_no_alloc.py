"""The allocation-free decode entry point ``attn_decode_fwd_noalloc`` (through
the C ABI) against ``attn_decode_fwd``, the entry point it mirrors: the same
kernels and plan, so the outputs must be bit-identical.  Two calls in a row,
the second on a smaller input, show that the static split-KV array keeps no
state that a later call depends on; a long-cache call is also checked
against the fp64 oracle.
"""

import pytest
import torch

import oracle
from workloads import inputs as wi

from .gpu_util import assert_close, canary_empty, canary_intact, f64, to_dev

pytestmark = pytest.mark.gpu

D = 64
SCRATCH_BYTES = 8650752  # the static array's size stated in include/attnvar.h


def _inputs(B, Hq, Hkv, Sq, Skv, seed):
    x = wi.attention_inputs(B, Hq, Hkv, Sq, Skv, D, seeds=seed)
    return x, tuple(to_dev(x[n]) for n in ("q", "k", "v"))


def _both(av, B, Hq, Hkv, Sq, Skv, score_mod, mask, seed):
    """Run the allocation-free call, then the workspace call; return both outputs."""
    print(f"noalloc decode B{B} Hq{Hq} Hkv{Hkv} Sq{Sq} Skv{Skv} {score_mod}/{mask}", flush=True)
    x, (q, k, v) = _inputs(B, Hq, Hkv, Sq, Skv, seed)
    out, big = canary_empty((B, Hq, Sq, D), torch.bfloat16)
    lse, bigl = canary_empty((B, Hq, Sq), torch.float32)
    av.attn_decode_fwd_noalloc(q, k, v, out, score_mod=score_mod, mask=mask, lse=lse)
    torch.cuda.synchronize()
    assert canary_intact(big, out.numel()) and canary_intact(bigl, lse.numel())
    ref_out, ref_lse = av.attn_decode_fwd(q, k, v, score_mod=score_mod, mask=mask, return_lse=True)
    torch.cuda.synchronize()
    return x, out, lse, ref_out, ref_lse


def test_noalloc_matches_workspace_entry_point(gpu_lib):
    # (B, Hq, Hkv, Sq, Skv): the first uses 4.3 MB of the array (64 key
    # splits), the second, smaller one 1.35 MB (10 splits), the third none
    # (512 (batch, KV head) units fill the chip without a split)
    cases = [((1, 32, 8, 1, 16384), "softcap", "causal", (5, 6, 7)),
             ((2, 32, 8, 2, 3001), "alibi", "none", (8, 9, 10)),
             ((64, 32, 8, 1, 700), "none", "causal", (11, 12, 13))]
    for i, (shape, sm, mk, seed) in enumerate(cases):
        need = gpu_lib.attn_decode_workspace_bytes(*shape, D)
        assert need <= SCRATCH_BYTES
        if i < 2:
            assert need > 0, "the case must exercise the static array"
        x, out, lse, ref_out, ref_lse = _both(gpu_lib, *shape, sm, mk, seed)
        assert torch.equal(out, ref_out), f"case {i}: outputs differ from attn_decode_fwd"
        assert torch.equal(lse, ref_lse), f"case {i}: lse differs from attn_decode_fwd"
        if i == 0:
            B, Hq, Hkv, Sq, Skv = shape
            ref, _ = oracle.attention(f64(x["q"]), f64(x["k"]), f64(x["v"]), score_mod=sm, mask=mk,
                                      q_offset=Skv - Sq)
            assert_close(out.float().cpu().numpy(), ref, "noalloc decode vs oracle")

