"""GPU parity of ``attn_decode_paged_fwd`` (decoding against a paged key/value
cache with per-sequence lengths) against the fp64 oracle, through the C ABI.

Pages are handed out in a random order, lengths are not multiples of the page
size, and every query row is checked.  Gate: |gpu - oracle| <= 1e-2 +
1e-2 |oracle|; LSE within 1e-3.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import inputs as wi

from .gpu_util import assert_close, canary_empty, canary_intact, f64, to_dev

pytestmark = pytest.mark.gpu

LSE_ATOL = 1e-3


def _paged_case(B, Hq, Hkv, Sq, lens, ps, seed=9):
    """Random cache content, pages assigned to sequences in a shuffled order."""
    D = 64
    maxp = max((n + ps - 1) // ps for n in lens) + 1  # one spare column in the table
    npages = sum((n + ps - 1) // ps for n in lens) + 3  # a few pages nobody uses
    x = wi.attention_inputs(npages, Hkv, Hkv, ps, ps, D, seeds=(seed, seed + 1, seed + 2))
    kc, vc = x["k"], x["v"]                 # [npages, Hkv, ps, D] bf16 bits
    q = wi.attention_inputs(B, Hq, Hkv, Sq, 1, D, seeds=(seed + 3, seed + 4, seed + 5))["q"]
    rng = np.random.default_rng(seed)
    order = rng.permutation(npages)
    bt = np.full((B, maxp), -1, dtype=np.int32)  # unused entries hold -1 (never read)
    nxt = 0
    for b, n in enumerate(lens):
        for p in range((n + ps - 1) // ps):
            bt[b, p] = order[nxt]
            nxt += 1
    return q, kc, vc, bt, np.asarray(lens, dtype=np.int32), npages


def _run(av, B, Hq, Hkv, Sq, lens, ps, score_mod, mask):
    q, kc, vc, bt, sl, npages = _paged_case(B, Hq, Hkv, Sq, lens, ps)
    out, big = canary_empty((B, Hq, Sq, 64), torch.bfloat16)
    lse, bigl = canary_empty((B, Hq, Sq), torch.float32)
    av.attn_decode_paged_fwd(to_dev(q), to_dev(kc), to_dev(vc), torch.from_numpy(bt).cuda(),
                             torch.from_numpy(sl).cuda(), score_mod=score_mod, mask=mask, out=out, lse=lse)
    torch.cuda.synchronize()
    assert canary_intact(big, out.numel()) and canary_intact(bigl, lse.numel())
    ref, ref_lse = oracle.paged_decode_attention(f64(q), f64(kc), f64(vc), np.where(bt < 0, 0, bt), sl,
                                                 page_size=ps, score_mod=score_mod, mask=mask)
    what = f"paged {score_mod}/{mask} B{B} Hq{Hq} Hkv{Hkv} Sq{Sq} ps{ps} lens{list(lens)[:4]}"
    assert_close(out.float().cpu().numpy(), ref, what)
    assert_close(lse.cpu().numpy(), ref_lse, what + " lse", atol=LSE_ATOL, rtol=1e-5)


@pytest.mark.parametrize("ps", [16, 32, 64])
@pytest.mark.parametrize("score_mod", ["none", "alibi", "softcap"])
def test_paged_parity(gpu_lib, ps, score_mod):
    for mask in ("none", "causal"):
        _run(gpu_lib, 3, 32, 8, 1, [700, 1, 129], ps, score_mod, mask)
        _run(gpu_lib, 2, 8, 2, 4, [64, 333], ps, score_mod, mask)


def test_paged_long_and_many(gpu_lib):
    _run(gpu_lib, 1, 32, 8, 1, [16000], 16, "softcap", "causal")   # keys split over workgroups
    rng = np.random.default_rng(3)
    lens = rng.integers(1, 2000, size=48).tolist()
    _run(gpu_lib, 48, 32, 8, 2, lens, 32, "none", "causal")


def test_paged_equals_dense(gpu_lib):
    """A cache whose pages are stored in order equals the dense decode path."""
    B, Hq, Hkv, Sq, S, ps = 2, 16, 4, 2, 512, 64
    x = wi.attention_inputs(B, Hq, Hkv, Sq, S, 64)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    npg = S // ps
    kc = k.view(B, Hkv, npg, ps, 64).permute(0, 2, 1, 3, 4).reshape(B * npg, Hkv, ps, 64).contiguous()
    vc = v.view(B, Hkv, npg, ps, 64).permute(0, 2, 1, 3, 4).reshape(B * npg, Hkv, ps, 64).contiguous()
    bt = torch.arange(B * npg, dtype=torch.int32, device="cuda").view(B, npg)
    sl = torch.full((B,), S, dtype=torch.int32, device="cuda")
    a = gpu_lib.attn_decode_paged_fwd(q, kc, vc, bt, sl, score_mod="softcap", mask="causal")
    b = gpu_lib.attn_decode_fwd(q, k, v, score_mod="softcap", mask="causal")
    torch.cuda.synchronize()
    assert torch.equal(a, b)
