"""GPU tests of the document-mask work order (``attn_doc_order``) and of
``attn_fwd`` visiting its query tiles in that order, through the C ABI.

The order is unique (descending key-tile count, ties by ascending index), so
it is compared exactly with a host recomputation of each 128-row query
tile's key range from the document ids: keys from the start of the first
row's document to the end of the last row's, in 64-key tiles.  The order
changes only when each workgroup runs, so ``attn_fwd`` with it must equal
``attn_fwd`` without it bit for bit; one case is also checked against the
fp64 oracle.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import inputs as wi

from .gpu_util import assert_close, f64, to_dev

pytestmark = pytest.mark.gpu

BM, BN = 128, 64


def expected_order(doc):
    B, S = doc.shape
    nM, nKV = -(-S // BM), -(-S // BN)
    cost = np.empty(B * nM, dtype=np.int64)
    for b in range(B):
        row = doc[b]
        for t in range(nM):
            q0, ql = t * BM, min(S, t * BM + BM) - 1
            kstart = int(np.searchsorted(row, row[q0], "left"))
            kend = int(np.searchsorted(row, row[ql], "right"))
            cost[b * nM + t] = min(nKV, -(-kend // BN)) - kstart // BN
    return np.array(sorted(range(B * nM), key=lambda i: (-cost[i], i)), dtype=np.int64), cost


def _check_order(av, doc):
    got = av.attn_doc_order(torch.from_numpy(doc).cuda())
    torch.cuda.synchronize()
    want, cost = expected_order(doc)
    g = got.cpu().numpy().astype(np.int64)
    assert np.array_equal(np.sort(g), np.arange(len(want))), "not a permutation"
    assert np.array_equal(g, want), f"first difference at {int(np.argmax(g != want))}"
    return g, cost


@pytest.mark.parametrize("B,S,lo", [(4, 4096, 64), (32, 512, 64), (1, 16384, 64), (3, 300, 4), (2, 1, 1),
                                    (8, 2048, 64), (2, 1000, 700)])
def test_order_matches_key_ranges(gpu_lib, B, S, lo):
    _check_order(gpu_lib, wi.doc_ids(4, B, S, lo=lo))


def test_order_degenerate_layouts(gpu_lib):
    # one document per row: every tile spans every key, the order is the identity
    g, _ = _check_order(gpu_lib, np.zeros((3, 1000), dtype=np.int32))
    assert np.array_equal(g, np.arange(len(g)))
    # every token its own document
    _check_order(gpu_lib, np.tile(np.arange(777, dtype=np.int32), (2, 1)))
    # document ids that skip values and start above zero
    _check_order(gpu_lib, (wi.doc_ids(5, 2, 900, lo=10) * 7 + 3).astype(np.int32))


def test_order_largest(gpu_lib):
    """16384 query tiles, the most one order holds (2^21 tokens in one row)."""
    S = 16384 * BM
    doc = wi.doc_ids(6, 1, S, lo=4096, hi=1 << 18)
    _check_order(gpu_lib, doc)


def _fwd_pair(av, B, Hq, Hkv, S, D, score_mod="none", seed=4, lo=64, bias=None):
    x = wi.attention_inputs(B, Hq, Hkv, S, S, D)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    doc = torch.from_numpy(wi.doc_ids(seed, B, S, lo=lo)).cuda()
    order = av.attn_doc_order(doc)
    kw = dict(score_mod=score_mod, mask="document", doc_id=doc, softcap=20.0, bias=bias, return_lse=True)
    o0, l0 = av.attn_fwd(q, k, v, **kw)
    o1, l1 = av.attn_fwd(q, k, v, doc_order=order, **kw)
    torch.cuda.synchronize()
    what = f"{score_mod}/document B{B} Hq{Hq} Hkv{Hkv} S{S} D{D}"
    assert torch.equal(o0, o1), what + ": output differs with the order"
    assert torch.equal(l0, l1), what + ": lse differs with the order"
    return x, doc, o1, l1


@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("score_mod", ["none", "alibi", "softcap"])
def test_fwd_same_bits_with_order(gpu_lib, D, score_mod):
    for (B, Hq, Hkv, S, lo) in ((2, 4, 2, 300, 16), (3, 8, 8, 1000, 64), (1, 2, 1, 129, 8)):
        _fwd_pair(gpu_lib, B, Hq, Hkv, S, D, score_mod, lo=lo)


def test_fwd_same_bits_with_order_bias(gpu_lib):
    B, H, S = 2, 4, 500
    bias = to_dev(wi.normal_bf16(18, (B, H, S, S), 2.0))
    _fwd_pair(gpu_lib, B, H, H, S, 64, "bias", lo=32, bias=bias)


@pytest.mark.parametrize("Hkv", [16, 2])
def test_fwd_benchmark_shape_with_order(gpu_lib, Hkv):
    """16k tokens (B = 4, S = 4096), 16 query heads, MHA and GQA."""
    _fwd_pair(gpu_lib, 4, 16, Hkv, 4096, 64)


def test_fwd_with_order_against_oracle(gpu_lib):
    B, Hq, Hkv, S, D = 2, 4, 2, 640, 64
    x, doc, out, lse = _fwd_pair(gpu_lib, B, Hq, Hkv, S, D, lo=40)
    ref, ref_lse = oracle.attention(f64(x["q"]), f64(x["k"]), f64(x["v"]), mask="document",
                                    doc_id=doc.cpu().numpy())
    assert_close(out.float().cpu().numpy(), ref, "document with order")
    assert_close(lse.cpu().numpy(), ref_lse, "document with order lse", atol=1e-3, rtol=1e-5)
