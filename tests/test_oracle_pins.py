"""Pins for the fp64 oracle: checks against things other than the oracle itself.

The Flashlight pages print no worked example, so the oracle is pinned by
hand-derived closed forms (``tests/golden/hand_cases.json``), invariants,
special cases that reduce to simpler attention, a test-only tiled online
softmax (the algebraic transformation the pages describe), and a scalar
brute force on tiny inputs.  Each pin is chosen so that a plausible slip in
the oracle (a dropped scale, a wrong mask inequality, a transposed operand, a
wrong GQA head map, a sign error in ALiBi) fails at least one test.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from workloads import inputs as wi

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")

VARIANTS = [(sm, mk) for sm in oracle.SCORE_MODS for mk in oracle.MASKS]


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _variant_kwargs(mask, S, seed=0):
    kw = {}
    if mask == "sliding_window":
        kw["window"] = max(1, S // 3)
    if mask == "prefix_lm":
        kw["prefix_len"] = S // 4
    if mask == "document":
        kw["doc_id"] = wi.doc_ids(seed + 40, 2, S, lo=1, hi=max(1, S // 2))
    return kw


# ---------------------------------------------------------------- golden
def test_hand_cases():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    assert len(cases) >= 10
    for c in cases:
        if c["kind"] == "attention":
            kw = {kk: c[kk] for kk in ("window", "prefix_len", "softcap", "alibi_max_bias") if kk in c}
            if "doc_id" in c:
                kw["doc_id"] = np.array(c["doc_id"])
            out, lse = oracle.attention(np.array(c["q"]), np.array(c["k"]), np.array(c["v"]),
                                        score_mod=c["score_mod"], mask=c["mask"], scale=c["scale"], **kw)
            np.testing.assert_allclose(out, np.array(c["out"]), rtol=0, atol=1e-12, err_msg=c["name"])
            np.testing.assert_allclose(lse, np.array(c["lse"]), rtol=0, atol=1e-12, err_msg=c["name"])
        elif c["kind"] == "diff":
            out = oracle.diff_attention(np.array(c["q"]), np.array(c["k"]), np.array(c["v"]),
                                        lam=c["lam"], scale=c["scale"], causal=c["causal"])
            np.testing.assert_allclose(out, np.array(c["out"]), rtol=0, atol=1e-12, err_msg=c["name"])
        elif c["kind"] == "evoformer":
            out = oracle.evoformer_row_gated_attention(
                np.array(c["m"]), np.array(c["wq"]), np.array(c["wk"]), np.array(c["wv"]),
                np.array(c["wg"]), np.array(c["bias"]), H=c["H"], dh=c["dh"], scale=c["scale"])
            np.testing.assert_allclose(out, np.array(c["out"]), rtol=0, atol=1e-12, err_msg=c["name"])
        else:
            raise AssertionError(c["kind"])


# ---------------------------------------------------------------- P1
@pytest.mark.parametrize("score_mod,mask", VARIANTS)
def test_p1_rows_sum_to_one(score_mod, mask):
    S, D = 37, 8
    q, k = _rand((S, D), 1), _rand((S, D), 2)
    rows = np.arange(S)
    kw = _variant_kwargs(mask, S)
    s = oracle.raw_scores(q, k, 1 / math.sqrt(D))
    s = oracle.apply_score_mod(s, score_mod, rows, rows, slope=0.3, softcap=2.0)
    a = oracle.allowed_matrix(mask, rows, S, window=kw.get("window", 0), prefix_len=kw.get("prefix_len", 0),
                              doc_row=kw["doc_id"][0] if "doc_id" in kw else None)
    p, lse = oracle.softmax_two_pass(s, a)
    assert np.all(np.abs(p.sum(axis=1) - 1) <= 1e-12)
    assert np.all(p[~a] == 0)
    assert np.all(p >= 0)
    # lse is the log of the partition function over the allowed entries
    ref = np.log(np.where(a, np.exp(s), 0).sum(axis=1))
    np.testing.assert_allclose(lse, ref, rtol=0, atol=1e-12)


def test_p1_fully_masked_row_is_zero():
    s = np.array([[1.0, 2.0], [3.0, 4.0]])
    a = np.array([[False, False], [True, False]])
    p, lse = oracle.softmax_two_pass(s, a)
    assert np.all(p[0] == 0) and lse[0] == -np.inf
    assert p[1, 0] == 1 and lse[1] == 3.0


# ---------------------------------------------------------------- P2
def _online_attention(q, k, v, allowed_fn, mod_fn, scale, block):
    """Test-only fp64 tiled *online* softmax: running max m and running sum l,
    rescaled by exp(m_old - m_new) whenever the max grows (the one-pass form
    that the pages derive from the two-pass one via exp(a - b) = exp(a)/exp(b))."""
    Sq, Skv = q.shape[0], k.shape[0]
    out = np.zeros((Sq, v.shape[1]))
    lse = np.zeros(Sq)
    for i in range(Sq):
        m, l, o = -np.inf, 0.0, np.zeros(v.shape[1])
        for j0 in range(0, Skv, block):
            js = np.arange(j0, min(Skv, j0 + block))
            s = mod_fn(scale * (k[js] @ q[i]), i, js)
            ok = allowed_fn(i, js)
            if not ok.any():
                continue
            m_new = max(m, s[ok].max())
            alpha = math.exp(m - m_new) if m != -np.inf else 0.0
            p = np.where(ok, np.exp(np.where(ok, s, 0) - m_new), 0.0)
            l = alpha * l + p.sum()
            o = alpha * o + p @ v[js]
            m = m_new
        out[i] = o / l if l > 0 else 0.0
        lse[i] = m + math.log(l) if l > 0 else -np.inf
    return out, lse


@pytest.mark.parametrize("score_mod,mask", VARIANTS)
@pytest.mark.parametrize("block", [1, 3, 16])
def test_p2_online_equals_two_pass(score_mod, mask, block):
    S, D = 29, 6
    q, k, v = _rand((1, 1, S, D), 3), _rand((1, 1, S, D), 4), _rand((1, 1, S, 5), 5)
    kw = _variant_kwargs(mask, S)
    slope, cap = oracle.alibi_slope(0, 1, 8.0), 20.0
    ref, ref_lse = oracle.attention(q, k, v, score_mod=score_mod, mask=mask, **kw)
    doc = kw["doc_id"][0] if "doc_id" in kw else None

    def allowed_fn(i, js):
        return oracle.allowed_matrix(mask, np.array([i]), S, window=kw.get("window", 0),
                                     prefix_len=kw.get("prefix_len", 0), doc_row=doc)[0, js]

    def mod_fn(s, i, js):
        if score_mod == "alibi":
            return s + slope * (js - i)
        if score_mod == "softcap":
            return cap * np.tanh(s / cap)
        return s

    out, lse = _online_attention(q[0, 0], k[0, 0], v[0, 0], allowed_fn, mod_fn, 1 / math.sqrt(D), block)
    np.testing.assert_allclose(out, ref[0, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse[0, 0], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- P3
def _allowed_sets(mask, S, window=0, prefix_len=0, doc=None):
    sets = []
    for i in range(S):
        if mask == "none":
            js = range(S)
        elif mask == "causal":
            js = range(0, i + 1)
        elif mask == "sliding_window":
            js = range(max(0, i - window + 1), i + 1)
        elif mask == "prefix_lm":
            js = sorted(set(range(prefix_len)) | set(range(i + 1)))
        elif mask == "document":
            js = [j for j in range(S) if doc[j] == doc[i]]
        sets.append(list(js))
    return sets


@pytest.mark.parametrize("mask", oracle.MASKS)
def test_p3_uniform_scores_give_mean_of_v(mask):
    S, D = 23, 4
    kw = _variant_kwargs(mask, S)
    q = np.zeros((2, 1, S, D))
    k = _rand((2, 1, S, D), 7)
    v = _rand((2, 1, S, 3), 8)
    out, lse = oracle.attention(q, k, v, mask=mask, **kw)
    for b in range(2):
        doc = kw["doc_id"][b] if "doc_id" in kw else None
        sets = _allowed_sets(mask, S, kw.get("window", 0), kw.get("prefix_len", 0), doc)
        for i, js in enumerate(sets):
            np.testing.assert_allclose(out[b, 0, i], v[b, 0, js].mean(axis=0), rtol=0, atol=1e-12)
            assert abs(lse[b, 0, i] - math.log(len(js))) <= 1e-12


# ---------------------------------------------------------------- P4
def test_p4_boundary_special_cases():
    S, D = 19, 8
    q, k, v = _rand((1, 2, S, D), 9), _rand((1, 2, S, D), 10), _rand((1, 2, S, D), 11)
    out, _ = oracle.attention(q, k, v, mask="causal")
    np.testing.assert_allclose(out[0, :, 0], v[0, :, 0], rtol=0, atol=1e-12)
    out, _ = oracle.attention(q, k, v, mask="sliding_window", window=1)
    np.testing.assert_allclose(out, v, rtol=0, atol=1e-12)
    doc = np.arange(S)[None, :]
    out, _ = oracle.attention(q, k, v, mask="document", doc_id=doc)
    np.testing.assert_allclose(out, v, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- P5
def _brute(q, k, v, score_mod, mask, scale, slope, cap, window, prefix_len, doc):
    """Scalar pure-Python attention for one head (lists of lists, math module only)."""
    Sq, Skv, Dv = len(q), len(k), len(v[0])
    out, lses = [], []
    for i in range(Sq):
        scores, ok = [], []
        for j in range(Skv):
            s = 0.0
            for d in range(len(q[i])):
                s += q[i][d] * k[j][d]
            s *= scale
            if score_mod == "alibi":
                s += slope * (j - i)
            elif score_mod == "softcap":
                s = cap * math.tanh(s / cap)
            if mask == "none":
                a = True
            elif mask == "causal":
                a = j <= i
            elif mask == "sliding_window":
                a = 0 <= i - j < window
            elif mask == "prefix_lm":
                a = j < prefix_len or j <= i
            else:
                a = doc[i] == doc[j]
            scores.append(s)
            ok.append(a)
        mx = max(s for s, a in zip(scores, ok) if a)
        w = [math.exp(s - mx) if a else 0.0 for s, a in zip(scores, ok)]
        tot = sum(w)
        out.append([sum(w[j] * v[j][e] for j in range(Skv)) / tot for e in range(Dv)])
        lses.append(mx + math.log(tot))
    return out, lses


@pytest.mark.parametrize("score_mod,mask", VARIANTS)
@pytest.mark.parametrize("S,D", [(1, 1), (2, 4), (3, 64), (5, 4), (8, 1), (16, 64)])
def test_p5_brute_force_tiny(score_mod, mask, S, D):
    Hq, Hkv = 4, 2
    q, k, v = _rand((1, Hq, S, D), 12), _rand((1, Hkv, S, D), 13), _rand((1, Hkv, S, 3), 14)
    kw = _variant_kwargs(mask, S)
    if mask == "sliding_window":
        kw["window"] = max(1, S // 2)
    if mask == "prefix_lm":
        kw["prefix_len"] = S // 3
    cap = 1.5
    out, lse = oracle.attention(q, k, v, score_mod=score_mod, mask=mask, softcap=cap, **kw)
    for hq in range(Hq):
        hk = hq // (Hq // Hkv)
        slope = 2.0 ** (-8.0 * (hq + 1) / Hq)
        doc = list(kw["doc_id"][0]) if "doc_id" in kw else None
        bo, bl = _brute(q[0, hq].tolist(), k[0, hk].tolist(), v[0, hk].tolist(), score_mod, mask,
                        1 / math.sqrt(D), slope, cap, kw.get("window", 0), kw.get("prefix_len", 0), doc)
        np.testing.assert_allclose(out[0, hq], np.array(bo), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[0, hq], np.array(bl), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- P5b: the bias tensor modifier
@pytest.mark.parametrize("mask", oracle.MASKS)
@pytest.mark.parametrize("bshape", ["full", "batch_shared", "head_shared", "shared"])
def test_p5b_bias_brute_force(mask, bshape):
    """Scalar loops with the bias element added to each scaled score."""
    B, Hq, Hkv, S, D = 2, 4, 2, 7, 5
    q, k, v = _rand((B, Hq, S, D), 60), _rand((B, Hkv, S, D), 61), _rand((B, Hkv, S, 3), 62)
    Bb = 1 if bshape in ("batch_shared", "shared") else B
    Hb = 1 if bshape in ("head_shared", "shared") else Hq
    bias = 2.0 * _rand((Bb, Hb, S, S), 63)
    kw = _variant_kwargs(mask, S)
    out, lse = oracle.attention(q, k, v, score_mod="bias", mask=mask, bias=bias, **kw)
    for b in range(B):
        for hq in range(Hq):
            hk = hq // (Hq // Hkv)
            bm = bias[b % Bb, hq % Hb]
            doc = kw["doc_id"][b] if "doc_id" in kw else None
            for i in range(S):
                sc, ok = [], []
                for j in range(S):
                    x = sum(q[b, hq, i, t] * k[b, hk, j, t] for t in range(D)) / math.sqrt(D) + bm[i, j]
                    if mask == "none":
                        a = True
                    elif mask == "causal":
                        a = j <= i
                    elif mask == "sliding_window":
                        a = 0 <= i - j < kw["window"]
                    elif mask == "prefix_lm":
                        a = j < kw["prefix_len"] or j <= i
                    else:
                        a = doc[i] == doc[j]
                    sc.append(x)
                    ok.append(a)
                mx = max(x for x, a in zip(sc, ok) if a)
                w = [math.exp(x - mx) if a else 0.0 for x, a in zip(sc, ok)]
                z = sum(w)
                for e in range(3):
                    assert out[b, hq, i, e] == pytest.approx(sum(w[j] * v[b, hk, j, e] for j in range(S)) / z,
                                                             abs=1e-12)
                assert lse[b, hq, i] == pytest.approx(mx + math.log(z), abs=1e-12)


def test_p5b_bias_reductions():
    """ALiBi written out as a tensor equals the ALiBi modifier (a transposed
    bias flips its sign and fails); a per-row constant leaves the output and
    shifts lse by that constant; a large bias on one key selects that key."""
    B, H, S, D = 1, 3, 19, 8
    q, k, v = _rand((B, H, S, D), 64), _rand((B, H, S, D), 65), _rand((B, H, S, 4), 66)
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    al = np.stack([oracle.alibi_slope(h, H, 8.0) * (j - i) for h in range(H)])[None].astype(np.float64)
    for mask in ("none", "causal"):
        o1, l1 = oracle.attention(q, k, v, score_mod="bias", mask=mask, bias=al)
        o2, l2 = oracle.attention(q, k, v, score_mod="alibi", mask=mask)
        np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)
    o3, _ = oracle.attention(q, k, v, score_mod="bias", bias=al.transpose(0, 1, 3, 2))
    assert np.abs(o3 - o2).max() > 1e-2
    c = 5.0 * _rand((1, 1, S, 1), 67)
    o4, l4 = oracle.attention(q, k, v, score_mod="bias", bias=np.broadcast_to(c, (1, 1, S, S)))
    o5, l5 = oracle.attention(q, k, v)
    np.testing.assert_allclose(o4, o5, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l4, l5 + c[0, 0, :, 0][None, None], rtol=0, atol=1e-12)
    onehot = np.zeros((1, 1, S, S))
    onehot[0, 0, :, 7] = 1e3
    o6, _ = oracle.attention(q, k, v, score_mod="bias", bias=onehot)
    np.testing.assert_allclose(o6, np.broadcast_to(v[:, :, 7:8, :], o6.shape), rtol=0, atol=1e-12)


def test_p5b_bias_rejects_bad_shapes():
    q = np.zeros((2, 4, 5, 3))
    for shape in [(3, 4, 5, 5), (2, 2, 5, 5), (2, 4, 5, 4), (4, 5, 5)]:
        with pytest.raises(ValueError):
            oracle.attention(q, q, q, score_mod="bias", bias=np.zeros(shape))


# ---------------------------------------------------------------- P6
def test_p6_gqa_equals_mha_with_repeated_kv():
    S, D = 21, 8
    q, k, v = _rand((2, 6, S, D), 15), _rand((2, 2, S, D), 16), _rand((2, 2, S, D), 17)
    for mask in oracle.MASKS:
        kw = _variant_kwargs(mask, S)
        a, la = oracle.attention(q, k, v, mask=mask, score_mod="alibi", **kw)
        b, lb = oracle.attention(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), mask=mask,
                                 score_mod="alibi", **kw)
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
        np.testing.assert_allclose(la, lb, rtol=0, atol=1e-12)
    # and a different group map (interleaved) must NOT match in general
    k_inter = np.stack([k[:, 0], k[:, 1]] * 3, axis=1)
    v_inter = np.stack([v[:, 0], v[:, 1]] * 3, axis=1)
    a, _ = oracle.attention(q, k, v)
    c, _ = oracle.attention(q, k_inter, v_inter)
    assert np.abs(a - c).max() > 1e-3


def test_p6_score_mod_reductions():
    S, D = 25, 8
    q, k, v = _rand((1, 3, S, D), 18), _rand((1, 3, S, D), 19), _rand((1, 3, S, D), 20)
    van, lvan = oracle.attention(q, k, v)
    big, lbig = oracle.attention(q, k, v, score_mod="softcap", softcap=1e9)
    np.testing.assert_allclose(big, van, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lbig, lvan, rtol=0, atol=1e-12)
    z, lz = oracle.attention(q, k, v, score_mod="alibi", alibi_max_bias=3000.0)  # slope underflows to 0
    np.testing.assert_allclose(z, van, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lz, lvan, rtol=0, atol=1e-12)
    # steep ALiBi + causal: the nearest key (j = i) dominates -> out[i] = v[i]
    steep, _ = oracle.attention(q[:, :1], k[:, :1], v[:, :1], score_mod="alibi", mask="causal",
                                alibi_max_bias=-math.log2(1e4))
    np.testing.assert_allclose(steep, v[:, :1], rtol=0, atol=1e-12)
    # ALiBi sign: with zero scores and no mask, larger j is favoured (bias grows with j - i)
    zq = np.zeros((1, 1, S, D))
    al, _ = oracle.attention(zq, k[:, :1], np.arange(S, dtype=float).reshape(1, 1, S, 1), score_mod="alibi")
    assert np.all(al[0, 0, :, 0] > (S - 1) / 2)
    # ALiBi slopes: geometric, head h (0-based) gets 2^(-8(h+1)/H)
    assert oracle.alibi_slope(0, 16) == 2.0 ** -0.5 and oracle.alibi_slope(15, 16) == 2.0 ** -8


def test_p6_softcap_via_inverse():
    """Scores chosen as cap*atanh(y) must come out of the soft cap as cap*y."""
    cap = 2.0
    ys = np.array([-0.9, -0.25, 0.0, 0.5, 0.95])
    x = cap * np.arctanh(ys)  # scaled scores before the cap
    S = len(ys)
    q = np.ones((1, 1, 1, 1))
    k = x.reshape(1, 1, S, 1)
    v = np.eye(S).reshape(1, 1, S, S)
    out, lse = oracle.attention(q, k, v, score_mod="softcap", softcap=cap, scale=1.0)
    w = np.exp(cap * ys)
    np.testing.assert_allclose(out[0, 0, 0], w / w.sum(), rtol=0, atol=1e-12)
    assert abs(lse[0, 0, 0] - math.log(w.sum())) < 1e-12
    # the capped score never exceeds the cap
    s = oracle.apply_score_mod(np.array([[1e6, -1e6, 3.0]]), "softcap", np.array([0]), np.arange(3), softcap=cap)
    assert np.all(np.abs(s) <= cap)


def test_p6_mask_reductions():
    S, D = 31, 8
    q, k, v = _rand((1, 2, S, D), 21), _rand((1, 2, S, D), 22), _rand((1, 2, S, D), 23)
    causal, lc = oracle.attention(q, k, v, mask="causal")
    none, ln_ = oracle.attention(q, k, v)
    for P, ref, lref in ((0, causal, lc), (S, none, ln_)):
        o, l_ = oracle.attention(q, k, v, mask="prefix_lm", prefix_len=P)
        np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l_, lref, rtol=0, atol=1e-12)
    for W in (S, S + 5):
        o, l_ = oracle.attention(q, k, v, mask="sliding_window", window=W)
        np.testing.assert_allclose(o, causal, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l_, lc, rtol=0, atol=1e-12)
    o, l_ = oracle.attention(q, k, v, mask="document", doc_id=np.zeros((1, S), dtype=np.int32))
    np.testing.assert_allclose(o, none, rtol=0, atol=1e-12)
    # window W sees exactly W keys once i >= W-1 (off-by-one guard)
    a = oracle.allowed_matrix("sliding_window", np.arange(S), S, window=4)
    assert a.sum(axis=1)[3:].tolist() == [4] * (S - 3) and a.sum(axis=1)[:3].tolist() == [1, 2, 3]
    a = oracle.allowed_matrix("prefix_lm", np.arange(S), S, prefix_len=5)
    assert a[0].sum() == 5 and a[10].sum() == 11


def test_scale_and_rows_sampling():
    S, D = 40, 16
    q, k, v = _rand((1, 1, S, D), 24), _rand((1, 1, S, D), 25), _rand((1, 1, S, D), 26)
    a, _ = oracle.attention(q, k, v, scale=0.5)
    b, _ = oracle.attention(q * 0.5, k, v, scale=1.0)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    d, _ = oracle.attention(q, k, v)
    e, _ = oracle.attention(q / 4.0, k, v, scale=1.0)  # default scale is 1/sqrt(16)
    np.testing.assert_allclose(d, e, rtol=0, atol=1e-12)
    rows = np.array([0, 7, 39])
    f, lf = oracle.attention(q, k, v, mask="causal", rows=rows, row_block=2)
    g, lg = oracle.attention(q, k, v, mask="causal")
    np.testing.assert_allclose(f, g[:, :, rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lf, lg[:, :, rows], rtol=0, atol=1e-12)


def test_oracle_rejects_bad_shapes():
    q = np.zeros((1, 3, 4, 2))
    k = np.zeros((1, 2, 4, 2))
    with pytest.raises(ValueError):
        oracle.attention(q, k, k)
    with pytest.raises(ValueError):
        oracle.attention(np.zeros((1, 2, 4, 2)), np.zeros((1, 2, 5, 2)), np.zeros((1, 2, 5, 2)), mask="causal")


# ---------------------------------------------------------------- P7
def test_p7_diff_reductions():
    S, Dh = 27, 8
    q, k, v = _rand((1, 2, S, 2 * Dh), 27), _rand((1, 2, S, 2 * Dh), 28), _rand((1, 2, S, 12), 29)
    o0 = oracle.diff_attention(q, k, v, lam=0.0)
    ref, _ = oracle.attention(q[..., :Dh], k[..., :Dh], v, mask="causal")
    np.testing.assert_allclose(o0, ref, rtol=0, atol=1e-12)
    o1 = oracle.diff_attention(q, k, v, lam=1.0)
    ref2, _ = oracle.attention(q[..., Dh:], k[..., Dh:], v, mask="causal")
    np.testing.assert_allclose(o1, ref - ref2, rtol=0, atol=1e-12)
    qq = np.concatenate([q[..., :Dh], q[..., :Dh]], axis=-1)
    kk = np.concatenate([k[..., :Dh], k[..., :Dh]], axis=-1)
    o2 = oracle.diff_attention(qq, kk, v, lam=0.8)
    np.testing.assert_allclose(o2, 0.2 * ref, rtol=0, atol=1e-12)
    # default scale is 1/sqrt(half width), not 1/sqrt(full width)
    o3 = oracle.diff_attention(q, k, v, lam=0.0, scale=1 / math.sqrt(Dh))
    np.testing.assert_allclose(o3, o0, rtol=0, atol=1e-12)
    # causal row 0 is (1 - lambda) v[0]
    np.testing.assert_allclose(oracle.diff_attention(q, k, v, lam=0.8)[:, :, 0], 0.2 * v[:, :, 0], atol=1e-12)


# ---------------------------------------------------------------- P7b: full differential head
def _scalar_causal_attention(q, k, v, scale):
    """One head, scalar loops, no max subtraction (tiny, well-scaled inputs)."""
    S, d = q.shape
    out = np.zeros((S, v.shape[1]))
    for i in range(S):
        w = [math.exp(scale * sum(q[i, t] * k[j, t] for t in range(d))) for j in range(i + 1)]
        z = sum(w)
        for e in range(v.shape[1]):
            out[i, e] = sum(w[j] * v[j, e] for j in range(i + 1)) / z
    return out


def test_p7b_lambda_init_schedule():
    # first layer 0.2, approaches 0.8 with depth, increasing
    assert oracle.diff_lambda_init(1) == pytest.approx(0.2, abs=1e-15)
    assert oracle.diff_lambda_init(200) == pytest.approx(0.8, abs=1e-12)
    vals = [oracle.diff_lambda_init(l) for l in range(1, 25)]
    assert all(b > a for a, b in zip(vals, vals[1:]))


def test_p7b_lambda_reparameterisation():
    ln3 = math.log(3.0)
    # exp(ln 3) - exp(0) + 0.2 = 2.2, and with the two pairs swapped 1 - 3 + 0.2
    assert oracle.diff_lambda([ln3, 0, 0], [1, 0, 5], [0, 0, 0], [4, 4, 4], 0.2) == pytest.approx(2.2, abs=1e-12)
    assert oracle.diff_lambda([0, 0, 0], [4, 4, 4], [ln3, 0, 0], [1, 0, 5], 0.2) == pytest.approx(-1.8, abs=1e-12)
    # the dot product, not an elementwise or first-component product
    assert oracle.diff_lambda([0.5, 0.25], [2.0, 4.0], [0, 0], [0, 0], 0.0) == pytest.approx(math.e ** 2 - 1, abs=1e-12)


@pytest.mark.parametrize("a,b,lam_init,eps", [
    (math.log(1.9), 0.0, 0.2, 0.0),   # lambda = 1.1: the head flips the sign of attention
    (0.0, math.log(1.5), 0.2, 0.0),   # lambda = -0.3: same sign
    (math.log(1.9), 0.0, 0.0, 0.0),   # without lambda_init, lambda = 0.9: same sign
    (0.0, math.log(1.5), 0.35, 0.3),  # eps matters: the magnitude of (1 - lambda) survives the norm
])
def test_p7b_identical_halves_closed_form(a, b, lam_init, eps):
    """Q2 = Q1, K2 = K1 make A = (1 - lambda) attn(Q1, K1, V); with attention
    from scalar loops, y = (1 - lambda_init) gamma (1 - lambda) attn / sqrt((1 - lambda)^2 mean(attn^2) + eps)."""
    S, Dh, Dv = 6, 3, 4
    q1, k1, v = _rand((S, Dh), 80) * 0.7, _rand((S, Dh), 81) * 0.7, _rand((S, Dv), 82)
    gamma = 1.0 + 0.3 * _rand(Dv, 83)
    q = np.concatenate([q1, q1], axis=-1)[None, None]
    k = np.concatenate([k1, k1], axis=-1)[None, None]
    lq1, lk1 = np.array([a, 0.0, 0.0]), np.array([1.0, 2.0, 3.0])
    lq2, lk2 = np.array([0.0, 7.0, 0.0]), np.array([9.0, b / 7.0, 1.0])  # lq2 . lk2 = b
    lam = math.exp(a) - math.exp(b) + lam_init
    y = oracle.diff_head(q, k, v[None, None], lq1, lk1, lq2, lk2, lambda_init=lam_init, gamma=gamma, eps=eps)
    att = _scalar_causal_attention(q1, k1, v, 1 / math.sqrt(Dh))
    A = (1.0 - lam) * att
    want = np.zeros((S, Dv))
    for i in range(S):
        rms = math.sqrt(sum(x * x for x in A[i]) / Dv + eps)
        for e in range(Dv):
            want[i, e] = (1.0 - lam_init) * gamma[e] * A[i, e] / rms
    np.testing.assert_allclose(y[0, 0], want, rtol=0, atol=1e-12)
    if eps == 0.0:  # sign of (1 - lambda) decides the sign of every output
        assert np.all(np.sign(y[0, 0] * gamma * att) == np.sign(1.0 - lam))


def test_p7b_row_rms_and_gamma():
    """With eps = 0 and gamma = 1 every output row has RMS |1 - lambda_init|;
    gamma multiplies channelwise after the norm."""
    S, Dh, Dv = 41, 8, 12
    q, k, v = _rand((2, 3, S, 2 * Dh), 84), _rand((2, 3, S, 2 * Dh), 85), _rand((2, 3, S, Dv), 86)
    lv = [0.3 * _rand(Dh, 87 + i) for i in range(4)]
    y = oracle.diff_head(q, k, v, *lv, lambda_init=0.35, eps=0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=-1)), 0.65, rtol=1e-12)
    gamma = 1.0 + 0.2 * _rand(Dv, 91)
    yg = oracle.diff_head(q, k, v, *lv, lambda_init=0.35, eps=0.0, gamma=gamma)
    np.testing.assert_allclose(yg, y * gamma, rtol=1e-12, atol=1e-14)
    # the norm removes any positive scale of V
    np.testing.assert_allclose(oracle.diff_head(q, k, 7.5 * v, *lv, lambda_init=0.35, eps=0.0), y, rtol=1e-10)


def test_p7b_scalar_brute_force():
    """The whole head by scalar loops on a tiny input (distinct halves)."""
    S, Dh, Dv = 5, 2, 3
    q, k, v = _rand((S, 2 * Dh), 92), _rand((S, 2 * Dh), 93), _rand((S, Dv), 94)
    lq1, lk1, lq2, lk2 = (0.4 * _rand(Dh, 95 + i) for i in range(4))
    gamma, lam_init, eps = 1.0 + 0.3 * _rand(Dv, 99), 0.45, 1e-3
    y = oracle.diff_head(q[None, None], k[None, None], v[None, None], lq1, lk1, lq2, lk2,
                         lambda_init=lam_init, gamma=gamma, eps=eps)
    lam = (math.exp(sum(lq1[t] * lk1[t] for t in range(Dh))) - math.exp(sum(lq2[t] * lk2[t] for t in range(Dh)))
           + lam_init)
    a1 = _scalar_causal_attention(q[:, :Dh], k[:, :Dh], v, 1 / math.sqrt(Dh))
    a2 = _scalar_causal_attention(q[:, Dh:], k[:, Dh:], v, 1 / math.sqrt(Dh))
    for i in range(S):
        A = [a1[i, e] - lam * a2[i, e] for e in range(Dv)]
        rms = math.sqrt(sum(x * x for x in A) / Dv + eps)
        for e in range(Dv):
            assert y[0, 0, i, e] == pytest.approx((1 - lam_init) * gamma[e] * A[e] / rms, abs=1e-12)


# ---------------------------------------------------------------- P8
def test_p8_evoformer_reductions():
    Ns, Nr, Cm, H, dh = 3, 11, 16, 2, 4
    m = _rand((Ns, Nr, Cm), 30)
    wq, wk, wv, wg = (_rand((Cm, H * dh), 31 + i) / 4 for i in range(4))
    bias = _rand((H, Nr, Nr), 35)
    base = oracle.evoformer_row_gated_attention(m, wq, wk, wv, wg, bias, H=H, dh=dh)
    # zero gate weights -> sigmoid(0) = 1/2 times the ungated attention
    half = oracle.evoformer_row_gated_attention(m, wq, wk, wv, np.zeros_like(wg), bias, H=H, dh=dh)
    # row-constant bias shifts every score of a row equally: no change
    shifted = oracle.evoformer_row_gated_attention(m, wq, wk, wv, wg, bias + _rand((H, Nr, 1), 36), H=H, dh=dh)
    np.testing.assert_allclose(shifted, base, rtol=0, atol=1e-12)
    # zero bias and zero gate == 1/2 * MHA on the projected q, k, v (head-major channels)
    q, k, v, _ = oracle.evoformer_projections(m, wq, wk, wv, wg)

    def heads(x):
        return x.reshape(Ns, Nr, H, dh).transpose(0, 2, 1, 3)

    mha, _ = oracle.attention(heads(q), heads(k), heads(v))
    z = oracle.evoformer_row_gated_attention(m, wq, wk, wv, np.zeros_like(wg), np.zeros_like(bias), H=H, dh=dh)
    np.testing.assert_allclose(z, 0.5 * mha.transpose(0, 2, 1, 3).reshape(Ns, Nr, H * dh), rtol=0, atol=1e-12)
    # with bias: ungated attention equals 2 * half
    np.testing.assert_allclose(2 * half, _evo_ungated(m, wq, wk, wv, bias, H, dh), rtol=0, atol=1e-12)
    # rows / seqs sampling is exact
    part = oracle.evoformer_row_gated_attention(m, wq, wk, wv, wg, bias, H=H, dh=dh,
                                                rows=np.array([0, 5, 10]), seqs=np.array([2]))
    np.testing.assert_allclose(part, base[[2]][:, [0, 5, 10]], rtol=0, atol=1e-12)


def test_p8_evoformer_column_pins():
    """Column-wise form: every column equals the row-wise form applied to
    the transposed MSA with a zero bias; one sequence gives sigmoid(g) * v;
    zero gate weights halve it; a scalar loop agrees; sampling is exact."""
    Ns, Nr, Cm, H, dh = 5, 4, 16, 2, 4
    m = _rand((Ns, Nr, Cm), 40)
    wq, wk, wv, wg = (_rand((Cm, H * dh), 41 + i) / 4 for i in range(4))
    col = oracle.evoformer_col_gated_attention(m, wq, wk, wv, wg, H=H, dh=dh)
    assert col.shape == (Ns, Nr, H * dh)
    mt = m.transpose(1, 0, 2)
    row_t = oracle.evoformer_row_gated_attention(mt, wq, wk, wv, wg, np.zeros((H, Ns, Ns)), H=H, dh=dh)
    np.testing.assert_allclose(col, row_t.transpose(1, 0, 2), rtol=0, atol=1e-12)
    # a single sequence attends only to itself
    one = oracle.evoformer_col_gated_attention(m[:1], wq, wk, wv, wg, H=H, dh=dh)
    g = m[0] @ wg
    np.testing.assert_allclose(one[0], (1 / (1 + np.exp(-g))) * (m[0] @ wv), rtol=0, atol=1e-12)
    # zero gate weights: half of the ungated attention, checked by a scalar loop
    half = oracle.evoformer_col_gated_attention(m, wq, wk, wv, np.zeros_like(wg), H=H, dh=dh)
    for r in range(Nr):
        q, k, v = m[:, r] @ wq, m[:, r] @ wk, m[:, r] @ wv
        for h in range(H):
            c = slice(h * dh, (h + 1) * dh)
            for i in range(Ns):
                z = [float(q[i, c] @ k[j, c]) / math.sqrt(dh) for j in range(Ns)]
                zm = max(z)
                e = [math.exp(t - zm) for t in z]
                want = sum(e[j] * v[j, c] for j in range(Ns)) / sum(e)
                np.testing.assert_allclose(half[i, r, c], 0.5 * want, rtol=0, atol=1e-12)
    part = oracle.evoformer_col_gated_attention(m, wq, wk, wv, wg, H=H, dh=dh, cols=np.array([3, 1]),
                                                seqs=np.array([0, 4]))
    np.testing.assert_allclose(part, col[[0, 4]][:, [3, 1]], rtol=0, atol=1e-12)


@pytest.mark.parametrize("score_mod", ["none", "alibi", "softcap"])
def test_decode_queries_at_the_end(score_mod):
    """Queries placed at the end of the keys (q_offset = Skv - Sq) equal the
    last rows of the full prefill; one query under the causal mask equals the
    unmasked attention of that query; a scalar loop agrees on a tiny case."""
    B, Hq, Hkv, S, D = 2, 4, 2, 37, 8
    q = _rand((B, Hq, S, D), 50)
    k = _rand((B, Hkv, S, D), 51)
    v = _rand((B, Hkv, S, D), 52)
    for mask in ("none", "causal"):
        full, full_lse = oracle.attention(q, k, v, score_mod=score_mod, mask=mask)
        for Sq in (1, 3, S):
            dec, dec_lse = oracle.attention(q[:, :, S - Sq:], k, v, score_mod=score_mod, mask=mask, q_offset=S - Sq)
            np.testing.assert_allclose(dec, full[:, :, S - Sq:], rtol=0, atol=1e-12)
            np.testing.assert_allclose(dec_lse, full_lse[:, :, S - Sq:], rtol=0, atol=1e-12)
    one_c, _ = oracle.attention(q[:, :, -1:], k, v, score_mod=score_mod, mask="causal", q_offset=S - 1)
    one_n, _ = oracle.attention(q[:, :, -1:], k, v, score_mod=score_mod, mask="none", q_offset=S - 1)
    np.testing.assert_allclose(one_c, one_n, rtol=0, atol=1e-12)
    # scalar loop: two queries at positions 5, 6 over 7 keys, causal
    qs, ks, vs = q[0, 0, :2], k[0, 0, :7], v[0, 0, :7]
    dec, _ = oracle.attention(qs[None, None], ks[None, None], vs[None, None], score_mod=score_mod, mask="causal",
                              q_offset=5)
    slope = oracle.alibi_slope(0, 1)
    for i in range(2):
        pos = 5 + i
        z = []
        for j in range(pos + 1):
            t = float(qs[i] @ ks[j]) / math.sqrt(D)
            if score_mod == "alibi":
                t += slope * (j - pos)
            if score_mod == "softcap":
                t = 20.0 * math.tanh(t / 20.0)
            z.append(t)
        zm = max(z)
        e = [math.exp(t - zm) for t in z]
        want = sum(e[j] * vs[j] for j in range(pos + 1)) / sum(e)
        np.testing.assert_allclose(dec[0, 0, i], want, rtol=0, atol=1e-12)
    with pytest.raises(ValueError):
        oracle.attention(q[:, :, :3], k, v, mask="causal", q_offset=0)


def test_paged_decode_pins():
    """A paged cache equals the dense cache it stores; shuffling the pages
    (with the block table) changes nothing; each sequence only sees its own
    length."""
    B, Hq, Hkv, Sq, D, ps = 3, 4, 2, 2, 8, 4
    lens = [9, 2, 12]
    maxp = 3
    rng = np.random.default_rng(60)
    dense_k = [_rand((1, Hkv, n, D), 61 + b) for b, n in enumerate(lens)]
    dense_v = [_rand((1, Hkv, n, D), 71 + b) for b, n in enumerate(lens)]
    q = _rand((B, Hq, Sq, D), 80)
    npages = B * maxp
    perm = rng.permutation(npages)
    kc = np.zeros((npages, Hkv, ps, D))
    vc = np.zeros((npages, Hkv, ps, D))
    bt = np.zeros((B, maxp), dtype=np.int32)
    for b, n in enumerate(lens):
        for p in range(maxp):
            bt[b, p] = perm[b * maxp + p]
            for s in range(ps):
                j = p * ps + s
                if j < n:
                    kc[bt[b, p], :, s] = dense_k[b][0, :, j]
                    vc[bt[b, p], :, s] = dense_v[b][0, :, j]
    for mask in ("none", "causal"):
        out, lse = oracle.paged_decode_attention(q, kc, vc, bt, lens, page_size=ps, score_mod="softcap", mask=mask)
        for b, n in enumerate(lens):
            ref, ref_lse = oracle.attention(q[b:b + 1], dense_k[b], dense_v[b], score_mod="softcap", mask=mask,
                                            q_offset=n - Sq)
            np.testing.assert_allclose(out[b:b + 1], ref, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse[b:b + 1], ref_lse, rtol=0, atol=1e-12)
    # relabel the pages once more: same result
    perm2 = rng.permutation(npages)
    inv = np.empty_like(perm2)
    inv[perm2] = np.arange(npages)
    out2, _ = oracle.paged_decode_attention(q, kc[perm2], vc[perm2], inv[bt], lens, page_size=ps, mask="causal",
                                            score_mod="softcap")
    out1, _ = oracle.paged_decode_attention(q, kc, vc, bt, lens, page_size=ps, mask="causal", score_mod="softcap")
    np.testing.assert_allclose(out2, out1, rtol=0, atol=1e-12)


@pytest.mark.parametrize("score_mod", ["none", "alibi", "softcap"])
@pytest.mark.parametrize("mask", ["none", "causal", "sliding_window", "prefix_lm", "document"])
def test_backward_matches_finite_differences(score_mod, mask):
    """Central differences of L = sum(out * dout) in float64 pin every gradient
    entry of the backward oracle (GQA 4/2, tiny shapes, softcap cap 2 so that
    the tanh derivative matters)."""
    B, Hq, Hkv, S, D = 1, 4, 2, 6, 3
    q = _rand((B, Hq, S, D), 90)
    k = _rand((B, Hkv, S, D), 91)
    v = _rand((B, Hkv, S, D), 92)
    dout = _rand((B, Hq, S, D), 93)
    kw = dict(score_mod=score_mod, mask=mask, softcap=2.0, alibi_max_bias=8.0, window=3, prefix_len=2,
              doc_id=np.array([[0, 0, 1, 1, 1, 2]]))
    dq, dk, dv = oracle.attention_backward(q, k, v, dout, **kw)

    def loss(qq, kk, vv):
        o, _ = oracle.attention(qq, kk, vv, **kw)
        return float(np.sum(o * dout))

    eps = 1e-6
    for x, gx, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [q, k, v]
            args_m = [q, k, v]
            args_p[which], args_m[which] = xp, xm
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        np.testing.assert_allclose(gx, num, rtol=1e-6, atol=1e-7)


def test_backward_reductions():
    """GQA gradients equal the repeated-MHA gradients summed per KV head; with
    q = 0 (uniform attention, no mask) dv is the column mean of dout."""
    B, Hq, Hkv, S, D = 2, 4, 2, 9, 5
    q = _rand((B, Hq, S, D), 94)
    k = _rand((B, Hkv, S, D), 95)
    v = _rand((B, Hkv, S, D), 96)
    dout = _rand((B, Hq, S, D), 97)
    dq, dk, dv = oracle.attention_backward(q, k, v, dout, mask="causal")
    kr, vr = np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1)
    dq2, dk2, dv2 = oracle.attention_backward(q, kr, vr, dout, mask="causal")
    np.testing.assert_allclose(dq, dq2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, dk2.reshape(B, Hkv, 2, S, D).sum(2), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, dv2.reshape(B, Hkv, 2, S, D).sum(2), rtol=0, atol=1e-12)
    _, _, dv0 = oracle.attention_backward(np.zeros_like(q), k, v, dout)
    want = dout.reshape(B, Hkv, 2, S, D).sum(2).mean(axis=2, keepdims=True)
    np.testing.assert_allclose(dv0, np.broadcast_to(want, dv0.shape), rtol=0, atol=1e-12)


def _evo_ungated(m, wq, wk, wv, bias, H, dh):
    """Independent loop form: per sequence, head and row."""
    Ns, Nr, _ = m.shape
    out = np.zeros((Ns, Nr, H * dh))
    for s in range(Ns):
        q, k, v = m[s] @ wq, m[s] @ wk, m[s] @ wv
        for h in range(H):
            c = slice(h * dh, (h + 1) * dh)
            for i in range(Nr):
                z = np.array([q[i, c] @ k[j, c] / math.sqrt(dh) + bias[h, i, j] for j in range(Nr)])
                w = np.exp(z - z.max())
                out[s, i, c] = (w / w.sum()) @ v[:, c]
    return out


def test_sigmoid_closed_forms():
    assert oracle.sigmoid(np.array(0.0)) == 0.5
    assert abs(oracle.sigmoid(np.array(math.log(3.0))) - 0.75) < 1e-15


# ---------------------------------------------------------------- inputs
def test_bf16_rounding_matches_torch_and_hand_values():
    import torch

    x = np.random.default_rng(0).standard_normal(100000, dtype=np.float32) * 3
    x = np.concatenate([x, np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 65504.0, 1e-40, 0.0, -0.0],
                                    dtype=np.float32)])
    ours = wi.bf16_bits_from_f32(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    hand = wi.bf16_bits_to_f64(wi.bf16_bits_from_f32(np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8], np.float32)))
    assert hand.tolist() == [1.0, 1.015625]  # ties to even


def test_doc_ids_recipe():
    S = 4096
    ids = wi.doc_ids(4, 4, S)
    lens = wi.doc_lengths(4, 4, S)
    assert ids.shape == (4, S) and ids.dtype == np.int32
    for b in range(4):
        assert np.all(np.diff(ids[b]) >= 0) and ids[b, 0] == 0
        assert sum(lens[b]) == S
        assert all(64 <= L <= S // 2 for L in lens[b][:-1])
        assert 1 <= lens[b][-1] <= S // 2
    assert np.array_equal(ids, wi.doc_ids(4, 4, S))
