"""C-ABI boundary tests that need no GPU: the library loads, exports every
function ``include/attnvar.h`` declares, and rejects every invalid argument
with the documented status before anything is launched."""

import ctypes
import os
import re

import pytest

import attention_variants_amd as av

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "attnvar.h")

# Fake, aligned, non-null device addresses: validation fails before any use.
P = 0x10000
P2 = 0x20000
P3 = 0x30000
P4 = 0x40000


@pytest.fixture(scope="module")
def lib():
    return av.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char\s*\*|const char\s*\*)\s*\*?\s*(\w+)\s*\(", text, re.M)
    return sorted(set(names))


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert set(declared) == set(av.EXPORTED), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings(lib):
    assert lib.av_abi_version() == 4
    for code, name in av.STATUS.items():
        assert lib.av_status_string(code).decode().startswith(name)
    assert lib.av_status_string(12345).decode() == "unknown av_status"


def _attn(lib, var=None, q=P, k=P2, v=P3, o=P4, lse=None, B=1, Hq=2, Hkv=2, Sq=128, Skv=128, D=64):
    if var is None:
        var = av.make_variant()
    ref = None if var == "null" else ctypes.byref(var)
    return lib.attn_fwd(ref, q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, D, None)


def test_attn_fwd_rejections(lib):
    assert _attn(lib, var="null") == -1
    assert _attn(lib, q=None) == -1
    assert _attn(lib, k=None) == -1
    assert _attn(lib, v=None) == -1
    assert _attn(lib, o=None) == -1
    assert _attn(lib, k=None, v=None, Skv=0, Sq=0) == 0  # empty tensors may be NULL
    assert _attn(lib, av.make_variant(mask="document")) == -1  # doc_id missing
    # shapes
    assert _attn(lib, B=0) == -2
    assert _attn(lib, Hq=3, Hkv=2) == -2
    assert _attn(lib, Sq=-1) == -2
    assert _attn(lib, av.make_variant(kv_group=3), Hq=4, Hkv=2) == -2
    assert _attn(lib, av.make_variant(kv_group=2), Hq=4, Hkv=2, Sq=0) == 0  # empty: nothing launched
    assert _attn(lib, av.make_variant(mask="causal"), Sq=128, Skv=64) == -2
    # unsupported
    assert _attn(lib, D=48) == -3
    assert _attn(lib, D=256) == -3
    bad = av.make_variant()
    bad.score_mod = 7
    assert _attn(lib, bad) == -3
    bad = av.make_variant()
    bad.mask = -1
    assert _attn(lib, bad) == -3
    # params
    assert _attn(lib, av.make_variant(score_mod="softcap", softcap=0.0)) == -7
    assert _attn(lib, av.make_variant(score_mod="softcap", softcap=float("nan"))) == -7
    assert _attn(lib, av.make_variant(scale=-1.0)) == -7
    assert _attn(lib, av.make_variant(scale=float("inf"))) == -7
    assert _attn(lib, av.make_variant(score_mod="alibi", alibi_max_bias=float("inf"))) == -7
    assert _attn(lib, av.make_variant(mask="sliding_window", window=0)) == -7
    assert _attn(lib, av.make_variant(mask="prefix_lm", prefix_len=129)) == -7
    assert _attn(lib, av.make_variant(mask="prefix_lm", prefix_len=-1)) == -7
    # alignment
    assert _attn(lib, q=P + 8) == -4
    assert _attn(lib, o=P4 + 2) == -4
    assert _attn(lib, lse=P + 2) == -4
    # sizes beyond 32-bit slice addressing
    assert _attn(lib, Sq=1 << 24, Skv=1 << 24, D=128) == -8
    assert _attn(lib, Skv=1 << 24, D=128) == -8
    # empty query set is a no-op success
    assert _attn(lib, Sq=0, Skv=0) == 0


def test_bias_score_mod_rejections(lib):
    def var(bias=0x60000, bs=0, hs=128 * 128, mask="none"):
        v = av.make_variant("bias", mask)
        v.bias = bias
        v.bias_batch_stride = bs
        v.bias_head_stride = hs
        return v

    assert _attn(lib, var(bias=None)) == -1
    assert _attn(lib, var(bias=None), Sq=0, Skv=0) == 0          # nothing to read
    assert _attn(lib, var(bs=-4)) == -7
    assert _attn(lib, var(hs=-1)) == -7
    assert _attn(lib, var(bias=0x60000 + 4)) == -4              # 8-byte alignment
    assert _attn(lib, var(hs=128 * 128 + 2)) == -4              # Skv % 4 == 0: strides multiple of 4
    assert _attn(lib, var(hs=0), Sq=1 << 15, Skv=1 << 15) == -8  # one slice beyond 32-bit offsets
    # Skv odd: rows are read 16 bits at a time and any stride passes the
    # alignment check (the call still stops at the size check, before a launch)
    assert _attn(lib, var(hs=7, bs=3), Sq=1 << 15, Skv=(1 << 15) + 1) == -8
    bad = var()
    bad.score_mod = 4
    assert _attn(lib, bad) == -3
    # the decode and backward entry points do not take the bias modifier
    ref = ctypes.byref(var())
    assert lib.attn_decode_fwd(ref, P, P2, P3, P4, None, 0x200000, 1 << 30, 1, 32, 8, 1, 4096, 64, None) == -3
    assert lib.attn_bwd(ref, P, P2, P3, P4, 0x70000, P, P2, P3, 0x200000, 1 << 30, 1, 2, 2, 64, 64, 64,
                        None) == -3


def test_doc_order_rejections(lib):
    assert lib.attn_doc_order_len(0, 128) == -2
    assert lib.attn_doc_order_len(2, -1) == -2
    assert lib.attn_doc_order_len(1, 0) == 0
    assert lib.attn_doc_order_len(4, 4096) == 4 * 32
    assert lib.attn_doc_order_len(3, 129) == 3 * 2                  # ragged last tile
    assert lib.attn_doc_order_len(1, 16384 * 128) == 16384          # the largest order
    assert lib.attn_doc_order_len(1, 16384 * 128 + 1) == -8
    assert lib.attn_doc_order_len(2, 2**31 - 1) == -8               # no int overflow
    assert lib.attn_doc_order(None, 1, 0, None, 0, None) == 0       # empty: nothing launched
    assert lib.attn_doc_order(None, 2, 256, P2, 4, None) == -1
    assert lib.attn_doc_order(P, 2, 256, None, 4, None) == -1
    assert lib.attn_doc_order(P + 2, 2, 256, P2, 4, None) == -4
    assert lib.attn_doc_order(P, 2, 256, P2 + 2, 4, None) == -4
    assert lib.attn_doc_order(P, 2, 256, P2, 3, None) == -5          # order_len < B * ceil(S/128)
    assert lib.attn_doc_order(P, 0, 256, P2, 4, None) == -2
    assert lib.attn_doc_order(P, 200, 16384, P2, 1 << 30, None) == -8
    # attn_fwd takes an order only with the document mask, 4-byte aligned
    v = av.make_variant(mask="causal")
    v.doc_order = 0x80000
    assert _attn(lib, v) == -7
    v = av.make_variant(mask="document")
    v.doc_id = 0x90000
    v.doc_order = 0x80002
    assert _attn(lib, v) == -4
    # the order's length must be attn_doc_order_len(B, Sq) of this call
    v.doc_order = 0x80000
    for n in (0, 1, 3, 5, 1 << 20):
        v.doc_order_len = n
        assert _attn(lib, v, B=2, Sq=256, Skv=256) == -7, n
    v.doc_order_len = 2
    assert _attn(lib, v, B=1, Sq=257, Skv=257) == -7      # 3 tiles of 128 rows
    v.doc_order_len = 4
    assert _attn(lib, v, B=2, Sq=256, Skv=256, Hq=2, Hkv=4) == -2  # shape errors come first
    assert av.attn_doc_order_len(4, 4096) == 128
    with pytest.raises(RuntimeError):
        av.attn_doc_order_len(1, 16384 * 128 + 1)


def test_diff_attn_rejections(lib):
    def call(q=P, k=P2, v=P3, o=P4, B=1, H=2, S=64, Dh=64, Dv=128, lam=0.8, scale=0.0):
        return lib.diff_attn_fwd(q, k, v, o, B, H, S, Dh, Dv, lam, scale, 1, None)

    assert call(q=None) == -1
    assert call(o=None) == -1
    assert call(B=0) == -2
    assert call(S=-3) == -2
    assert call(Dh=16) == -3
    assert call(Dv=96) == -3
    assert call(lam=float("nan")) == -7
    assert call(scale=-2.0) == -7
    assert call(k=P2 + 4) == -4
    assert call(S=0) == 0


def test_diff_head_rejections(lib):
    L1, L2, L3, L4, G = 0x50000, 0x50100, 0x50200, 0x50300, 0x50400

    def call(q=P, k=P2, v=P3, lq1=L1, lk1=L2, lq2=L3, lk2=L4, gamma=G, o=P4, B=1, H=2, S=64, Dh=64, Dv=128,
             lam_init=0.2, eps=1e-5, scale=0.0):
        return lib.diff_head_fwd(q, k, v, lq1, lk1, lq2, lk2, gamma, o, B, H, S, Dh, Dv, lam_init, eps, scale, 1,
                                 None)

    assert call(q=None) == -1
    assert call(lq1=None) == -1
    assert call(lk2=None) == -1
    assert call(B=0) == -2
    assert call(Dh=48) == -3
    assert call(Dv=96) == -3
    assert call(lam_init=float("inf")) == -7
    assert call(eps=0.0) == -7
    assert call(eps=-1e-5) == -7
    assert call(eps=float("nan")) == -7
    assert call(lk1=L2 + 2) == -4
    assert call(gamma=G + 1) == -4
    assert call(v=P3 + 8) == -4
    assert call(S=0) == 0
    assert call(S=0, gamma=None) == 0


def test_evoformer_rejections(lib):
    need = lib.evoformer_workspace_bytes(128, 256, 8, 32)
    assert need == 4 * 128 * 256 * 8 * 32 * 2
    assert lib.evoformer_workspace_bytes(0, 256, 8, 32) == 0

    def call(m=P, w=P2, bias=P3, out=P4, ws=0x100000, wsb=None, Ns=2, Nr=16, Cm=64, H=4, dh=32, scale=0.0):
        if wsb is None:
            wsb = lib.evoformer_workspace_bytes(max(Ns, 1), max(Nr, 1), max(H, 1), max(dh, 1))
        return lib.evoformer_gated_attn_fwd(m, w, w, w, w, bias, out, ws, wsb, Ns, Nr, Cm, H, dh, scale, None)

    assert call(m=None) == -1
    assert call(w=None) == -1
    assert call(bias=None) == -1
    assert call(Ns=0) == -2
    assert call(dh=48) == -3
    assert call(Cm=48) == -3
    assert call(H=2) == -3  # H*dh must be a multiple of 128
    assert call(scale=float("nan")) == -7
    assert call(m=P + 2) == -4
    assert call(ws=None) == -5
    assert call(wsb=100) == -5
    assert call(ws=0x100000 + 16) == -4


def test_decode_rejections(lib):
    assert lib.attn_decode_workspace_bytes(1, 32, 8, 1, 4096, 64) > 0     # few KV heads: keys split
    assert lib.attn_decode_workspace_bytes(64, 32, 8, 1, 4096, 64) == 0   # enough workgroups: one split
    assert lib.attn_decode_workspace_bytes(0, 32, 8, 1, 4096, 64) == 0

    def call(score_mod=0, mask=1, q=P, k=P2, v=P3, out=P4, lse=None, ws=0x200000, wsb=1 << 30, B=1, Hq=32,
             Hkv=8, Sq=1, Skv=4096, D=64, scale=0.0):
        var = av.AvVariant(score_mod, mask, scale, 20.0, 8.0, 256, 0, None, 0)
        return lib.attn_decode_fwd(ctypes.byref(var), q, k, v, out, lse, ws, wsb, B, Hq, Hkv, Sq, Skv, D, None)

    assert call(q=None) == -1
    assert call(k=None) == -1
    assert call(mask=2) == -3          # only none and causal
    assert call(score_mod=7) == -3
    assert call(Hq=30) == -2           # Hq not a multiple of Hkv
    assert call(Skv=0, Sq=1) == -2     # causal queries must lie inside the keys
    assert call(D=128) == -3
    assert call(Sq=9) == -3            # 4 heads x 9 queries > 32 rows
    assert call(scale=float("nan")) == -7
    assert call(out=P4 + 2) == -4
    assert call(ws=None) == -5         # B=1: the keys are split, a workspace is needed
    assert call(wsb=16) == -5
    assert call(ws=0x200000 + 8) == -4
    assert call(Sq=0) == 0


def test_paged_decode_rejections(lib):
    assert lib.attn_decode_paged_workspace_bytes(1, 32, 8, 1, 64, 16, 1024) > 0
    assert lib.attn_decode_paged_workspace_bytes(1, 32, 8, 1, 64, 0, 1024) == 0

    def call(score_mod=2, mask=1, q=P, k=P2, v=P3, bt=0x50000, sl=0x60000, out=P4, ws=0x200000, wsb=1 << 30, B=1,
             Hq=32, Hkv=8, Sq=1, D=64, ps=16, maxp=64, npages=64):
        var = av.AvVariant(score_mod, mask, 0.0, 20.0, 8.0, 256, 0, None, 0)
        return lib.attn_decode_paged_fwd(ctypes.byref(var), q, k, v, bt, sl, out, None, ws, wsb, B, Hq, Hkv, Sq, D,
                                         ps, maxp, npages, None)

    assert call(bt=None) == -1
    assert call(sl=None) == -1
    assert call(k=None) == -1
    assert call(mask=3) == -3
    assert call(ps=8) == -3
    assert call(ps=48) == -3
    assert call(D=128) == -3
    assert call(Sq=9) == -3
    assert call(maxp=0) == -2
    assert call(npages=0) == -2
    assert call(bt=0x50000 + 2) == -4
    assert call(k=P2 + 8) == -4
    assert call(ws=None) == -5
    assert call(Sq=0) == 0


def test_backward_rejections(lib):
    assert lib.attn_bwd_workspace_bytes(2, 16, 4, 100, 100, 64) == 2 * 16 * 100 * 8

    def call(score_mod=0, mask=1, lse=0x70000, dq=0x80000, ws=0x200000, wsb=1 << 30, B=1, Hq=4, Hkv=2, Sq=128,
             Skv=128, D=64):
        var = av.AvVariant(score_mod, mask, 0.0, 20.0, 8.0, 256, 0, None, 0)
        return lib.attn_bwd(ctypes.byref(var), P, P2, P3, P4, lse, dq, 0x90000, 0xA0000, ws, wsb, B, Hq,
                            Hkv, Sq, Skv, D, None)

    assert call(lse=None) == -1
    assert call(dq=None) == -1
    assert call(mask=5) == -3
    assert call(mask=4) == -1          # the document mask needs doc_id
    assert call(Skv=64) == -2          # a mask needs Sq == Skv
    assert call(mask=2, Skv=64) == -2
    assert call(D=128) == -3
    assert call(Hq=3) == -2
    assert call(ws=None) == -5
    assert call(wsb=8) == -5
    assert call(dq=0x80000 + 4) == -4
    assert call(lse=0x70000 + 2) == -4

    # the document work order, as for attn_fwd: only with the document mask,
    # 4-byte aligned, of attn_doc_order_len(B, Sq) entries
    def call_v(var, B=2, S=256):
        return lib.attn_bwd(ctypes.byref(var), P, P2, P3, P4, 0x70000, 0x80000, 0x90000, 0xA0000, 0x200000,
                            1 << 30, B, 4, 2, S, S, 64, None)

    v = av.make_variant(mask="causal")
    v.doc_order, v.doc_order_len = 0x80000, 4
    assert call_v(v) == -7
    v = av.make_variant(mask="document")
    v.doc_id = 0x90000
    v.doc_order, v.doc_order_len = 0x80002, 4
    assert call_v(v) == -4
    v.doc_order = 0x80000
    for n in (0, 3, 5, 1 << 20):
        v.doc_order_len = n
        assert call_v(v) == -7, n
    v.doc_order_len = 2
    assert call_v(v, B=1, S=257) == -7          # 3 tiles of 128 rows


def test_evoformer_column_rejections(lib):
    def call(m=P, w=P2, out=P4, ws=0x100000, wsb=None, Ns=2, Nr=16, Cm=64, H=4, dh=32, scale=0.0):
        if wsb is None:
            wsb = lib.evoformer_workspace_bytes(max(Ns, 1), max(Nr, 1), max(H, 1), max(dh, 1))
        return lib.evoformer_col_gated_attn_fwd(m, w, w, w, w, out, ws, wsb, Ns, Nr, Cm, H, dh, scale, None)

    assert call(m=None) == -1
    assert call(w=None) == -1
    assert call(out=None) == -1
    assert call(Nr=0) == -2
    assert call(dh=16) == -3
    assert call(Cm=96) == -3
    assert call(H=1) == -3
    assert call(scale=float("inf")) == -7
    assert call(out=P4 + 8) == -4
    assert call(ws=None) == -5
    assert call(wsb=1) == -5
    assert call(ws=0x100000 + 128) == -4


class _FakeDevice:
    """Lets the binding's checks accept host tensors, so that a wrong caller
    buffer can be shown to raise before anything reaches the library (with a
    host pointer the library call itself would fail with a HIP error)."""

    def __init__(self, monkeypatch):
        monkeypatch.setattr(av, "_on_device", lambda t: True)


def _bf(*shape):
    import torch

    return torch.zeros(*shape, dtype=torch.bfloat16)


def test_binding_rejects_wrong_output_buffers(monkeypatch):
    import torch

    _FakeDevice(monkeypatch)
    q, kv = _bf(2, 4, 8, 64), _bf(2, 2, 8, 64)
    f32 = torch.float32
    bad = [
        dict(out=_bf(2, 4, 8, 32)),                      # wrong shape
        dict(out=_bf(2, 4, 7, 64)),
        dict(out=torch.zeros(2, 4, 8, 64)),              # wrong dtype (TypeError)
        dict(lse=torch.zeros(2, 4, 7, dtype=f32)),
        dict(lse=torch.zeros(2, 4, 8, 1, dtype=f32)),
        dict(out=_bf(2, 4, 64, 8).transpose(2, 3)),      # not contiguous
    ]
    for kw in bad:
        with pytest.raises((ValueError, TypeError)):
            av.attn_fwd(q, kv, kv, **kw)
    with pytest.raises(ValueError):
        av.attn_fwd(q, kv, _bf(2, 2, 7, 64))             # v shorter than k
    with pytest.raises(ValueError):
        av.attn_fwd(q, kv, kv, mask="document", doc_id=torch.zeros(2, 7, dtype=torch.int32))
    with pytest.raises(ValueError):
        av.attn_decode_fwd(q, kv, kv, out=_bf(2, 4, 8, 63))
    with pytest.raises(ValueError):
        av.attn_decode_fwd(q, kv, kv, lse=torch.zeros(2, 4, 9, dtype=f32))


def test_binding_rejects_wrong_backward_buffers(monkeypatch):
    import torch

    _FakeDevice(monkeypatch)
    q, kv = _bf(1, 4, 16, 64), _bf(1, 2, 16, 64)
    lse = torch.zeros(1, 4, 16)
    for kw in (dict(dq=_bf(1, 4, 15, 64)), dict(dk=_bf(1, 4, 16, 64)), dict(dv=_bf(1, 2, 16, 32)),
               dict(workspace=torch.zeros(8, dtype=torch.uint8))):
        with pytest.raises(ValueError):
            av.attn_bwd(q, kv, kv, q, lse, **kw)
    with pytest.raises(ValueError):
        av.attn_bwd(q, kv, _bf(1, 2, 15, 64), q, lse)  # v and k disagree
    with pytest.raises(ValueError):
        av.attn_bwd(q, kv, _bf(1, 1, 16, 64), q, lse)
    with pytest.raises(ValueError):
        av.attn_bwd(q, kv, kv, q, torch.zeros(1, 4, 17))


def test_binding_rejects_wrong_diff_and_evoformer_buffers(monkeypatch):
    import torch

    _FakeDevice(monkeypatch)
    q, v = _bf(1, 2, 8, 128), _bf(1, 2, 8, 128)
    with pytest.raises(ValueError):
        av.diff_attn_fwd(q, q, v, out=_bf(1, 2, 8, 64))
    lam = torch.zeros(64)
    with pytest.raises(ValueError):
        av.diff_head_fwd(q, q, v, lam, lam, lam, lam, lambda_init=0.2, out=_bf(1, 2, 9, 128))
    with pytest.raises(ValueError):
        av.diff_head_fwd(q, q, v, lam, lam, lam, torch.zeros(32), lambda_init=0.2)
    m, w, b = _bf(2, 16, 64), _bf(64, 128), _bf(4, 16, 16)
    with pytest.raises(ValueError):
        av.evoformer_gated_attn_fwd(m, w, w, w, w, b, H=4, dh=32, out=_bf(2, 16, 64))
    with pytest.raises(ValueError):
        av.evoformer_gated_attn_fwd(m, w, w, w, w, b, H=4, dh=32,
                                    workspace=torch.zeros(100, dtype=torch.uint8))
    with pytest.raises(ValueError):
        av.evoformer_gated_attn_fwd(m, w, w, w, _bf(64, 64), b, H=4, dh=32)
    with pytest.raises(ValueError):
        av.evoformer_col_gated_attn_fwd(m, w, w, w, w, H=4, dh=32, out=_bf(2, 15, 128))


def test_python_binding_rejects_cpu_tensors():
    import torch

    x = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        av.attn_fwd(x, x, x)
    with pytest.raises(ValueError):
        av.make_variant(mask="bogus")


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError):
        av.load_library(str(tmp_path / "nope.so"))


def test_binding_has_every_exported_function():
    """Each C entry point has a Python function of the same name in the binding."""
    for name in av.EXPORTED:
        if name.startswith("av_"):
            continue
        assert callable(getattr(av, name, None)), name


def test_decode_partials_fit_the_static_array(lib):
    """Every decode plan's split-KV partials fit the 8650752-byte array of the
    allocation-free entry point: exhaustive over 1..1100 (batch, KV head)
    units at key counts from one tile to 2^20 keys."""
    worst = 0
    for units in range(1, 1101):
        for skv in (1, 64 * 4, 64 * 4 * 7 + 1, 4096, 16384, 100003, 1 << 20):
            worst = max(worst, lib.attn_decode_workspace_bytes(1, units, units, 1, skv, 64))
    assert 0 < worst <= 8650752
