"""MI355X-native fused attention variants -- Python binding of ``libattnvar.so``.

Thin ctypes layer over the C ABI declared in ``include/attnvar.h``: it checks
tensor dtypes, devices and shapes, allocates outputs with ``torch.empty`` and
passes raw device pointers plus torch's current HIP stream.  Every step of the
computation runs in the library's HIP kernels; there is no fallback.  If the
library has not been built, every entry point raises.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattnvar.so")

SCORE_MODS = {"none": 0, "alibi": 1, "softcap": 2, "bias": 3}
MASKS = {"none": 0, "causal": 1, "sliding_window": 2, "prefix_lm": 3, "document": 4}

AV_OK = 0
STATUS = {
    0: "AV_OK",
    -1: "AV_ERR_NULL",
    -2: "AV_ERR_SHAPE",
    -3: "AV_ERR_UNSUPPORTED",
    -4: "AV_ERR_ALIGN",
    -5: "AV_ERR_WORKSPACE",
    -6: "AV_ERR_HIP",
    -7: "AV_ERR_PARAM",
    -8: "AV_ERR_TOO_LARGE",
}

# Names the header declares; tests check that the library exports each one.
EXPORTED = (
    "attn_fwd",
    "attn_doc_order_len",
    "attn_doc_order",
    "attn_decode_workspace_bytes",
    "attn_decode_fwd",
    "attn_decode_fwd_noalloc",
    "attn_decode_paged_workspace_bytes",
    "attn_decode_paged_fwd",
    "attn_bwd_workspace_bytes",
    "attn_bwd",
    "diff_attn_fwd",
    "diff_head_fwd",
    "evoformer_workspace_bytes",
    "evoformer_gated_attn_fwd",
    "evoformer_col_gated_attn_fwd",
    "av_status_string",
    "av_abi_version",
)


class AvVariant(ctypes.Structure):
    """Mirror of ``av_variant`` in ``include/attnvar.h``."""

    _fields_ = [
        ("score_mod", ctypes.c_int32),
        ("mask", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("softcap", ctypes.c_float),
        ("alibi_max_bias", ctypes.c_float),
        ("window", ctypes.c_int32),
        ("prefix_len", ctypes.c_int32),
        ("doc_id", ctypes.c_void_p),
        ("kv_group", ctypes.c_int32),
        ("bias", ctypes.c_void_p),
        ("bias_batch_stride", ctypes.c_int64),
        ("bias_head_stride", ctypes.c_int64),
        ("doc_order", ctypes.c_void_p),
        ("doc_order_len", ctypes.c_int32),
    ]


_lib = None
_vp = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float


def load_library(path: str | None = None):
    """Load the in-tree ``libattnvar.so`` (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"attention_variants_amd: HIP library missing at {p}; build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(p)
    lib.attn_fwd.argtypes = [ctypes.POINTER(AvVariant), _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp]
    lib.attn_fwd.restype = _i
    lib.attn_doc_order_len.argtypes = [_i, _i]
    lib.attn_doc_order_len.restype = _i
    lib.attn_doc_order.argtypes = [_vp, _i, _i, _vp, _i, _vp]
    lib.attn_doc_order.restype = _i
    lib.attn_decode_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i]
    lib.attn_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_decode_fwd.argtypes = [ctypes.POINTER(AvVariant), _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                                    _i, _i, _i, _i, _i, _i, _vp]
    lib.attn_decode_fwd.restype = _i
    lib.attn_decode_fwd_noalloc.argtypes = [ctypes.POINTER(AvVariant), _vp, _vp, _vp, _vp, _vp,
                                            _i, _i, _i, _i, _i, _i, _vp]
    lib.attn_decode_fwd_noalloc.restype = _i
    lib.attn_decode_paged_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i, _i]
    lib.attn_decode_paged_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_decode_paged_fwd.argtypes = [ctypes.POINTER(AvVariant), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                          ctypes.c_size_t, _i, _i, _i, _i, _i, _i, _i, _i, _vp]
    lib.attn_decode_paged_fwd.restype = _i
    lib.attn_bwd_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i]
    lib.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_bwd.argtypes = [ctypes.POINTER(AvVariant), _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                             ctypes.c_size_t, _i, _i, _i, _i, _i, _i, _vp]
    lib.attn_bwd.restype = _i
    lib.diff_attn_fwd.argtypes = [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _f, _i, _vp]
    lib.diff_attn_fwd.restype = _i
    lib.diff_head_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _f, _f, _i,
                                  _vp]
    lib.diff_head_fwd.restype = _i
    lib.evoformer_workspace_bytes.argtypes = [_i, _i, _i, _i]
    lib.evoformer_workspace_bytes.restype = ctypes.c_size_t
    lib.evoformer_gated_attn_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                                             _i, _i, _i, _i, _i, _f, _vp]
    lib.evoformer_gated_attn_fwd.restype = _i
    lib.evoformer_col_gated_attn_fwd.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                                                 _i, _i, _i, _i, _i, _f, _vp]
    lib.evoformer_col_gated_attn_fwd.restype = _i
    lib.av_status_string.argtypes = [_i]
    lib.av_status_string.restype = ctypes.c_char_p
    lib.av_abi_version.argtypes = []
    lib.av_abi_version.restype = _i
    if path is None:
        _lib = lib
    return lib


def status_string(rc: int) -> str:
    return load_library().av_status_string(rc).decode()


def _check(rc: int, what: str):
    if rc != AV_OK:
        raise RuntimeError(f"{what}: {status_string(rc)}")


def _stream_ptr(device):
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _on_device(t) -> bool:
    """True when ``t`` lives in HIP device memory (the kernels dereference its pointer)."""
    return t.is_cuda


def _need(t, name, dtype, ndim, device=None):
    """Check a tensor argument: type, HIP device (the same one as ``device`` when
    given), dtype, rank and contiguity."""
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not _on_device(t):
        raise ValueError(f"{name} must be on a HIP device")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _need_shape(t, name, dtype, shape, device):
    """A caller-supplied output: exactly ``shape``, ``dtype``, contiguous, on ``device``.
    The kernels write every element of that shape through the raw pointer."""
    _need(t, name, dtype, len(shape), device)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {tuple(shape)}, got {tuple(t.shape)}")


def _need_workspace(ws, name, nbytes, device):
    """A caller-supplied workspace: contiguous device memory of at least ``nbytes`` bytes."""
    import torch

    if not isinstance(ws, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not _on_device(ws) or ws.device != device:
        raise ValueError(f"{name} must be on {device}")
    if not ws.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    have = ws.numel() * ws.element_size()
    if have < nbytes:
        raise ValueError(f"{name} holds {have} bytes, {nbytes} needed")
    return have


def make_variant(score_mod="none", mask="none", *, scale=0.0, softcap=20.0, alibi_max_bias=8.0,
                 window=256, prefix_len=0, doc_id=None, kv_group=0, bias=None, bias_batch_stride=0,
                 bias_head_stride=0, doc_order=None) -> AvVariant:
    if score_mod not in SCORE_MODS:
        raise ValueError(f"unknown score_mod {score_mod!r}")
    if mask not in MASKS:
        raise ValueError(f"unknown mask {mask!r}")
    return AvVariant(SCORE_MODS[score_mod], MASKS[mask], float(scale or 0.0), float(softcap),
                     float(alibi_max_bias), int(window), int(prefix_len),
                     None if doc_id is None else int(doc_id.data_ptr()), int(kv_group),
                     None if bias is None else int(bias.data_ptr()), int(bias_batch_stride), int(bias_head_stride),
                     None if doc_order is None else int(doc_order.data_ptr()),
                     0 if doc_order is None else int(doc_order.numel()))


def attn_fwd(q, k, v, *, score_mod="none", mask="none", scale=0.0, softcap=20.0, alibi_max_bias=8.0,
             window=256, prefix_len=0, doc_id=None, kv_group=0, bias=None, return_lse=False, out=None, lse=None,
             doc_order=None):
    """Fused attention forward.  q [B,Hq,Sq,D], k/v [B,Hkv,Skv,D] bf16 -> out [B,Hq,Sq,D] (bf16).

    ``score_mod="bias"`` adds ``bias`` (bf16 [Bb, Hb, Sq, Skv], Bb in {1, B},
    Hb in {1, Hq}; a size-1 axis is shared) to the scaled scores.
    ``doc_order`` (document mask only): the work order ``attn_doc_order(doc_id)`` returns.
    With ``return_lse`` also returns the fp32 natural-log sum-exp per row.
    """
    import torch

    lib = load_library()
    _need(q, "q", torch.bfloat16, 4)
    dev = q.device
    for t, n in ((k, "k"), (v, "v")):
        _need(t, n, torch.bfloat16, 4, dev)
    B, Hq, Sq, D = q.shape
    Bk, Hkv, Skv, Dk = k.shape
    if Bk != B or Dk != D or tuple(v.shape) != (B, Hkv, Skv, D):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if doc_id is not None:
        _need_shape(doc_id, "doc_id", torch.int32, (B, Sq), dev)
    if doc_order is not None:
        _need(doc_order, "doc_order", torch.int32, 1, dev)
        if doc_order.numel() != attn_doc_order_len(B, Sq):
            raise ValueError("doc_order must come from attn_doc_order(doc_id) of this shape")
    bs = hs = 0
    if score_mod == "bias":
        if bias is None:
            raise ValueError("score_mod='bias' needs a bias tensor")
        _need(bias, "bias", torch.bfloat16, 4, dev)
        Bb, Hb = bias.shape[:2]
        if Bb not in (1, B) or Hb not in (1, Hq) or tuple(bias.shape[2:]) != (Sq, Skv):
            raise ValueError(f"bias must be [1 or B, 1 or Hq, Sq, Skv], got {tuple(bias.shape)}")
        hs = Sq * Skv if Hb > 1 else 0
        bs = Hb * Sq * Skv if Bb > 1 else 0
    elif bias is not None:
        raise ValueError("bias given without score_mod='bias'")
    if out is None:
        out = torch.empty((B, Hq, Sq, D), dtype=torch.bfloat16, device=dev)
    else:
        _need_shape(out, "out", torch.bfloat16, (B, Hq, Sq, D), dev)
    if lse is not None:
        _need_shape(lse, "lse", torch.float32, (B, Hq, Sq), dev)
    elif return_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=dev)
    var = make_variant(score_mod, mask, scale=scale, softcap=softcap, alibi_max_bias=alibi_max_bias,
                       window=window, prefix_len=prefix_len, doc_id=doc_id, kv_group=kv_group, bias=bias,
                       bias_batch_stride=bs, bias_head_stride=hs, doc_order=doc_order)
    rc = lib.attn_fwd(ctypes.byref(var), q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                      None if lse is None else lse.data_ptr(), B, Hq, Hkv, Sq, Skv, D, _stream_ptr(q.device))
    _check(rc, "attn_fwd")
    return (out, lse) if return_lse else out


def attn_doc_order_len(B, S) -> int:
    n = int(load_library().attn_doc_order_len(B, S))
    _check(min(n, 0), "attn_doc_order_len")
    return n


def attn_doc_order(doc_id, out=None):
    """Heaviest-first work order of attn_fwd's query tiles under the document
    mask, from ``doc_id`` [B, S] int32: an int32 tensor of attn_doc_order_len(B, S)."""
    import torch

    lib = load_library()
    _need(doc_id, "doc_id", torch.int32, 2)
    B, S = doc_id.shape
    n = attn_doc_order_len(B, S)
    if out is None:
        out = torch.empty((n,), dtype=torch.int32, device=doc_id.device)
    else:
        _need_shape(out, "out", torch.int32, (n,), doc_id.device)
    rc = lib.attn_doc_order(doc_id.data_ptr(), B, S, out.data_ptr(), out.numel(), _stream_ptr(doc_id.device))
    _check(rc, "attn_doc_order")
    return out


def attn_decode_workspace_bytes(B, Hq, Hkv, Sq, Skv, D) -> int:
    return int(load_library().attn_decode_workspace_bytes(B, Hq, Hkv, Sq, Skv, D))


def attn_decode_fwd(q, k, v, *, score_mod="none", mask="none", scale=0.0, softcap=20.0, alibi_max_bias=8.0,
                    kv_group=0, return_lse=False, out=None, lse=None, workspace=None):
    """Decoding / short-query attention: q [B,Hq,Sq,D] are the last Sq positions of
    k/v [B,Hkv,Skv,D] (bf16) -> out [B,Hq,Sq,D].  Masks: none or causal.
    ``workspace`` (uint8 device tensor) is allocated when needed and not given.
    """
    import torch

    lib = load_library()
    _need(q, "q", torch.bfloat16, 4)
    dev = q.device
    for t, n in ((k, "k"), (v, "v")):
        _need(t, n, torch.bfloat16, 4, dev)
    B, Hq, Sq, D = q.shape
    Bk, Hkv, Skv, Dk = k.shape
    if Bk != B or Dk != D or tuple(v.shape) != (B, Hkv, Skv, D):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if out is None:
        out = torch.empty((B, Hq, Sq, D), dtype=torch.bfloat16, device=dev)
    else:
        _need_shape(out, "out", torch.bfloat16, (B, Hq, Sq, D), dev)
    if lse is not None:
        _need_shape(lse, "lse", torch.float32, (B, Hq, Sq), dev)
    elif return_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=dev)
    need = lib.attn_decode_workspace_bytes(B, Hq, Hkv, Sq, Skv, D) if Sq > 0 else 0
    ws_bytes = 0
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        ws_bytes = _need_workspace(workspace, "workspace", need, dev)
    var = make_variant(score_mod, mask, scale=scale, softcap=softcap, alibi_max_bias=alibi_max_bias,
                       kv_group=kv_group)
    rc = lib.attn_decode_fwd(ctypes.byref(var), q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                             None if lse is None else lse.data_ptr(),
                             None if workspace is None else workspace.data_ptr(),
                             ws_bytes, B, Hq, Hkv, Sq, Skv, D, _stream_ptr(dev))
    _check(rc, "attn_decode_fwd")
    return (out, lse) if return_lse else out


def attn_decode_fwd_noalloc(q, k, v, out, *, score_mod="none", mask="none", scale=0.0, softcap=20.0,
                            alibi_max_bias=8.0, kv_group=0, lse=None):
    """attn_decode_fwd without a workspace: the library keeps the split-KV
    partials in its static per-GPU array, so the call allocates nothing.  The
    caller passes ``out`` (and optionally ``lse``); calls that overlap on one
    GPU race."""
    import torch

    lib = load_library()
    _need(q, "q", torch.bfloat16, 4)
    dev = q.device
    for t, n in ((k, "k"), (v, "v")):
        _need(t, n, torch.bfloat16, 4, dev)
    B, Hq, Sq, D = q.shape
    Bk, Hkv, Skv, Dk = k.shape
    if Bk != B or Dk != D or tuple(v.shape) != (B, Hkv, Skv, D):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    _need_shape(out, "out", torch.bfloat16, (B, Hq, Sq, D), dev)
    if lse is not None:
        _need_shape(lse, "lse", torch.float32, (B, Hq, Sq), dev)
    var = make_variant(score_mod, mask, scale=scale, softcap=softcap, alibi_max_bias=alibi_max_bias,
                       kv_group=kv_group)
    rc = lib.attn_decode_fwd_noalloc(ctypes.byref(var), q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                     None if lse is None else lse.data_ptr(), B, Hq, Hkv, Sq, Skv, D,
                                     _stream_ptr(dev))
    _check(rc, "attn_decode_fwd_noalloc")
    return out


def attn_decode_paged_workspace_bytes(B, Hq, Hkv, Sq, D, page_size, max_pages) -> int:
    return int(load_library().attn_decode_paged_workspace_bytes(B, Hq, Hkv, Sq, D, page_size, max_pages))


def attn_decode_paged_fwd(q, k_cache, v_cache, block_table, seq_lens, *, score_mod="none", mask="none", scale=0.0,
                          softcap=20.0, alibi_max_bias=8.0, kv_group=0, return_lse=False, out=None, lse=None,
                          workspace=None):
    """Decoding against a paged cache: k_cache/v_cache [num_pages, Hkv, page_size, D] bf16,
    block_table [B, max_pages] int32, seq_lens [B] int32; q [B, Hq, Sq, D] are the last Sq
    positions of each sequence -> out [B, Hq, Sq, D].
    """
    import torch

    lib = load_library()
    _need(q, "q", torch.bfloat16, 4)
    dev = q.device
    _need(k_cache, "k_cache", torch.bfloat16, 4, dev)
    _need(v_cache, "v_cache", torch.bfloat16, 4, dev)
    _need(block_table, "block_table", torch.int32, 2, dev)
    _need(seq_lens, "seq_lens", torch.int32, 1, dev)
    B, Hq, Sq, D = q.shape
    num_pages, Hkv, page_size, Dk = k_cache.shape
    if Dk != D or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_cache / v_cache must be [num_pages, Hkv, page_size, D]")
    if block_table.shape[0] != B or tuple(seq_lens.shape) != (B,):
        raise ValueError("block_table must be [B, max_pages] and seq_lens [B]")
    max_pages = block_table.shape[1]
    if out is None:
        out = torch.empty((B, Hq, Sq, D), dtype=torch.bfloat16, device=dev)
    else:
        _need_shape(out, "out", torch.bfloat16, (B, Hq, Sq, D), dev)
    if lse is not None:
        _need_shape(lse, "lse", torch.float32, (B, Hq, Sq), dev)
    elif return_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=dev)
    need = lib.attn_decode_paged_workspace_bytes(B, Hq, Hkv, Sq, D, page_size, max_pages) if Sq > 0 else 0
    ws_bytes = 0
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        ws_bytes = _need_workspace(workspace, "workspace", need, dev)
    var = make_variant(score_mod, mask, scale=scale, softcap=softcap, alibi_max_bias=alibi_max_bias,
                       kv_group=kv_group)
    rc = lib.attn_decode_paged_fwd(ctypes.byref(var), q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                                   block_table.data_ptr(), seq_lens.data_ptr(), out.data_ptr(),
                                   None if lse is None else lse.data_ptr(),
                                   None if workspace is None else workspace.data_ptr(),
                                   ws_bytes, B, Hq, Hkv, Sq, D, page_size, max_pages, num_pages, _stream_ptr(dev))
    _check(rc, "attn_decode_paged_fwd")
    return (out, lse) if return_lse else out


def attn_bwd_workspace_bytes(B, Hq, Hkv, Sq, Skv, D) -> int:
    return int(load_library().attn_bwd_workspace_bytes(B, Hq, Hkv, Sq, Skv, D))


def attn_bwd(q, k, v, dout, lse, *, score_mod="none", mask="none", scale=0.0, softcap=20.0,
             alibi_max_bias=8.0, window=256, prefix_len=0, doc_id=None, kv_group=0, dq=None, dk=None, dv=None,
             workspace=None, doc_order=None):
    """Gradients (dq, dk, dv) of attn_fwd's output for an upstream ``dout``; ``lse``
    is attn_fwd's (``return_lse=True``).  Every mask of attn_fwd, with the same
    ``window`` / ``prefix_len`` / ``doc_id``; ``doc_order`` (document mask only)
    is the work order ``attn_doc_order(doc_id)`` returns, as for attn_fwd."""
    import torch

    lib = load_library()
    _need(q, "q", torch.bfloat16, 4)
    dev = q.device
    for t, n in ((k, "k"), (v, "v"), (dout, "dout")):
        _need(t, n, torch.bfloat16, 4, dev)
    B, Hq, Sq, D = q.shape
    Bk, Hkv, Skv, Dk = k.shape
    if Bk != B or Dk != D or tuple(v.shape) != (B, Hkv, Skv, D):
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if tuple(dout.shape) != tuple(q.shape):
        raise ValueError("dout must match q")
    _need_shape(lse, "lse", torch.float32, (B, Hq, Sq), dev)
    if dq is None:
        dq = torch.empty_like(q)
    else:
        _need_shape(dq, "dq", torch.bfloat16, (B, Hq, Sq, D), dev)
    if dk is None:
        dk = torch.empty_like(k)
    else:
        _need_shape(dk, "dk", torch.bfloat16, (B, Hkv, Skv, D), dev)
    if dv is None:
        dv = torch.empty_like(v)
    else:
        _need_shape(dv, "dv", torch.bfloat16, (B, Hkv, Skv, D), dev)
    if doc_id is not None:
        _need_shape(doc_id, "doc_id", torch.int32, (B, Sq), dev)
    if doc_order is not None:
        _need(doc_order, "doc_order", torch.int32, 1, dev)
        if doc_order.numel() != attn_doc_order_len(B, Sq):
            raise ValueError("doc_order must come from attn_doc_order(doc_id) of this shape")
    need = lib.attn_bwd_workspace_bytes(B, Hq, Hkv, Sq, Skv, D)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    ws_bytes = _need_workspace(workspace, "workspace", need, dev)
    var = make_variant(score_mod, mask, scale=scale, softcap=softcap, alibi_max_bias=alibi_max_bias,
                       window=window, prefix_len=prefix_len, doc_id=doc_id, kv_group=kv_group, doc_order=doc_order)
    rc = lib.attn_bwd(ctypes.byref(var), q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(),
                      lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
                      ws_bytes, B, Hq, Hkv, Sq, Skv, D, _stream_ptr(dev))
    _check(rc, "attn_bwd")
    return dq, dk, dv


def diff_attn_fwd(q, k, v, *, lam=0.8, scale=0.0, causal=True, out=None):
    """Differential attention.  q, k [B,H,S,2*Dh], v [B,H,S,Dv] bf16 -> out [B,H,S,Dv]."""
    import torch

    lib = load_library()
    _need(q, "q", torch.bfloat16, 4)
    dev = q.device
    for t, n in ((k, "k"), (v, "v")):
        _need(t, n, torch.bfloat16, 4, dev)
    B, H, S, D2 = q.shape
    if tuple(k.shape) != (B, H, S, D2) or v.shape[:3] != (B, H, S) or D2 % 2:
        raise ValueError("shape mismatch")
    Dv = v.shape[3]
    if out is None:
        out = torch.empty((B, H, S, Dv), dtype=torch.bfloat16, device=dev)
    else:
        _need_shape(out, "out", torch.bfloat16, (B, H, S, Dv), dev)
    rc = lib.diff_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, S, D2 // 2, Dv,
                           float(lam), float(scale or 0.0), int(bool(causal)), _stream_ptr(q.device))
    _check(rc, "diff_attn_fwd")
    return out


def diff_head_fwd(q, k, v, lambda_q1, lambda_k1, lambda_q2, lambda_k2, *, lambda_init, gamma=None, eps=1e-5,
                  scale=0.0, causal=True, out=None):
    """Full differential-attention head: the differential core with
    lambda = exp(lq1.lk1) - exp(lq2.lk2) + lambda_init, then per-row RMSNorm
    (weight ``gamma``, ones when None) times (1 - lambda_init).
    q, k [B,H,S,2*Dh], v [B,H,S,Dv] bf16; lambda_* [Dh], gamma [Dv] float32 on
    the same device -> out [B,H,S,Dv] bf16."""
    import torch

    lib = load_library()
    _need(q, "q", torch.bfloat16, 4)
    dev = q.device
    for t, n in ((k, "k"), (v, "v")):
        _need(t, n, torch.bfloat16, 4, dev)
    B, H, S, D2 = q.shape
    if tuple(k.shape) != (B, H, S, D2) or v.shape[:3] != (B, H, S) or D2 % 2:
        raise ValueError("shape mismatch")
    Dv = v.shape[3]
    for t, n in ((lambda_q1, "lambda_q1"), (lambda_k1, "lambda_k1"), (lambda_q2, "lambda_q2"),
                 (lambda_k2, "lambda_k2")):
        _need_shape(t, n, torch.float32, (D2 // 2,), dev)
    if gamma is not None:
        _need_shape(gamma, "gamma", torch.float32, (Dv,), dev)
    if out is None:
        out = torch.empty((B, H, S, Dv), dtype=torch.bfloat16, device=dev)
    else:
        _need_shape(out, "out", torch.bfloat16, (B, H, S, Dv), dev)
    rc = lib.diff_head_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), lambda_q1.data_ptr(), lambda_k1.data_ptr(),
                           lambda_q2.data_ptr(), lambda_k2.data_ptr(), None if gamma is None else gamma.data_ptr(),
                           out.data_ptr(), B, H, S, D2 // 2, Dv, float(lambda_init), float(eps), float(scale or 0.0),
                           int(bool(causal)), _stream_ptr(q.device))
    _check(rc, "diff_head_fwd")
    return out


def evoformer_workspace_bytes(Ns, Nr, H, dh) -> int:
    return int(load_library().evoformer_workspace_bytes(Ns, Nr, H, dh))


def evoformer_gated_attn_fwd(m, wq, wk, wv, wg, bias, *, H, dh, scale=0.0, workspace=None, out=None):
    """Evoformer row-wise gated self-attention with pair bias.

    m [Ns,Nr,Cm], w* [Cm,H*dh], bias [H,Nr,Nr] bf16 -> out [Ns,Nr,H*dh] bf16.
    ``workspace`` (uint8 device tensor) is allocated when not given.
    """
    import torch

    lib = load_library()
    _need(m, "m", torch.bfloat16, 3)
    dev = m.device
    Ns, Nr, Cm = m.shape
    for t, n in ((wq, "wq"), (wk, "wk"), (wv, "wv"), (wg, "wg")):
        _need_shape(t, n, torch.bfloat16, (Cm, H * dh), dev)
    _need_shape(bias, "bias", torch.bfloat16, (H, Nr, Nr), dev)
    need = evoformer_workspace_bytes(Ns, Nr, H, dh)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = _need_workspace(workspace, "workspace", need, dev)
    if out is None:
        out = torch.empty((Ns, Nr, H * dh), dtype=torch.bfloat16, device=dev)
    else:
        _need_shape(out, "out", torch.bfloat16, (Ns, Nr, H * dh), dev)
    rc = lib.evoformer_gated_attn_fwd(m.data_ptr(), wq.data_ptr(), wk.data_ptr(), wv.data_ptr(), wg.data_ptr(),
                                      bias.data_ptr(), out.data_ptr(), workspace.data_ptr(), ws_bytes,
                                      Ns, Nr, Cm, H, dh, float(scale or 0.0), _stream_ptr(m.device))
    _check(rc, "evoformer_gated_attn_fwd")
    return out


def evoformer_col_gated_attn_fwd(m, wq, wk, wv, wg, *, H, dh, scale=0.0, workspace=None, out=None):
    """Evoformer column-wise gated self-attention (over the sequences of each
    residue column, no pair bias).

    m [Ns,Nr,Cm], w* [Cm,H*dh] bf16 -> out [Ns,Nr,H*dh] bf16.
    ``workspace`` (uint8 device tensor) is allocated when not given.
    """
    import torch

    lib = load_library()
    _need(m, "m", torch.bfloat16, 3)
    dev = m.device
    Ns, Nr, Cm = m.shape
    for t, n in ((wq, "wq"), (wk, "wk"), (wv, "wv"), (wg, "wg")):
        _need_shape(t, n, torch.bfloat16, (Cm, H * dh), dev)
    need = evoformer_workspace_bytes(Ns, Nr, H, dh)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = _need_workspace(workspace, "workspace", need, dev)
    if out is None:
        out = torch.empty((Ns, Nr, H * dh), dtype=torch.bfloat16, device=dev)
    else:
        _need_shape(out, "out", torch.bfloat16, (Ns, Nr, H * dh), dev)
    rc = lib.evoformer_col_gated_attn_fwd(m.data_ptr(), wq.data_ptr(), wk.data_ptr(), wv.data_ptr(), wg.data_ptr(),
                                          out.data_ptr(), workspace.data_ptr(), ws_bytes,
                                          Ns, Nr, Cm, H, dh, float(scale or 0.0), _stream_ptr(m.device))
    _check(rc, "evoformer_col_gated_attn_fwd")
    return out

