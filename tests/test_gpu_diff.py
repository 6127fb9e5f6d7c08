"""GPU parity of ``diff_attn_fwd`` against the fp64 oracle (through the C ABI).

Shapes: 16 heads, Q/K halves of 64, V width 128 (and 64), scale 1/8; and 32
heads, halves of 32, V width 64, scale 1/sqrt(32) (the talk notes' two
differential shapes); causal, lambda 0.8; the benchmark sizes (16k tokens)
are checked on sampled rows.
Gate: |gpu - oracle| <= 1e-2 + 1e-2 |oracle| elementwise.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import inputs as wi

from .gpu_util import assert_close, canary_empty, canary_intact, f64, sample_rows, to_dev

pytestmark = pytest.mark.gpu


def _run(av, B, H, S, Dv=128, lam=0.8, causal=True, rows=None, Dh=64):
    x = wi.diff_inputs(B, H, S, Dh, Dv)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    out, big = canary_empty((B, H, S, Dv), torch.bfloat16)
    av.diff_attn_fwd(q, k, v, lam=lam, causal=causal, out=out)
    torch.cuda.synchronize()
    assert canary_intact(big, out.numel()), "write past the end of out"
    ref = oracle.diff_attention(f64(x["q"]), f64(x["k"]), f64(x["v"]), lam=lam, causal=causal, rows=rows)
    got = out.float().cpu().numpy()
    if rows is not None:
        got = got[:, :, rows]
    return assert_close(got, ref, f"diff B{B} H{H} S{S} Dh{Dh} Dv{Dv} lam{lam} causal{causal}"), out


@pytest.mark.parametrize("S", [1, 17, 32, 100, 129, 300])
@pytest.mark.parametrize("causal", [True, False])
def test_small_all_rows(gpu_lib, S, causal):
    _run(gpu_lib, 2, 3, S, causal=causal)
    _run(gpu_lib, 1, 2, S, Dv=64, causal=causal)
    _run(gpu_lib, 2, 3, S, Dh=32, Dv=64, causal=causal)
    _run(gpu_lib, 1, 2, S, Dh=32, Dv=128, causal=causal)


def test_lambda_values(gpu_lib):
    for lam in (0.0, 0.5, 1.0, -0.3):
        _run(gpu_lib, 1, 2, 200, lam=lam)


def test_reductions_on_gpu(gpu_lib):
    """lambda = 0 equals causal attention on the first halves; identical halves give (1 - lambda) attn."""
    B, H, S = 1, 4, 257
    x = wi.diff_inputs(B, H, S)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    d0 = gpu_lib.diff_attn_fwd(q, k, v, lam=0.0).float()
    a = gpu_lib.attn_fwd(q[..., :64].contiguous(), k[..., :64].contiguous(), v[..., :64].contiguous(),
                         mask="causal", scale=0.125).float()
    d0_64 = gpu_lib.diff_attn_fwd(q, k, v[..., :64].contiguous(), lam=0.0).float()
    assert (d0_64 - a).abs().max().item() < 2e-2
    qq = torch.cat([q[..., :64], q[..., :64]], dim=-1).contiguous()
    kk = torch.cat([k[..., :64], k[..., :64]], dim=-1).contiguous()
    d = gpu_lib.diff_attn_fwd(qq, kk, v, lam=0.8).float()
    d1 = gpu_lib.diff_attn_fwd(qq, kk, v, lam=0.0).float()
    assert (d - 0.2 * d1).abs().max().item() < 1e-2
    # causal row 0 is (1 - lambda) v[0]
    assert (d[:, :, 0] - 0.2 * v[:, :, 0].float()).abs().max().item() < 1e-2
    assert torch.isfinite(d0).all()


def test_deterministic(gpu_lib):
    x = wi.diff_inputs(2, 4, 500)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    r = [gpu_lib.diff_attn_fwd(q, k, v) for _ in range(3)]
    assert torch.equal(r[0], r[1]) and torch.equal(r[1], r[2])


@pytest.mark.parametrize("S", [1024, 4096, 16384])
def test_benchmark_shapes(gpu_lib, S):
    rows = sample_rows(S, tiles=(32, 128), extra=24, seed=5) if S > 1024 else None
    if rows is not None and S == 16384:
        rows = rows[::3]
    _run(gpu_lib, 16384 // S, 16, S, rows=rows)


@pytest.mark.parametrize("S", [1024, 4096, 16384])
def test_benchmark_shapes_32x64(gpu_lib, S):
    """32 heads, Q/K halves of 32, V width 64 (the talk notes' "nhead 32,
    headdim 64" differential shape), 16k tokens, sampled rows beyond S = 1k."""
    rows = sample_rows(S, tiles=(32, 128), extra=24, seed=6) if S > 1024 else None
    if rows is not None and S == 16384:
        rows = rows[::3]
    _run(gpu_lib, 16384 // S, 32, S, Dh=32, Dv=64, rows=rows)


def test_reductions_dh32(gpu_lib):
    """Halves of 32: lambda = 0 equals causal attention on the first halves at scale 1/sqrt(32)."""
    B, H, S = 1, 4, 257
    x = wi.diff_inputs(B, H, S, 32, 64)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    d0 = gpu_lib.diff_attn_fwd(q, k, v, lam=0.0).float()
    a = gpu_lib.attn_fwd(q[..., :32].contiguous(), k[..., :32].contiguous(), v[..., :32].contiguous(),
                         mask="causal").float()
    assert (d0[..., :32] - a).abs().max().item() < 2e-2
