"""GPU parity of ``diff_head_fwd`` (the full differential-attention head)
against the fp64 oracle, through the C ABI.

The head normalises every output row, so an error in A is amplified by
1/rms(A); the gate stays |gpu - oracle| <= 1e-2 + 1e-2 |oracle| elementwise.
Shapes: 16 heads, Q/K halves of 64, V width 128 (and 64), causal and not;
the benchmark sizes (16k tokens) are checked on sampled rows.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from workloads import inputs as wi

from .gpu_util import assert_close, canary_empty, canary_intact, f64, sample_rows, to_dev

pytestmark = pytest.mark.gpu


def _params(Dv, seed=17, scale_lam=1.0, Dh=64):
    p = wi.diff_head_params(Dh, Dv, seed)
    for n in ("lq1", "lk1", "lq2", "lk2"):
        p[n] = (p[n] * np.float32(scale_lam)).astype(np.float32)
    return p


def _run(av, B, H, S, Dv=128, causal=True, rows=None, p=None, lambda_init=None, use_gamma=True, eps=1e-5,
         Dh=64):
    x = wi.diff_inputs(B, H, S, Dh, Dv)
    p = _params(Dv, Dh=Dh) if p is None else p
    lambda_init = oracle.diff_lambda_init(3) if lambda_init is None else lambda_init
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    dp = {n: torch.from_numpy(p[n]).cuda() for n in p}
    out, big = canary_empty((B, H, S, Dv), torch.bfloat16)
    av.diff_head_fwd(q, k, v, dp["lq1"], dp["lk1"], dp["lq2"], dp["lk2"], lambda_init=lambda_init,
                     gamma=dp["gamma"] if use_gamma else None, eps=eps, causal=causal, out=out)
    torch.cuda.synchronize()
    assert canary_intact(big, out.numel()), "write past the end of out"
    pf = {n: p[n].astype(np.float64) for n in p}
    ref = oracle.diff_head(f64(x["q"]), f64(x["k"]), f64(x["v"]), pf["lq1"], pf["lk1"], pf["lq2"], pf["lk2"],
                           lambda_init=lambda_init, gamma=pf["gamma"] if use_gamma else None, eps=eps,
                           causal=causal, rows=rows)
    got = out.float().cpu().numpy()
    if rows is not None:
        got = got[:, :, rows]
    return assert_close(got, ref, f"diff head B{B} H{H} S{S} Dh{Dh} Dv{Dv} causal{causal} gamma{use_gamma}"), out


@pytest.mark.parametrize("S", [1, 17, 32, 129, 300])
@pytest.mark.parametrize("causal", [True, False])
def test_small_all_rows(gpu_lib, S, causal):
    _run(gpu_lib, 2, 3, S, causal=causal)
    _run(gpu_lib, 1, 2, S, Dv=64, causal=causal, use_gamma=False)
    _run(gpu_lib, 2, 3, S, Dh=32, Dv=64, causal=causal)


@pytest.mark.parametrize("scale_lam,lambda_init", [(0.0, 0.2), (3.0, 0.8), (6.0, 0.35), (1.0, -0.5)])
def test_lambda_regimes(gpu_lib, scale_lam, lambda_init):
    """lambda vectors scaled from zero (lambda = lambda_init) up to dot products
    of order one, so lambda spans both signs of (1 - lambda)."""
    p = _params(128, seed=23, scale_lam=scale_lam)
    lam = oracle.diff_lambda(p["lq1"].astype(np.float64), p["lk1"].astype(np.float64), p["lq2"].astype(np.float64),
                             p["lk2"].astype(np.float64), lambda_init)
    assert math.isfinite(lam)
    _run(gpu_lib, 1, 4, 200, p=p, lambda_init=lambda_init)


def test_large_eps_and_zero_v(gpu_lib):
    """eps dominates when V is tiny; V = 0 gives exact zeros (no NaN)."""
    _run(gpu_lib, 1, 2, 100, eps=0.5)
    B, H, S, Dv = 1, 2, 70, 128
    x = wi.diff_inputs(B, H, S, 64, Dv)
    q, k = to_dev(x["q"]), to_dev(x["k"])
    v = torch.zeros((B, H, S, Dv), dtype=torch.bfloat16, device="cuda")
    p = {n: torch.from_numpy(a).cuda() for n, a in _params(Dv).items()}
    out = gpu_lib.diff_head_fwd(q, k, v, p["lq1"], p["lk1"], p["lq2"], p["lk2"], lambda_init=0.3, gamma=p["gamma"])
    torch.cuda.synchronize()
    assert torch.equal(out, torch.zeros_like(out))


def test_head_equals_normalised_core(gpu_lib):
    """With zero lambda vectors lambda = lambda_init, and the head is the core
    result (diff_attn_fwd, same lambda) normalised per row."""
    B, H, S, Dv = 1, 4, 257, 128
    x = wi.diff_inputs(B, H, S, 64, Dv)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    z = torch.zeros(64, dtype=torch.float32, device="cuda")
    li = 0.45
    y = gpu_lib.diff_head_fwd(q, k, v, z, z, z, z, lambda_init=li, eps=1e-5).float()
    a = gpu_lib.diff_attn_fwd(q, k, v, lam=li).float()
    want = (1 - li) * a / torch.sqrt(torch.mean(a * a, dim=-1, keepdim=True) + 1e-5)
    # the core output is rounded to bf16 before this normalisation, the head's is not
    assert (y - want).abs().max().item() < 2e-2
    rms = torch.sqrt(torch.mean(y * y, dim=-1))
    assert (rms - (1 - li)).abs().max().item() < 1e-2


def test_deterministic(gpu_lib):
    x = wi.diff_inputs(2, 4, 500)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    p = {n: torch.from_numpy(a).cuda() for n, a in _params(128).items()}
    r = [gpu_lib.diff_head_fwd(q, k, v, p["lq1"], p["lk1"], p["lq2"], p["lk2"], lambda_init=0.2, gamma=p["gamma"])
         for _ in range(3)]
    assert torch.equal(r[0], r[1]) and torch.equal(r[1], r[2])


@pytest.mark.parametrize("S", [1024, 4096, 16384])
def test_benchmark_shapes(gpu_lib, S):
    rows = sample_rows(S, tiles=(32, 128), extra=24, seed=6) if S > 1024 else None
    if rows is not None and S == 16384:
        rows = rows[::3]
    _run(gpu_lib, 16384 // S, 16, S, rows=rows)
