"""GPU parity of ``evoformer_gated_attn_fwd`` against the fp64 oracle (through the C ABI).

The oracle keeps the projections in fp64; the GPU rounds them to bf16 in the
workspace (fp32 accumulation), which stays far inside the gate
|gpu - oracle| <= 1e-2 + 1e-2 |oracle|.  Benchmark shapes (128 sequences,
256/384/768 residues, 8 heads x 32) are checked on sampled sequences and rows.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import inputs as wi

from .gpu_util import assert_close, canary_empty, canary_intact, f64, to_dev

pytestmark = pytest.mark.gpu


def _run(av, Ns, Nr, Cm=256, H=8, dh=32, seqs=None, rows=None, zero_gate=False, bias_shift=None):
    x = wi.evoformer_inputs(Ns, Nr, Cm, H, dh)
    if zero_gate:
        x["wg"] = np.zeros_like(x["wg"])
    t = {n: to_dev(x[n]) for n in x}
    out, big = canary_empty((Ns, Nr, H * dh), torch.bfloat16)
    av.evoformer_gated_attn_fwd(t["m"], t["wq"], t["wk"], t["wv"], t["wg"], t["bias"], H=H, dh=dh, out=out)
    torch.cuda.synchronize()
    assert canary_intact(big, out.numel()), "write past the end of out"
    ref = oracle.evoformer_row_gated_attention(f64(x["m"]), f64(x["wq"]), f64(x["wk"]), f64(x["wv"]), f64(x["wg"]),
                                               f64(x["bias"]), H=H, dh=dh, rows=rows, seqs=seqs)
    got = out.float().cpu().numpy()
    if seqs is not None:
        got = got[seqs]
    if rows is not None:
        got = got[:, rows]
    return assert_close(got, ref, f"evoformer Ns{Ns} Nr{Nr} Cm{Cm} H{H}"), out


@pytest.mark.parametrize("Nr", [1, 16, 17, 100, 129, 256])
def test_small_all_rows(gpu_lib, Nr):
    _run(gpu_lib, 3, Nr, Cm=128, H=4)


def test_channel_and_head_counts(gpu_lib):
    _run(gpu_lib, 2, 64, Cm=64, H=4)
    _run(gpu_lib, 2, 64, Cm=320, H=12)
    _run(gpu_lib, 130, 40, Cm=256, H=8)  # token count not a multiple of the GEMM tile
    # Cm = 256 takes the persistent projection when its 128-channel tiles
    # (H of them at dh = 32) divide 32: 4 and 16 tiles here; 12 take the tiled form
    _run(gpu_lib, 3, 100, Cm=256, H=4)
    _run(gpu_lib, 2, 72, Cm=256, H=16)
    _run(gpu_lib, 2, 72, Cm=256, H=12)


def test_zero_gate_is_half(gpu_lib):
    _, out = _run(gpu_lib, 2, 96, Cm=128, H=4, zero_gate=True)
    assert torch.isfinite(out.float()).all()


def test_deterministic(gpu_lib):
    x = wi.evoformer_inputs(4, 200, 256, 8, 32)
    t = {n: to_dev(x[n]) for n in x}
    r = [gpu_lib.evoformer_gated_attn_fwd(t["m"], t["wq"], t["wk"], t["wv"], t["wg"], t["bias"], H=8, dh=32)
         for _ in range(3)]
    assert torch.equal(r[0], r[1]) and torch.equal(r[1], r[2])


def test_workspace_too_small_is_rejected(gpu_lib):
    x = wi.evoformer_inputs(2, 32, 64, 4, 32)
    t = {n: to_dev(x[n]) for n in x}
    ws = torch.empty(100, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="bytes"):
        gpu_lib.evoformer_gated_attn_fwd(t["m"], t["wq"], t["wk"], t["wv"], t["wg"], t["bias"], H=4, dh=32,
                                         workspace=ws)


@pytest.mark.parametrize("Nr", [256, 384, 768])
def test_benchmark_shapes(gpu_lib, Nr):
    # 20 sequences spread over the grid (every 8th, the ends and random ones)
    # and about 46 residues per sequence, tile edges included
    rng = np.random.default_rng(7)
    seqs = np.unique(np.concatenate([np.arange(0, 128, 8), [1, 127], rng.integers(0, 128, 4)]))
    assert len(seqs) >= 16
    rows = np.unique(np.concatenate([[0, 1, Nr - 1, 127, 128, Nr // 2], rng.integers(0, Nr, 40)]))
    _run(gpu_lib, 128, Nr, seqs=seqs, rows=rows)


@pytest.mark.parametrize("Nr", [1, 17, 100, 129])
def test_head_width_64_all_rows(gpu_lib, Nr):
    """4 heads x 64 (the talk notes' Evoformer kernel-benchmark head shape), every row."""
    _run(gpu_lib, 3, Nr, Cm=128, H=4, dh=64)
    _run(gpu_lib, 2, Nr, Cm=256, H=4, dh=64)


@pytest.mark.parametrize("Nr", [256, 384, 768])
def test_benchmark_shapes_4x64(gpu_lib, Nr):
    """128 sequences, 4 heads x 64, Cm 256: sampled sequences and residues as above."""
    rng = np.random.default_rng(8)
    seqs = np.unique(np.concatenate([np.arange(0, 128, 8), [1, 127], rng.integers(0, 128, 4)]))
    rows = np.unique(np.concatenate([[0, 1, Nr - 1, 127, 128, Nr // 2], rng.integers(0, Nr, 40)]))
    _run(gpu_lib, 128, Nr, H=4, dh=64, seqs=seqs, rows=rows)


def test_pair_bias_minus_inf(gpu_lib):
    """A pair bias of -inf drops the pair (the bias enters the QK^T MFMA as its
    initial accumulator, where -inf stays -inf); about a third of the pairs
    are dropped, each row keeps its own residue."""
    Ns, Nr, Cm, H, dh = 3, 100, 128, 4, 32
    x = wi.evoformer_inputs(Ns, Nr, Cm, H, dh)
    drop = np.random.default_rng(41).random((H, Nr, Nr)) < 0.35
    drop[:, np.arange(Nr), np.arange(Nr)] = False
    x["bias"] = np.where(drop, np.uint16(0xFF80), x["bias"]).astype(np.uint16)
    t = {n: to_dev(x[n]) for n in x}
    out = gpu_lib.evoformer_gated_attn_fwd(t["m"], t["wq"], t["wk"], t["wv"], t["wg"], t["bias"], H=H, dh=dh)
    torch.cuda.synchronize()
    ref = oracle.evoformer_row_gated_attention(f64(x["m"]), f64(x["wq"]), f64(x["wk"]), f64(x["wv"]), f64(x["wg"]),
                                               f64(x["bias"]), H=H, dh=dh)
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all()
    assert_close(got, ref, "evoformer pair bias with -inf")


# Shapes that take the single-launch form (Cm = 256, N_res a multiple of 8,
# up to 256 residues, dh 32 or 64): every residue block count, odd and even,
# ragged last 64-key tiles, waves with no block, one block or two; and just
# past the limit (the two launches).
FUSED = [(8, 32, 8), (24, 32, 4), (64, 32, 8), (96, 64, 4), (200, 32, 8), (232, 64, 4), (256, 64, 4),
         (256, 32, 8), (264, 32, 8), (392, 32, 4)]


@pytest.mark.parametrize("Nr,dh,H", FUSED)
def test_fused_form_all_rows(gpu_lib, Nr, dh, H):
    _run(gpu_lib, 2, Nr, Cm=256, H=H, dh=dh)


def test_fused_form_pair_bias_minus_inf(gpu_lib):
    """As test_pair_bias_minus_inf, on the single-launch form."""
    Ns, Nr, Cm, H, dh = 3, 136, 256, 8, 32
    x = wi.evoformer_inputs(Ns, Nr, Cm, H, dh)
    drop = np.random.default_rng(42).random((H, Nr, Nr)) < 0.35
    drop[:, np.arange(Nr), np.arange(Nr)] = False
    x["bias"] = np.where(drop, np.uint16(0xFF80), x["bias"]).astype(np.uint16)
    t = {n: to_dev(x[n]) for n in x}
    out = gpu_lib.evoformer_gated_attn_fwd(t["m"], t["wq"], t["wk"], t["wv"], t["wg"], t["bias"], H=H, dh=dh)
    torch.cuda.synchronize()
    ref = oracle.evoformer_row_gated_attention(f64(x["m"]), f64(x["wq"]), f64(x["wk"]), f64(x["wv"]), f64(x["wg"]),
                                               f64(x["bias"]), H=H, dh=dh)
    got = out.float().cpu().numpy()
    assert np.isfinite(got).all()
    assert_close(got, ref, "evoformer single-launch form, pair bias with -inf")


def test_fused_form_deterministic(gpu_lib):
    x = wi.evoformer_inputs(4, 248, 256, 8, 32)
    t = {n: to_dev(x[n]) for n in x}
    r = [gpu_lib.evoformer_gated_attn_fwd(t["m"], t["wq"], t["wk"], t["wv"], t["wg"], t["bias"], H=8, dh=32)
         for _ in range(3)]
    assert torch.equal(r[0], r[1]) and torch.equal(r[1], r[2])


@pytest.mark.parametrize("Nr, Cm, one_launch", [(256, 256, True), (200, 256, True), (260, 256, False),
                                                (256, 128, False)])
def test_workspace_use_follows_the_path(gpu_lib, Nr, Cm, one_launch):
    """Cm 256 with N_res <= 256 (a multiple of 8) keeps the projections on
    chip and leaves the workspace bytes alone; the two-launch path writes its
    planes."""
    Ns, H, dh = 2, 8, 32
    x = wi.evoformer_inputs(Ns, Nr, Cm, H, dh)
    t = {n: to_dev(x[n]) for n in x}
    ws = torch.full((gpu_lib.evoformer_workspace_bytes(Ns, Nr, H, dh),), 0xA5, dtype=torch.uint8, device="cuda")
    out = gpu_lib.evoformer_gated_attn_fwd(t["m"], t["wq"], t["wk"], t["wv"], t["wg"], t["bias"], H=H, dh=dh,
                                           workspace=ws)
    torch.cuda.synchronize()
    untouched = bool((ws == 0xA5).all().item())
    assert untouched == one_launch
    ref = oracle.evoformer_row_gated_attention(f64(x["m"]), f64(x["wq"]), f64(x["wk"]), f64(x["wv"]), f64(x["wg"]),
                                               f64(x["bias"]), H=H, dh=dh)
    assert_close(out.float().cpu().numpy(), ref, f"evoformer row Nr{Nr} Cm{Cm}")
