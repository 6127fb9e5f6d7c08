"""GPU parity of ``evoformer_col_gated_attn_fwd`` (Evoformer column-wise gated
self-attention: per residue column and head, softmax attention over the
sequences, no pair bias) against the fp64 oracle, through the C ABI.

Gate: |gpu - oracle| <= 1e-2 + 1e-2 |oracle|.  The benchmark shapes (128
sequences, 256/384/768 residues, 8 heads x 32) are checked on sampled columns
and sequences, which is exact because columns are independent.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import inputs as wi

from .gpu_util import assert_close, canary_empty, canary_intact, f64, to_dev

pytestmark = pytest.mark.gpu


def _run(av, Ns, Nr, Cm=256, H=8, dh=32, seqs=None, cols=None, zero_gate=False):
    x = wi.evoformer_inputs(Ns, Nr, Cm, H, dh)
    if zero_gate:
        x["wg"] = np.zeros_like(x["wg"])
    t = {n: to_dev(x[n]) for n in ("m", "wq", "wk", "wv", "wg")}
    out, big = canary_empty((Ns, Nr, H * dh), torch.bfloat16)
    av.evoformer_col_gated_attn_fwd(t["m"], t["wq"], t["wk"], t["wv"], t["wg"], H=H, dh=dh, out=out)
    torch.cuda.synchronize()
    assert canary_intact(big, out.numel()), "write past the end of out"
    ref = oracle.evoformer_col_gated_attention(f64(x["m"]), f64(x["wq"]), f64(x["wk"]), f64(x["wv"]),
                                               f64(x["wg"]), H=H, dh=dh, cols=cols, seqs=seqs)
    got = out.float().cpu().numpy()
    if seqs is not None:
        got = got[seqs]
    if cols is not None:
        got = got[:, cols]
    return assert_close(got, ref, f"evoformer col Ns{Ns} Nr{Nr} Cm{Cm} H{H}"), out


@pytest.mark.parametrize("Ns", [1, 2, 16, 33, 128, 130])
def test_small_all_columns(gpu_lib, Ns):
    _run(gpu_lib, Ns, 7, Cm=128, H=4)


def test_channel_and_head_counts(gpu_lib):
    _run(gpu_lib, 64, 3, Cm=64, H=4)
    _run(gpu_lib, 40, 5, Cm=320, H=12)
    _run(gpu_lib, 257, 2, Cm=256, H=8)  # attention length past two 128-row tiles


def test_one_sequence_is_gated_v(gpu_lib):
    """Ns = 1: every column attends to itself only, out = sigmoid(g) * v."""
    _run(gpu_lib, 1, 300, Cm=128, H=4)


def test_zero_gate_is_half(gpu_lib):
    _, out = _run(gpu_lib, 50, 4, Cm=128, H=4, zero_gate=True)
    assert torch.isfinite(out.float()).all()


def test_column_equals_row_on_transposed_msa(gpu_lib):
    """The column form of m equals the row form of m^T with a zero bias (both GPU paths)."""
    Ns, Nr, Cm, H, dh = 40, 24, 128, 4, 32
    x = wi.evoformer_inputs(Ns, Nr, Cm, H, dh)
    t = {n: to_dev(x[n]) for n in ("m", "wq", "wk", "wv", "wg")}
    col = gpu_lib.evoformer_col_gated_attn_fwd(t["m"], t["wq"], t["wk"], t["wv"], t["wg"], H=H, dh=dh)
    mt = t["m"].transpose(0, 1).contiguous()
    zero = torch.zeros(H, Ns, Ns, dtype=torch.bfloat16, device="cuda")
    row = gpu_lib.evoformer_gated_attn_fwd(mt, t["wq"], t["wk"], t["wv"], t["wg"], zero, H=H, dh=dh)
    torch.cuda.synchronize()
    assert_close(col.float().cpu().numpy(), row.transpose(0, 1).float().cpu().numpy(), "col vs row(m^T)",
                 atol=1e-2, rtol=1e-2)


def test_deterministic(gpu_lib):
    x = wi.evoformer_inputs(64, 20, 256, 8, 32)
    t = {n: to_dev(x[n]) for n in ("m", "wq", "wk", "wv", "wg")}
    r = [gpu_lib.evoformer_col_gated_attn_fwd(t["m"], t["wq"], t["wk"], t["wv"], t["wg"], H=8, dh=32)
         for _ in range(3)]
    assert torch.equal(r[0], r[1]) and torch.equal(r[1], r[2])


@pytest.mark.parametrize("Nr", [256, 384, 768])
def test_benchmark_shapes(gpu_lib, Nr):
    rng = np.random.default_rng(8)
    seqs = np.unique(np.concatenate([[0, 1, 63, 64, 127], rng.integers(0, 128, 12)]))
    cols = np.unique(np.concatenate([[0, 1, Nr - 1, Nr // 2], rng.integers(0, Nr, 12)]))
    _run(gpu_lib, 128, Nr, seqs=seqs, cols=cols)


@pytest.mark.parametrize("Ns", [1, 33, 128, 130])
def test_head_width_64(gpu_lib, Ns):
    """4 heads x 64, every column of a small MSA."""
    _run(gpu_lib, Ns, 7, Cm=128, H=4, dh=64)
    _run(gpu_lib, Ns, 5, Cm=256, H=4, dh=64)


@pytest.mark.parametrize("dh", [32, 64])
@pytest.mark.parametrize("Ns", [127, 128, 129, 255, 256, 257, 300])
def test_sequence_counts_at_the_kernel_limits(gpu_lib, Ns, dh):
    """Cm 256 on both sides of each limit: the one-kernel path over 128 tokens
    and over 256 tokens, then the two launches past 256 sequences."""
    _run(gpu_lib, Ns, 3, Cm=256, H=8 if dh == 32 else 4, dh=dh)


@pytest.mark.parametrize("Nr", [256, 768])
def test_benchmark_shapes_4x64(gpu_lib, Nr):
    rng = np.random.default_rng(9)
    seqs = np.unique(np.concatenate([[0, 1, 63, 64, 127], rng.integers(0, 128, 12)]))
    cols = np.unique(np.concatenate([[0, 1, Nr - 1, Nr // 2], rng.integers(0, Nr, 28)]))
    _run(gpu_lib, 128, Nr, H=4, dh=64, seqs=seqs, cols=cols)


@pytest.mark.parametrize("Ns, Cm, one_launch", [(128, 256, True), (256, 256, True), (257, 256, False),
                                                (128, 128, False)])
def test_workspace_use_follows_the_path(gpu_lib, Ns, Cm, one_launch):
    """Cm 256 with at most 256 sequences keeps the projections on chip and
    leaves the workspace bytes alone; the two-launch path writes its planes."""
    Nr, H, dh = 5, 4, 64
    x = wi.evoformer_inputs(Ns, Nr, Cm, H, dh)
    t = {n: to_dev(x[n]) for n in ("m", "wq", "wk", "wv", "wg")}
    ws = torch.full((gpu_lib.evoformer_workspace_bytes(Ns, Nr, H, dh),), 0xA5, dtype=torch.uint8, device="cuda")
    out = gpu_lib.evoformer_col_gated_attn_fwd(t["m"], t["wq"], t["wk"], t["wv"], t["wg"], H=H, dh=dh, workspace=ws)
    torch.cuda.synchronize()
    untouched = bool((ws == 0xA5).all().item())
    assert untouched == one_launch
    ref = oracle.evoformer_col_gated_attention(f64(x["m"]), f64(x["wq"]), f64(x["wk"]), f64(x["wv"]),
                                               f64(x["wg"]), H=H, dh=dh)
    assert_close(out.float().cpu().numpy(), ref, f"evoformer col Ns{Ns} Cm{Cm}")
