"""CPU checks of bench.py's work model and bookkeeping (no GPU).

The visible-pair counts that every TFLOP/s figure divides by are pinned
against the oracle's explicit mask matrices; the traffic lookup must return a
number only for the kernel source it was measured on; more than one GPU is
refused before anything touches a device.
"""

import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import oracle
from workloads import inputs as wi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("S", [1, 5, 64, 300, 1000])
@pytest.mark.parametrize("mask", oracle.MASKS)
def test_visible_pairs_match_mask_matrices(S, mask):
    window, prefix = max(1, S // 3), S // 4
    rows = np.arange(S)
    if mask == "document":
        lens = wi.doc_lengths(4, 1, S, lo=1, hi=max(1, S // 2))[0]
        doc = np.repeat(np.arange(len(lens)), lens)
        want = int(oracle.allowed_matrix(mask, rows, S, doc_row=doc).sum())
        assert bench.visible_pairs(mask, S, doc_lens=lens) == want
    else:
        want = int(oracle.allowed_matrix(mask, rows, S, window=window, prefix_len=prefix).sum())
        assert bench.visible_pairs(mask, S, window=window, prefix_len=prefix) == want


def test_flops_and_bytes_formulas():
    B, H, S, D = 4, 16, 4096, 64
    assert bench.attn_flops(B, H, S, D, "none") == 274877906944  # 4 * D per pair, S^2 pairs per head
    assert bench.attn_bytes(B, H, H, S, D) == 134217728          # Q, K, V, O once in bf16
    assert bench.attn_bytes(B, H, 2, S, D) == 2 * (2 * B * H * S * D + 2 * B * 2 * S * D)
    lens = wi.doc_lengths(4, B, S)
    assert bench.attn_flops(B, H, S, D, "document", doc_lens=lens) == \
        sum(sum(int(L) * int(L) for L in row) for row in lens) * H * 4 * D


def test_traffic_lookup_follows_the_source_hash(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    f = prof / "attn_fwd_S4096_hbm_traffic.txt"
    f.write_text(f"# comment\nkernel_source_sha={bench.kernel_source_sha()}\n"
                 "traffic_bytes_per_launch.alibi=123\n")
    for rel in bench.KERNEL_SOURCES:  # the hash reads the kernel sources under ROOT
        os.makedirs(tmp_path / os.path.dirname(rel), exist_ok=True)
        (tmp_path / rel).write_bytes(open(os.path.join(ROOT, rel), "rb").read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("alibi") == 123.0
    assert bench.measured_traffic("softcap") is None          # no line for it
    f.write_text("kernel_source_sha=0000000000000000\ntraffic_bytes_per_launch.alibi=123\n")
    assert bench.measured_traffic("alibi") is None            # measured on another source


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
