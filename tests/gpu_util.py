"""Helpers shared by the GPU parity tests (host side only)."""

import numpy as np
import torch

from workloads import inputs as wi

ATOL = 1e-2  # parity gate: |gpu - ref| <= ATOL + RTOL * |ref|, elementwise
RTOL = 1e-2


def to_dev(bits, dev="cuda"):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def f64(bits):
    return wi.bf16_bits_to_f64(bits)


def assert_close(got, ref, what, atol=ATOL, rtol=RTOL):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bad = err > atol + rtol * np.abs(ref)
    if bad.any():
        idx = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} elements out of tolerance; max|err| {err.max():.3e}; "
                             f"first at {tuple(idx)} got {got[tuple(idx)]} ref {ref[tuple(idx)]}")
    return float(err.max())


def assert_rms_rel(got, ref, what, bound=0.05):
    """Diagnostic beside the elementwise gate: for every output row (last axis),
    max|err| / rms(ref row) <= bound.  At long sequences attention outputs are
    small (rms ~ sqrt(e / S)), where the 1e-2 absolute term alone would pass
    almost anything.  Per row, because masked rows differ in scale by orders of
    magnitude (causal row 0 is V[0]); within a row of D values max <= sqrt(D)
    rms, so the bf16 output rounding alone stays below 2^-9 sqrt(64) = 1.6 %."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref, axis=-1))
    err = np.abs(got - ref).max(axis=-1)
    live = rms > 0
    if not live.any():
        return 0.0
    r = err[live] / rms[live]
    worst = float(r.max())
    assert worst <= bound, (f"{what}: max over rows of max|err| / rms(ref row) = {worst:.3e} > {bound} "
                            f"at row {tuple(np.argwhere(live)[int(r.argmax())])}")
    return worst


def sample_rows_at_least(S, n=512, tiles=(64, 128), seed=0, must=()):
    """sample_rows() topped up with random rows until at least n distinct rows."""
    extra = 0
    while True:
        rows = sample_rows(S, tiles=tiles, extra=extra, seed=seed, must=must)
        if len(rows) >= min(n, S):
            return rows
        extra += max(16, min(n, S) - len(rows))


def sample_rows(S, tiles=(64, 128), extra=64, seed=0, must=()):
    """Exact-check row sample: edges, every tile boundary +-1, given rows, plus random rows."""
    rows = {0, 1, S - 1, S - 2}
    for t in tiles:
        for m in range(t, S, t):
            rows.update((m - 1, m, m + 1))
    rows.update(int(r) for r in must)
    rng = np.random.default_rng(seed)
    rows.update(rng.integers(0, S, size=extra).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < S), dtype=np.int64)


def canary_empty(shape, dtype, dev="cuda", pad=4096):
    """Tensor of `shape` carved from a larger buffer whose tail holds a canary pattern."""
    n = int(np.prod(shape))
    if dtype == torch.bfloat16:
        big = torch.full((n + pad,), -12345.0, dtype=dtype, device=dev)
    else:
        big = torch.full((n + pad,), 7.25e30, dtype=dtype, device=dev)
    return big[:n].view(shape), big


def canary_intact(big, n):
    tail = big[n:]
    expect = -12345.0 if big.dtype == torch.bfloat16 else 7.25e30
    return bool(torch.all(tail == torch.tensor(expect, dtype=big.dtype, device=big.device)).item())
