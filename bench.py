#!/usr/bin/env python3
"""Benchmark of the fused attention forward on one MI355X.

One step = the hot path over the headline workload: the MHA score-modifier
shape at S = 4096 (B = 4, H = 16, D = 64, 16k tokens), run once per score
modifier (vanilla, ALiBi, tanh softcap).  Inputs are seeded synthetic bf16
N(0,1) tensors resident in HBM before timing starts.  Prints ONE JSON line.

Throughput is visible (unmasked) FLOPs / time: 4 * D flops per visible
(query, key) pair (QK^T and PV).  The roofline block covers the slowest of
the three kernels, timed with HIP events on the launch stream; the CPU
baseline is the fp64 oracle timed on a bounded sample of the same workload.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
  python bench.py --sweep OUT.jsonl     (all shapes of every variant, one line each)
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

from workloads import inputs as wi  # noqa: E402

METRIC = "attention fwd TFLOP/s (visible FLOPs) & % bf16 MFMA peak, per variant"
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = (
    "attention_variants_amd/csrc/attn_fwd.hip",
    "attention_variants_amd/csrc/attn_tile.hpp",
    "attention_variants_amd/csrc/av_device.hpp",
    "attention_variants_amd/csrc/av_kernels.hpp",    # the kernel's argument block and tile shapes
    "attention_variants_amd/csrc/attnvar_api.cpp",   # launch choices and host-computed constants (softcap form)
)


# ----------------------------------------------------------------- work model
def visible_pairs(mask, S, *, window=256, prefix_len=0, doc_lens=None):
    """Number of visible (query, key) pairs of one head."""
    if mask == "none":
        return S * S
    if mask == "causal":
        return S * (S + 1) // 2
    if mask == "sliding_window":
        W = min(window, S)
        return W * (W + 1) // 2 + (S - W) * W
    if mask == "prefix_lm":
        P = prefix_len
        return P * P + (S * (S + 1) // 2 - P * (P + 1) // 2)
    if mask == "document":
        return sum(L * L for L in doc_lens)
    raise ValueError(mask)


def attn_flops(B, Hq, S, D, mask, **kw):
    if mask == "document":
        return sum(visible_pairs(mask, S, doc_lens=lens) for lens in kw["doc_lens"]) * Hq * 4 * D
    return B * Hq * visible_pairs(mask, S, **kw) * 4 * D


def attn_bytes(B, Hq, Hkv, S, D):
    return 2 * (2 * B * Hq * S * D + 2 * B * Hkv * S * D)


def kernel_source_sha():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(score_mod="none"):
    """HBM bytes per launch of the kernel of `score_mod` from the committed
    counter summary, if it was taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "attn_fwd_S4096_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.strip().split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha") != kernel_source_sha():
        return None
    try:
        return float(kv[f"traffic_bytes_per_launch.{score_mod}"])
    except (KeyError, ValueError):
        return None


# ----------------------------------------------------------------- GPU timing
def _dev(bits, dev):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def time_launches(fns, steps, warmup, min_warm_s=0.2):
    """Run each callable of `fns` once per step; return (total_ms, [per-fn mean ms]).

    Warm-up runs at least `warmup` rounds and at least `min_warm_s` seconds, so
    the GPU clock has ramped up after any idle gap (input generation on the
    host) before timing starts."""
    import torch

    t_end = time.perf_counter() + min_warm_s
    n = 0
    while n < warmup or time.perf_counter() < t_end:
        for f in fns:
            f()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    starts = [[torch.cuda.Event(enable_timing=True) for _ in range(steps)] for _ in fns]
    ends = [[torch.cuda.Event(enable_timing=True) for _ in range(steps)] for _ in fns]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for s in range(steps):
        for i, f in enumerate(fns):
            starts[i][s].record()
            f()
            ends[i][s].record()
    t1.record()
    torch.cuda.synchronize()
    total = t0.elapsed_time(t1)
    per = [sum(starts[i][s].elapsed_time(ends[i][s]) for s in range(steps)) / steps for i in range(len(fns))]
    return total, per


# ----------------------------------------------------------------- CPU baseline
_CPU_X = None
CPU_ROW_BLOCK = 1024


def _cpu_worker_init(S, D):
    """Pool worker: one BLAS thread (the pool supplies the parallelism) and the
    seeded inputs of one batch entry, two heads, of the S x D shape."""
    global _CPU_X
    try:
        from threadpoolctl import threadpool_limits

        threadpool_limits(1)
    except Exception:  # noqa: BLE001
        pass
    x = wi.attention_inputs(1, 2, 2, S, S, D)
    _CPU_X = tuple(wi.bf16_bits_to_f64(x[n]) for n in ("q", "k", "v"))


def _cpu_task(task):
    """One (head, 1024-row query block) of the oracle; returns its visible FLOPs."""
    import oracle

    h, sm, r0 = task
    q, k, v = _CPU_X
    S, D = q.shape[2], q.shape[3]
    rows = np.arange(r0, min(r0 + CPU_ROW_BLOCK, S))
    oracle.attention(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], score_mod=sm, rows=rows)
    return len(rows) * S * 4 * D


def cpu_baseline(budget_s=15.0):
    """The fp64 oracle, unchanged, on a bounded sample of the workload: blocks
    of 1024 query rows of (batch entry, head) slices of the S = 4096, D = 64
    shape, cycling vanilla / ALiBi / softcap, spread over a process pool of
    one worker per host core (at most 16, the machine's CPU share), each worker
    with one BLAS thread, until the time budget is spent.  Rate = visible
    FLOPs of the blocks done / wall time.  Run before the GPU is touched, so
    the pool forks a process that holds no device state."""
    import multiprocessing as mp

    S, D = 4096, 64
    workers = max(1, min(os.cpu_count() or 1, 16))
    mods = ("none", "alibi", "softcap")
    nblk = S // CPU_ROW_BLOCK

    def task(i):
        return ((i // nblk) % 2, mods[(i // (2 * nblk)) % 3], (i % nblk) * CPU_ROW_BLOCK)

    ctx = mp.get_context("fork")
    with ctx.Pool(workers, initializer=_cpu_worker_init, initargs=(S, D)) as pool:
        pool.map(_cpu_task, [(0, "none", 0)] * workers)  # every worker has its inputs
        # one block in flight per worker; a new one is issued only while time remains
        t0 = time.perf_counter()
        deadline = t0 + budget_s
        pending = [pool.apply_async(_cpu_task, (task(i),)) for i in range(workers)]
        issued, done, flops = workers, 0, 0
        while pending:
            r = pending.pop(0)
            flops += r.get()
            done += 1
            if time.perf_counter() < deadline:
                pending.append(pool.apply_async(_cpu_task, (task(issued),)))
                issued += 1
        dt = time.perf_counter() - t0
    return {
        "value": round(flops / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": int(workers),
        "kind": "oracle",
        "blas_threads_per_worker": 1,
        "host_cpu_count": os.cpu_count(),
        "sample": f"{done} blocks of {CPU_ROW_BLOCK} query rows x {S} keys (D={D}) of the S={S} shape, "
                  f"cycling vanilla/ALiBi/softcap, on a pool of {workers} processes, {dt:.1f} s wall, "
                  f"fp64 numpy",
    }


# ----------------------------------------------------------------- main bench
def run_headline(args, cpu_rec=None):
    import torch

    import attention_variants_amd as av

    av.load_library()
    dev = torch.device("cuda:0")
    B, H, S, D = 4, 16, 4096, 64
    x = wi.attention_inputs(B, H, H, S, S, D)
    q, k, v = (_dev(x[n], dev) for n in ("q", "k", "v"))
    out = torch.empty_like(q)
    mods = ("none", "alibi", "softcap")
    fns = [(lambda sm=sm: av.attn_fwd(q, k, v, score_mod=sm, out=out)) for sm in mods]
    total_ms, per_ms = time_launches(fns, args.steps, args.warmup)
    fl = attn_flops(B, H, S, D, "none")
    ms_step = total_ms / args.steps
    value = 3 * fl / (ms_step * 1e-3) / 1e12
    variants = {}
    for sm, ms in zip(mods, per_ms):
        tf = fl / (ms * 1e-3) / 1e12
        variants[sm] = {"us": round(ms * 1e3, 2), "tflops": round(tf, 1), "frac_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
    dom = max(range(3), key=lambda i: per_ms[i])
    achieved = fl / (per_ms[dom] * 1e-3) / 1e12
    traffic = measured_traffic(mods[dom])
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "mha_score_mod_S4096",
            "B": B, "H": H, "S": S, "D": D,
            "variants": list(mods),
            "step": "one attn_fwd per score modifier (vanilla, ALiBi, softcap), no mask",
        },
        "roofline": {
            "bound": "mfma",
            "kernel": f"attn_fwd_kernel<D=64, score_mod={mods[dom]}, mask=none>",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "avg_launch_us": round(per_ms[dom] * 1e3, 2),
            "algorithmic_flops_per_launch": fl,
            "algorithmic_bytes_per_launch": attn_bytes(B, H, H, S, D),
        },
        "variants": variants,
    }
    rec["cpu_baseline"] = cpu_rec
    return rec


def run_sweep(path, steps, warmup):
    """Every shape of every variant (score mods, masks MHA/GQA, diff, Evoformer); one JSON line each."""
    import torch

    import attention_variants_amd as av

    av.load_library()
    dev = torch.device("cuda:0")
    f = open(path, "w")

    def emit(rec):
        f.write(json.dumps(rec) + "\n")
        f.flush()
        print(json.dumps(rec), file=sys.stderr, flush=True)

    for S in (512, 1024, 2048, 4096, 8192, 16384):
        B = 16384 // S
        for Hkv in (16, 2):
            x = wi.attention_inputs(B, 16, Hkv, S, S, 64)
            q, k, v = (_dev(x[n], dev) for n in ("q", "k", "v"))
            out = torch.empty_like(q)
            doc_np = wi.doc_ids(4, B, S)
            doc = torch.from_numpy(doc_np).to(dev)
            doc_lens = wi.doc_lengths(4, B, S)
            cases = [("none", "none"), ("alibi", "none"), ("softcap", "none")] if Hkv == 16 else []
            cases += [("none", "causal"), ("none", "sliding_window"), ("none", "prefix_lm"), ("none", "document"),
                      ("none", "document+order")]
            # the document mask's heaviest-first work order: built once per
            # document layout (its own time is reported), reused by every call
            order = av.attn_doc_order(doc)
            _, per_order = time_launches([lambda: av.attn_doc_order(doc, out=order)], steps, warmup)
            for sm, case in cases:
                mk = case.split("+")[0]
                kw = dict(score_mod=sm, mask=mk, window=256, prefix_len=S // 4,
                          doc_id=doc if mk == "document" else None, out=out,
                          doc_order=order if case == "document+order" else None)
                _, per = time_launches([lambda kw=kw: av.attn_fwd(q, k, v, **kw)], steps, warmup)
                fl = attn_flops(B, 16, S, 64, mk, window=256, prefix_len=S // 4, doc_lens=doc_lens)
                by = attn_bytes(B, 16, Hkv, S, 64)
                tf = fl / (per[0] * 1e-3) / 1e12
                rec = {"kernel": "attn_fwd", "score_mod": sm, "mask": case, "B": B, "Hq": 16, "Hkv": Hkv, "S": S,
                       "D": 64, "us": round(per[0] * 1e3, 2), "visible_tflops": round(tf, 1),
                       "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                       "hbm_gbs": round(by / (per[0] * 1e-3) / 1e9, 1)}
                if case == "document+order":
                    rec["order_build_us"] = round(per_order[0] * 1e3, 2)
                emit(rec)
    # the bias-tensor score modifier at S = 4096: one bias per head shared over
    # the batch ([1, 16, S, S], 537 MB) and one per (batch, head) ([4, 16, S, S], 2.1 GB)
    S, B = 4096, 4
    x = wi.attention_inputs(B, 16, 16, S, S, 64)
    q, k, v = (_dev(x[n], dev) for n in ("q", "k", "v"))
    out = torch.empty_like(q)
    for Bb in (1, B):
        bias = torch.randn((Bb, 16, S, S), device=dev, generator=torch.Generator(dev).manual_seed(18),
                           dtype=torch.float32).to(torch.bfloat16)
        for mk in ("none", "causal"):
            _, per = time_launches([lambda mk=mk: av.attn_fwd(q, k, v, score_mod="bias", mask=mk, bias=bias,
                                                              out=out)], steps, warmup)
            fl = attn_flops(B, 16, S, 64, mk)
            by = attn_bytes(B, 16, 16, S, 64) + bias.numel() * 2 * (0.5 if mk == "causal" else 1.0)
            tf = fl / (per[0] * 1e-3) / 1e12
            emit({"kernel": "attn_fwd", "score_mod": "bias", "bias_shape": list(bias.shape), "mask": mk, "B": B,
                  "Hq": 16, "Hkv": 16, "S": S, "D": 64, "us": round(per[0] * 1e3, 2),
                  "visible_tflops": round(tf, 1), "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                  "hbm_gbs_incl_bias_once": round(by / (per[0] * 1e-3) / 1e9, 1)})
        del bias
    # differential attention: 16 heads with halves of 64 and V of 128, and 32
    # heads with halves of 32 and V of 64 (visible work 2 * 2*Dh + 2*Dv per pair)
    for (H, Dh, Dv) in ((16, 64, 128), (32, 32, 64)):
        for S in (1024, 4096, 16384):
            B = 16384 // S
            x = wi.diff_inputs(B, H, S, Dh, Dv)
            q, k, v = (_dev(x[n], dev) for n in ("q", "k", "v"))
            out = torch.empty_like(v)
            _, per = time_launches([lambda: av.diff_attn_fwd(q, k, v, out=out)], steps, warmup)
            pairs = B * H * S * (S + 1) // 2
            fpp = 4 * Dh + 2 * Dv
            tf = pairs * fpp / (per[0] * 1e-3) / 1e12
            emit({"kernel": "diff_attn_fwd", "B": B, "H": H, "S": S, "Dh": Dh, "Dv": Dv,
                  "us": round(per[0] * 1e3, 2), "visible_tflops": round(tf, 1),
                  "executed_tflops": round(tf * (fpp + 2 * Dv) / fpp, 1),
                  "frac_mfma_peak_visible": round(tf / PEAK_BF16_TFLOPS, 4)})
            # the full head (lambda re-parameterisation and per-row RMSNorm fused in the epilogue)
            hp = {n: torch.from_numpy(a).to(dev) for n, a in wi.diff_head_params(Dh, Dv).items()}
            _, per = time_launches([lambda: av.diff_head_fwd(q, k, v, hp["lq1"], hp["lk1"], hp["lq2"], hp["lk2"],
                                                             lambda_init=0.2, gamma=hp["gamma"], out=out)],
                                   steps, warmup)
            tf = pairs * fpp / (per[0] * 1e-3) / 1e12
            emit({"kernel": "diff_head_fwd", "B": B, "H": H, "S": S, "Dh": Dh, "Dv": Dv,
                  "us": round(per[0] * 1e3, 2), "visible_tflops": round(tf, 1),
                  "frac_mfma_peak_visible": round(tf / PEAK_BF16_TFLOPS, 4)})
    # backward at the headline shape (algorithmic work: 5 products of 2*S*S*D
    # per head, i.e. 2.5x the forward's visible FLOPs)
    for (sm, mk_case) in (("none", "none"), ("softcap", "causal"), ("none", "causal"), ("none", "sliding_window"),
                          ("none", "prefix_lm"), ("none", "document"), ("none", "document+order")):
        mk = "document" if mk_case == "document+order" else mk_case
        B, H, S, D = 4, 16, 4096, 64
        x = wi.attention_inputs(B, H, H, S, S, D)
        q, k, v = (_dev(x[n], dev) for n in ("q", "k", "v"))
        dout = _dev(wi.normal_bf16(5, (B, H, S, D), 1.0), dev)
        mkw = dict(window=256, prefix_len=S // 4,
                   doc_id=torch.from_numpy(wi.doc_ids(4, B, S)).to(dev) if mk == "document" else None)
        out, lse = av.attn_fwd(q, k, v, score_mod=sm, mask=mk, return_lse=True, **mkw)
        if mk_case == "document+order":
            # the forward's heaviest-first order, built once per document layout
            mkw["doc_order"] = av.attn_doc_order(mkw["doc_id"])
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(av.attn_bwd_workspace_bytes(B, H, H, S, S, D), dtype=torch.uint8, device=dev)
        _, per = time_launches([lambda: av.attn_bwd(q, k, v, dout, lse, score_mod=sm, mask=mk, dq=dq, dk=dk, dv=dv,
                                                    workspace=ws, **mkw)], steps, warmup)
        fl = 2.5 * attn_flops(B, H, S, D, mk, window=256, prefix_len=S // 4, doc_lens=wi.doc_lengths(4, B, S))
        tf = fl / (per[0] * 1e-3) / 1e12
        emit({"kernel": "attn_bwd", "score_mod": sm, "mask": mk_case, "B": B, "H": H, "S": S, "D": D,
              "us": round(per[0] * 1e3, 2), "algorithmic_tflops": round(tf, 1),
              "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4)})
    # decoding: one new query per sequence against its key/value cache
    # (LLaMA-3.2-1B attention shape: 32 query heads, 8 KV heads, D = 64)
    for (B, Skv) in ((64, 4096), (8, 16384), (1, 16384)):
        Hq, Hkv, D = 32, 8, 64
        x = wi.attention_inputs(B, Hq, Hkv, 1, Skv, D)
        q, k, v = (_dev(x[n], dev) for n in ("q", "k", "v"))
        out = torch.empty_like(q)
        ws = torch.empty(max(1, av.attn_decode_workspace_bytes(B, Hq, Hkv, 1, Skv, D)), dtype=torch.uint8, device=dev)
        for sm, mk in (("none", "causal"), ("softcap", "causal")):
            _, per = time_launches([lambda: av.attn_decode_fwd(q, k, v, score_mod=sm, mask=mk, out=out,
                                                                workspace=ws)], steps, warmup)
            byts = 2 * (2 * B * Hkv * Skv * D + 2 * B * Hq * D)
            emit({"kernel": "attn_decode_fwd", "score_mod": sm, "mask": mk, "B": B, "Hq": Hq, "Hkv": Hkv, "Sq": 1,
                  "Skv": Skv, "D": D, "us": round(per[0] * 1e3, 2), "hbm_gbs": round(byts / (per[0] * 1e-3) / 1e9, 1),
                  "frac_hbm_peak": round(byts / (per[0] * 1e-3) / 8e12, 4)})
    # the same against a paged cache (16-key pages handed out in a shuffled order)
    for (B, Skv, ps) in ((64, 4096, 16), (8, 16384, 64)):
        Hq, Hkv, D = 32, 8, 64
        npg = B * Skv // ps
        x = wi.attention_inputs(npg, Hkv, Hkv, ps, ps, D)
        kc, vc = _dev(x["k"], dev), _dev(x["v"], dev)
        q = _dev(wi.attention_inputs(B, Hq, Hkv, 1, 1, D)["q"], dev)
        bt = torch.from_numpy(np.random.default_rng(0).permutation(npg).astype(np.int32).reshape(B, Skv // ps)).to(dev)
        sl = torch.full((B,), Skv, dtype=torch.int32, device=dev)
        out = torch.empty_like(q)
        ws = torch.empty(max(1, av.attn_decode_paged_workspace_bytes(B, Hq, Hkv, 1, D, ps, Skv // ps)),
                         dtype=torch.uint8, device=dev)
        _, per = time_launches([lambda: av.attn_decode_paged_fwd(q, kc, vc, bt, sl, score_mod="softcap",
                                                                  mask="causal", out=out, workspace=ws)],
                               steps, warmup)
        byts = 2 * (2 * B * Hkv * Skv * D + 2 * B * Hq * D)
        emit({"kernel": "attn_decode_paged_fwd", "score_mod": "softcap", "mask": "causal", "B": B, "Hq": Hq,
              "Hkv": Hkv, "Sq": 1, "Skv": Skv, "page_size": ps, "D": D, "us": round(per[0] * 1e3, 2),
              "hbm_gbs": round(byts / (per[0] * 1e-3) / 1e9, 1), "frac_hbm_peak": round(byts / (per[0] * 1e-3) / 8e12, 4)})
    # Evoformer: the AlphaFold2 head shape 8 x 32 and the kernel-benchmark 4 x 64
    for (Hh, dh, Nr) in [(8, 32, n) for n in (256, 384, 768)] + [(4, 64, n) for n in (256, 384, 768)]:
        Ns, Cm = 128, 256
        x = wi.evoformer_inputs(Ns, Nr, Cm, Hh, dh)
        t = {n: _dev(x[n], dev) for n in x}
        ws = torch.empty(av.evoformer_workspace_bytes(Ns, Nr, Hh, dh), dtype=torch.uint8, device=dev)
        out = torch.empty((Ns, Nr, Hh * dh), dtype=torch.bfloat16, device=dev)
        try:
            _, per = time_launches([lambda: av.evoformer_gated_attn_fwd(t["m"], t["wq"], t["wk"], t["wv"], t["wg"],
                                                                        t["bias"], H=Hh, dh=dh, workspace=ws,
                                                                        out=out)], steps, warmup)
        except RuntimeError as e:
            emit({"kernel": "evoformer", "Nr": Nr, "error": str(e)})
            continue
        fl = 2 * Ns * Nr * Cm * 4 * Hh * dh + 4 * Ns * Hh * Nr * Nr * dh
        tf = fl / (per[0] * 1e-3) / 1e12
        emit({"kernel": "evoformer_gated_attn_fwd", "Ns": Ns, "Nr": Nr, "H": Hh, "dh": dh,
              "us": round(per[0] * 1e3, 2),
              "visible_tflops": round(tf, 1), "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4)})
        # column-wise form on the same MSA: attention over the 128 sequences of each residue column
        _, per = time_launches([lambda: av.evoformer_col_gated_attn_fwd(t["m"], t["wq"], t["wk"], t["wv"], t["wg"],
                                                                        H=Hh, dh=dh, workspace=ws, out=out)],
                               steps, warmup)
        fl = 2 * Ns * Nr * Cm * 4 * Hh * dh + 4 * Nr * Hh * Ns * Ns * dh
        tf = fl / (per[0] * 1e-3) / 1e12
        emit({"kernel": "evoformer_col_gated_attn_fwd", "Ns": Ns, "Nr": Nr, "H": Hh, "dh": dh,
              "us": round(per[0] * 1e3, 2),
              "visible_tflops": round(tf, 1), "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4)})
    f.close()


def run_profile(what, steps, nres=256, evo_heads=8):
    """Launch one kernel `steps` times with nothing else on the stream."""
    import torch

    dev = torch.device("cuda:0")
    if what == "copy":
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"profile": "copy", "bytes_read_per_launch": n, "bytes_written_per_launch": n}))
        return
    import attention_variants_amd as av

    av.load_library()
    if what == "evoformer":
        Ns, Nr, Cm, Hh, dh = 128, nres, 256, evo_heads, 256 // evo_heads
        x = wi.evoformer_inputs(Ns, Nr, Cm, Hh, dh)
        t = {n: _dev(x[n], dev) for n in x}
        ws = torch.empty(av.evoformer_workspace_bytes(Ns, Nr, Hh, dh), dtype=torch.uint8, device=dev)
        out = torch.empty((Ns, Nr, Hh * dh), dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()
        for _ in range(steps):
            av.evoformer_gated_attn_fwd(t["m"], t["wq"], t["wk"], t["wv"], t["wg"], t["bias"], H=Hh, dh=dh,
                                        workspace=ws, out=out)
        torch.cuda.synchronize()
        print(json.dumps({"profile": "evoformer", "Ns": Ns, "Nr": Nr, "H": Hh, "dh": dh, "launches": steps}))
        return
    if what == "evoformer_col":
        Ns, Nr, Cm, Hh, dh = 128, nres, 256, evo_heads, 256 // evo_heads
        x = wi.evoformer_inputs(Ns, Nr, Cm, Hh, dh)
        t = {n: _dev(x[n], dev) for n in x}
        ws = torch.empty(av.evoformer_workspace_bytes(Ns, Nr, Hh, dh), dtype=torch.uint8, device=dev)
        out = torch.empty((Ns, Nr, Hh * dh), dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()
        for _ in range(steps):
            av.evoformer_col_gated_attn_fwd(t["m"], t["wq"], t["wk"], t["wv"], t["wg"], H=Hh, dh=dh,
                                            workspace=ws, out=out)
        torch.cuda.synchronize()
        print(json.dumps({"profile": "evoformer_col", "Ns": Ns, "Nr": Nr, "H": Hh, "dh": dh, "launches": steps}))
        return
    if what in ("decode", "decode_b1"):
        B, Hq, Hkv, Skv, D = (64, 32, 8, 4096, 64) if what == "decode" else (1, 32, 8, 16384, 64)
        x = wi.attention_inputs(B, Hq, Hkv, 1, Skv, D)
        q, k, v = (_dev(x[n], dev) for n in ("q", "k", "v"))
        out = torch.empty_like(q)
        ws = torch.empty(max(1, av.attn_decode_workspace_bytes(B, Hq, Hkv, 1, Skv, D)), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        for _ in range(steps):
            av.attn_decode_fwd(q, k, v, score_mod="softcap", mask="causal", out=out, workspace=ws)
        torch.cuda.synchronize()
        print(json.dumps({"profile": what, "B": B, "Hq": Hq, "Hkv": Hkv, "Skv": Skv, "launches": steps}))
        return
    if what == "bwd":
        B, H, S, D = 4, 16, 4096, 64
        x = wi.attention_inputs(B, H, H, S, S, D)
        q, k, v = (_dev(x[n], dev) for n in ("q", "k", "v"))
        dout = _dev(wi.normal_bf16(5, (B, H, S, D), 1.0), dev)
        out, lse = av.attn_fwd(q, k, v, return_lse=True)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(av.attn_bwd_workspace_bytes(B, H, H, S, S, D), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        for _ in range(steps):
            av.attn_bwd(q, k, v, dout, lse, dq=dq, dk=dk, dv=dv, workspace=ws)
        torch.cuda.synchronize()
        print(json.dumps({"profile": "bwd", "B": B, "H": H, "S": S, "D": D, "launches": steps}))
        return
    if what == "bwd_document":
        # the document mask, natural order then the heaviest-first order
        B, H, S, D = 4, 16, 4096, 64
        x = wi.attention_inputs(B, H, H, S, S, D)
        q, k, v = (_dev(x[n], dev) for n in ("q", "k", "v"))
        dout = _dev(wi.normal_bf16(5, (B, H, S, D), 1.0), dev)
        doc = torch.from_numpy(wi.doc_ids(4, B, S)).to(dev)
        out, lse = av.attn_fwd(q, k, v, mask="document", doc_id=doc, return_lse=True)
        order = av.attn_doc_order(doc)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(av.attn_bwd_workspace_bytes(B, H, H, S, S, D), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        for o in (None, order):
            for _ in range(steps):
                av.attn_bwd(q, k, v, dout, lse, mask="document", doc_id=doc, doc_order=o, dq=dq, dk=dk, dv=dv,
                            workspace=ws)
        torch.cuda.synchronize()
        print(json.dumps({"profile": "bwd_document", "B": B, "H": H, "S": S, "D": D,
                          "launches": steps, "orders": ["natural", "heaviest-first"]}))
        return
    if what == "bias":
        B, H, S, D = 4, 16, 4096, 64
        x = wi.attention_inputs(B, H, H, S, S, D)
        q, k, v = (_dev(x[n], dev) for n in ("q", "k", "v"))
        bias = _dev(wi.normal_bf16(18, (1, H, S, S), 2.0), dev)
        out = torch.empty_like(q)
        torch.cuda.synchronize()
        for _ in range(steps):
            av.attn_fwd(q, k, v, score_mod="bias", bias=bias, out=out)
        torch.cuda.synchronize()
        print(json.dumps({"profile": "bias", "B": B, "H": H, "S": S, "bias": [1, H, S, S], "launches": steps}))
        return
    if what == "document":
        # document mask at S = 4096 (16 heads, seeded lengths 64..S/2): the
        # heaviest-first order is built once per step, then the ordered forward
        B, H, S, D = 4, 16, 4096, 64
        x = wi.attention_inputs(B, H, H, S, S, D)
        q, k, v = (_dev(x[n], dev) for n in ("q", "k", "v"))
        doc = torch.from_numpy(wi.doc_ids(4, B, S)).to(dev)
        order = av.attn_doc_order(doc)
        out = torch.empty_like(q)
        torch.cuda.synchronize()
        for _ in range(steps):
            av.attn_doc_order(doc, out=order)
            av.attn_fwd(q, k, v, mask="document", doc_id=doc, doc_order=order, out=out)
        torch.cuda.synchronize()
        print(json.dumps({"profile": "document", "B": B, "H": H, "S": S, "D": D, "launches": steps}))
        return
    if what in ("window", "causal"):
        # sliding window 256 (causal) or plain causal at S = 4096, 16 heads
        B, H, S, D = 4, 16, 4096, 64
        x = wi.attention_inputs(B, H, H, S, S, D)
        q, k, v = (_dev(x[n], dev) for n in ("q", "k", "v"))
        out = torch.empty_like(q)
        mask = "sliding_window" if what == "window" else "causal"
        torch.cuda.synchronize()
        for _ in range(steps):
            av.attn_fwd(q, k, v, mask=mask, window=256, out=out)
        torch.cuda.synchronize()
        print(json.dumps({"profile": what, "B": B, "H": H, "S": S, "D": D, "window": 256, "launches": steps}))
        return
    if what == "kernels":
        # one launch family after another, `steps` launches each, for counters
        # that compare the instantiations (16k tokens: B = 4, S = 4096): the
        # forward at D = 32 and 128 with softcap under four masks (GQA 16/2,
        # document mask in natural order), the bias tensor, ALiBi causal and
        # PrefixLM at D = 64, both differential shapes, the column-wise
        # Evoformer at N_res 256 and dense decode (64 x 4096 keys)
        B, S = 4, 4096
        for D in (32, 128):
            x = wi.attention_inputs(B, 16, 2, S, S, D)
            q, k, v = (_dev(x[n], dev) for n in ("q", "k", "v"))
            for mk in ("none", "causal", "sliding_window", "document"):
                kw = dict(mask=mk, score_mod="softcap")
                if mk == "document":
                    kw["doc_id"] = torch.from_numpy(wi.doc_ids(4, B, S)).to(dev)
                for _ in range(steps):
                    av.attn_fwd(q, k, v, **kw)
        x = wi.attention_inputs(B, 16, 16, S, S, 64)
        q, k, v = (_dev(x[n], dev) for n in ("q", "k", "v"))
        bias = _dev(wi.normal_bf16(18, (1, 16, S, S), 2.0), dev)
        for _ in range(steps):
            av.attn_fwd(q, k, v, score_mod="bias", bias=bias)
        del bias
        for mk in ("causal", "prefix_lm"):
            for _ in range(steps):
                av.attn_fwd(q, k, v, mask=mk, score_mod="alibi", prefix_len=S // 4)
        for Dh, Dv, H in ((64, 128, 16), (32, 64, 32)):
            x = wi.diff_inputs(B, H, S, Dh, Dv)
            q, k, v = (_dev(x[n], dev) for n in ("q", "k", "v"))
            for _ in range(steps):
                av.diff_attn_fwd(q, k, v)
        x = wi.evoformer_inputs(128, 256, 256, 8, 32)
        t = {n: _dev(x[n], dev) for n in x}
        for _ in range(steps):
            av.evoformer_col_gated_attn_fwd(t["m"], t["wq"], t["wk"], t["wv"], t["wg"], H=8, dh=32)
        x = wi.attention_inputs(64, 32, 8, 1, 4096, 64)
        q, k, v = (_dev(x[n], dev) for n in ("q", "k", "v"))
        for _ in range(steps):
            av.attn_decode_fwd(q, k, v, score_mod="softcap", mask="causal")
        torch.cuda.synchronize()
        print(json.dumps({"profile": "kernels", "launches_each": steps}))
        return
    if what == "diff":
        x = wi.diff_inputs(4, 16, 4096)
        q, k, v = (_dev(x[n], dev) for n in ("q", "k", "v"))
        out = torch.empty_like(v)
        torch.cuda.synchronize()
        for _ in range(steps):
            av.diff_attn_fwd(q, k, v, out=out)
        torch.cuda.synchronize()
        print(json.dumps({"profile": "diff", "B": 4, "H": 16, "S": 4096, "launches": steps}))
        return
    B, H, S, D = 4, 16, 4096, 64
    x = wi.attention_inputs(B, H, H, S, S, D)
    q, k, v = (_dev(x[n], dev) for n in ("q", "k", "v"))
    out = torch.empty_like(q)
    torch.cuda.synchronize()
    for _ in range(steps):
        av.attn_fwd(q, k, v, score_mod=what, out=out)
    torch.cuda.synchronize()
    print(json.dumps({"profile": f"attn_fwd {what}", "B": B, "H": H, "S": S, "D": D, "launches": steps,
                      "algorithmic_bytes_per_launch": attn_bytes(B, H, H, S, D)}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--nres", type=int, default=256, help="N_res of the Evoformer profile run")
    ap.add_argument("--evo-heads", type=int, default=8, choices=[8, 4],
                    help="heads of the Evoformer profile run: 8 x 32 or 4 x 64")
    ap.add_argument("--sweep", default=None, help="write one JSON line per shape/variant to this file")
    ap.add_argument("--profile", choices=["none", "alibi", "softcap", "copy", "evoformer", "evoformer_col", "diff",
                                          "document", "window", "causal",
                                          "decode", "decode_b1", "bwd", "bwd_document", "bias", "kernels"],
                    default=None,
                    help="launch only this kernel --steps times (for counter collection); 'copy' is a "
                         "plain 1 GiB device copy used to calibrate the HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: measures one GPU only; --gpus must be 1 (the library has no multi-GPU path; "
              "sharding is a design note, not code)", file=sys.stderr)
        sys.exit(2)
    if args.sweep:
        run_sweep(args.sweep, args.steps, args.warmup)
        return
    if args.profile:
        run_profile(args.profile, args.steps, args.nres, args.evo_heads)
        return
    # the CPU baseline runs first: its pool forks a process that has not touched the GPU
    cpu_rec = None if args.no_cpu_baseline else cpu_baseline(args.cpu_budget)
    rec = run_headline(args, cpu_rec)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
