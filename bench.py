#!/usr/bin/env python3
"""Lighthouse attention layer benchmark on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input: pool+score,
chunked top-K, map, causal attention reading its rows through the map, scatter (forward),
then scatter backward, the two attention backward passes and gather+pool backward.  The
steps run through the library's stage entry points (the same kernels lh_forward /
lh_backward launch, in the same order) with HIP events recorded between stages on the launch
stream, so every kernel's time comes from the timed steps themselves.  Inputs are resident
in HBM before timing starts.

Prints ONE JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import dataclasses
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Lighthouse fwd+bwd tokens/sec/layer at {n} on 1 GPU; % HBM and MFMA peak"


def metric_name(n_tokens):
    """The metric string, labelled with the token count actually run (512K for 524,288)."""
    if n_tokens % 1024 == 0:
        label = f"{n_tokens // 1024}K" if n_tokens < 1 << 20 else f"{n_tokens / 2**20:g}M"
    else:
        label = f"{n_tokens} tokens"
    return METRIC.format(n=label)
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(w, info):
    """Per-launch algorithmic work of each stage (bytes for HBM stages, flops for attention).

    Each stage counts its own inputs read once and outputs written once, at the dtypes the
    path stores: pooled levels bf16, scores float32, indices int32, Og / LSE / gathered
    gradients float32, dOg bf16; index maps count one read per pyramid entry (inv) or slot
    (gmap).  The attention reads its rows through gmap, so no gather stage exists.
    """
    B, N, H, D = w.batch, w.n_tokens, w.heads, w.head_dim
    S, P, P1, K = info.gathered_len, info.pyramid_total, info.pooled_rows, info.sel_total
    e = 2 if w.dtype == "bf16" else 4  # token-tensor element size
    BH = B * H
    pairs = BH * S * (S + 1) / 2
    # scored entries: the pooled levels, plus the raw tokens under the DIRECT reading; the
    # top-K reads the scores of the selected levels (REFINE: 1..L-1, DIRECT: 0..L-2)
    n_top = info.level_size[w.levels - 1]
    scored = P if w.mode == "direct" else P - N
    selected = P - n_top if w.mode == "direct" else P - N
    by = {
        "pool_score": 3 * B * N * H * D * e + 3 * B * P1 * H * D * 2 + BH * scored * 4,
        "topk": BH * selected * 4 + BH * K * 4,
        "build_map": BH * K * 4 + BH * P * 4 + BH * S * 4,
        "scatter": BH * S * D * 4 + BH * P * 4 + B * N * H * D * e,
        "scatter_bwd": B * N * H * D * e + BH * S * 4 + BH * S * D * 4 + BH * S * D * 2
                       + BH * S * 4,
        "gather_pool_bwd": 3 * BH * S * D * 4 + BH * P * 4 + 3 * B * N * H * D * e,
    }
    fl = {
        "attn_fwd": 2 * 2 * D * pairs,        # Q K^T and P V
        "attn_bwd_dkdv": 4 * 2 * D * pairs,   # Q K^T, dO V^T, P^T dO, dS^T Q
        "attn_bwd_dq": 1 * 2 * D * pairs,     # dS K (its two recomputed products are overhead)
    }
    return by, fl


KERNEL_OF_STAGE = {"attn_fwd": "attn_fwd_mapped_d{d}", "attn_bwd_dkdv": "attn_bwd_kv_mapped_d{d}",
                   "attn_bwd_dq": "attn_bwd_q_mapped_d{d}"}


def measured_traffic(workload, stage, head_dim):
    """HBM bytes per launch of a stage's kernel from the committed rocprofv3 counter runs,
    or None when there are none or the kernel sources changed since they were taken."""
    import glob
    import hashlib

    path = os.path.join(ROOT, "profiles", f"{workload}_counters.json")
    if not os.path.exists(path) or stage not in KERNEL_OF_STAGE:
        return None
    with open(path) as f:
        rec = json.load(f)
    h = hashlib.sha256()
    for src in sorted(glob.glob(os.path.join(ROOT, "hierarchical_sparse_attention_lh_amd", "csrc", "*"))):
        with open(src, "rb") as f:
            h.update(f.read())
    if h.hexdigest()[:16] != rec.get("csrc_sha256_16"):
        return None
    t = rec["per_launch"].get(KERNEL_OF_STAGE[stage].format(d=head_dim))
    return None if t is None else int(t["read_bytes"] + t["write_bytes"])


def time_staged(layer, steps, warmup, torch):
    names = [n for n, _ in layer.stages_fwd + layer.stages_bwd]
    stages = layer.stages_fwd + layer.stages_bwd
    for i in range(warmup):
        layer.run(stages)
        torch.cuda.synchronize()
        log(f"warmup step {i + 1}/{warmup} done")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        ev[s][0].record()
        layer.run(stages, between=lambda i, n, s=s: ev[s][i + 1].record())
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # per-stage medians over the timed steps; the step time is the mean
    per = {n: statistics.median(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps))
           for i, n in enumerate(names)}
    gpu_step = sum(ev[s][0].elapsed_time(ev[s][-1]) for s in range(steps)) / steps
    return wall / steps * 1e3, gpu_step, per


def time_monolithic(torch, ops, cfg, t, steps, with_bwd=True):
    bufs = ops.Buffers(cfg)
    y = torch.empty_like(t["q"])
    dx = [torch.empty_like(t["q"]) for _ in range(3)]

    def step():
        ops.lh_forward(cfg, t["q"], t["k"], t["v"], bufs=bufs, y=y)
        if with_bwd:
            ops.lh_backward(cfg, t["q"], t["k"], t["v"], bufs, t["dy"], *dx)

    step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        step()
    b.record()
    torch.cuda.synchronize()
    del bufs
    return a.elapsed_time(b) / steps


def time_dense(torch, ops, t, steps):
    """This library's dense causal attention straight on the [B, N, H, D] token tensors (the
    stage-2 dense-resumption call): forward, and forward + backward, with HIP events."""
    q, k, v, dy = t["q"], t["k"], t["v"], t["dy"]
    o, lse = ops.lh_attn_fwd(q, k, v, layout="bshd")
    ops.lh_attn_bwd(q, k, v, o, lse, dy, layout="bshd")
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    fwd, bwd = [], []
    for _ in range(steps):
        ev[0].record()
        o, lse = ops.lh_attn_fwd(q, k, v, layout="bshd")
        ev[1].record()
        ops.lh_attn_bwd(q, k, v, o, lse, dy, layout="bshd")
        ev[2].record()
        torch.cuda.synchronize()
        fwd.append(ev[0].elapsed_time(ev[1]))
        bwd.append(ev[1].elapsed_time(ev[2]))
    return statistics.median(fwd), statistics.median(bwd)


def cpu_baseline(w, x):
    """The oracle, as it stands, on head 0 of batch 0 of the same inputs (fwd + bwd)."""
    import numpy as np

    import oracle as O

    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = 1
    ocfg = O.Config(w.levels, w.pool, w.k, w.chunk,
                    mode=O.DIRECT if w.mode == "direct" else O.REFINE, scorer=w.scorer)
    q, k, v, dy = (x[n][0, :, 0].astype(np.float64) for n in ("q", "k", "v", "dy"))
    t0 = time.perf_counter()
    _, st = O.head_forward(q, k, v, ocfg)
    O.head_backward(dy, st, ocfg)
    t = time.perf_counter() - t0
    # heads are independent and the oracle runs them one after another
    return {"value": w.batch * w.n_tokens / (t * w.heads * w.batch), "unit": "tokens/s/layer",
            "cores": int(cores), "kind": "oracle",
            "sample": f"head 0 of {w.heads} (batch 0) of the {w.name} workload, forward + "
                      f"backward, {t:.1f} s; scaled by the head count"}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="lh-512k")
    ap.add_argument("--select", choices=("refine", "direct"), default="refine",
                    help="selection reading (the metric is quoted on refine)")
    ap.add_argument("--scorer", choices=("k", "qk", "qkv"), default="k",
                    help="score of a pooled entry (the metric is quoted on k)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense-attention baseline")
    ap.add_argument("--out", default=None, help="also write the JSON line to this file")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 1 GiB device copy (reference for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported by this "
              "build (the multi-GPU sharding is a design note, not code).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from hierarchical_sparse_attention_lh_amd import _lib, ops, synth

    if args.copy_calibration:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 1 GiB read + 1 GiB written by one copy kernel")
        del src, dst

    w = synth.WORKLOADS[args.workload]
    if args.select != w.mode:
        w = dataclasses.replace(w, name=f"{w.name}-{args.select}", mode=args.select)
    if args.scorer != w.scorer:
        w = dataclasses.replace(w, name=f"{w.name}-{args.scorer}", scorer=args.scorer)
    log(f"workload {w}")
    t0 = time.perf_counter()
    x = synth.workload_inputs(w, with_grad=True)
    log(f"inputs generated in {time.perf_counter() - t0:.1f} s")
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    t = {n: torch.from_numpy(a).to("cuda").to(dt) for n, a in x.items()}
    torch.cuda.synchronize()
    cfg = ops.config_for(w)
    info = ops.lh_plan(cfg)
    layer = ops.StagedLayer(cfg, t["q"], t["k"], t["v"], t["dy"])
    log(f"S = {info.gathered_len}, buffers ready; hip runtimes: {_lib.hip_runtimes_mapped()}")

    wall_ms, gpu_ms, per = time_staged(layer, args.steps, args.warmup, torch)
    ms = max(wall_ms, gpu_ms)
    tokens = w.batch * w.n_tokens
    log(f"staged step: {ms:.3f} ms ({per})")
    fwd_names = [n for n, _ in layer.stages_fwd]
    fwd_ms = sum(per[n] for n in fwd_names)
    mono_fb = time_monolithic(torch, ops, cfg, t, max(1, args.steps // 2))
    mono_f = time_monolithic(torch, ops, cfg, t, max(1, args.steps // 2), with_bwd=False)
    log(f"lh_forward+lh_backward: {mono_fb:.3f} ms; lh_forward: {mono_f:.3f} ms")
    del layer
    torch.cuda.empty_cache()

    by, fl = algorithmic(w, info)
    stages = {}
    for n, v in per.items():
        if n in fl:
            stages[n] = {"ms": round(v, 4), "tflops": round(fl[n] / (v * 1e-3) / 1e12, 2),
                         "mfma_frac": round(fl[n] / (v * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
        else:
            stages[n] = {"ms": round(v, 4), "gbs": round(by[n] / (v * 1e-3) / 1e9, 1),
                         "hbm_frac": round(by[n] / (v * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    hbm_names = [n for n in per if n in by]
    hbm_bytes = sum(by[n] for n in hbm_names)
    hbm_ms = sum(per[n] for n in hbm_names)
    dom = max(per, key=per.get)
    if dom in fl:
        ach = fl[dom] / (per[dom] * 1e-3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2),
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(w.name, dom, w.head_dim),
                "avg_ms": round(per[dom], 4)}
    else:
        ach = by[dom] / (per[dom] * 1e-3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
                "avg_ms": round(per[dom], 4)}

    dense = None
    if not args.no_dense:
        log("timing the dense causal attention on the token tensors (S = N)")
        d_f, d_b = time_dense(torch, ops, t, 2)
        dpairs = w.batch * w.heads * w.n_tokens * (w.n_tokens + 1) / 2
        dfl_f, dfl_b = 2 * 2 * w.head_dim * dpairs, 5 * 2 * w.head_dim * dpairs
        dense = {"fwd_ms": round(d_f, 2), "fwd_bwd_ms": round(d_f + d_b, 2),
                 "speedup_fwd": round(d_f / mono_f, 2),
                 "speedup_fwd_bwd": round((d_f + d_b) / mono_fb, 2),
                 "roofline_fwd": {"bound": "mfma", "achieved": round(dfl_f / (d_f * 1e-3) / 1e12, 1),
                                  "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                  "frac": round(dfl_f / (d_f * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)},
                 "roofline_bwd": {"bound": "mfma", "achieved": round(dfl_b / (d_b * 1e-3) / 1e12, 1),
                                  "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                  "frac": round(dfl_b / (d_b * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}}
        log(f"dense: {dense}")
        torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on one head")
        cpu = cpu_baseline(w, x)
        log(f"cpu baseline: {cpu}")

    out = {
        "metric": metric_name(w.n_tokens), "value": round(tokens / (ms * 1e-3), 1),
        "unit": "tokens/s/layer",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "n_tokens": w.n_tokens, "heads": w.heads,
                   "head_dim": w.head_dim, "levels": w.levels, "pool": w.pool, "k": w.k,
                   "chunk": w.chunk, "gathered_len": info.gathered_len,
                   "input_dtype": w.dtype, "seed": w.seed, "select": w.mode,
                   "scorer": w.scorer},
        "roofline": roof,
        "cpu_baseline": cpu,
        "forward_tokens_per_s": round(tokens / (fwd_ms * 1e-3), 1),
        "forward_ms": round(fwd_ms, 4),
        "monolithic_ms": {"fwd_bwd": round(mono_fb, 4), "fwd": round(mono_f, 4)},
        "hbm_stages": {"bytes": int(hbm_bytes), "ms": round(hbm_ms, 4),
                       "gbs": round(hbm_bytes / (hbm_ms * 1e-3) / 1e9, 1),
                       "frac": round(hbm_bytes / (hbm_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                       "bytes_per_token": round(hbm_bytes / tokens, 1)},
        "stages": stages,
        "dense_baseline": dense,
    }
    line = json.dumps(out)
    print(line, flush=True)
    if args.out:
        with open(args.out, "w") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
