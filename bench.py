#!/usr/bin/env python3
"""Throughput of batched speculative-decoding verification on one MI355X.

Default workload: B=256 sequences, K=7 drafted positions, V=128256 tokens,
bf16 target and draft logits, stochastic verification at T=1.0 (the shifted-
draft configuration). A step is one spec_verify call over one batch: the
streaming softmax-statistics pass over all 2K+1 logit rows per sequence, the
acceptance scan with emit/histogram/EMA, and the residual or bonus draw.
Inputs are synthetic, seeded and resident in HBM before the timed region;
two input sets are rotated.

Prints one JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "verified seqs/sec + achieved HBM GB/s (% of MI355X peak), V=128256 B=256 K=7"
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_rowstats_sum_c3.json")
CSRC = os.path.join(ROOT, "speculative_decoding_verification_temp_amd", "csrc")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# the sources that define the streaming kernels whose traffic is recorded
STREAM_SOURCES = ("sv_device.hpp", "sv_rowstats.hpp")


def source_digest() -> str:
    h = hashlib.sha256()
    for name in STREAM_SOURCES:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(workload: str, kernel: str):
    """HBM bytes per dispatch from committed rocprofv3 counter runs, or None
    when they were taken on other kernel source or another workload."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except OSError:
        return None
    if t.get("source_digest") != source_digest() or t.get("workload") != workload \
            or t.get("kernel") != kernel:
        return None
    fetch = t["fetch_kib_per_dispatch"] * 1024.0 * t["copy_factor_fetch"]
    write = t["write_kib_per_dispatch"] * 1024.0 * t["copy_factor_write"]
    return fetch + write


def cpu_baseline(sets, gpu_outs, cfg, mode, seconds: float, kb=None):
    """Time the fp64 CPU oracle on a bounded sample of the same workload, one
    sequence at a time on one core, cycling over the input sets until about
    `seconds` of oracle time, and compare its outputs with the GPU's for those
    sequences (gpu_outs[i] holds the GPU's tokens and accept lengths for set i)."""
    import numpy as np
    from oracle import spec_oracle as O
    from workloads import to_host_f64

    m = {"stochastic": O.MODE_STOCHASTIC, "greedy": O.MODE_GREEDY, "margin": O.MODE_MARGIN}[mode]
    n, mism, t_cpu, k = 0, 0, 0.0, 0
    while t_cpu < seconds and k < 64 * cfg.B:
        i, b = (k // cfg.B) % len(sets), k % cfg.B
        x = sets[i]
        tok_g, len_g = gpu_outs[i]
        tgt = to_host_f64(x["target"][b:b + 1])
        drf = to_host_f64(x["draft"][b:b + 1]) if mode == "stochastic" else None
        tok = x["tokens"][b:b + 1].cpu().numpy()
        uni = x["uniforms"][b:b + 1].cpu().double().numpy()
        t0 = time.perf_counter()
        r = O.verify_batch(tgt, drf, tok, uni, cfg.T, m, cfg.tau,
                           draft_len=None if kb is None else kb[b:b + 1])
        t_cpu += time.perf_counter() - t0
        if r.min_dist[0] >= 1e-6 and (r.accept_len[0] != len_g[b]
                                      or not np.array_equal(r.tokens[0], tok_g[b])):
            mism += 1
        n += 1
        k += 1
    return dict(value=n / t_cpu, unit="seqs/s", cores=1, kind="oracle",
                sample=f"{n} sequence verifications cycling over the {len(sets)} input set(s) of "
                       f"the timed batch, fp64 numpy, one thread ({t_cpu:.1f} s of oracle time)",
                parity_mismatches=mism)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c3")
    ap.add_argument("--mode", default="stochastic", choices=["stochastic", "greedy", "margin"])
    ap.add_argument("--sets", type=int, default=2, help="input sets rotated across steps")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--stops", default="none", choices=["none", "varlen"],
                    help="varlen: per-sequence draft counts k_b drawn uniformly from 1..K "
                         "(seeded), no end-of-sequence token, no budget")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a 1 GiB device copy (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); sequences "
              "shard over GPUs with no exchange, so run one process per GPU.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import speculative_decoding_verification_temp_amd as sv
    from workloads import CONFIGS, make_inputs

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    cfg = CONFIGS[args.config]
    mode = args.mode
    if mode not in cfg.modes:
        sys.exit(f"config {cfg.name} runs modes {cfg.modes}")
    B, K, V = cfg.B, cfg.K, cfg.V
    s = cfg.elem_bytes
    gen_mode = "stochastic" if mode == "stochastic" else "greedy" if cfg.name != "c4" else mode
    log(f"generating {args.sets} input set(s) for {cfg.name} {mode} B={B} K={K} V={V} {cfg.dtype}")
    sets = [make_inputs(cfg, step, dev, gen_mode) for step in range(args.sets)]
    torch.cuda.synchronize()

    v = sv.SpecVerifier(B, K, V, cfg.torch_dtype, ema_decay=cfg.ema_decay)
    kb = np.full(B, K, dtype=np.int64)
    if args.stops == "varlen":
        kb = np.random.default_rng([20260923, cfg.index, 7]).integers(1, K + 1, B)
        kb_dev = torch.as_tensor(kb.astype(np.int32), device=dev).contiguous()
        v.set_stops(-1, kb_dev, None)
    out = (torch.empty((B, K + 1), dtype=torch.int32, device=dev),
           torch.empty((B,), dtype=torch.int32, device=dev),
           torch.empty((K + 1,), dtype=torch.int32, device=dev))

    def step(i):
        x = sets[i % len(sets)]
        v.verify(x["target"], x["draft"], x["tokens"], x["uniforms"], cfg.T, mode, cfg.tau,
                 out=out)

    # draw rows re-read per set (data dependent): 2 rows per rejection, 1 per bonus
    draw_bytes = []
    for i in range(len(sets)):
        step(i)
        torch.cuda.synchronize()
        a = out[1].cpu()
        valid = a >= 0
        kbt = torch.as_tensor(kb)
        if mode == "stochastic":
            rows = int(((a < kbt) & valid).sum()) * 2 + int((a == kbt).sum())
        else:
            rows = 0
        draw_bytes.append(rows * V * s)
    log(f"warmup {args.warmup}")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    v.profile(True)
    log(f"timing {args.steps} steps")
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(args.steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    ms_total = t0.elapsed_time(t1)
    pass_ms, call_ms, ncalls = v.profile_read()
    v.profile(False)
    ms_step = ms_total / args.steps
    pass_avg = pass_ms / max(1, ncalls)

    rows_total = int((2 * kb + 1).sum()) if mode == "stochastic" else int((kb + 1).sum())
    pass_bytes = rows_total * V * s
    io_bytes = B * (K * 4 + (K + 1) * 4 + (K + 1) * 4 + 4) + 2 * B * K * s
    call_bytes = pass_bytes + sum(draw_bytes) / len(draw_bytes) + io_bytes
    kernel = "rowstats_sum" if mode == "stochastic" else "rowstats_max"
    achieved = pass_bytes / (pass_avg * 1e-3) / 1e9
    traffic = traffic_for(f"{cfg.name}/{mode}", kernel) if args.stops == "none" else None
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                "traffic": traffic, "kernel": kernel,
                "kernel_ms": round(pass_avg, 5),
                "algorithmic_bytes_per_launch": pass_bytes}
    res = {
        "metric": METRIC,
        "value": round(B / (ms_step * 1e-3), 1),
        "unit": "verified seqs/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": f"{cfg.name} {mode}: B={B} K={K} V={V} {cfg.dtype} logits, "
                               f"T={cfg.T}" + (f", tau={cfg.tau}" if mode == "margin" else "")
                               + (", per-sequence draft counts 1..K" if args.stops == "varlen"
                                  else ""),
                   "B": B, "K": K, "V": V, "mode": mode, "parallelism": "single GPU"},
        "achieved_hbm_gbs": round(call_bytes / (ms_step * 1e-3) / 1e9, 1),
        "frac_of_peak": round(call_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "algorithmic_bytes_per_step": int(call_bytes),
        "roofline": roofline,
    }
    if args.copy_probe:
        # a plain 1 GiB device copy: counter calibration and a bandwidth reference
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(3):
            dst.copy_(src)
        c1.record()
        torch.cuda.synchronize()
        ms = c0.elapsed_time(c1) / 3
        res["copy_probe"] = {"bytes_read": 1 << 30, "bytes_written": 1 << 30,
                             "ms": round(ms, 4), "gbs": round(2 * (1 << 30) / (ms * 1e-3) / 1e9, 1)}
    if not args.no_cpu:
        log("cpu baseline (oracle)")
        gpu_outs = []
        for i in range(len(sets)):
            step(i)
            torch.cuda.synchronize()
            gpu_outs.append((out[0].cpu().numpy(), out[1].cpu().numpy()))
        res["cpu_baseline"] = cpu_baseline(sets, gpu_outs, cfg, mode, args.cpu_seconds,
                                           kb if args.stops == "varlen" else None)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
