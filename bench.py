#!/usr/bin/env python3
"""Throughput of batched speculative-decoding verification on one MI355X.

Default workload: B=256 sequences, K=7 drafted positions, V=128256 tokens,
bf16 target and draft logits, stochastic verification at T=1.0 (the shifted-
draft configuration). A step is one spec_verify call over one batch: the
streaming softmax-statistics pass over all 2K+1 logit rows per sequence, the
acceptance scan with emit/histogram/EMA, and the residual or bonus draw.
Inputs are synthetic, seeded and resident in HBM before the timed region;
input sets are rotated, as many as make them span at least twice the 256 MB
last-level cache (two for the large configurations). With --graph the timed
calls are replayed from a HIP graph (the launch-bound small configurations).

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
MALL_BYTES = 256 << 20       # MI355X last-level (Infinity) cache
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "speculative_decoding_verification_temp_amd", "csrc")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# the sources that define each streaming kernel whose traffic is recorded
STREAM_SOURCES = {
    "rowstats_sum": ("sv_device.hpp", "sv_topm.hpp", "sv_rowstats.hpp"),
    "rowstats_max": ("sv_device.hpp", "sv_topm.hpp", "sv_rowstats.hpp"),
    "rowstats_trunc_win": ("sv_device.hpp", "sv_topm.hpp", "sv_rowstats.hpp", "sv_kernels.hpp",
                           "sv_fused.hpp", "sv_trunc.hpp"),
    "rowstats_trunc32": ("sv_device.hpp", "sv_topm.hpp", "sv_rowstats.hpp", "sv_kernels.hpp",
                         "sv_fused.hpp", "sv_trunc.hpp", "sv_trunc32.hpp"),
}


def traffic_file(kernel: str, workload: str) -> str:
    return os.path.join(PROFILES, f"traffic_{kernel}_{workload.replace('/', '_')}.json")


def source_digest(kernel: str = "rowstats_sum") -> str:
    h = hashlib.sha256()
    for name in STREAM_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(workload: str, kernel: str):
    """HBM bytes per dispatch from committed rocprofv3 counter runs, or None
    when they were taken on other kernel source or another workload."""
    try:
        with open(traffic_file(kernel, workload)) as f:
            t = json.load(f)
    except OSError:
        return None
    if t.get("source_digest") != source_digest(kernel) or t.get("workload") != workload \
            or t.get("kernel") != kernel:
        return None
    fetch = t["fetch_kib_per_dispatch"] * 1024.0 * t["copy_factor_fetch"]
    write = t["write_kib_per_dispatch"] * 1024.0 * t["copy_factor_write"]
    return fetch + write


# ---- CPU baseline: the oracle on host cores --------------------------------
# Worker processes are spawned (fresh interpreters that import numpy and the
# oracle only, never the GPU runtime) and read the sampled inputs from shared
# memory, so a task is just a sequence index.
_W = {}


def walk_rows_read(accept_len, kb, mode: str) -> int:
    """Logit rows one walk-order call reads: position 0's rows (target row 0,
    and draft row 0 when k_b > 0 for stochastic calls) of every sequence, then
    every other needed row (target rows 1..k_b, and draft rows 1..k_b-1 for
    stochastic calls) of the sequences whose walk keeps position 0, i.e. those
    with j >= 1 (no invalid sequences in these workloads)."""
    import numpy as np
    n = 0
    for j, k in zip(np.asarray(accept_len, dtype=np.int64), np.asarray(kb, dtype=np.int64)):
        if j < 0:
            continue
        if mode == "stochastic":
            n += 1 + int(k > 0) + ((k + max(k - 1, 0)) if j >= 1 else 0)
        else:
            n += 1 + (k if j >= 1 else 0)
    return int(n)


def _worker_init(specs, T, mode, tau, trunc=(0, 1.0), walk=False):
    from multiprocessing import shared_memory
    import numpy as np
    from oracle import spec_oracle as O
    _W["shm"] = []
    for name, (shm_name, shape, dtype) in specs.items():
        if shm_name is None:
            _W[name] = None
            continue
        shm = shared_memory.SharedMemory(name=shm_name)
        _W["shm"].append(shm)
        _W[name] = np.ndarray(shape, dtype=dtype, buffer=shm.buf)
    _W["args"] = (T, mode, tau)
    _W["trunc"] = trunc
    _W["walk"] = walk
    _W["O"] = O


def _worker_task(k):
    O = _W["O"]
    T, mode, tau = _W["args"]
    n = _W["tgt"].shape[0]
    q = k % n
    kb = _W["kb"]
    tk, tp = _W["trunc"]
    r = O.verify_batch(_W["tgt"][q:q + 1], None if _W["drf"] is None else _W["drf"][q:q + 1],
                       _W["tok"][q:q + 1], _W["uni"][q:q + 1], T, mode, tau,
                       draft_len=None if kb is None else kb[q:q + 1],
                       top_k=[tk], top_p=[tp], walk_order=_W["walk"])
    return q, int(r.accept_len[0]), r.tokens[0].tolist(), float(r.min_dist[0])


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(sets, gpu_outs, cfg, mode, seconds: float, kb=None, trunc=(0, 1.0),
                 walk=False):
    """Time the fp64 CPU oracle on a bounded sample of the same workload, one
    sequence per task: first in this process on one core, then on a pool of
    worker processes (one per core of this process's CPU set, at most 16: the
    host share of one GPU), about seconds/2 each,
    cycling over up to 64 sequences of the timed input sets. Every verified
    sequence is compared with the GPU's output for it (gpu_outs[i] holds the
    GPU's tokens and accept lengths for set i)."""
    import concurrent.futures as cf
    import multiprocessing as mp
    from multiprocessing import shared_memory
    import numpy as np
    import torch
    from oracle import spec_oracle as O

    m = {"stochastic": O.MODE_STOCHASTIC, "greedy": O.MODE_GREEDY, "margin": O.MODE_MARGIN}[mode]
    n = min(64, len(sets) * cfg.B)
    where = [(k % len(sets), (k // len(sets)) % cfg.B) for k in range(n)]
    arrays = {
        "tgt": np.stack([sets[i]["target"][b].to(torch.float32).cpu().numpy() for i, b in where]),
        "drf": (np.stack([sets[i]["draft"][b].to(torch.float32).cpu().numpy() for i, b in where])
                if mode == "stochastic" else None),
        "tok": np.stack([sets[i]["tokens"][b].cpu().numpy() for i, b in where]),
        "uni": np.stack([sets[i]["uniforms"][b].cpu().double().numpy() for i, b in where]),
        "kb": None if kb is None else np.asarray([kb[b] for _, b in where]),
    }

    def check(q, alen, toks, dist):
        i, b = where[q]
        tok_g, len_g = gpu_outs[i]
        return int(dist >= 1e-6 and (alen != len_g[b] or not np.array_equal(toks, tok_g[b])))

    # one core, in this process
    mism, n1 = 0, 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds / 2 or n1 == 0:
        q = n1 % n
        r = O.verify_batch(arrays["tgt"][q:q + 1],
                           None if arrays["drf"] is None else arrays["drf"][q:q + 1],
                           arrays["tok"][q:q + 1], arrays["uni"][q:q + 1], cfg.T, m, cfg.tau,
                           draft_len=None if kb is None else arrays["kb"][q:q + 1],
                           top_k=[trunc[0]], top_p=[trunc[1]], walk_order=walk)
        mism += check(q, int(r.accept_len[0]), r.tokens[0], float(r.min_dist[0]))
        n1 += 1
    t1 = time.perf_counter() - t0

    # all usable cores (at most 16), worker processes over shared memory
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    nproc = max(1, min(16, avail))
    shms, specs = [], {}
    try:
        for name, a in arrays.items():
            if a is None:
                specs[name] = (None, None, None)
                continue
            shm = shared_memory.SharedMemory(create=True, size=max(1, a.nbytes))
            shms.append(shm)
            np.ndarray(a.shape, dtype=a.dtype, buffer=shm.buf)[...] = a
            specs[name] = (shm.name, a.shape, a.dtype.str)
        ctx = mp.get_context("spawn")
        with cf.ProcessPoolExecutor(nproc, mp_context=ctx, initializer=_worker_init,
                                    initargs=(specs, cfg.T, m, cfg.tau, trunc, walk)) as ex:
            list(ex.map(_worker_task, range(nproc)))          # start-up, not timed
            nn, k = 0, 0
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < seconds / 2 or nn == 0:
                for q, alen, toks, dist in ex.map(_worker_task, range(k, k + 2 * nproc)):
                    mism += check(q, alen, np.asarray(toks), dist)
                k += 2 * nproc
                nn += 2 * nproc
            tn = time.perf_counter() - t0
    finally:
        for shm in shms:
            shm.close()
            shm.unlink()
    return dict(value=nn / tn, unit="seqs/s", cores=nproc, kind="oracle",
                cores_available=avail, cpu_model=cpu_model(),
                single_core_value=n1 / t1,
                sample=f"{n1} sequence verifications on one core ({t1:.1f} s), then {nn} on "
                       f"{nproc} worker processes ({tn:.1f} s), cycling over {n} sequences of "
                       f"the timed input sets; fp64 numpy"
                       + ("; rows read in walk order" if walk else ""),
                parity_mismatches=mism)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c3")
    ap.add_argument("--mode", default="stochastic", choices=["stochastic", "greedy", "margin"])
    ap.add_argument("--sets", type=int, default=0,
                    help="input sets rotated across steps (0: enough to span twice the 256 MB "
                         "last-level cache, between 2 and 64)")
    ap.add_argument("--graph", action="store_true",
                    help="time the calls as replays of a HIP graph that holds one call per "
                         "input set (the streaming-pass time then comes from the same calls "
                         "run eagerly right after)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--stops", default="none", choices=["none", "varlen"],
                    help="varlen: per-sequence draft counts k_b drawn uniformly from 1..K "
                         "(seeded), no end-of-sequence token, no budget")
    ap.add_argument("--top-k", type=int, default=0,
                    help="stochastic mode: top-k truncation of every target and draft row "
                         "(every sequence); 0 = off")
    ap.add_argument("--top-p", type=float, default=1.0,
                    help="stochastic mode: top-p truncation after top-k; 1 = off")
    ap.add_argument("--residual", type=int, default=0,
                    help="stochastic mode: draft residual side output on the draft's top-m "
                         "support (m = this value, 0 = off)")
    ap.add_argument("--walk", action="store_true",
                    help="walk-order reading (the rows of a position are read only when the "
                         "walk reaches it; nothing past the first rejection); no effect on "
                         "stochastic calls with the residual side output")
    ap.add_argument("--no-walk-report", action="store_true",
                    help="leave out the walk-order timing reported beside a plain line "
                         "(counter and trace runs that should see the line's calls only)")
    ap.add_argument("--policy", action="store_true",
                    help="run the tree-shape policy epilogue (seeded draft confidences, d = 0.5)")
    ap.add_argument("--read-probe", action="store_true",
                    help="also time a plain 2 GiB streaming read with the streaming pass's "
                         "access pattern (achievable-bandwidth reference)")
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
    read_rows = 2 * K + 1 if mode == "stochastic" else K + 1
    set_bytes = B * read_rows * V * s
    nsets = args.sets or max(2, min(64, -(-2 * MALL_BYTES // set_bytes)))
    log(f"generating {nsets} input set(s) for {cfg.name} {mode} B={B} K={K} V={V} {cfg.dtype}")
    sets = [make_inputs(cfg, step, dev, gen_mode) for step in range(nsets)]
    torch.cuda.synchronize()

    v = sv.SpecVerifier(B, K, V, cfg.torch_dtype, ema_decay=cfg.ema_decay)
    kb = np.full(B, K, dtype=np.int64)
    if args.stops == "varlen":
        kb = np.random.default_rng([20260923, cfg.index, 7]).integers(1, K + 1, B)
        kb_dev = torch.as_tensor(kb.astype(np.int32), device=dev).contiguous()
        v.set_stops(-1, kb_dev, None)
    trunc = mode == "stochastic" and (0 < args.top_k < V or args.top_p < 1.0)
    trunc_args = (torch.full((B,), args.top_k, dtype=torch.int32, device=dev),
                  torch.full((B,), args.top_p, dtype=torch.float32, device=dev))
    if trunc:
        v.set_truncation(*trunc_args)
    # (the library reads calls with the residual side output in full
    # whatever the setting)
    walk_ok = not (mode == "stochastic" and args.residual)
    if args.residual and mode == "stochastic":
        v.set_residual(args.residual)
    walk = args.walk and walk_ok
    if walk:
        v.set_walk_order(True)
    if args.policy:
        conf = np.random.default_rng([20260923, cfg.index, 8]).uniform(0.0, 1.0, B)
        v.set_policy(torch.as_tensor(conf.astype(np.float32), device=dev), 0.5)
    out = (torch.empty((B, K + 1), dtype=torch.int32, device=dev),
           torch.empty((B,), dtype=torch.int32, device=dev),
           torch.empty((K + 1,), dtype=torch.int32, device=dev))

    def step(i):
        x = sets[i % len(sets)]
        v.verify(x["target"], x["draft"], x["tokens"], x["uniforms"], cfg.T, mode, cfg.tau,
                 out=out)

    # draw rows re-read per set (data dependent): 2 rows per rejection, 1 per bonus
    draw_bytes = []
    walk_rows = []      # walk-order reading: rows the staged streaming pass reads per set
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
        if walk:
            walk_rows.append(walk_rows_read(a.numpy(), kb, mode))
    log(f"warmup {args.warmup}")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    if args.graph:
        # one graph holding one call per input set, replayed; the library's
        # own timing events stay out of the graph
        g = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream(dev)
        cap.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(cap):
            for i in range(len(sets)):
                step(i)
        torch.cuda.current_stream(dev).wait_stream(cap)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(len(sets)):
                step(i)
        reps = max(1, -(-args.steps // len(sets)))
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        log(f"timing {reps} graph replays of {len(sets)} calls")
        t0.record()
        for _ in range(reps):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        ms_step = t0.elapsed_time(t1) / (reps * len(sets))
        v.profile(True)
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
        pass_ms, call_ms, ncalls = v.profile_read()
        v.profile(False)
        args.steps = reps * len(sets)
    else:
        v.profile(True)
        log(f"timing {args.steps} steps")
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
    if walk:
        rows_total = sum(walk_rows) / len(walk_rows)
    pass_bytes = int(rows_total * V * s)
    io_bytes = B * (K * 4 + (K + 1) * 4 + (K + 1) * 4 + 4) + 2 * B * K * s
    call_bytes = pass_bytes + sum(draw_bytes) / len(draw_bytes) + io_bytes
    trunc_kernel = "rowstats_trunc32" if cfg.dtype == "f32" else "rowstats_trunc_win"
    kernel = (trunc_kernel if trunc else "rowstats_sum") if mode == "stochastic" \
        else "rowstats_max"
    achieved = pass_bytes / (pass_avg * 1e-3) / 1e9
    workload = f"{cfg.name}/{mode}" + (f"/top-k{args.top_k}-top-p{args.top_p}" if trunc else "") \
        + (f"/residual{args.residual}" if args.residual and mode == "stochastic" else "") \
        + ("/walk" if walk else "")
    traffic = traffic_for(workload, kernel) if args.stops == "none" else None
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
                                  else "")
                               + (f", top-k {args.top_k}, top-p {args.top_p}" if trunc else "")
                               + (", tree-shape policy" if args.policy else "")
                               + (f", draft residual m={args.residual}"
                                  if args.residual and mode == "stochastic" else "")
                               + (", walk-order reading" if walk else ""),
                   "B": B, "K": K, "V": V, "mode": mode, "parallelism": "single GPU",
                   "input_sets": len(sets), "input_bytes_rotated": int(set_bytes * len(sets)),
                   "timing": "hip graph replays" if args.graph else "eager calls"},
        "achieved_hbm_gbs": round(call_bytes / (ms_step * 1e-3) / 1e9, 1),
        "frac_of_peak": round(call_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "algorithmic_bytes_per_step": int(call_bytes),
        "roofline": roofline,
    }
    if (not walk and walk_ok and not args.graph and not args.policy
            and not args.no_walk_report):
        # the same calls with walk-order reading, reported beside the line:
        # rows past each sequence's first rejection are not read
        vw = sv.SpecVerifier(B, K, V, cfg.torch_dtype, ema_decay=cfg.ema_decay)
        if args.stops == "varlen":
            vw.set_stops(-1, kb_dev, None)
        if trunc:
            vw.set_truncation(*trunc_args)
        vw.set_walk_order(True)
        outw = tuple(torch.empty_like(t) for t in out)
        same, rows_w = True, []
        for i in range(len(sets)):
            step(i)
            x = sets[i]
            vw.verify(x["target"], x["draft"], x["tokens"], x["uniforms"], cfg.T, mode,
                      cfg.tau, out=outw)
            torch.cuda.synchronize()
            same = same and torch.equal(out[0], outw[0]) and torch.equal(out[1], outw[1])
            rows_w.append(walk_rows_read(outw[1].cpu().numpy(), kb, mode))
        for i in range(args.warmup):
            x = sets[i % len(sets)]
            vw.verify(x["target"], x["draft"], x["tokens"], x["uniforms"], cfg.T, mode,
                      cfg.tau, out=outw)
        torch.cuda.synchronize()
        t0.record()
        for i in range(args.steps):
            x = sets[i % len(sets)]
            vw.verify(x["target"], x["draft"], x["tokens"], x["uniforms"], cfg.T, mode,
                      cfg.tau, out=outw)
        t1.record()
        torch.cuda.synchronize()
        ms_w = t0.elapsed_time(t1) / args.steps
        res["walk_order_reading"] = {
            "value": round(B / (ms_w * 1e-3), 1), "unit": "verified seqs/s",
            "ms_per_step": round(ms_w, 5),
            "logit_rows_read_per_call": round(sum(rows_w) / len(rows_w), 1),
            "logit_rows_per_call": int(rows_total),
            "outputs_equal_full_reading": bool(same),
            "note": "spec_verify_set_walk_order(1): a position's rows are read only once the "
                    "walk reaches it; same calls and inputs as the line"}
        vw.close()
    if args.read_probe:
        buf = torch.zeros(2 << 30, dtype=torch.uint8, device=dev)
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        for _ in range(3):
            sv.read_probe(buf, sink)
        r0 = torch.cuda.Event(enable_timing=True)
        r1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        r0.record()
        for _ in range(20):
            sv.read_probe(buf, sink)
        r1.record()
        torch.cuda.synchronize()
        ms = r0.elapsed_time(r1) / 20
        gbs = buf.numel() / (ms * 1e-3) / 1e9
        res["read_probe"] = {"bytes": buf.numel(), "ms": round(ms, 4), "gbs": round(gbs, 1),
                             "frac": round(gbs / PEAK_HBM_GBS, 4),
                             "streaming_pass_vs_probe": round(achieved / gbs, 4)}
        del buf
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
        res["cpu_baseline"] = cpu_baseline(
            sets, gpu_outs, cfg, mode, args.cpu_seconds, kb if args.stops == "varlen" else None,
            (args.top_k, float(np.float32(args.top_p))) if trunc else (0, 1.0), walk)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
