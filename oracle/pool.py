"""Run the CPU oracle over many sequences at once, in worker processes.

TEST INFRASTRUCTURE ONLY, under the same rule as spec_oracle: only the test
suite and the benchmark's CPU-baseline leg use it; the product path never
does. It adds no arithmetic of its own. The caller's host arrays are placed in
shared memory once; each worker process calls spec_oracle.verify_batch on a
chunk of sequences (the `rows` it is given) and returns that BatchResult; the
chunks are merged in order. EMA state travels with each chunk as the slots of
its rows (slots are batch rows and chunks are disjoint), so the merged state is
what one sequential verify_batch call would have left.

Workers are spawned (never forked: the parent may hold a GPU context) and
import numpy and the oracle only.
"""

from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os
from multiprocessing import shared_memory

import numpy as np

from oracle import spec_oracle as O

_W: dict = {}


def usable_cores(cap: int = 16) -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(cap, n))


def _attach(specs):
    for name, (shm_name, shape, dtype) in specs.items():
        if shm_name is None:
            _W[name] = None
            continue
        shm = shared_memory.SharedMemory(name=shm_name)
        _W["_shm_" + name] = shm
        _W[name] = np.ndarray(shape, dtype=np.dtype(dtype), buffer=shm.buf)


def _task(job):
    rows, args, per_row, ema = job
    T, mode, tau, eos = args
    kw = {k: (None if v is None else v) for k, v in per_row.items()}
    sub = None
    if ema is not None:
        decay, vals, steps = ema
        sub = O.EmaState(_W["target"].shape[0], decay)
        sub.ema[rows] = vals
        sub.steps[rows] = steps
    r = O.verify_batch(_W["target"], _W["draft"], _W["tokens"], _W["uniforms"], T, mode, tau,
                       ema=sub, rows=rows, eos=eos, **kw)
    return r, (None if sub is None else (sub.ema[rows], sub.steps[rows]))


def merge(parts):
    """Concatenate BatchResults of consecutive row chunks."""
    out = parts[0]
    for p in parts[1:]:
        for k in ("tokens", "accept_len", "p_d", "q_d", "z", "argmax", "min_dist"):
            setattr(out, k, np.concatenate([getattr(out, k), getattr(p, k)]))
        out.hist = out.hist + p.hist
        out.zero_q_accepts += p.zero_q_accepts
        out.z0_fallbacks += p.z0_fallbacks
        out.invalid += p.invalid
        out.n_decisions += p.n_decisions
    return out


class OraclePool:
    """A pool of oracle workers over fixed-shape host arrays.

    arrays: target [B, K+1, V], draft [B, K, V] or None, tokens [B, K],
    uniforms [B, K+1] or None (any dtype the oracle widens exactly to float64;
    fp32 holds bf16 exactly). `load` copies new contents of the same shapes in
    place, so one pool serves many steps.
    """

    def __init__(self, shapes: dict, nproc: int | None = None):
        self.nproc = nproc or usable_cores()
        self._shms, specs, self.arrays = [], {}, {}
        for name, spec in shapes.items():
            if spec is None:
                specs[name] = (None, None, None)
                self.arrays[name] = None
                continue
            shape, dtype = spec
            dtype = np.dtype(dtype)
            size = int(np.prod(shape)) * dtype.itemsize
            shm = shared_memory.SharedMemory(create=True, size=max(1, size))
            self._shms.append(shm)
            self.arrays[name] = np.ndarray(shape, dtype=dtype, buffer=shm.buf)
            specs[name] = (shm.name, tuple(shape), dtype.str)
        self._ex = cf.ProcessPoolExecutor(self.nproc, mp_context=mp.get_context("spawn"),
                                          initializer=_attach, initargs=(specs,))

    def load(self, **arrays):
        for name, a in arrays.items():
            if a is not None:
                self.arrays[name][...] = a

    def verify(self, rows, T: float, mode: int, tau: float = 0.0, ema: O.EmaState | None = None,
               eos: int = -1, draft_len=None, max_emit=None, top_k=None, top_p=None,
               chunk: int | None = None) -> O.BatchResult:
        """verify_batch over the listed rows of the loaded arrays, split into
        chunks across the workers; per-row arrays are indexed by batch row."""
        rows = np.asarray(rows, dtype=np.int64)
        if chunk is None:
            chunk = max(1, -(-len(rows) // (4 * self.nproc)))
        per_row = dict(draft_len=draft_len, max_emit=max_emit, top_k=top_k, top_p=top_p)
        jobs = []
        for c0 in range(0, len(rows), chunk):
            r = rows[c0:c0 + chunk]
            e = None if ema is None else (ema.decay, ema.ema[r].copy(), ema.steps[r].copy())
            jobs.append((r, (T, mode, tau, eos), per_row, e))
        parts = []
        for (r, _, _, _), (res, e) in zip(jobs, self._ex.map(_task, jobs)):
            parts.append(res)
            if e is not None:
                ema.ema[r], ema.steps[r] = e
        return merge(parts)

    def close(self):
        self._ex.shutdown(wait=True)
        for shm in self._shms:
            shm.close()
            shm.unlink()
        self._shms = []

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
