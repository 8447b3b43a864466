"""The fp64 oracle over every channel of a full-size workload, in parallel
processes -- TEST INFRASTRUCTURE (it runs the oracle).

A full-size configuration has thousands of channels; the oracle takes about a
second per 64 channels of 32k tokens.  Work is cut into channel ranges.  Each
task regenerates its range from the seeded generator
(workloads.make(..., channels=...)), so no input crosses a process boundary,
computes each oracle it needs once, and compares every result handed to it
with oracle.channel_stats; the parent combines the per-channel statistics with
oracle.from_stats, which gives exactly what oracle.compare gives on the whole
array.  Workers are spawned fresh (no GPU state is inherited) and import only
numpy, scipy, the oracle and the generator.  A spawned worker imports the
parent's main script first (unless it is a package's __main__, as under
`python -m pytest`), so a script that uses the pool keeps its own work under
`if __name__ == "__main__":`.

Jobs (one per result to check), each with the result restricted to the task's
channels (host arrays: bf16 bit patterns as uint16, or float32):
    ("modal", label, y)                 y against oracle.hyena_fwd
    ("modal_state", label, s)           s against oracle.modal_state
    ("chunk", label, C, y, s)           y and s against oracle.chunk_fwd(C)
    ("fir", label, K, y)                y against oracle.fir_fwd with taps K
"""
from __future__ import annotations

import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

MAX_WORKERS = 16            # host cores that go with one GPU on the test boxes
_POOL = None


def _init_worker():
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)          # one BLAS thread per worker process


def pool() -> ProcessPoolExecutor:
    global _POOL
    if _POOL is None:
        n = max(1, min(MAX_WORKERS, os.cpu_count() or 1))
        _POOL = ProcessPoolExecutor(n, mp_context=mp.get_context("spawn"),
                                    initializer=_init_worker)
    return _POOL


def shutdown():
    global _POOL
    if _POOL is not None:
        _POOL.shutdown(wait=True)
        _POOL = None


def _state_rel_sq(s, ref):
    """Per (b, c) row: (||s - ref|| / ||ref||)^2 over the modes."""
    s = np.asarray(s, dtype=np.float64).reshape(-1, ref.shape[-1])
    r = np.asarray(ref, dtype=np.float64).reshape(-1, ref.shape[-1])
    num = np.sum((s - r) ** 2, axis=-1)
    den = np.sum(r ** 2, axis=-1)
    out = np.where(den > 0, num / np.where(den > 0, den, 1.0), num)
    return np.where(np.isfinite(s).all(axis=-1), out, np.inf)


def run_block(name, overrides, c0, c1, jobs):
    """Worker: the oracle on channels [c0, c1) of workload `name` and the
    statistics of every job's result.  Returns {label: {"y": stats,
    "state": per-row squared relative errors}}."""
    import oracle
    import workloads as W

    w = W.make(name, channels=(c0, c1), **(overrides or {}))
    x1, x2, v = w.f64("x1"), w.f64("x2"), w.f64("v")
    lam = w.log_poles.astype(np.float64)
    R = w.residues.astype(np.float64)
    sk = w.skip.astype(np.float64)
    cache = {}

    def ref(key):
        if key not in cache:
            kind = key[0]
            if kind == "modal":
                cache[key] = oracle.hyena_fwd(x1, x2, v, lam, R, sk)
            elif kind == "modal_state":
                cache[key] = oracle.modal_state(x1 * v, lam)
            elif kind == "chunk":
                cache[key] = oracle.chunk_fwd(x1, x2, v, lam, R, sk, key[1])
            elif kind == "fir":
                cache[key] = oracle.fir_fwd(x1, x2, v, w.taps[key[1]].astype(np.float64), sk)
        return cache[key]

    def dec(y):
        y = np.asarray(y)
        return W.to_f64(y, "bf16") if y.dtype == np.uint16 else y.astype(np.float64)

    out = {}
    for job in jobs:
        kind, label = job[0], job[1]
        if kind == "modal":
            out[label] = {"y": oracle.channel_stats(dec(job[2]), ref(("modal",)))}
        elif kind == "modal_state":
            out[label] = {"state": _state_rel_sq(job[2], ref(("modal_state",)))}
        elif kind == "chunk":
            ry, rs = ref(("chunk", int(job[2])))
            out[label] = {"y": oracle.channel_stats(dec(job[3]), ry),
                          "state": _state_rel_sq(job[4], rs)}
        elif kind == "fir":
            out[label] = {"y": oracle.channel_stats(dec(job[3]), ref(("fir", int(job[2]))))}
        else:
            raise ValueError(kind)
    return out


def _slice(job, c0, c1):
    """The job with its result arrays cut to channels [c0, c1) (axis 1)."""
    kind = job[0]
    if kind in ("modal", "modal_state"):
        return (kind, job[1], np.ascontiguousarray(job[2][:, c0:c1]))
    if kind == "chunk":
        return (kind, job[1], job[2], np.ascontiguousarray(job[3][:, c0:c1]),
                np.ascontiguousarray(job[4][:, c0:c1]))
    if kind == "fir":
        return (kind, job[1], job[2], np.ascontiguousarray(job[3][:, c0:c1]))
    raise ValueError(kind)


def check(name, jobs, channels, overrides=None, block=64):
    """Statistics of every job over the given channels of workload `name`.

    channels: an iterable of channel indices (any order; consecutive ones are
    grouped into ranges of at most `block`, aligned to multiples of `block`).
    Returns {label: {"y": metrics dict (oracle.compare's keys), "state":
    channel-equalised relative L2 of the state}}."""
    import oracle

    ch = np.unique(np.asarray(list(channels), dtype=np.int64))
    ranges = []
    for c in ch:
        c = int(c)
        if ranges and ranges[-1][1] == c and c % block != 0:
            ranges[-1][1] = c + 1
        else:
            ranges.append([c, c + 1])
    futs = [pool().submit(run_block, name, overrides, a, b, [_slice(j, a, b) for j in jobs])
            for a, b in ranges]
    parts = [f.result() for f in futs]
    out = {}
    for job in jobs:
        label = job[1]
        res = {}
        ys = [p[label]["y"] for p in parts if "y" in p[label]]
        if ys:
            res["y"] = oracle.from_stats(ys)
        ss = [p[label]["state"] for p in parts if "state" in p[label]]
        if ss:
            res["state"] = float(np.sqrt(np.mean(np.concatenate(ss))))
        out[label] = res
    return out
