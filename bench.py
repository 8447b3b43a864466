"""Benchmark of the Hyena operator on one MI355X.

One step = one pass of the operator over the 32 kb chunked-prefill workload
(B=1, D=4096, L=32768, bf16 I/O, N=16 modes, chunk 1024 with carried state):
modal filter generation, input gate, causal long convolution, output gate and
skip, and the carried modal state -- all in one launch of hyena_chunk_fwd
(whose automatic choice at 16 modes is the matrix-core algorithm).  Inputs
are resident in HBM before timing starts; consecutive steps take four
different input sets in turn (and write four outputs), so no step reads data
an earlier step left in the last-level cache.  The same step repeated on one
input set is reported beside it as `same_input_set` with --same-input.
`step_ms` gives the median, min and max of single steps, each timed on its
own in a separate pass after the headline's timed region.  Before the W
warm-up steps the step runs untimed for 0.3 s, which brings an idle GPU back
to the clocks of back-to-back work (see settle()); the timed region is then
exactly K steps.

Prints ONE JSON line.  Besides the headline it reports
  roofline      the dominant kernel's algorithmic bytes over its HIP-event
                time, and its HBM bytes and fp32-vector / bf16-matrix flops
                per launch from rocprofv3 counters kept in
                profiles/traffic.json while the kernel sources are unchanged;
  components    the other entry points at the headline shape;
  configs       every workload configuration (tiny fp32, the 7B layer set,
                32k, 40B-shaped, 262K) through each of its entry points:
                median / min / max time per call, Gtoken-channels/s, the
                fraction of 8 TB/s (algorithmic bytes) and of 157.3 TFLOP/s
                (nominal flops of the FFT algorithm), and the fp64 oracle's
                rate on a bounded sample of the same configuration;
  cpu_baseline  the fp64 oracle of the headline workload on the host's
                cores (one worker process per core, up to 16), and on one.

    python bench.py [--gpus 1] [--steps 100] [--warmup 100] [--no-cpu-baseline]
                    [--no-components] [--no-configs] [--same-input]
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
sys.path.insert(0, ROOT)

METRIC = "Hyena op Gtoken·channels/s at D=4096 L=32768 bf16; % HBM roofline"
HBM_PEAK_GBS = 8000.0
FP32_PEAK_TFLOPS = 157.3                     # MI355X fp32 vector (packed FP32)
BF16_MFMA_PEAK_TFLOPS = 2500.0               # MI355X dense bf16 matrix cores
WORKLOAD = "32k_chunked"
CHUNK = 1024
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# device code of the timed kernel; the HBM counters in TRAFFIC_FILE are used
# only while these files are unchanged
KERNEL_SOURCES = ["genomic_lm_amd/csrc/chunk_mfma.hip", "genomic_lm_amd/csrc/mfma_common.hpp",
                  "genomic_lm_amd/csrc/common.hpp", "genomic_lm_amd/csrc/pow_pair.hpp"]
INPUT_SETS = 4                               # activation sets the timed steps rotate over
CONFIG_SETS = 3                              # input sets of each configuration entry
CPU_WORKERS_MAX = 16                         # host cores that go with one GPU
CPU_BUDGET_S = 30.0                          # wall time the all-core oracle pass may take
CPU_SINGLE_S = 6.0                           # wall time of the one-core sample


def kernel_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--algo", default="auto", choices=["mfma", "fft", "auto"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-components", action="store_true")
    ap.add_argument("--no-configs", action="store_true")
    ap.add_argument("--same-input", action="store_true",
                    help="also time the step repeated on one input set (last-level cache hits)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (counter calibration)")
    return ap.parse_args()


# ------------------------------------------------------------------ timing
def copy_calibration(steps):
    """A plain copy of known size, for scaling HBM byte counters."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": steps}), flush=True)


def settle(fn, seconds):
    """fn called back to back for `seconds`, untimed.  An idle MI355X lowers
    its clocks (while the host draws the inputs, say) and a few milliseconds
    of work do not bring them back: 20 headline steps after 5 warm-up steps
    measured 0.23-0.26 ms after an idle pause, 0.209-0.215 ms after 0.3 s of
    1 GiB copies, and 0.202-0.204 ms after 0.3 s of the step itself -- the
    rate of 500 steps after 100 (0.203 ms)."""
    import torch
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def copy_bandwidth(stream):
    """Bytes moved per second (1 GiB read + 1 GiB written) by a plain
    device-to-device copy on this GPU: the streaming rate the box delivers,
    beside the published peak."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    src.fill_(1)
    t = timed(lambda: dst.copy_(src), 10, 3, stream)
    del src, dst
    return 2 * n / t / 1e9


def per_step_ms(fn, steps, stream):
    """Each of `steps` calls timed on its own (an event after every call on
    `stream`): the spread of single steps, beside the headline's average."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))


def timed(fn, steps, warmup, stream):
    """Average per-call time (s) over `steps` calls, HIP events on `stream`."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3 / steps


def measure(fn, stream, blocks=5, block_s=0.03):
    """fn run untimed for 0.2 s (settle), then `blocks` runs of n back-to-back
    calls between HIP events, n chosen so a run lasts about block_s (at
    least 3 calls): the median, min and max of the per-call averages (s) and
    the calls timed."""
    settle(fn, 0.2)
    t1 = timed(fn, 1, 0, stream)
    n = max(3, min(400, int(math.ceil(block_s / max(t1, 1e-6)))))
    ts = sorted(timed(fn, n, 0, stream) for _ in range(blocks))
    return ts[len(ts) // 2], ts[0], ts[-1], n * blocks


def rotating(f, k):
    n = [0]

    def g():
        f(n[0] % k)
        n[0] += 1
    return g


# ------------------------------------------------------------------ CPU oracle
def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_block(name, c0, c1, kind, arg):
    """Worker: the fp64 oracle on channels [c0, c1) of workload `name`, the
    inputs regenerated from the seeded generator.  Returns (token-channels,
    seconds spent in the oracle call)."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    import workloads as W

    w = W.make(name, channels=(c0, c1))
    x1, x2, v = w.f64("x1"), w.f64("x2"), w.f64("v")
    lam, R, sk = (a.astype(np.float64) for a in (w.log_poles, w.residues, w.skip))
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        if kind == "chunk":
            oracle.chunk_fwd(x1, x2, v, lam, R, sk, arg)
        elif kind == "fftconv":
            oracle.hyena_fwd(x1, x2, v, lam, R, sk)
        elif kind == "fir":
            oracle.fir_fwd(x1, x2, v, w.taps[arg].astype(np.float64), sk)
        else:
            raise ValueError(kind)
        dt = time.perf_counter() - t0
    return w.B * (c1 - c0) * w.L, dt


class OraclePool:
    """Worker processes for the oracle, one thread each, spawned fresh (no
    GPU state inherited): min(16, cores) of them."""

    def __init__(self):
        import multiprocessing as mp
        from concurrent.futures import ProcessPoolExecutor
        self.n = max(1, min(CPU_WORKERS_MAX, os.cpu_count() or 1))
        self.ex = ProcessPoolExecutor(self.n, mp_context=mp.get_context("spawn"))

    def run(self, name, D, kind, arg, block, budget_s):
        """Channel blocks [0, D) in order until they are done or budget_s of
        wall time has passed (blocks not started by then are cancelled).
        Returns (token-channels done, channels done, wall seconds)."""
        from concurrent.futures import wait, FIRST_COMPLETED
        t0 = time.perf_counter()
        futs = {self.ex.submit(_oracle_block, name, c, min(c + block, D), kind, arg): c
                for c in range(0, D, block)}
        tc = ch = 0
        pending = set(futs)
        while pending:
            done, pending = wait(pending, timeout=max(0.0, budget_s - (time.perf_counter() - t0)),
                                 return_when=FIRST_COMPLETED)
            for f in done:
                if not f.cancelled():
                    n_tc, _ = f.result()
                    tc += n_tc
                    c = futs[f]
                    ch += min(c + block, D) - c
            if time.perf_counter() - t0 > budget_s:
                for f in pending:
                    f.cancel()
                for f in pending:
                    if not f.cancelled():       # already running: let it finish and count it
                        n_tc, _ = f.result()
                        tc += n_tc
                        c = futs[f]
                        ch += min(c + block, D) - c
                break
        return tc, ch, time.perf_counter() - t0

    def close(self):
        self.ex.shutdown(wait=True)


def cpu_baseline(pool, w):
    """The fp64 oracle's chunked prefill (oracle.chunk_fwd, chunk 1024) of the
    headline workload: all channels over the worker processes (within
    CPU_BUDGET_S; fewer channels are labelled extrapolated), and a one-core
    sample in this process."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle

    # one core: blocks of 16 channels until CPU_SINGLE_S has passed
    done, dt, blk = 0, 0.0, 16
    with threadpool_limits(limits=1):
        while dt < CPU_SINGLE_S and done < w.D:
            rows = np.arange(done, min(done + blk, w.D))
            x1, x2, v = (w.f64(k, rows) for k in ("x1", "x2", "v"))
            lam = w.log_poles[rows].astype(np.float64)
            R = w.residues[rows].astype(np.float64)
            sk = w.skip[rows].astype(np.float64)
            t0 = time.perf_counter()
            oracle.chunk_fwd(x1, x2, v, lam, R, sk, CHUNK)
            dt += time.perf_counter() - t0
            done = int(rows[-1]) + 1
    one = w.B * done * w.L / dt / 1e9
    tc, ch, wall = pool.run(WORKLOAD, w.D, "chunk", CHUNK, 64, CPU_BUDGET_S)
    extrapolated = ch < w.D
    model = cpu_model()
    return {
        "value": round(tc / wall / 1e9, 6), "unit": "Gtoken·channels/s", "cores": pool.n,
        "kind": "oracle",
        "sample": (f"oracle.chunk_fwd (fp64, chunk {CHUNK}) on {ch} of {w.D} channels x {w.L} "
                   f"tokens (B={w.B}) in 64-channel blocks over {pool.n} worker processes of one "
                   f"thread each, inputs regenerated per block inside the timed wall "
                   f"{wall:.1f} s; {model}, {os.cpu_count()} logical cores"
                   + ("; rate over the channels done, extrapolated to the workload"
                      if extrapolated else "; the whole workload")),
        "extrapolated": extrapolated,
        "cpu_model": model,
        "wall_s": round(wall, 2),
        "single_core": {"value": round(one, 6), "cores": 1,
                        "sample": f"channels 0..{done - 1} ({done} of {w.D}), {dt:.1f} s of "
                                  f"oracle time, BLAS held to 1 thread; extrapolated"},
    }


# ------------------------------------------------------------------ configurations
def nominal_flops(kind, L, C=None, K=None):
    """Nominal fp32 flops per token-channel of the FFT algorithm (radix-2
    counts, real transforms at 2.5 N log2 N): single pass 15 log2(2L) + 42,
    chunked 10 log2(2C) + 74, FIR 2K + 4."""
    if kind == "fftconv":
        return 15 * math.log2(2 * L) + 42
    if kind == "chunk":
        return 10 * math.log2(2 * C) + 74
    return 2 * K + 4


def run_configs(stream, pool, oracle_s):
    """Every configuration through each of its entry points."""
    import numpy as np
    import torch
    import genomic_lm_amd as G
    import workloads as W

    dev = torch.device("cuda:0")
    plan = [
        ("tiny", [("fftconv", {})], ("fftconv", None)),
        ("7b_layer_set", [("fir", {"K": 7}), ("fir", {"K": 128}), ("fftconv", {})], ("fir", 128)),
        ("32k_chunked", [("chunk", {"C": 1024}), ("chunk", {"C": 1024, "algo": "fft"}),
                         ("chunk_calls", {"C": 1024}), ("fftconv", {})], ("chunk", 1024)),
        ("40b_shaped", [("chunk", {"C": 1024}), ("fftconv", {})], ("chunk", 1024)),
        ("262k", [("fftconv", {}), ("chunk", {"C": 4096}), ("chunk", {"C": 4096, "algo": "fft"})],
         ("fftconv", None)),
    ]
    out = {}
    for name, entries, oracle_kind in plan:
        w = W.make(name)
        B, D, L = w.B, w.D, w.L
        bf16 = w.io == "bf16"
        esz = 2 if bf16 else 4
        to = (lambda a: torch.from_numpy(np.ascontiguousarray(a)).view(torch.bfloat16).to(dev)) if bf16 \
            else (lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev))
        par = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
        base = (to(w.x1), to(w.x2), to(w.v))
        lam, res, skip = par(w.log_poles), par(w.residues), par(w.skip)
        taps = {K: par(t) for K, t in w.taps.items()}
        # input sets: the workload's streams and copies with the channels rotated
        sets = [base] + [tuple(torch.roll(t, shifts=k * (D // CONFIG_SETS) + 1, dims=1).contiguous()
                               for t in base) for k in range(1, CONFIG_SETS)]
        ys = [torch.empty_like(base[0]) for _ in sets]
        st = torch.empty((B, D, w.N), dtype=torch.float32, device=dev)
        ws = torch.empty(max(G.fftconv_workspace_size(B, D, L, w.N, base[0].dtype), 16),
                         dtype=torch.uint8, device=dev)
        tc = B * D * L
        res_cfg = {"workload": w.cfg.desc, "B": B, "D": D, "L": L, "io": w.io, "modes": w.N,
                   "entries": {}}
        for kind, opt in entries:
            if kind == "fftconv":
                label = f"fftconv N_fft={next_pow2(2 * L)}"
                fn = lambda k: G.fftconv_fwd(*sets[k], lam, res, skip, out=ys[k], workspace=ws)
                flops = nominal_flops("fftconv", L)
            elif kind == "fir":
                K = opt["K"]
                label = f"fir K={K}"
                fn = lambda k, K=K: G.fir_fwd(*sets[k], taps[K], skip, out=ys[k])
                flops = nominal_flops("fir", L, K=K)
            elif kind == "chunk":
                C, algo = opt["C"], opt.get("algo", "auto")
                label = f"chunk C={C}" + ("" if algo == "auto" else f" algo={algo}")
                fn = lambda k, C=C, algo=algo: G.chunk_fwd(*sets[k], lam, res, C, skip, algo=algo,
                                                           out=ys[k], state_out=st)
                flops = nominal_flops("chunk", L, C=C)
            else:                                   # chunk_calls: one call per chunk, state handed over
                C = opt["C"]
                label = f"chunk C={C} x{(L + C - 1) // C} calls"
                xs = [[tuple(t[..., t0:t0 + C].contiguous() for t in sk) for t0 in range(0, L, C)]
                      for sk in sets]
                ycs = [[torch.empty_like(c[0]) for c in xk] for xk in xs]
                sts = [torch.empty_like(st), torch.empty_like(st)]

                def fn(k, xs=xs, ycs=ycs, sts=sts, C=C):
                    s_in = None
                    for i, (a, b, c) in enumerate(xs[k]):
                        G.chunk_fwd(a, b, c, lam, res, C, skip, state_in=s_in, out=ycs[k][i],
                                    state_out=sts[i & 1])
                        s_in = sts[i & 1]
                flops = nominal_flops("chunk", L, C=C)
            med, lo, hi, n = measure(rotating(fn, len(sets)), stream)
            res_cfg["entries"][label] = {
                "ms": round(med * 1e3, 4), "ms_min": round(lo * 1e3, 4), "ms_max": round(hi * 1e3, 4),
                "calls": n, "Gtc_per_s": round(tc / med / 1e9, 2),
                "hbm_frac": round(4 * esz * tc / med / 1e9 / HBM_PEAK_GBS, 4),
                "fp32_frac_nominal": round(flops * tc / med / 1e12 / FP32_PEAK_TFLOPS, 4),
            }
        if pool is not None:
            okind, oarg = oracle_kind
            blk = max(1, min(64, int(4e6 // L)))
            tc_o, ch_o, wall = pool.run(name, D, okind, oarg, blk, oracle_s)
            res_cfg["cpu_oracle"] = {
                "value": round(tc_o / wall / 1e9, 6), "unit": "Gtoken·channels/s", "cores": pool.n,
                "function": {"chunk": f"oracle.chunk_fwd (chunk {oarg})", "fftconv": "oracle.hyena_fwd",
                             "fir": f"oracle.fir_fwd (K={oarg})"}[okind],
                "sample": f"{ch_o} of {D} channels in {wall:.1f} s"
                          + ("" if ch_o == D else ", extrapolated to the workload"),
                "extrapolated": ch_o < D,
            }
        out[name] = res_cfg
        del sets, ys, ws, base, st
        torch.cuda.empty_cache()
    return out


def next_pow2(n):
    p = 1
    while p < n:
        p <<= 1
    return p


# ------------------------------------------------------------------ main
def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (--gpus {args.gpus} requested): the operator "
              "shards over channels with no communication, so N GPUs run N independent copies "
              "of this single-GPU workload.", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.steps)
        return

    import numpy as np
    import torch
    import genomic_lm_amd as G
    import workloads as W

    G.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = W.make(WORKLOAD)
    B, D, L = w.B, w.D, w.L
    algo_used = args.algo if args.algo != "auto" else ("mfma" if w.N <= 16 else "fft")
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).view(torch.bfloat16).to(dev)
    par = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)
    x1, x2, v = to(w.x1), to(w.x2), to(w.v)
    lam, res, skip = par(w.log_poles), par(w.residues), par(w.skip)
    st = torch.empty((B, D, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    # Consecutive steps take consecutive input sets (the workload's streams,
    # then copies with the channels rotated) and write separate outputs, so
    # that no step reads what an earlier one left in the 256 MB last-level
    # cache: a model's layers never see the same activations twice.
    sets = [(x1, x2, v)]
    for k in range(1, INPUT_SETS):
        sets.append(tuple(torch.roll(t, shifts=k * (D // INPUT_SETS) + 1, dims=1).contiguous()
                          for t in (x1, x2, v)))
    ys = [torch.empty_like(x1) for _ in range(INPUT_SETS)]

    def head(k):
        G.chunk_fwd(*sets[k], lam, res, CHUNK, skip, algo=args.algo, out=ys[k], state_out=st)

    step = rotating(head, INPUT_SETS)
    # the streaming rate of a plain copy; then the GPU brought to its working
    # clocks by 0.3 s of untimed steps, the W warm-up steps and the K timed
    # steps
    copy_gbs = copy_bandwidth(stream)
    settle(step, 0.3)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t_wall0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    t_step = e0.elapsed_time(e1) / 1e3 / args.steps
    for yk in ys:
        if not torch.isfinite(yk.float()).all():
            raise RuntimeError("non-finite output")
    # for context (--same-input): the same step repeated on one input set,
    # whose reads then partly hit the last-level cache
    t_same = timed(lambda: head(0), args.steps, 2, stream) if args.same_input else None
    # single steps of the same rotation, timed after the headline's region
    spread = per_step_ms(step, args.steps, stream)

    tc = B * D * L
    alg_bytes = 8 * tc                       # x1, x2, v read + y written, bf16
    achieved = alg_bytes / t_step / 1e9
    traffic = None
    compute = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("kernel_hash") == kernel_hash() and tr.get("algo") == algo_used:
            traffic = tr.get("bytes_per_launch")
            fl = tr.get("compute")
            if fl:
                # flops per launch from the SQ counters (fp32 VALU: 64 lanes x
                # (add + mul + transcendental + 2 fma) instructions; bf16 MFMA:
                # 512 x MFMA_MOPS_BF16) over this run's launch time
                compute = {}
                for key, n, peak in (("valu_fp32", fl["valu_fp32_flops"], FP32_PEAK_TFLOPS),
                                     ("mfma_bf16", fl["mfma_bf16_flops"], BF16_MFMA_PEAK_TFLOPS)):
                    a = n / t_step / 1e12
                    compute[key] = {"achieved": round(a, 2), "peak": peak, "unit": "TFLOP/s",
                                    "frac": round(a / peak, 4), "flops": n}

    comps = {}
    if not args.no_components:
        comp_steps = max(3, args.steps // 4)
        taps7, taps128 = par(w.taps[7]), par(w.taps[128])
        fft_ws = torch.empty(max(G.fftconv_workspace_size(B, D, L, w.N, x1.dtype), 16),
                             dtype=torch.uint8, device=dev)
        runs = {
            "chunk_fft": rotating(lambda k: G.chunk_fwd(*sets[k], lam, res, CHUNK, skip, algo="fft",
                                                        out=ys[k], state_out=st), INPUT_SETS),
            "chunk_mfma": rotating(lambda k: G.chunk_fwd(*sets[k], lam, res, CHUNK, skip, algo="mfma",
                                                         out=ys[k], state_out=st), INPUT_SETS),
            "fftconv_single_pass": rotating(lambda k: G.fftconv_fwd(*sets[k], lam, res, skip,
                                                                    out=ys[k], workspace=fft_ws),
                                            INPUT_SETS),
            "fftconv_single_pass_noalloc": rotating(lambda k: G.fftconv_fwd_noalloc(
                *sets[k], lam, res, skip, out=ys[k]), INPUT_SETS),
            "fir7": rotating(lambda k: G.fir_fwd(*sets[k], taps7, skip, out=ys[k]), INPUT_SETS),
            "fir128": rotating(lambda k: G.fir_fwd(*sets[k], taps128, skip, out=ys[k]), INPUT_SETS),
        }
        # the same prefill as 32 calls of one chunk each, the state handed over
        nch = (L + CHUNK - 1) // CHUNK
        xs = [[tuple(t[..., t0:t0 + CHUNK].contiguous() for t in sk) for t0 in range(0, L, CHUNK)]
              for sk in sets]
        ycs = [[torch.empty_like(c[0]) for c in xk] for xk in xs]
        sts = [torch.empty_like(st), torch.empty_like(st)]

        def per_chunk_calls(k):
            s_in = None
            for i, (a, b, c) in enumerate(xs[k]):
                G.chunk_fwd(a, b, c, lam, res, CHUNK, skip, state_in=s_in, algo=args.algo,
                            out=ycs[k][i], state_out=sts[i & 1])
                s_in = sts[i & 1]

        runs[f"chunk_{algo_used}_x{nch}_calls"] = rotating(per_chunk_calls, INPUT_SETS)
        # the same calls captured once per input set in a HIP graph and
        # replayed, as a serving loop would issue them: the kernels back to
        # back without the binding's per-call host work (argument checks,
        # stream lookup, the foreign call)
        graphs = []
        for k in range(INPUT_SETS):
            per_chunk_calls(k)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                per_chunk_calls(k)
            graphs.append(g)
        runs[f"chunk_{algo_used}_x{nch}_calls_graph"] = rotating(lambda k: graphs[k].replay(),
                                                                 INPUT_SETS)
        # one decode step per row from the caches (B=1, D=4096: latency-bound)
        tok = [t[..., L - 1].contiguous() for t in (x1, x2, v)]
        y1 = torch.empty_like(tok[0])
        st1 = st.clone()
        runs["modal_decode_step"] = lambda: G.modal_decode(*tok, lam, res, skip, state_in=st1,
                                                           out=y1, state_out=st1)
        tok3 = [t[..., L - 1:].contiguous() for t in (x1, x2, v)]
        y3 = torch.empty_like(tok3[0])
        win = torch.zeros((B, D, 127), dtype=torch.float32, device=dev)
        runs["fir128_window_step"] = lambda: G.fir_fwd_window(*tok3, taps128, skip, window_in=win,
                                                              out=y3, window_out=win)
        # complex-pole modes (Evo 1 form, 8 per channel) at the same shape
        lc, rc = W.complex_modes(D, 8, seed=5)
        lc_d, rc_d = torch.from_numpy(lc).to(dev), torch.from_numpy(rc).to(dev)
        stc = torch.empty((B, D, 8), dtype=torch.complex64, device=dev)
        runs["fftconv_cpx_single_pass"] = rotating(lambda k: G.fftconv_fwd_cpx(
            *sets[k], lc_d, rc_d, skip, out=ys[k], workspace=fft_ws), INPUT_SETS)
        # 32 real modes (the workload's 16 and the same poles scaled by 0.7,
        # residues halved and negated): the matrix cores' one-mode-per-lane
        # form, and the per-chunk FFTs that serve larger mode counts
        lam32 = torch.cat([lam, 0.7 * lam], 1).contiguous()
        res32 = torch.cat([res, -0.5 * res], 1).contiguous()
        st32 = torch.empty((B, D, 32), dtype=torch.float32, device=dev)
        runs["chunk_mfma_32modes"] = rotating(lambda k: G.chunk_fwd(
            *sets[k], lam32, res32, CHUNK, skip, algo="mfma", out=ys[k], state_out=st32), INPUT_SETS)
        runs["chunk_fft_32modes"] = rotating(lambda k: G.chunk_fwd(
            *sets[k], lam32, res32, CHUNK, skip, algo="fft", out=ys[k], state_out=st32), INPUT_SETS)
        runs["chunk_cpx_fft"] = rotating(lambda k: G.chunk_fwd_cpx(
            *sets[k], lc_d, rc_d, CHUNK, skip, algo="fft", out=ys[k], state_out=stc), INPUT_SETS)
        runs["chunk_cpx_mfma"] = rotating(lambda k: G.chunk_fwd_cpx(
            *sets[k], lc_d, rc_d, CHUNK, skip, algo="mfma", out=ys[k], state_out=stc), INPUT_SETS)
        # the same prefill read straight from in_proj's token-major layout
        # (B, L, 3D), channels interleaved per triple, y written (B, L, D)
        xins = [torch.stack(sk, -1).permute(0, 2, 1, 3).contiguous().view(B, L, 3 * D) for sk in sets]
        y_tms = [torch.empty((B, L, D), dtype=torch.bfloat16, device=dev) for _ in sets]
        tm_ws = torch.empty(max(G.chunk_tokmajor_workspace_size(B, D, L, w.N), 16),
                            dtype=torch.uint8, device=dev)
        runs["chunk_tokmajor"] = rotating(lambda k: G.chunk_fwd_tokmajor(
            xins[k], lam, res, skip, out=y_tms[k], state_out=st, workspace=tm_ws), INPUT_SETS)
        runs["chunk_tokmajor_mfma"] = rotating(lambda k: G.chunk_fwd_tokmajor(
            xins[k], lam, res, skip, out=y_tms[k], state_out=st, algo="mfma"), INPUT_SETS)
        win6 = torch.empty((B, D, 6), dtype=torch.float32, device=dev)
        win127 = torch.empty((B, D, 127), dtype=torch.float32, device=dev)
        runs["fir7_tokmajor"] = rotating(lambda k: G.fir_fwd_tokmajor(
            xins[k], taps7, skip, out=y_tms[k], window_out=win6), INPUT_SETS)
        runs["fir128_tokmajor"] = rotating(lambda k: G.fir_fwd_tokmajor(
            xins[k], taps128, skip, out=y_tms[k], window_out=win127), INPUT_SETS)
        one_token = {"modal_decode_step", "fir128_window_step"}   # B*D token·channels
        for name, fn in runs.items():
            t = timed(fn, comp_steps, 2, stream)
            n_tc = B * D if name in one_token else tc
            comps[name] = {"ms": round(t * 1e3, 4), "Gtc_per_s": round(n_tc / t / 1e9, 2),
                           "hbm_frac": round(8 * n_tc / t / 1e9 / HBM_PEAK_GBS, 4)}
        del xs, ycs, xins, y_tms, tm_ws, fft_ws, graphs
        torch.cuda.empty_cache()

    pool = None if args.no_cpu_baseline else OraclePool()
    configs = None
    if not args.no_configs:
        del sets, ys
        torch.cuda.empty_cache()
        configs = run_configs(stream, pool, oracle_s=3.0)

    out = {
        "metric": METRIC,
        "value": round(tc / t_step / 1e9, 3),
        "unit": "Gtoken·channels/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "32k chunked prefill (B=1 D=4096 L=32768, bf16 I/O, N=16, chunk 1024)",
                   "entry": "hyena_chunk_fwd" if args.algo == "auto" else "hyena_chunk_fwd_algo",
                   "algo": algo_used, "B": B, "D": D, "L": L, "chunk": CHUNK, "modes": w.N,
                   "io": "bf16", "input_sets": INPUT_SETS},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "compute": compute,
        "hbm_copy": {"measured_GBps": round(copy_gbs, 1),
                     "frac": round(achieved / copy_gbs, 4)},
        "wall_s_timed": round(t_wall, 3),
        "step_ms": {"median": round(spread[len(spread) // 2], 4), "min": round(spread[0], 4),
                    "max": round(spread[-1], 4), "n": len(spread)},
        "components": comps,
    }
    if configs is not None:
        out["configs"] = configs
    if t_same is not None:
        out["same_input_set"] = {"ms_per_step": round(t_same * 1e3, 4),
                                 "value": round(tc / t_same / 1e9, 3)}
    if pool is not None:
        out["cpu_baseline"] = cpu_baseline(pool, w)
        pool.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
