"""Benchmark of the Hyena operator on one MI355X.

One step = one pass of the operator over the 32 kb chunked-prefill workload
(B=1, D=4096, L=32768, bf16 I/O, N=16 modes, chunk 1024 with carried state):
modal filter generation, input gate, causal long convolution, output gate and
skip, and the carried modal state -- all in one launch of hyena_chunk_fwd.
Inputs are resident in HBM before timing starts; consecutive steps take four
different input sets in turn (and write four outputs), so no step reads data
an earlier step left in the last-level cache.  The same step repeated on one
input set is reported beside it as `same_input_set` with --same-input.
`step_ms` gives the median, min and max of single steps, each timed on its
own in a separate pass after the headline's timed region.

Prints ONE JSON line.  Besides the headline it reports the roofline of the
dominant kernel (HIP-event timing of the same launches; HBM bytes and the
fp32 vector / bf16 matrix-core flops per launch from rocprofv3 counters kept
in profiles/traffic.json, while the kernel sources are unchanged), the other
entry points at the same shape, and the fp64 CPU oracle timed on a bounded
sample.

    python bench.py [--gpus 1] [--steps 100] [--warmup 100] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
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
                  "genomic_lm_amd/csrc/common.hpp"]
CPU_SAMPLE_S = 12.0                          # wall time the CPU oracle is given
INPUT_SETS = 4                               # activation sets the timed steps rotate over


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
    ap.add_argument("--algo", default="mfma", choices=["mfma", "fft", "auto"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-components", action="store_true")
    ap.add_argument("--same-input", action="store_true",
                    help="also time the step repeated on one input set (last-level cache hits)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (counter calibration)")
    return ap.parse_args()


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


def cpu_baseline(w):
    """The fp64 oracle's chunked prefill on a bounded sample of channels.

    Blocks of 16 channels (all L tokens each) are run until CPU_SAMPLE_S of
    wall time has passed or every channel is done; BLAS is held to one thread
    so that `cores` is what was used.
    """
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    done, dt, blk = 0, 0.0, 16
    with threadpool_limits(limits=1):
        while dt < CPU_SAMPLE_S and done < w.D:
            rows = np.arange(done, min(done + blk, w.D))
            x1, x2, v = (w.f64(k, rows) for k in ("x1", "x2", "v"))
            lam = w.log_poles[rows].astype(np.float64)
            R = w.residues[rows].astype(np.float64)
            sk = w.skip[rows].astype(np.float64)
            t0 = time.perf_counter()
            oracle.chunk_fwd(x1, x2, v, lam, R, sk, CHUNK)
            dt += time.perf_counter() - t0
            done = int(rows[-1]) + 1
    tc = w.B * done * w.L
    return {
        "value": round(tc / dt / 1e9, 6), "unit": "Gtoken·channels/s", "cores": 1, "kind": "oracle",
        "sample": f"oracle.chunk_fwd (fp64, chunk {CHUNK}) on channels 0..{done - 1} of {w.D} "
                  f"x {w.L} tokens (B={w.B}), {dt:.1f} s wall, numpy with BLAS held to 1 thread",
    }


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

    def rotating(f):
        n = [0]

        def g():
            f(n[0] % INPUT_SETS)
            n[0] += 1
        return g

    def head(k):
        G.chunk_fwd(*sets[k], lam, res, CHUNK, skip, algo=args.algo, out=ys[k], state_out=st)

    step = rotating(head)
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
        if tr.get("kernel_hash") == kernel_hash() and tr.get("algo") == args.algo:
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

    copy_gbs = copy_bandwidth(stream)
    comps = {}
    if not args.no_components:
        comp_steps = max(3, args.steps // 4)
        taps7, taps128 = par(w.taps[7]), par(w.taps[128])
        fft_ws = torch.empty(max(G.fftconv_workspace_size(B, D, L, w.N, x1.dtype), 16),
                             dtype=torch.uint8, device=dev)
        runs = {
            "chunk_fft": rotating(lambda k: G.chunk_fwd(*sets[k], lam, res, CHUNK, skip, algo="fft",
                                                        out=ys[k], state_out=st)),
            "chunk_mfma": rotating(lambda k: G.chunk_fwd(*sets[k], lam, res, CHUNK, skip, algo="mfma",
                                                         out=ys[k], state_out=st)),
            "fftconv_single_pass": rotating(lambda k: G.fftconv_fwd(*sets[k], lam, res, skip,
                                                                    out=ys[k], workspace=fft_ws)),
            "fir7": rotating(lambda k: G.fir_fwd(*sets[k], taps7, skip, out=ys[k])),
            "fir128": rotating(lambda k: G.fir_fwd(*sets[k], taps128, skip, out=ys[k])),
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

        runs[f"chunk_{args.algo}_x{nch}_calls"] = rotating(per_chunk_calls)
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
            *sets[k], lc_d, rc_d, skip, out=ys[k], workspace=fft_ws))
        runs["chunk_cpx_fft"] = rotating(lambda k: G.chunk_fwd_cpx(
            *sets[k], lc_d, rc_d, CHUNK, skip, algo="fft", out=ys[k], state_out=stc))
        runs["chunk_cpx_mfma"] = rotating(lambda k: G.chunk_fwd_cpx(
            *sets[k], lc_d, rc_d, CHUNK, skip, algo="mfma", out=ys[k], state_out=stc))
        # the same prefill read straight from in_proj's token-major layout
        # (B, L, 3D), channels interleaved per triple, y written (B, L, D)
        xins = [torch.stack(sk, -1).permute(0, 2, 1, 3).contiguous().view(B, L, 3 * D) for sk in sets]
        y_tms = [torch.empty((B, L, D), dtype=torch.bfloat16, device=dev) for _ in sets]
        tm_ws = torch.empty(max(G.chunk_tokmajor_workspace_size(B, D, L, w.N), 16),
                            dtype=torch.uint8, device=dev)
        runs["chunk_tokmajor"] = rotating(lambda k: G.chunk_fwd_tokmajor(
            xins[k], lam, res, skip, out=y_tms[k], state_out=st, workspace=tm_ws))
        win6 = torch.empty((B, D, 6), dtype=torch.float32, device=dev)
        win127 = torch.empty((B, D, 127), dtype=torch.float32, device=dev)
        runs["fir7_tokmajor"] = rotating(lambda k: G.fir_fwd_tokmajor(
            xins[k], taps7, skip, out=y_tms[k], window_out=win6))
        runs["fir128_tokmajor"] = rotating(lambda k: G.fir_fwd_tokmajor(
            xins[k], taps128, skip, out=y_tms[k], window_out=win127))
        one_token = {"modal_decode_step", "fir128_window_step"}   # B*D token·channels
        for name, fn in runs.items():
            t = timed(fn, comp_steps, 2, stream)
            n_tc = B * D if name in one_token else tc
            comps[name] = {"ms": round(t * 1e3, 4), "Gtc_per_s": round(n_tc / t / 1e9, 2),
                           "hbm_frac": round(8 * n_tc / t / 1e9 / HBM_PEAK_GBS, 4)}

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
                   "entry": "hyena_chunk_fwd", "algo": args.algo, "B": B, "D": D, "L": L,
                   "chunk": CHUNK, "modes": w.N, "io": "bf16", "input_sets": INPUT_SETS},
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
    if t_same is not None:
        out["same_input_set"] = {"ms_per_step": round(t_same * 1e3, 4),
                                 "value": round(tc / t_same / 1e9, 3)}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
