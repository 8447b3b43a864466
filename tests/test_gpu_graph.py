"""Entry points inside a HIP graph: a chunked prefill, single passes (on
chip, and in two launches through a workspace), decode steps and FIR window
steps (channel- and token-major) captured once and replayed several times, with the program's own eager work in between; every replay must give
the eager results bit for bit (every kernel here is deterministic).  Nothing
in these calls allocates, clears memory with a memset or synchronises, which
is what capture needs."""
import numpy as np
import pytest
import torch

import genomic_lm_amd as G
import workloads as W
from tests.gpu_util import DevWorkload, act_to_dev, gate, log, oracle_modal, state_gate

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.lib()
    yield


def _program(d, xin, bufs, n_pre, steps):
    """Prefill n_pre tokens, then `steps` single-token steps, into bufs."""
    x1, x2, v = d.x1, d.x2, d.v
    G.chunk_fwd(*(t[..., :n_pre] for t in bufs["pre"]), d.lam, d.res, 1024, d.skip,
                out=bufs["y_pre"], state_out=bufs["s"])
    G.fir_fwd_window(*(t[..., :n_pre] for t in bufs["pre"]), d.taps[128], d.skip,
                     out=bufs["yf_pre"], window_out=bufs["win"])
    G.chunk_fwd_tokmajor(bufs["xin_pre"], d.lam, d.res, d.skip, out=bufs["yt_pre"],
                         state_out=bufs["st"], workspace=bufs["ws"])
    G.fftconv_fwd(*bufs["pre"], d.lam, d.res, d.skip, out=bufs["yc_pre"])
    G.fftconv_fwd(*bufs["long"], d.lam, d.res, d.skip, out=bufs["yc_long"],
                  workspace=bufs["fws"])
    for i in range(steps):
        tok = bufs["tok"][i]
        G.modal_decode(*tok, d.lam, d.res, d.skip, state_in=bufs["s"], out=bufs["y_dec"][i],
                       state_out=bufs["s"])
        G.fir_fwd_window(*(t[..., None] for t in tok), d.taps[128], d.skip,
                         window_in=bufs["win"], out=bufs["yf_dec"][i][..., None],
                         window_out=bufs["win"])
        G.fir_fwd_tokmajor(bufs["xin_tok"][i], d.taps[7], d.skip, window_in=bufs["wt"],
                           out=bufs["yt_dec"][i], window_out=bufs["wt"])


def test_graph_capture_and_replay():
    n_pre, steps = 3000, 4
    w = W.make("7b_layer_set", D=256, L=n_pre + steps)
    d = DevWorkload(w)
    dev = d.x1.device
    xin = act_to_dev(W.interleave_triples(w.x1, w.x2, w.v), "bf16")
    B, D = 1, w.D
    pre = [t[..., :n_pre].contiguous() for t in (d.x1, d.x2, d.v)]
    ws_bytes = max(16, G.chunk_tokmajor_workspace_size(B, D, n_pre, w.N))
    n_long = 12000                                   # single pass in two launches
    wl = W.make("7b_layer_set", D=256, L=n_long)
    long = [act_to_dev(a, "bf16") for a in (wl.x1, wl.x2, wl.v)]
    fws_bytes = G.fftconv_workspace_size(B, D, n_long, w.N)
    assert fws_bytes > 0

    def fresh():
        return {
            "pre": pre,
            "xin_pre": xin[:, :n_pre].contiguous(),
            "tok": [[t[..., n_pre + i].contiguous() for t in (d.x1, d.x2, d.v)] for i in range(steps)],
            "xin_tok": [xin[:, n_pre + i:n_pre + i + 1].contiguous() for i in range(steps)],
            "y_pre": torch.empty_like(pre[0]), "yf_pre": torch.empty_like(pre[0]),
            "yt_pre": torch.empty((B, n_pre, D), dtype=torch.bfloat16, device=dev),
            "s": torch.empty((B, D, w.N), device=dev), "st": torch.empty((B, D, w.N), device=dev),
            "win": torch.empty((B, D, 127), device=dev), "wt": torch.zeros((B, D, 6), device=dev),
            "ws": torch.empty(ws_bytes, dtype=torch.uint8, device=dev),
            "long": long, "yc_pre": torch.empty_like(pre[0]),
            "yc_long": torch.empty_like(long[0]),
            "fws": torch.empty(fws_bytes, dtype=torch.uint8, device=dev),
            "y_dec": [torch.empty((B, D), dtype=torch.bfloat16, device=dev) for _ in range(steps)],
            "yf_dec": [torch.empty((B, D), dtype=torch.bfloat16, device=dev) for _ in range(steps)],
            "yt_dec": [torch.empty((B, 1, D), dtype=torch.bfloat16, device=dev) for _ in range(steps)],
        }

    outs = ("y_pre", "yf_pre", "yt_pre", "yc_pre", "yc_long", "s", "st", "win", "wt")
    lists = ("y_dec", "yf_dec", "yt_dec")

    def snapshot(b):
        snap = {k: b[k].clone() for k in outs}
        for k in lists:
            snap[k] = [t.clone() for t in b[k]]
        return snap

    eager = fresh()
    _program(d, xin, eager, n_pre, steps)
    torch.cuda.synchronize()
    ref = snapshot(eager)

    cap = fresh()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        _program(d, xin, cap, n_pre, steps)           # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            _program(d, xin, cap, n_pre, steps)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    for rep in range(3):
        cap["wt"].zero_()                             # the token-major FIR window starts empty
        for k in outs + lists:                        # poison the outputs between replays
            for t in (cap[k] if k in lists else [cap[k]]):
                if k != "wt":
                    t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _program(d, xin, fresh(), n_pre, 1)          # eager work between the replays
        torch.cuda.synchronize()
        log(f"graph replay {rep}")
        for k in outs:
            assert torch.equal(cap[k], ref[k]), (rep, k)
        for k in lists:
            for a, b in zip(cap[k], ref[k]):
                assert torch.equal(a, b), (rep, k)


@pytest.mark.parametrize("C", [1024, 512, 3072])
def test_chunk_calls_graph_replay(C):
    """A prefill as one call per chunk, the state handed from call to call
    (the form a serving loop replays without per-call host work): every
    replay equals the eager calls bit for bit, and those pass the oracle
    gates.  C = 1024 and 512 run the one-tile kernel (whole and partial
    tiles), 3072 the general one."""
    w = W.make("7b_layer_set", B=2, D=48, L=6 * 1024)
    d = DevWorkload(w)
    dev = d.x1.device
    chunks = [[t[..., t0:t0 + C].contiguous() for t in (d.x1, d.x2, d.v)]
              for t0 in range(0, w.L, C)]
    ys = [torch.empty_like(c[0]) for c in chunks]
    sts = [torch.empty((w.B, w.D, w.N), dtype=torch.float32, device=dev) for _ in range(2)]
    last = (len(chunks) - 1) & 1

    def calls():
        s_in = None
        for i, (a, b, c) in enumerate(chunks):
            G.chunk_fwd(a, b, c, d.lam, d.res, C, d.skip, state_in=s_in, out=ys[i],
                        state_out=sts[i & 1])
            s_in = sts[i & 1]

    log(f"graph replay of {len(chunks)} chunk calls, C={C}: eager")
    calls()
    torch.cuda.synchronize()
    y_eager = torch.cat(ys, -1)
    s_eager = sts[last].clone()
    ref, ref_s = oracle_modal(w)
    gate(y_eager, ref, "bf16", label=f"chunk calls C={C} eager")
    state_gate(s_eager, ref_s, label=f"chunk calls C={C} eager")

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for rep in range(3):
        for t in ys + sts:
            t.fill_(float("nan"))
        G.fftconv_fwd(d.x1, d.x2, d.v, d.lam, d.res, d.skip)     # unrelated eager work
        torch.cuda.synchronize()
        log(f"  replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(torch.cat(ys, -1), y_eager), f"replay {rep}: y differs"
        assert torch.equal(sts[last], s_eager), f"replay {rep}: state differs"
