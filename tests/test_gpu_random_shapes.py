"""Seeded random shapes through the channel-major entry points, against the
fp64 oracle: lengths off the tile and power-of-two grids, batch sizes, mode
counts, chunk sizes, FIR lengths and both I/O types, drawn once from a fixed
seed so that every run checks the same cases.  Each case runs the single
pass, the chunked entry with both algorithms (a random initial state, and the
matrix-core one only where its mode limit allows) and the explicit FIR.
Every case has at least MIN_OUTPUTS outputs (below).
"""
import numpy as np
import pytest
import torch

import genomic_lm_amd as G
import workloads as W
from tests.gpu_util import DevWorkload, gate, log, oracle_fir, oracle_modal, par_to_dev, state_gate

pytestmark = pytest.mark.gpu

MFMA_MAX_MODES = 32
# The relative-L2 gate is a statistic over the outputs: rounding y to bf16
# alone costs up to 2^-8 relative per element (about 1.2e-3 rms), so a case
# with a few dozen outputs can exceed 2e-3 on rounding noise (seen at 36 and
# 160 outputs).  Short rows therefore get more channels.
MIN_OUTPUTS = 4096
FFT_MAX_CHUNK = 8192


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.lib()
    yield


def _cases(n=40, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        io = "bf16" if rng.random() < 0.75 else "f32"
        B = int(rng.integers(1, 4))
        D = int(rng.integers(1, 33))
        band = int(rng.integers(0, 3))
        L = int((rng.integers(1, 64), rng.integers(64, 1100), rng.integers(1100, 6000))[band])
        N = int(rng.choice([1, 2, 5, 8, 13, 16, 23, 32, 40, 64]))
        C = int(rng.choice([1, 7, 64, 100, 512, 1000, 1024, 2048, 4096]))
        K = int(rng.choice([1, 2, 7, 31, 64, 100, 128, 300]))
        D = min(4096, max(D, -(-MIN_OUTPUTS // (B * L))))
        out.append((i, io, B, D, L, N, C, K))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "r{}-{}-B{}-D{}-L{}-N{}-C{}-K{}".format(*c))
def test_random_shape(case):
    i, io, B, D, L, N, C, K = case
    w = W.make("tiny" if io == "f32" else "7b_layer_set", B=B, D=D, L=L, N=N)
    d = DevWorkload(w)
    log(f"random case {i}: io={io} B={B} D={D} L={L} N={N} C={C} K={K}")

    ref, _ = oracle_modal(w)
    gate(G.fftconv_fwd(d.x1, d.x2, d.v, d.lam, d.res, d.skip), ref, io, label="fftconv")

    s0 = W.random_state(B, D, N, seed=1000 + i)
    ref_c, ref_s = oracle_modal(w, C=C, state_in=s0)
    algos = (["fft"] if C <= FFT_MAX_CHUNK else []) + (["mfma"] if N <= MFMA_MAX_MODES else [])
    for algo in algos:
        y, s = G.chunk_fwd(d.x1, d.x2, d.v, d.lam, d.res, C, d.skip, state_in=par_to_dev(s0),
                           algo=algo)
        gate(y, ref_c, io, label=f"chunk/{algo}")
        state_gate(s, ref_s, label=f"chunk/{algo}")

    taps = W.random_taps(K, D, seed=2000 + i, bf16=(io == "bf16"))
    ref_f = oracle_fir(w, K, taps=taps)
    gate(G.fir_fwd(d.x1, d.x2, d.v, par_to_dev(taps), d.skip), ref_f, io, label=f"fir K={K}")
