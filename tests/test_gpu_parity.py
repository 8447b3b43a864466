"""HIP path against the fp64 oracle, element by element, through the C ABI.

Small cases cover every kernel variant (each FFT size, FIR tap counts, chunk
sizes, ragged lengths, batch > 1, carried state); the full-size cases run the
configurations the benchmark uses, in the same launch configuration, into
NaN-filled buffers, and compare every channel (all time steps) with the
oracle, run in parallel processes on the host.
"""
import numpy as np
import pytest
import torch

import genomic_lm_amd as G
import oracle
import workloads as W
from tests.gpu_util import (DevWorkload, act_to_dev, all_finite, gate, host, log, oracle_fir,
                            oracle_modal, offset_copy, par_to_dev, poisoned, pool_gate,
                            sample_rows, state_gate, to_f64, compare_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.lib()                                   # loud failure if the library is missing
    yield


def small(io, D=8, L=1024, B=1, seed_cfg=None, lam_lo=None):
    name = seed_cfg or ("tiny" if io == "f32" else "7b_layer_set")
    return W.make(name, B=B, D=D, L=L, lam_lo=lam_lo)


# ------------------------------------------------------------------ filter
@pytest.mark.parametrize("L", [1, 777, 8192])
def test_modal_filter(L):
    w = small("f32", D=16, L=L)
    d = DevWorkload(w)
    log(f"modal_filter D=16 L={L}")
    h = to_f64(G.modal_filter(d.lam, d.res, L))
    ref = oracle.modal_filter(w.log_poles, w.residues, L)
    err = np.sqrt(np.sum((h - ref) ** 2, -1) / np.sum(ref ** 2, -1))
    assert np.max(err) < 1e-5, err


# ------------------------------------------------------------------ fftconv
@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("L", [1, 2, 7, 100, 512, 777, 1000, 1024, 2049, 4096, 8192, 8193, 12000,
                               16384, 32768])
def test_fftconv_small(io, L):
    B = 2 if L in (777, 4096) else 1
    w = small(io, D=4, L=L, B=B)
    d = DevWorkload(w)
    log(f"fftconv io={io} B={B} D=4 L={L}")
    y = G.fftconv_fwd(d.x1, d.x2, d.v, d.lam, d.res, d.skip)
    ref, _ = oracle_modal(w)
    gate(y, ref, io, label=f"fftconv L={L}")


# Rows longer than 8192 go through a workspace: up to L = 32768 one launch
# per parity half, beyond it the three-kernel four-step path.  Lengths cover
# the two-launch sizes (S = 16384 here; 8192 in test_fftconv_small), each
# row-transform size of the four-step (S/256 = 128 ... 1024), odd lengths
# (the pair loads' ragged tail), and B*D above one row batch.
@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("L,B,D", [(16385, 1, 3), (20001, 2, 2), (32768, 1, 2),
                                   (32769, 1, 3), (40000, 2, 2), (65536, 1, 2), (65001, 1, 2),
                                   (131072, 1, 2), (262143, 1, 1), (300000, 1, 1)])
def test_fftconv_large(io, L, B, D):
    w = small(io, D=D, L=L, B=B)
    d = DevWorkload(w)
    ws = G.fftconv_workspace_size(B, D, L, w.N, d.x1.dtype)
    log(f"fftconv large io={io} B={B} D={D} L={L} workspace={ws}")
    assert ws > 0
    y = G.fftconv_fwd(d.x1, d.x2, d.v, d.lam, d.res, d.skip)
    ref, _ = oracle_modal(w)
    gate(y, ref, io, label=f"fftconv L={L}")


def test_fftconv_large_row_batches():
    # 1200 rows of S = 32768 (1 MiB of workspace each): two row batches
    # (1024 + 176) through one workspace; sampled channels, every batch row
    w = small("bf16", D=400, L=33000, B=3)
    d = DevWorkload(w)
    log("fftconv large B=3 D=400 L=33000")
    y = G.fftconv_fwd(d.x1, d.x2, d.v, d.lam, d.res, d.skip)
    rows = sample_rows(w.D, k=12)
    ref, _ = oracle_modal(w, rows)
    gate(y, ref, "bf16", rows, label="fftconv 1200 rows")


def test_fftconv_split_row_batches():
    # 8200 rows of S = 16384 (128 KiB of workspace each): two row batches
    # (8192 + 8) of the two-launch form through one workspace; the sampled
    # channels include the last, whose rows lie in the second batch
    w = small("bf16", D=4100, L=16385, B=2)
    d = DevWorkload(w)
    log("fftconv split B=2 D=4100 L=16385")
    assert G.fftconv_workspace_size(2, 4100, 16385, w.N) == 8192 * 8 * 16384
    y = G.fftconv_fwd(d.x1, d.x2, d.v, d.lam, d.res, d.skip)
    rows = sample_rows(w.D, k=6)
    ref, _ = oracle_modal(w, rows)
    gate(y, ref, "bf16", rows, label="fftconv 8200 rows")


def test_fftconv_large_workspace_errors():
    w = small("bf16", D=1, L=40000)
    d = DevWorkload(w)
    need = G.fftconv_workspace_size(1, 1, 40000, w.N, d.x1.dtype)
    short = torch.empty(need - 16, dtype=torch.uint8, device=d.x1.device)
    with pytest.raises(G.HyenaError, match="WORKSPACE"):
        G.fftconv_fwd(d.x1, d.x2, d.v, d.lam, d.res, d.skip, workspace=short)


# ------------------------------------------------------------------ FIR
@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("K,L", [(1, 100), (3, 1), (7, 2048), (7, 3001), (8, 4096), (9, 100),
                                 (128, 2048), (128, 5000), (129, 300), (1024, 4096)])
def test_fir_small(io, K, L):
    w = small(io, D=4, L=L, B=2 if K == 7 else 1)
    d = DevWorkload(w)
    taps = W.random_taps(K, w.D, seed=K, bf16=(io == "bf16"))
    log(f"fir io={io} K={K} L={L}")
    y = G.fir_fwd(d.x1, d.x2, d.v, par_to_dev(taps), d.skip)
    gate(y, oracle_fir(w, K, taps=taps), io, label=f"fir K={K} L={L}")


@pytest.mark.parametrize("K", [1, 2, 7, 33, 64, 100, 128])
@pytest.mark.parametrize("L,B", [(1024, 1), (3000, 2), (4096, 1), (777, 1), (100, 1), (5120, 1),
                                 (8, 32), (512, 2), (2056, 1)])
def test_fir_mfma_cases(K, L, B):
    """bf16 FIR with K <= 128 runs on the matrix cores: every diagonal count
    (1..5), whole tiles, a ragged last tile, rows shorter than a tile, rows not
    16-byte aligned (odd L), batch > 1."""
    w = small("bf16", D=4, L=L, B=B)
    d = DevWorkload(w)
    taps = W.random_taps(K, w.D, seed=K + 1000, bf16=True)
    log(f"fir/mfma K={K} L={L} B={B}")
    y = G.fir_fwd(d.x1, d.x2, d.v, par_to_dev(taps), d.skip)
    gate(y, oracle_fir(w, K, taps=taps), "bf16", label=f"fir/mfma K={K} L={L}")


@pytest.mark.parametrize("K", [7, 128])
def test_fir_mfma_fp32_taps(K):
    """Taps that are not bf16 values take the two-part product path."""
    w = small("bf16", D=8, L=4096)
    d = DevWorkload(w)
    taps = W.random_taps(K, w.D, seed=K + 2000, bf16=False)
    assert not np.array_equal(W.bf16_bits_to_f32(W.f32_to_bf16_bits(taps)), taps)
    y = G.fir_fwd(d.x1, d.x2, d.v, par_to_dev(taps), d.skip)
    gate(y, oracle_fir(w, K, taps=taps), "bf16", label=f"fir/mfma fp32 taps K={K}")


# ------------------------------------------------------------------ chunked
# (256, 3000) and (257, 3000): the FFT chunk algorithm's last chunk length
# with the state decayed by an fp32 pair, and the first with one fp32 factor
CHUNK_CASES = [(1, 50), (7, 300), (64, 1000), (128, 1024), (256, 3000), (257, 3000),
               (1000, 4096), (1024, 3000), (1024, 5000), (4096, 8192), (8192, 8192),
               (2048, 1500)]


@pytest.mark.parametrize("algo", ["mfma", "fft"])
@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("C,L", CHUNK_CASES)
def test_chunk_small(algo, io, C, L):
    w = small(io, D=4, L=L, B=2 if C == 64 else 1)
    d = DevWorkload(w)
    s0 = W.random_state(w.B, w.D, w.N, seed=C + L)
    log(f"chunk algo={algo} io={io} C={C} L={L}")
    for state in (None, s0):
        sin = None if state is None else par_to_dev(state)
        y, s = G.chunk_fwd(d.x1, d.x2, d.v, d.lam, d.res, C, d.skip, state_in=sin, algo=algo)
        ref_y, ref_s = oracle_modal(w, C=C, state_in=state)
        gate(y, ref_y, io, label=f"chunk/{algo} C={C} L={L} state={'yes' if state is not None else 'no'}")
        state_gate(s, ref_s, label=f"chunk/{algo} C={C} L={L}")


# bf16 rows whose length is a multiple of 8 but not of 1024: the matrix-core
# kernel stages the partial last tile like a full one (chunks past L re-read
# an in-bounds chunk and are zeroed); lengths below one tile, one chunk past
# a tile, one chunk short of one, and a 32-tile row with a partial 33rd.
@pytest.mark.parametrize("L", [8, 512, 1016, 1032, 2056, 32768 + 744])
def test_chunk_mfma_partial_tile(L):
    w = small("bf16", D=5, L=L, B=2)
    d = DevWorkload(w)
    s0 = W.random_state(w.B, w.D, w.N, seed=L)
    log(f"chunk/mfma partial tile L={L}")
    rows = np.arange(w.D) if L <= 4096 else sample_rows(w.D, k=3)
    for state in (None, s0):
        sin = None if state is None else par_to_dev(state)
        y, s = G.chunk_fwd(d.x1, d.x2, d.v, d.lam, d.res, 1024, d.skip, state_in=sin, algo="mfma")
        ref_y, ref_s = oracle_modal(w, rows, C=1024, state_in=state)
        gate(y, ref_y, "bf16", rows, label=f"chunk/mfma L={L} state={'yes' if state is not None else 'no'}")
        state_gate(s, ref_s, rows, label=f"chunk/mfma L={L}")


def test_chunk_mfma_one_tile_rows_many():
    # one 1024-token chunk per row and more rows than the chip holds waves
    # at once (2 per SIMD), so later waves start as earlier ones retire;
    # sampled channels of both batch items, state in and out
    w = small("bf16", D=3000, L=1024, B=2)
    d = DevWorkload(w)
    s0 = W.random_state(w.B, w.D, w.N, seed=11)
    rows = sample_rows(w.D, k=10)
    log("chunk/mfma one tile, B=2 D=3000 L=1024")
    for state in (None, s0):
        sin = None if state is None else par_to_dev(state)
        y, s = G.chunk_fwd(d.x1, d.x2, d.v, d.lam, d.res, 1024, d.skip, state_in=sin, algo="mfma")
        ref_y, ref_s = oracle_modal(w, rows, C=1024, state_in=state)
        gate(y, ref_y, "bf16", rows, label=f"chunk/mfma rows>waves state={'yes' if state is not None else 'no'}")
        state_gate(s, ref_s, rows, label="chunk/mfma rows>waves")


@pytest.mark.parametrize("N", [1, 5, 16])
@pytest.mark.parametrize("L", [1024, 520])
def test_chunk_one_tile_mode_counts(N, L):
    """Rows of at most one 1024-token tile (one chunk per call) with fewer
    modes than scan lanes: the padded lanes' states reach neither y nor
    state_out; a whole tile and a partial one, state in and out."""
    w = W.make("7b_layer_set", B=2, D=6, L=L, N=N)
    d = DevWorkload(w)
    s0 = W.random_state(w.B, w.D, w.N, seed=N + L)
    for state in (None, s0):
        sin = None if state is None else par_to_dev(state)
        log(f"chunk one tile N={N} L={L} state={'yes' if state is not None else 'no'}")
        y, s = G.chunk_fwd(d.x1, d.x2, d.v, d.lam, d.res, 1024, d.skip, state_in=sin, algo="mfma")
        ref_y, ref_s = oracle_modal(w, C=1024, state_in=state)
        gate(y, ref_y, "bf16", label=f"chunk one tile N={N} L={L}")
        state_gate(s, ref_s, label=f"chunk one tile N={N} L={L}")


@pytest.mark.parametrize("N", [1, 3, 17, 24, 32, 33, 64])
def test_mode_counts(N):
    """From one mode to the maximum of 64: single pass, chunked with AUTO (the
    matrix-core path up to 32 modes -- one scan lane per mode from 17 on --
    FFT beyond), and each algorithm it has."""
    w = W.make("7b_layer_set", B=2, D=4, L=3000, N=N)
    d = DevWorkload(w)
    log(f"modes N={N}")
    ref, ref_s = oracle_modal(w)
    gate(G.fftconv_fwd(d.x1, d.x2, d.v, d.lam, d.res, d.skip), ref, "bf16", label=f"fftconv N={N}")
    for algo in (["auto", "fft", "mfma"] if N <= 32 else ["auto", "fft"]):
        y, s = G.chunk_fwd(d.x1, d.x2, d.v, d.lam, d.res, 1024, d.skip, algo=algo)
        gate(y, ref, "bf16", label=f"chunk/{algo} N={N}")
        state_gate(s, ref_s, label=f"chunk/{algo} N={N}")
    if N > 32:
        with pytest.raises(G.HyenaError, match="UNSUPPORTED"):
            G.chunk_fwd(d.x1, d.x2, d.v, d.lam, d.res, 1024, d.skip, algo="mfma")


# The split single pass (L > 4096) forms h on the matrix cores, 16 modes per
# block of products: mode counts on both sides of a block boundary and the
# maximum, both split sizes (S = 4096 and 16384), bf16 and fp32 rows; then
# modes at the extremes of the exponent range: two slow modes with nearly
# equal poles and opposite residues (h a small difference of two large
# terms), and fast ones whose terms underflow within a few tokens.
@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("L", [5000, 20001])
@pytest.mark.parametrize("N", [1, 3, 15, 16, 17, 33, 64])
def test_fftconv_split_mode_counts(N, L, io):
    w = W.make("tiny" if io == "f32" else "7b_layer_set", B=1, D=3, L=L, N=N)
    d = DevWorkload(w)
    log(f"fftconv split modes N={N} L={L} io={io}")
    ref, _ = oracle_modal(w)
    gate(G.fftconv_fwd(d.x1, d.x2, d.v, d.lam, d.res, d.skip), ref, io, label=f"fftconv N={N} L={L}")


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_fftconv_split_extreme_modes(io):
    w = W.make("tiny" if io == "f32" else "7b_layer_set", B=1, D=6, L=32768, N=16)
    rng = np.random.default_rng(23)
    lam = w.log_poles.astype(np.float64).copy()
    res = w.residues.astype(np.float64).copy()
    lam[:, 0] = -1.0e-4 * (1.0 + 0.3 * rng.random(w.D))
    lam[:, 1] = lam[:, 0] * (1.0 + 0.05 * rng.random(w.D))
    res[:, 0], res[:, 1] = 0.4, -0.4
    lam[:, 2:6] = -rng.uniform(5.0, 80.0, (w.D, 4))
    w.log_poles, w.residues = lam.astype(np.float32), res.astype(np.float32)
    d = DevWorkload(w)
    log(f"fftconv split extreme modes io={io}")
    ref, _ = oracle_modal(w)
    gate(G.fftconv_fwd(d.x1, d.x2, d.v, d.lam, d.res, d.skip), ref, io, label="fftconv extreme modes")


# The 32-slot form (17 to 32 real modes): fp32 and bf16 rows, whole tiles, a
# partial last tile, rows of at most one tile, unaligned rows, carried state.
@pytest.mark.parametrize("io,L,offset", [("bf16", 5000, False), ("bf16", 1016, False),
                                         ("bf16", 2048, False), ("bf16", 777, True),
                                         ("f32", 3000, False), ("f32", 640, True)])
@pytest.mark.parametrize("N", [20, 32])
def test_chunk_mfma_32_slots(N, io, L, offset):
    w = W.make("tiny" if io == "f32" else "7b_layer_set", B=2, D=5, L=L, N=N)
    d = DevWorkload(w)
    s0 = W.random_state(w.B, w.D, w.N, seed=N + L)
    xs = [offset_copy(t) for t in (d.x1, d.x2, d.v)] if offset else [d.x1, d.x2, d.v]
    log(f"chunk/mfma 32 slots N={N} io={io} L={L} offset={offset}")
    for state in (None, s0):
        sin = None if state is None else par_to_dev(state)
        y, s = G.chunk_fwd(*xs, d.lam, d.res, 1024, d.skip, state_in=sin, algo="mfma")
        ref_y, ref_s = oracle_modal(w, C=1024, state_in=state)
        gate(y, ref_y, io, label=f"chunk/mfma N={N} L={L} {io}")
        state_gate(s, ref_s, label=f"chunk/mfma N={N} L={L} {io}")


@pytest.mark.parametrize("algo", ["mfma", "fft"])
def test_chunk_resume_matches_single_call(algo):
    """Split anywhere, carry the state through the host, continue."""
    w = small("bf16", D=8, L=5000)
    d = DevWorkload(w)
    C = 1024
    y_all, s_all = G.chunk_fwd(d.x1, d.x2, d.v, d.lam, d.res, C, d.skip, algo=algo)
    for cut in (1024, 2048, 1500, 4999):
        log(f"resume algo={algo} cut={cut}")
        parts = [t[..., :cut].contiguous() for t in (d.x1, d.x2, d.v)]
        ya, sa = G.chunk_fwd(*parts, d.lam, d.res, C, d.skip, algo=algo)
        sa_host = sa.cpu()                      # the cache leaves the device and comes back
        parts = [t[..., cut:].contiguous() for t in (d.x1, d.x2, d.v)]
        yb, sb = G.chunk_fwd(*parts, d.lam, d.res, C, d.skip, state_in=sa_host.cuda(), algo=algo)
        y = torch.cat([ya, yb], dim=-1)
        ref, ref_s = oracle_modal(w)
        gate(y, ref, "bf16", label=f"resume cut={cut}")
        state_gate(sb, ref_s, label=f"resume cut={cut}")
        d_ = (y.float() - y_all.float()).abs().max().item()
        scale = y_all.float().abs().max().item()
        assert d_ <= 2e-2 * scale


@pytest.mark.parametrize("algo", ["mfma", "fft"])
def test_chunk_state_in_place(algo):
    """state_out may be the state_in buffer: per-chunk calls updating one cache."""
    w = small("bf16", D=8, L=3072)
    d = DevWorkload(w)
    C = 1024
    ref, ref_s = oracle_modal(w)
    st = torch.zeros((1, w.D, w.N), dtype=torch.float32, device=d.x1.device)
    ys = []
    for t0 in range(0, w.L, C):
        log(f"in-place state algo={algo} t0={t0}")
        sl = [t[..., t0:t0 + C].contiguous() for t in (d.x1, d.x2, d.v)]
        yc, s_out = G.chunk_fwd(*sl, d.lam, d.res, C, d.skip, state_in=st, state_out=st, algo=algo)
        assert s_out.data_ptr() == st.data_ptr()
        ys.append(yc)
    gate(torch.cat(ys, -1), ref, "bf16", label=f"in-place state {algo}")
    state_gate(st, ref_s, label=f"in-place state {algo}")


def test_chunked_equals_single_pass_on_gpu():
    w = small("bf16", D=8, L=32768)
    d = DevWorkload(w)
    y_full = G.fftconv_fwd(d.x1, d.x2, d.v, d.lam, d.res, d.skip)
    ref, _ = oracle_modal(w)
    for algo in ("mfma", "fft"):
        for C in (1024, 4096):
            y, _ = G.chunk_fwd(d.x1, d.x2, d.v, d.lam, d.res, C, d.skip, algo=algo)
            gate(y, ref, "bf16", label=f"chunk/{algo} C={C}")
            # chunked = single pass: the two GPU results agree within the gates
            m = oracle.compare(to_f64(y), to_f64(y_full))
            log(f"  chunk/{algo} C={C} vs fftconv: {m}")
            assert oracle.passes(m), m


@pytest.mark.parametrize("algo,C", [("mfma", 1024), ("mfma", 4096), ("fft", 1024), ("fft", 4096),
                                    ("fftconv", 0), ("mfma_calls", 1024)])
def test_slow_cancelling_modes(algo, C):
    """Two slow modes (|lam| ~ 1e-5, remembered for ~1e5 tokens) with nearly
    equal poles and opposite residues: each mode's carried term is many times
    the output, so a relative error of the carried state that a long scan
    compounds (a decay factor rounded once and applied thousands of times)
    shows up in the output at full size.  mfma_calls: 128 calls of one
    1024-token chunk each, the fp32 state handed from call to call (the
    one-tile kernel, whose decay factors are single fp32 values)."""
    w = W.make("262k", D=8, L=131072)
    rng = np.random.default_rng(17)
    lam = w.log_poles.copy()
    res = w.residues.copy()
    lam[:, 0] = -1.0e-5 * (1.0 + 0.3 * rng.random(w.D))
    lam[:, 1] = lam[:, 0] * (1.0 + 0.05 * rng.random(w.D))
    res[:, 0] = 0.4
    res[:, 1] = -0.4
    w.log_poles, w.residues = lam.astype(np.float32), res.astype(np.float32)
    d = DevWorkload(w)
    log(f"slow cancelling modes: {algo} C={C}")
    ref, ref_s = oracle_modal(w)
    if algo == "fftconv":
        y = G.fftconv_fwd(d.x1, d.x2, d.v, d.lam, d.res, d.skip)
        gate(y, ref, "bf16", label="fftconv slow modes")
        return
    if algo == "mfma_calls":
        ys, s = [], None
        for t0 in range(0, w.L, C):
            sl = [t[..., t0:t0 + C].contiguous() for t in (d.x1, d.x2, d.v)]
            yc, s = G.chunk_fwd(*sl, d.lam, d.res, C, d.skip, state_in=s, algo="mfma")
            ys.append(yc)
        y = torch.cat(ys, -1)
    else:
        y, s = G.chunk_fwd(d.x1, d.x2, d.v, d.lam, d.res, C, d.skip, algo=algo)
    gate(y, ref, "bf16", label=f"chunk/{algo} C={C} slow modes")
    state_gate(s, ref_s, label=f"chunk/{algo} C={C} slow modes")


# ------------------------------------------------------------------ exact special cases
def test_impulse_is_causal():
    """x1 = delta at t0, v = x2 = 1, skip = 0: y = h shifted by t0.

    Direct evaluations (MFMA blocks, FIR) give exact zeros before t0; FFT
    evaluations give rounding noise there, except in chunks that end before
    t0, whose input is all zero."""
    D, L = 4, 4096
    w = small("bf16", D=D, L=L)
    t0 = 1500
    x1 = np.zeros((1, D, L), dtype=np.float32)
    x1[..., t0] = 1.0
    one = W.f32_to_bf16_bits(np.ones((1, D, L), dtype=np.float32))
    dx1 = act_to_dev(W.f32_to_bf16_bits(x1), "bf16")
    dv = act_to_dev(one, "bf16")
    lam, res = par_to_dev(w.log_poles), par_to_dev(w.residues)
    h = oracle.modal_filter(w.log_poles, w.residues, L)
    ref = np.zeros((1, D, L))
    ref[0, :, t0:] = h[:, :L - t0]
    outs = {   # name -> (output, first index that must be exactly zero-free of noise)
        "fftconv": (G.fftconv_fwd(dx1, dv, dv, lam, res), 0),
        "chunk/mfma": (G.chunk_fwd(dx1, dv, dv, lam, res, 1024, algo="mfma")[0], t0),
        "chunk/fft": (G.chunk_fwd(dx1, dv, dv, lam, res, 1024, algo="fft")[0], 1024),
    }
    for name, (y, exact_until) in outs.items():
        yy = to_f64(y)
        assert np.all(yy[..., :exact_until] == 0.0), name
        assert np.max(np.abs(yy[..., :t0])) <= 1e-6 * np.max(np.abs(ref)), name
        gate(y, ref, "bf16", label=f"impulse {name}")
    taps = par_to_dev(W.random_taps(7, D, seed=1, bf16=True))
    yf = to_f64(G.fir_fwd(dx1, dv, dv, taps))
    assert np.all(yf[..., :t0] == 0.0) and np.all(yf[..., t0 + 7:] == 0.0)


def test_zero_residues_give_exact_skip_path():
    w = small("bf16", D=4, L=3000)
    d = DevWorkload(w)
    zero = torch.zeros_like(d.res)
    u = w.f64("x1") * w.f64("v")
    expect = W.f32_to_bf16_bits((w.skip[None, :, None].astype(np.float64) * u).astype(np.float32))
    for name, y in {
        "fftconv": G.fftconv_fwd(d.x1, d.x2, d.v, d.lam, zero, d.skip),
        "chunk/mfma": G.chunk_fwd(d.x1, d.x2, d.v, d.lam, zero, 512, d.skip, algo="mfma")[0],
        "chunk/fft": G.chunk_fwd(d.x1, d.x2, d.v, d.lam, zero, 512, d.skip, algo="fft")[0],
        "fir": G.fir_fwd(d.x1, d.x2, d.v, torch.zeros(w.D, 7, device=d.x1.device), d.skip),
    }.items():
        got = y.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, expect), name


def test_outputs_fully_written_and_deterministic():
    w = small("bf16", D=8, L=5000)
    d = DevWorkload(w)
    runs = {
        "fftconv": lambda out: G.fftconv_fwd(d.x1, d.x2, d.v, d.lam, d.res, d.skip, out=out),
        "chunk/mfma": lambda out: G.chunk_fwd(d.x1, d.x2, d.v, d.lam, d.res, 1024, d.skip, algo="mfma", out=out)[0],
        "chunk/fft": lambda out: G.chunk_fwd(d.x1, d.x2, d.v, d.lam, d.res, 1024, d.skip, algo="fft", out=out)[0],
        "fir128": lambda out: G.fir_fwd(d.x1, d.x2, d.v, d.taps[128], d.skip, out=out),
    }
    for name, run in runs.items():
        first = None
        for rep in range(3):
            out = torch.full_like(d.x1, float("nan"))
            run(out)
            assert torch.isfinite(out.float()).all(), name
            bits = out.view(torch.int16).cpu()
            if first is None:
                first = bits
            else:
                assert torch.equal(bits, first), name


def test_empty_sequences():
    dv = torch.device("cuda:0")
    D, N = 4, 16
    lam = torch.full((D, N), -0.1, device=dv)
    res = torch.ones((D, N), device=dv)
    x = torch.empty((1, D, 0), dtype=torch.bfloat16, device=dv)
    s0 = torch.randn(1, D, N, device=dv)
    y, s = G.chunk_fwd(x, x, x, lam, res, 1024, state_in=s0)
    assert y.shape == (1, D, 0) and torch.equal(s, s0)
    _, s = G.chunk_fwd(x, x, x, lam, res, 1024)
    assert torch.count_nonzero(s) == 0
    assert G.fftconv_fwd(x, x, x, lam, res).shape == (1, D, 0)


# ------------------------------------------------------------------ full-size configurations
# Every output buffer starts as NaN and must come back entirely finite.
# Every channel is compared with the single-pass definition (oracle.hyena_fwd,
# oracle.fir_fwd) by the oracle process pool, and the chunked results of
# N_RECURRENCE channels spread over the whole range (both halves of a
# 4096-row launch, which the matrix-core kernel runs as two rounds of waves)
# also with the chunk recurrence itself (oracle.chunk_fwd).
N_RECURRENCE = 64


@pytest.fixture(scope="module", autouse=True)
def stop_oracle_pool():
    yield
    from tests import oracle_pool
    oracle_pool.shutdown()


def _full(name):
    log(f"generating {name}")
    w = W.make(name)
    return w, DevWorkload(w)


def test_config_tiny_full():
    w, d = _full("tiny")
    ref, ref_s = oracle_modal(w)
    y = G.fftconv_fwd(d.x1, d.x2, d.v, d.lam, d.res, d.skip, out=poisoned(d.x1))
    all_finite(y, "tiny fftconv")
    gate(y, ref, "f32", label="tiny fftconv")
    ref_c, ref_cs = oracle_modal(w, C=128)
    for algo in ("mfma", "fft"):
        y, s = G.chunk_fwd(d.x1, d.x2, d.v, d.lam, d.res, 128, d.skip, algo=algo,
                           out=poisoned(d.x1))
        all_finite(y, f"tiny chunk/{algo}")
        gate(y, ref_c, "f32", label=f"tiny chunk/{algo} vs chunk recurrence")
        state_gate(s, ref_cs, label=f"tiny chunk/{algo} vs chunk recurrence")
        gate(y, ref, "f32", label=f"tiny chunk/{algo} vs single pass")
        state_gate(s, ref_s, label=f"tiny chunk/{algo} vs single pass")


def test_config_7b_layer_set():
    w, d = _full("7b_layer_set")
    jobs = []
    for K in (7, 128):
        y = G.fir_fwd(d.x1, d.x2, d.v, d.taps[K], d.skip, out=poisoned(d.x1))
        all_finite(y, f"7b FIR-{K}")
        jobs.append(("fir", f"7b FIR-{K}", K, host(y)))
    y = G.fftconv_fwd(d.x1, d.x2, d.v, d.lam, d.res, d.skip, out=poisoned(d.x1))
    all_finite(y, "7b modal fftconv")
    jobs.append(("modal", "7b modal fftconv", host(y)))
    pool_gate("7b_layer_set", jobs, range(w.D), "bf16")


def _prefill_results(name, w, d, C):
    """The modal operator's full-size results, each in a NaN-filled buffer:
    the chunked entry in one launch (both algorithms), the same prefill as
    per-chunk calls with the state handed over (AUTO), and the single pass.
    Returns {label: (y, state or None)} on the device."""
    res = {}
    for algo in ("mfma", "fft"):
        y, s = G.chunk_fwd(d.x1, d.x2, d.v, d.lam, d.res, C, d.skip, algo=algo,
                           out=poisoned(d.x1))
        res[f"{name} chunk/{algo} one launch"] = (y, s)
    ys, st = [], None
    for t0 in range(0, w.L, C):
        sl = [t[..., t0:t0 + C].contiguous() for t in (d.x1, d.x2, d.v)]
        yc, st = G.chunk_fwd(*sl, d.lam, d.res, C, d.skip, state_in=st, out=poisoned(sl[0]))
        ys.append(yc)
    res[f"{name} chunk x{len(ys)} calls"] = (torch.cat(ys, -1), st)
    y = G.fftconv_fwd(d.x1, d.x2, d.v, d.lam, d.res, d.skip, out=poisoned(d.x1))
    res[f"{name} fftconv"] = (y, None)
    for label, (y, _) in res.items():
        all_finite(y, label)
    return res


def _check_prefill(name, w, res, C, block=64):
    h = {label: (host(y), None if s is None else host(s)) for label, (y, s) in res.items()}
    jobs = [("modal", label, y) for label, (y, _) in h.items()]
    jobs += [("modal_state", f"{label} state", s) for label, (_, s) in h.items() if s is not None]
    pool_gate(name, jobs, range(w.D), "bf16", block=block)
    rows = sample_rows(w.D, k=N_RECURRENCE)
    assert np.any(rows < w.D // 2) and np.any(rows >= w.D // 2)
    jobs = [("chunk", f"{label} vs chunk recurrence", C, y, s)
            for label, (y, s) in h.items() if s is not None]
    pool_gate(name, jobs, rows, "bf16")


@pytest.mark.parametrize("name", ["32k_chunked", "40b_shaped"])
def test_config_32k(name):
    w, d = _full(name)
    C = 1024
    res = _prefill_results(name, w, d, C)
    _check_prefill(name, w, res, C)


def test_headline_shape_deterministic():
    """Ten runs of each entry point at the 32k x 4096 shape give the same bits."""
    w, d = _full("32k_chunked")
    runs = {
        "chunk/mfma": lambda out: G.chunk_fwd(d.x1, d.x2, d.v, d.lam, d.res, 1024, d.skip,
                                              algo="mfma", out=out)[0],
        "chunk/fft": lambda out: G.chunk_fwd(d.x1, d.x2, d.v, d.lam, d.res, 1024, d.skip,
                                             algo="fft", out=out)[0],
        "fftconv": lambda out: G.fftconv_fwd(d.x1, d.x2, d.v, d.lam, d.res, d.skip, out=out),
        "fir128": lambda out: G.fir_fwd(d.x1, d.x2, d.v, d.taps[128], d.skip, out=out),
    }
    for name, run in runs.items():
        first = run(poisoned(d.x1)).view(torch.int16).clone()
        all_finite(first.view(torch.bfloat16), name)
        for rep in range(9):
            y = run(poisoned(d.x1))
            assert torch.equal(y.view(torch.int16), first), (name, rep + 1)
        log(f"  {name}: 10 runs bit-identical")


def test_scale_equivariance_40b():
    """op(s x1) = s op(x1) on the 40B-shaped workload, whose channels already
    carry x1 scales up to 1e12.  With s = 2^10, s x1 is exact in bf16 and every
    step of the operator is linear in x1, so the scaled result must pass the
    gates against s times the unscaled one."""
    w, d = _full("40b_shaped")
    s = 1024.0
    x1s = (d.x1.float() * s).to(torch.bfloat16)
    assert torch.equal(x1s.float(), d.x1.float() * s)
    ops = {
        "chunk/mfma": lambda a: G.chunk_fwd(a, d.x2, d.v, d.lam, d.res, 1024, d.skip, algo="mfma",
                                            out=poisoned(d.x1))[0],
        "chunk/fft": lambda a: G.chunk_fwd(a, d.x2, d.v, d.lam, d.res, 1024, d.skip, algo="fft",
                                           out=poisoned(d.x1))[0],
        "fftconv": lambda a: G.fftconv_fwd(a, d.x2, d.v, d.lam, d.res, d.skip, out=poisoned(d.x1)),
    }
    for name, op in ops.items():
        y = op(d.x1)
        ys = op(x1s)
        all_finite(ys, f"40b {name} scaled")
        same = int(torch.sum(ys.float() == y.float() * s).item())
        m = compare_dev(ys, y, scale=s)
        log(f"  40b {name}: op(2^10 x1) vs 2^10 op(x1): {m}, {same} of {y.numel()} identical")
        assert oracle.passes(m), (name, m)


def test_config_262k():
    # the single pass as one FFT product of length 524288, and the chunked
    # entry with chunks of 4096 tokens (both algorithms)
    w, d = _full("262k")
    C = 4096
    res = {}
    for algo in ("mfma", "fft"):
        y, st = G.chunk_fwd(d.x1, d.x2, d.v, d.lam, d.res, C, d.skip, algo=algo, out=poisoned(d.x1))
        res[f"262k chunk/{algo} C={C}"] = (y, st)
    res["262k fftconv N=524288"] = (G.fftconv_fwd(d.x1, d.x2, d.v, d.lam, d.res, d.skip,
                                                  out=poisoned(d.x1)), None)
    for label, (y, _) in res.items():
        all_finite(y, label)
    del d
    _check_prefill("262k", w, res, C, block=32)


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_misaligned_rows(io):
    """Every entry point with activations one element off 16-byte alignment
    (and L a multiple of 8, so only the alignment disables the vector paths)."""
    w = small(io, D=4, L=4096, B=2)
    d = DevWorkload(w)
    x1, x2, v = (offset_copy(t) for t in (d.x1, d.x2, d.v))
    y = offset_copy(torch.zeros_like(d.x1))
    assert x1.data_ptr() % 16 != 0 and y.data_ptr() % 16 != 0
    ref, ref_s = oracle_modal(w)
    log(f"misaligned io={io}")
    gate(G.fftconv_fwd(x1, x2, v, d.lam, d.res, d.skip, out=y), ref, io, label="fftconv misaligned")
    for algo in ("mfma", "fft"):
        yy, s = G.chunk_fwd(x1, x2, v, d.lam, d.res, 1024, d.skip, algo=algo, out=y)
        gate(yy, ref, io, label=f"chunk/{algo} misaligned")
        state_gate(s, ref_s, label=f"chunk/{algo} misaligned")
    for K in (7, 128, 200):
        taps = d.taps[K] if K in d.taps else par_to_dev(
            W.random_taps(K, w.D, seed=K, bf16=(io == "bf16")))
        tp_np = w.taps[K] if K in w.taps else taps.cpu().numpy()
        ref_f = oracle_fir(w, K, taps=tp_np)
        gate(G.fir_fwd(x1, x2, v, taps, d.skip, out=y), ref_f, io, label=f"fir{K} misaligned")
        yw, _ = G.fir_fwd_window(x1, x2, v, taps, d.skip, out=y)
        gate(yw, ref_f, io, label=f"fir{K} window misaligned")
    # the single pass in two launches (L <= 32768) and through the four-step path
    for Ll, kind in ((20000, "two-launch"), (40000, "four-step")):
        wl = small(io, D=2, L=Ll)
        dl = DevWorkload(wl)
        yl = G.fftconv_fwd(*(offset_copy(t) for t in (dl.x1, dl.x2, dl.v)), dl.lam, dl.res, dl.skip)
        gate(yl, oracle_modal(wl)[0], io, label=f"fftconv {kind} misaligned")
