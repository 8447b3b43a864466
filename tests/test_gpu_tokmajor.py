"""The modal operator on in_proj's token-major layout, on the GPU, through the
C ABI, against the fp64 oracle.

xin (B, L, 3D) holds each channel's x1, x2, v side by side (triple order
`pos`), y is (B, L, D).  The cases cover both element types, both load paths
(16-byte chunks; single elements when rows are not a multiple of 16 bytes or
the input is misaligned), partial channel groups, ragged tails, every mode
count variant, carried and aliased states, and the 32 kb shape sampled; the
explicit FIR on the same layout, with its window carried between calls.
"""
import numpy as np
import pytest
import torch

import genomic_lm_amd as G
import oracle
import workloads as W
from tests.gpu_util import (DevWorkload, act_to_dev, gate, log, offset_copy, par_to_dev,
                            sample_rows, state_gate)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.lib()
    yield


def _setup(io, B, D, L, N=None, pos=(0, 1, 2)):
    w = W.make("tiny" if io == "f32" else "7b_layer_set", B=B, D=D, L=L, N=N)
    xin = W.interleave_triples(w.x1, w.x2, w.v, pos)
    return w, xin, act_to_dev(xin, w.io)


def _ref(w, xin, pos, rows=None, state_in=None):
    """Oracle on channel subset `rows`: y (B, L, len(rows)) and state."""
    rows = np.arange(w.D) if rows is None else np.asarray(rows)
    cols = (3 * rows[:, None] + np.arange(3)[None, :]).ravel()
    x = W.to_f64(xin[..., cols], w.io)
    s0 = None if state_in is None else np.asarray(state_in, np.float64)[:, rows]
    return oracle.chunk_fwd_tokmajor(x, w.log_poles[rows].astype(np.float64),
                                     w.residues[rows].astype(np.float64),
                                     w.skip[rows].astype(np.float64), pos, state_in=s0)


def _gate_tm(y_dev, ref, io, rows=None, label=""):
    """Gate a token-major output per channel: compare as (B, D, L)."""
    return gate(y_dev.transpose(1, 2), np.moveaxis(ref, 1, 2), io, rows, label=label)


def _mfma_applies(io, D, N=16):
    return io == "bf16" and D % 8 == 0 and N <= 16


@pytest.mark.parametrize("algo", ["auto", "mfma", "recurrence"])
@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("D,L", [(256, 1000), (300, 777), (64, 2048), (520, 67), (8, 5)])
@pytest.mark.parametrize("pos", [(0, 1, 2), (2, 0, 1)])
def test_tokmajor_small(io, D, L, pos, algo):
    w, xin, xd = _setup(io, B=2, D=D, L=L, pos=pos)
    d = DevWorkload(w)
    log(f"tokmajor io={io} D={D} L={L} pos={pos} algo={algo}")
    if algo == "mfma" and not _mfma_applies(io, D):
        with pytest.raises(G.HyenaError, match="UNSUPPORTED"):
            G.chunk_fwd_tokmajor(xd, d.lam, d.res, d.skip, pos=pos, algo=algo)
        return
    y, s = G.chunk_fwd_tokmajor(xd, d.lam, d.res, d.skip, pos=pos, algo=algo)
    ref, ref_s = _ref(w, xin, pos)
    assert y.shape == (2, L, D)
    _gate_tm(y, ref, io, label=f"tokmajor D={D} L={L} {algo}")
    state_gate(s, ref_s, label=f"tokmajor D={D} L={L} {algo}")


# The one-pass matrix-core evaluation: every triple order, lengths around the
# 1024-token tile (one token, partial tiles, whole tiles, one past, the
# two-tile pipeline and its odd tail), fewer modes than lanes, carried state.
@pytest.mark.parametrize("pos", [(0, 1, 2), (1, 0, 2), (2, 1, 0), (1, 2, 0)])
@pytest.mark.parametrize("L", [1, 3, 1023, 1024, 1025, 2048, 3071, 5000])
def test_tokmajor_mfma_lengths(pos, L):
    N = 16 if L != 1023 else 5
    w, xin, xd = _setup("bf16", B=1, D=16, L=L, N=N, pos=pos)
    d = DevWorkload(w)
    s0 = W.random_state(1, 16, N, seed=L)
    log(f"tokmajor mfma L={L} pos={pos}")
    y, s = G.chunk_fwd_tokmajor(xd, d.lam, d.res, d.skip, pos=pos, algo="mfma",
                                state_in=torch.from_numpy(s0).to(xd.device))
    ref, ref_s = _ref(w, xin, pos, state_in=s0)
    _gate_tm(y, ref, "bf16", label=f"tokmajor mfma L={L}")
    state_gate(s, ref_s, label=f"tokmajor mfma L={L}")


@pytest.mark.parametrize("D,algo", [(260, "auto"), (264, "mfma")])
@pytest.mark.parametrize("N", [1, 3, 8, 17, 33, 64])
def test_tokmajor_mode_counts(N, D, algo):
    """Every per-lane mode array size (8, 16, 32, 64), with padding; the
    matrix-core evaluation takes N <= 16."""
    w, xin, xd = _setup("bf16", B=1, D=D, L=2000, N=N)
    d = DevWorkload(w)
    log(f"tokmajor N={N} D={D} {algo}")
    if algo == "mfma" and N > 16:
        with pytest.raises(G.HyenaError, match="UNSUPPORTED"):
            G.chunk_fwd_tokmajor(xd, d.lam, d.res, d.skip, algo=algo)
        return
    y, s = G.chunk_fwd_tokmajor(xd, d.lam, d.res, d.skip, algo=algo)
    ref, ref_s = _ref(w, xin, (0, 1, 2))
    _gate_tm(y, ref, "bf16", label=f"tokmajor N={N}")
    state_gate(s, ref_s, label=f"tokmajor N={N}")


@pytest.mark.parametrize("io,algo", [("bf16", "auto"), ("f32", "auto"), ("bf16", "mfma")])
def test_tokmajor_state_in_and_in_place(io, algo):
    """A carried state in, updated in place (state_out is state_in)."""
    B, D, L = 2, 384, 1200
    w, xin, xd = _setup(io, B=B, D=D, L=L)
    d = DevWorkload(w)
    s0 = W.random_state(B, D, w.N, seed=3)
    s_dev = torch.from_numpy(s0).to(xd.device)
    y, s = G.chunk_fwd_tokmajor(xd, d.lam, d.res, d.skip, state_in=s_dev, state_out=s_dev,
                                algo=algo)
    assert s.data_ptr() == s_dev.data_ptr()
    ref, ref_s = _ref(w, xin, (0, 1, 2), state_in=s0)
    _gate_tm(y, ref, io, label="tokmajor state in place")
    state_gate(s, ref_s, label="tokmajor state in place")


def test_tokmajor_split_equals_whole_and_channel_major():
    """Two token-major calls with the state handed over equal one call, and
    both equal the channel-major chunk kernels on the same streams."""
    B, D, L, cut = 1, 512, 6000, 2345
    w, xin, xd = _setup("bf16", B=B, D=D, L=L, pos=(1, 2, 0))
    d = DevWorkload(w)
    ya, sa = G.chunk_fwd_tokmajor(xd[:, :cut].contiguous(), d.lam, d.res, d.skip, pos=(1, 2, 0))
    yb, sb = G.chunk_fwd_tokmajor(xd[:, cut:].contiguous(), d.lam, d.res, d.skip, pos=(1, 2, 0),
                                  state_in=sa)
    ref, ref_s = _ref(w, xin, (1, 2, 0))
    _gate_tm(torch.cat([ya, yb], 1), ref, "bf16", label="tokmajor split")
    state_gate(sb, ref_s, label="tokmajor split")
    yc, sc = G.chunk_fwd(d.x1, d.x2, d.v, d.lam, d.res, 1024, d.skip, algo="mfma")
    yt, st = G.chunk_fwd_tokmajor(xd, d.lam, d.res, d.skip, pos=(1, 2, 0))
    diff = (yc.float().transpose(1, 2) - yt.float()).abs().max().item()
    assert diff <= 2e-2 * yc.float().abs().max().item(), diff
    state_gate(st, ref_s, label="tokmajor whole")


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_tokmajor_prefill_then_decode(io):
    """Token-major prefill, then decode steps on the token's (B, D) slices."""
    B, D, L, T = 2, 256, 1500, 6
    pos = (2, 1, 0)
    w, xin, xd = _setup(io, B=B, D=D, L=L + T, pos=pos)
    d = DevWorkload(w)
    y, s = G.chunk_fwd_tokmajor(xd[:, :L].contiguous(), d.lam, d.res, d.skip, pos=pos)
    ys = [y]
    for t in range(L, L + T):
        x1, x2, v = (xd[:, t, p::3].contiguous() for p in pos)
        yt, s = G.modal_decode(x1, x2, v, d.lam, d.res, d.skip, state_in=s, state_out=s)
        ys.append(yt[:, None, :])
    ref, ref_s = _ref(w, xin, pos)
    _gate_tm(torch.cat(ys, 1), ref, io, label="tokmajor prefill + decode")
    state_gate(s, ref_s, label="tokmajor prefill + decode")


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_tokmajor_misaligned_and_tiny(io):
    """Input one element off 16-byte alignment (single-element loads), and
    L = 1 and L = 0 (the state passes through)."""
    w, xin, xd = _setup(io, B=2, D=264, L=700)
    d = DevWorkload(w)
    xm = offset_copy(xd)
    assert xm.data_ptr() % 16 != 0
    y, s = G.chunk_fwd_tokmajor(xm, d.lam, d.res, d.skip)
    ref, ref_s = _ref(w, xin, (0, 1, 2))
    _gate_tm(y, ref, io, label="tokmajor misaligned")
    state_gate(s, ref_s, label="tokmajor misaligned")
    y1, s1 = G.chunk_fwd_tokmajor(xd[:, :1].contiguous(), d.lam, d.res, d.skip, state_in=s)
    r1, rs1 = _ref(w, xin[:, :1], (0, 1, 2), state_in=s.cpu().numpy())
    _gate_tm(y1, r1, io, label="tokmajor L=1")
    state_gate(s1, rs1, label="tokmajor L=1", tol=1e-6)
    e = torch.empty((2, 0, 3 * 264), dtype=xd.dtype, device=xd.device)
    y0, s0 = G.chunk_fwd_tokmajor(e, d.lam, d.res, d.skip, state_in=s1)
    assert y0.shape == (2, 0, 264) and torch.equal(s0, s1)


@pytest.mark.parametrize("L,algo", [(32768, "auto"), (32768, "mfma"), (8192, "auto")])
def test_tokmajor_32k_shape(L, algo):
    """B = 1, D = 4096, bf16, N = 16: the 32 kb shape the benchmark times
    (AUTO takes the per-token segments there) and the matrix-core evaluation
    on it, and an 8 kb prefill, where AUTO takes the matrix cores; sampled
    channels of both halves of the channel range, every output finite."""
    w = W.make("32k_chunked", L=L)
    xin = W.interleave_triples(w.x1, w.x2, w.v)
    xd = act_to_dev(xin, "bf16")
    lam, res, skip = par_to_dev(w.log_poles), par_to_dev(w.residues), par_to_dev(w.skip)
    y = torch.full((1, L, w.D), float("nan"), dtype=torch.bfloat16, device=xd.device)
    y, s = G.chunk_fwd_tokmajor(xd, lam, res, skip, out=y, algo=algo)
    assert bool(torch.isfinite(y).all())
    rows = sample_rows(w.D, k=16)
    ref, ref_s = _ref(w, xin, (0, 1, 2), rows)
    _gate_tm(y, ref, "bf16", rows, label=f"{L} tokmajor {algo}")
    state_gate(s, ref_s, rows, label=f"{L} tokmajor {algo}")


# ------------------------------------------------------------------ FIR
def _taps(w, K, seed=None):
    if K in w.taps and seed is None:
        return w.taps[K]
    return W.random_taps(K, w.D, seed=K if seed is None else seed, bf16=(w.io == "bf16"))


def _ref_fir(w, xin, pos, taps, rows=None, window_in=None):
    rows = np.arange(w.D) if rows is None else np.asarray(rows)
    cols = (3 * rows[:, None] + np.arange(3)[None, :]).ravel()
    x = W.to_f64(xin[..., cols], w.io)
    wi = None if window_in is None else np.asarray(window_in, np.float64)[:, rows]
    return oracle.fir_fwd_tokmajor(x, np.asarray(taps, np.float64)[rows],
                                   w.skip[rows].astype(np.float64), pos, window_in=wi)


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("K", [1, 7, 20, 50, 128])
@pytest.mark.parametrize("D,L", [(256, 1000), (300, 777), (72, 3000), (40, 5)])
def test_tokmajor_fir(io, K, D, L):
    pos = (1, 0, 2)
    w, xin, xd = _setup(io, B=2, D=D, L=L, pos=pos)
    d = DevWorkload(w)
    taps = _taps(w, K)
    log(f"tokmajor fir io={io} K={K} D={D} L={L}")
    y, win = G.fir_fwd_tokmajor(xd, par_to_dev(taps), d.skip, pos=pos)
    ref, ref_w = _ref_fir(w, xin, pos, taps)
    assert y.shape == (2, L, D)
    _gate_tm(y, ref, io, label=f"tokmajor fir K={K} D={D} L={L}")
    if K > 1:
        assert np.array_equal(win.cpu().numpy(), ref_w.astype(np.float32))
    else:
        assert win is None


@pytest.mark.parametrize("K,D", [(7, 264), (128, 264), (128, 256)])
def test_tokmajor_fir_pieces_and_decode(K, D):
    """A prefill call, calls of assorted lengths and single-token steps with
    the window handed over (in place) equal one call over the sequence (D = 256:
    the 32-channel matrix-core form; 264: the 8-channel one)."""
    L = 2600
    w, xin, xd = _setup("bf16", B=1, D=D, L=L, pos=(2, 0, 1))
    d = DevWorkload(w)
    taps = par_to_dev(_taps(w, K))
    win = torch.zeros((1, w.D, K - 1), dtype=torch.float32, device=xd.device)
    # the first call spans several segments with the window updated in place
    # (written after the FIR kernel); later ones fit one segment (written by it)
    pts = [0, 2100, 2101, 2103, 2200, 2327, 2500] + list(range(2501, L + 1))
    ys = []
    for a, b in zip(pts[:-1], pts[1:]):
        yp, wo = G.fir_fwd_tokmajor(xd[:, a:b].contiguous(), taps, d.skip, pos=(2, 0, 1),
                                    window_in=win, window_out=win)
        assert wo.data_ptr() == win.data_ptr()
        ys.append(yp)
    ref, ref_w = _ref_fir(w, xin, (2, 0, 1), _taps(w, K))
    log(f"tokmajor fir pieces K={K} ({len(pts) - 1} calls)")
    _gate_tm(torch.cat(ys, 1), ref, "bf16", label=f"tokmajor fir pieces K={K}")
    assert np.array_equal(win.cpu().numpy(), ref_w.astype(np.float32))


@pytest.mark.parametrize("K", [50, 128])
def test_tokmajor_fir_fp32_taps_and_window(K):
    """Taps that are not bf16 values (their second bf16 part is not zero) and a
    window of arbitrary fp32 values, on the matrix-core path (bf16, D a
    multiple of 8, K > 32); the window comes out as [window_in, u] shifted."""
    w, xin, xd = _setup("bf16", B=2, D=64, L=3000, pos=(0, 2, 1))
    d = DevWorkload(w)
    taps = W.random_taps(K, w.D, seed=K + 7, bf16=False)
    assert not np.array_equal(W.bf16_bits_to_f32(W.f32_to_bf16_bits(taps)), taps)
    rng = np.random.default_rng(K)
    win0 = rng.standard_normal((2, w.D, K - 1)).astype(np.float32)
    wi = torch.from_numpy(win0).to(xd.device)
    log(f"tokmajor fir fp32 taps K={K}")
    for L in (3000, 40):
        y, wo = G.fir_fwd_tokmajor(xd[:, :L].contiguous(), par_to_dev(taps), d.skip, pos=(0, 2, 1),
                                   window_in=wi)
        ref, ref_w = _ref_fir(w, xin[:, :L], (0, 2, 1), taps, window_in=win0)
        _gate_tm(y, ref, "bf16", label=f"tokmajor fir fp32 taps K={K} L={L}")
        assert np.array_equal(wo.cpu().numpy(), ref_w.astype(np.float32))


@pytest.mark.parametrize("L", [5, 256, 700])
def test_tokmajor_fir_one_block(L):
    """D = 32: a single channel block; a row shorter than one 256-token tile,
    exactly one tile, and a partial second tile."""
    w, xin, xd = _setup("bf16", B=3, D=32, L=L, pos=(0, 1, 2))
    d = DevWorkload(w)
    taps = _taps(w, 128)
    y, win = G.fir_fwd_tokmajor(xd, par_to_dev(taps), d.skip, pos=(0, 1, 2))
    ref, ref_w = _ref_fir(w, xin, (0, 1, 2), taps)
    _gate_tm(y, ref, "bf16", label=f"tokmajor fir one block L={L}")
    assert np.array_equal(win.cpu().numpy(), ref_w.astype(np.float32))


@pytest.mark.parametrize("K", [33, 100, 128])
def test_tokmajor_fir_segments(K):
    """The 32-channel matrix-core form cuts the sequence into segments (here 4
    of 2304 tokens, the last one short and ending in a partial tile), each
    after the first refilling its halo from the inputs; B = 2, a window in,
    channel triples in a permuted order."""
    w, xin, xd = _setup("bf16", B=2, D=96, L=9000, pos=(2, 1, 0))
    d = DevWorkload(w)
    taps = _taps(w, K)
    rng = np.random.default_rng(K + 1)
    win0 = W.bf16_bits_to_f32(W.f32_to_bf16_bits(rng.standard_normal((2, w.D, K - 1)).astype(np.float32)))
    wi = torch.from_numpy(win0).to(xd.device)
    log(f"tokmajor fir segments K={K}")
    y, wo = G.fir_fwd_tokmajor(xd, par_to_dev(taps), d.skip, pos=(2, 1, 0), window_in=wi)
    ref, ref_w = _ref_fir(w, xin, (2, 1, 0), taps, window_in=win0)
    _gate_tm(y, ref, "bf16", label=f"tokmajor fir segments K={K}")
    assert np.array_equal(wo.cpu().numpy(), ref_w.astype(np.float32))


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_tokmajor_fir_misaligned(io):
    w, xin, xd = _setup(io, B=2, D=256, L=900)
    d = DevWorkload(w)
    xm = offset_copy(xd)
    for K in (7, 128):
        y, _ = G.fir_fwd_tokmajor(xm, par_to_dev(_taps(w, K)), d.skip)
        ref, _ = _ref_fir(w, xin, (0, 1, 2), _taps(w, K))
        _gate_tm(y, ref, io, label=f"tokmajor fir misaligned K={K}")
    with pytest.raises(G.HyenaError):
        G.fir_fwd_tokmajor(xd, par_to_dev(_taps(w, 129)), d.skip)


def test_tokmajor_fir_wide_d():
    """D = 8192 (256 blocks of 32 channels: one segment, the workgroups grouped
    in pairs per XCD), a ragged L, channels sampled over the whole width; every
    output written and finite."""
    w, xin, xd = _setup("bf16", B=1, D=8192, L=3000, pos=(1, 2, 0))
    d = DevWorkload(w)
    taps = _taps(w, 128)
    y = torch.full((1, 3000, 8192), float("nan"), dtype=torch.bfloat16, device=xd.device)
    y, win = G.fir_fwd_tokmajor(xd, par_to_dev(taps), d.skip, pos=(1, 2, 0), out=y)
    assert bool(torch.isfinite(y).all())
    rows = sample_rows(w.D, k=16)
    ref, ref_w = _ref_fir(w, xin, (1, 2, 0), taps, rows)
    _gate_tm(y, ref, "bf16", rows, label="tokmajor fir D=8192")
    assert np.array_equal(win.cpu().numpy()[:, rows], ref_w.astype(np.float32))


def test_tokmajor_fir_7b_shape():
    """D = 4096, L = 8192 (the 7B layer set), K = 7 and 128, sampled channels."""
    w = W.make("7b_layer_set")
    xin = W.interleave_triples(w.x1, w.x2, w.v)
    xd = act_to_dev(xin, "bf16")
    skip = par_to_dev(w.skip)
    rows = sample_rows(w.D)
    for K in (7, 128):
        y, win = G.fir_fwd_tokmajor(xd, par_to_dev(w.taps[K]), skip)
        ref, ref_w = _ref_fir(w, xin, (0, 1, 2), w.taps[K], rows)
        _gate_tm(y, ref, "bf16", rows, label=f"7b tokmajor fir K={K}")
        assert np.array_equal(win.cpu().numpy()[:, rows], ref_w.astype(np.float32))
