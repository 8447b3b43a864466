"""Complex-pole modal filters (Evo 1's poles / residues, in log form) on the
GPU, through the C ABI, against the fp64 oracle: the filter, the single pass
(on chip and four-step), chunked prefill with a complex state, and decode.
"""
import numpy as np
import pytest
import torch

import genomic_lm_amd as G
import oracle
import workloads as W
from tests.gpu_util import DevWorkload, gate, log, offset_copy, sample_rows, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.lib()
    yield


def _setup(io, D, L, B=1, N=8, seed=21, lam_lo=1e-3):
    w = W.make("tiny" if io == "f32" else "7b_layer_set", B=B, D=D, L=L)
    lam, R = W.complex_modes(D, N, seed, lam_lo)
    d = DevWorkload(w)
    dev = d.x1.device
    return w, d, lam, R, torch.from_numpy(lam).to(dev), torch.from_numpy(R).to(dev)


def _ref(w, lam, R, rows=None, C=None, state_in=None):
    rows = np.arange(w.D) if rows is None else np.asarray(rows)
    x1, x2, v = (w.f64(k, rows) for k in ("x1", "x2", "v"))
    s0 = None if state_in is None else state_in[:, rows]
    if C is None and s0 is None:
        y = oracle.hyena_fwd_cpx(x1, x2, v, lam[rows], R[rows], w.skip[rows])
        return y, oracle.modal_state_cpx(x1 * v, lam[rows])
    return oracle.chunk_fwd_cpx(x1, x2, v, lam[rows], R[rows], w.skip[rows], C or w.L, state_in=s0)


def _state_err(s_dev, ref):
    s = s_dev.cpu().numpy().astype(np.complex128)
    num = np.sqrt(np.sum(np.abs(s - ref) ** 2, axis=-1))
    den = np.sqrt(np.sum(np.abs(ref) ** 2, axis=-1))
    return float(np.sqrt(np.mean((num / np.where(den > 0, den, 1)) ** 2)))


@pytest.mark.parametrize("L", [1, 777, 8192, 40000])
def test_modal_filter_cpx(L):
    w, d, lam, R, lam_d, R_d = _setup("f32", D=16, L=8)
    log(f"modal_filter_cpx L={L}")
    h = to_f64(G.modal_filter_cpx(lam_d, R_d, L))
    ref = oracle.modal_filter_cpx(lam, R, L)
    err = np.sqrt(np.sum((h - ref) ** 2, -1) / np.sum(ref ** 2, -1))
    assert np.max(err) < 2e-5, err


@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("L", [100, 1024, 3001, 16384, 20001, 24000, 40000])
def test_fftconv_cpx(io, L):
    w, d, lam, R, lam_d, R_d = _setup(io, D=4, L=L, B=2 if L < 5000 else 1)
    log(f"fftconv_cpx io={io} L={L}")
    y = G.fftconv_fwd_cpx(d.x1, d.x2, d.v, lam_d, R_d, d.skip)
    ref, _ = _ref(w, lam, R)
    gate(y, ref, io, label=f"fftconv_cpx L={L}")


# The split single pass (L > 4096) forms h on the matrix cores, 8 complex
# modes (16 product slots) per block: counts on both sides of a block
# boundary and up to 32 modes, both split sizes, bf16 and fp32 rows, and a
# slow decay range (|Re log p| down to 1e-5).
@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("L", [5000, 20001])
@pytest.mark.parametrize("N", [1, 7, 8, 9, 17, 32])
def test_fftconv_cpx_split_mode_counts(N, L, io):
    w, d, lam, R, lam_d, R_d = _setup(io, D=3, L=L, N=N, seed=40 + N)
    log(f"fftconv_cpx split modes N={N} L={L} io={io}")
    y = G.fftconv_fwd_cpx(d.x1, d.x2, d.v, lam_d, R_d, d.skip)
    ref, _ = _ref(w, lam, R)
    gate(y, ref, io, label=f"fftconv_cpx N={N} L={L}")


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_fftconv_cpx_split_slow_modes(io):
    w, d, lam, R, lam_d, R_d = _setup(io, D=4, L=32768, N=8, seed=77, lam_lo=1e-5)
    log(f"fftconv_cpx split slow modes io={io}")
    y = G.fftconv_fwd_cpx(d.x1, d.x2, d.v, lam_d, R_d, d.skip)
    ref, _ = _ref(w, lam, R)
    gate(y, ref, io, label="fftconv_cpx slow modes")


@pytest.mark.parametrize("algo", ["fft", "mfma"])
@pytest.mark.parametrize("io", ["bf16", "f32"])
@pytest.mark.parametrize("C,L", [(64, 1000), (1024, 3000), (1000, 4096), (4096, 9000), (8192, 8192)])
@pytest.mark.parametrize("with_state", [False, True])
def test_chunk_cpx(algo, io, C, L, with_state):
    w, d, lam, R, lam_d, R_d = _setup(io, D=4, L=L, B=2)
    s0 = W.random_complex_state(2, w.D, 8, seed=C) if with_state else None
    s0_d = None if s0 is None else torch.from_numpy(s0).to(d.x1.device)
    log(f"chunk_cpx {algo} io={io} C={C} L={L} state={with_state}")
    y, s = G.chunk_fwd_cpx(d.x1, d.x2, d.v, lam_d, R_d, C, d.skip, state_in=s0_d, algo=algo)
    ref, ref_s = _ref(w, lam, R, C=C, state_in=s0)
    gate(y, ref, io, label=f"chunk_cpx {algo} C={C}")
    err = _state_err(s, ref_s)
    log(f"  state rel_l2_ch={err:.3e}")
    assert err < 1e-4


@pytest.mark.parametrize("N", [1, 3, 5, 8, 9, 12, 16, 17])
def test_chunk_cpx_mode_counts(N):
    """Complex mode counts through AUTO: N <= 16 on the matrix cores (padding
    slots included; 9 to 16 on the 32-slot form), N = 17 on the FFT
    algorithm; and the unaligned path."""
    w, d, lam, R, lam_d, R_d = _setup("bf16", D=6, L=2500, B=1, N=N, seed=30 + N)
    log(f"chunk_cpx auto N={N}")
    y, s = G.chunk_fwd_cpx(d.x1, d.x2, d.v, lam_d, R_d, 1024, d.skip)
    ref, ref_s = _ref(w, lam, R)
    gate(y, ref, "bf16", label=f"chunk_cpx auto N={N}")
    assert _state_err(s, ref_s) < 1e-4
    if N <= 16:
        y2, s2 = G.chunk_fwd_cpx(*(offset_copy(t) for t in (d.x1, d.x2, d.v)), lam_d, R_d, 1000,
                                 d.skip, algo="mfma")
        gate(y2, ref, "bf16", label=f"chunk_cpx mfma unaligned N={N}")
        assert _state_err(s2, ref_s) < 1e-4
    else:
        with pytest.raises(G.HyenaError):
            G.chunk_fwd_cpx(d.x1, d.x2, d.v, lam_d, R_d, 1024, d.skip, algo="mfma")


@pytest.mark.parametrize("algo", ["fft", "mfma"])
@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_decode_cpx_after_prefill(algo, io):
    L, T = 3000, 16
    w, d, lam, R, lam_d, R_d = _setup(io, D=16, L=L + T, B=2)
    pre = [t[..., :L].contiguous() for t in (d.x1, d.x2, d.v)]
    y_pre, s = G.chunk_fwd_cpx(*pre, lam_d, R_d, 1024, d.skip, algo=algo)
    ys = [y_pre]
    for t in range(L, L + T):
        yt, s = G.modal_decode_cpx(d.x1[..., t].contiguous(), d.x2[..., t].contiguous(),
                                   d.v[..., t].contiguous(), lam_d, R_d, d.skip,
                                   state_in=s, state_out=s)
        ys.append(yt[..., None])
    ref, ref_s = _ref(w, lam, R)
    gate(torch.cat(ys, -1), ref, io, label="cpx prefill+decode")
    assert _state_err(s, ref_s) < 1e-4


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_decode_cpx_long_run(io):
    """4096 one-token steps from a zero state (and the FFT chunk algorithm with
    C = 1): the complex pole is applied as an fp32 pair, so its rounding does
    not compound over a slow mode's memory.  What remains is the unbiased
    rounding of each step's complex product (state ~1e-5 after 4096 steps,
    inside the state tolerance of 1e-4)."""
    w, d, lam, R, lam_d, R_d = _setup(io, D=4, L=4096, B=1)
    log(f"decode_cpx long run io={io}")
    s = torch.zeros((1, w.D, 8), dtype=torch.complex64, device=d.x1.device)
    y = torch.empty_like(d.x1)
    for t in range(w.L):
        yt, s = G.modal_decode_cpx(d.x1[..., t].contiguous(), d.x2[..., t].contiguous(),
                                   d.v[..., t].contiguous(), lam_d, R_d, d.skip,
                                   state_in=s, state_out=s)
        y[..., t] = yt
    ref, ref_s = _ref(w, lam, R)
    gate(y, ref, io, label="decode_cpx x4096")
    assert _state_err(s, ref_s) < 1e-4
    y1, s1 = G.chunk_fwd_cpx(d.x1, d.x2, d.v, lam_d, R_d, 1, d.skip, algo="fft")
    gate(y1, ref, io, label="chunk_cpx fft C=1")
    assert _state_err(s1, ref_s) < 1e-4


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_cpx_misaligned_rows(io):
    """Complex entry points with activations one element off 16-byte alignment,
    on chip, in two launches and four-step, then a decode step from offset
    single tokens."""
    for L in (4096, 20000, 40000):
        w, d, lam, R, lam_d, R_d = _setup(io, D=4, L=L, B=2 if L < 5000 else 1)
        x1, x2, v = (offset_copy(t) for t in (d.x1, d.x2, d.v))
        assert x1.data_ptr() % 16 != 0
        ref, ref_s = _ref(w, lam, R)
        log(f"cpx misaligned io={io} L={L}")
        gate(G.fftconv_fwd_cpx(x1, x2, v, lam_d, R_d, d.skip), ref, io, label="fftconv_cpx misaligned")
        if L > 8192:
            continue
        n = L - 1
        pre = [offset_copy(t[..., :n].contiguous()) for t in (d.x1, d.x2, d.v)]
        y, s = G.chunk_fwd_cpx(*pre, lam_d, R_d, 1024, d.skip)
        tok = [offset_copy(t[..., n].contiguous()) for t in (d.x1, d.x2, d.v)]
        yt, s = G.modal_decode_cpx(*tok, lam_d, R_d, d.skip, state_in=s)
        gate(torch.cat([y, yt[..., None]], -1), ref, io, label="chunk_cpx + decode_cpx misaligned")
        assert _state_err(s, ref_s) < 1e-4


def test_cpx_with_real_modes_matches_real_entries():
    """Zero imaginary parts: the complex entry points equal the real ones."""
    w = W.make("7b_layer_set", D=8, L=5000)
    d = DevWorkload(w)
    lam_c = torch.complex(d.lam, torch.zeros_like(d.lam))
    R_c = torch.complex(d.res, torch.zeros_like(d.res))
    lam_c, R_c = lam_c[:, :8].contiguous(), R_c[:, :8].contiguous()   # MFMA: <= 8 complex
    lam8, res8 = d.lam[:, :8].contiguous(), d.res[:, :8].contiguous()
    ref = oracle.hyena_fwd(w.f64("x1"), w.f64("x2"), w.f64("v"), w.log_poles[:, :8],
                           w.residues[:, :8], w.skip)
    for name, y in (
        ("fftconv", G.fftconv_fwd_cpx(d.x1, d.x2, d.v, lam_c, R_c, d.skip)),
        ("chunk", G.chunk_fwd_cpx(d.x1, d.x2, d.v, lam_c, R_c, 1024, d.skip, algo="fft")[0]),
        ("chunk_mfma", G.chunk_fwd_cpx(d.x1, d.x2, d.v, lam_c, R_c, 1024, d.skip,
                                       algo="mfma")[0]),
    ):
        gate(y, ref, "bf16", label=f"real modes via {name}_cpx")
        y_real = (G.fftconv_fwd(d.x1, d.x2, d.v, lam8, res8, d.skip) if name == "fftconv"
                  else G.chunk_fwd(d.x1, d.x2, d.v, lam8, res8, 1024, d.skip,
                                   algo="mfma" if name == "chunk_mfma" else "fft")[0])
        diff = (y.float() - y_real.float()).abs().max().item()
        assert diff <= 2e-2 * y_real.float().abs().max().item(), (name, diff)


def test_cpx_7b_shape():
    """D = 4096, L = 8192, N = 8 complex modes: single pass and chunked, sampled rows."""
    w = W.make("7b_layer_set")
    lam, R = W.complex_modes(w.D, 8, seed=77)
    d = DevWorkload(w)
    lam_d, R_d = torch.from_numpy(lam).to(d.x1.device), torch.from_numpy(R).to(d.x1.device)
    rows = sample_rows(w.D)
    ref, ref_s = _ref(w, lam, R, rows)
    gate(G.fftconv_fwd_cpx(d.x1, d.x2, d.v, lam_d, R_d, d.skip), ref, "bf16", rows,
         label="7b cpx fftconv")
    for algo in ("fft", "mfma"):
        y, s = G.chunk_fwd_cpx(d.x1, d.x2, d.v, lam_d, R_d, 1024, d.skip, algo=algo)
        gate(y, ref, "bf16", rows, label=f"7b cpx chunk {algo}")
        assert _state_err(s[:, torch.as_tensor(rows, device=s.device)], ref_s) < 1e-4
