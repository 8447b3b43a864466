"""Index arithmetic of the on-chip Stockham FFT (genomic_lm_amd/csrc/fft.hpp),
checked on the host for every transform shape the kernels instantiate.

The LDS exchange of each pass pads every 32-element row by one element
(lds_pad(i) = i + i/32).  The kernels compute one padded base per butterfly
and reach its other elements through constant offsets, which is valid only if
lds_pad(base + r*NS) = lds_pad(base) + r*NS + (r*NS >> 5) for all of a pass's
indices.  This test walks every thread of every pass (stores and the next
pass's loads) and checks that identity, and that the stores of a pass write
each of the S elements exactly once.
"""
import pytest


def pad(i):
    return i + (i >> 5)


def radix(S, T, NS):
    P = min(S // T, 16)
    return P if S // NS >= P else S // NS


# (S, T) of every instantiation: fftconv.hip (two-half kernels S <= 4096,
# one-half kernels S = 8192, 16384), chunk_fft.hip (S = C/2), and
# fftconv_large.hip (size-256 column transforms; row transforms S1 = 128 ..
# 1024, forward with S1/8 threads, inverse with S1/4)
SHAPES = sorted({(256, 64), (512, 64), (1024, 128), (2048, 256), (4096, 512), (8192, 512),
                 (16384, 1024),
                 (1024, 64), (2048, 128), (4096, 256),
                 (256, 32), (128, 16), (256, 32), (512, 64), (1024, 128),
                 (128, 32), (256, 64), (512, 128), (1024, 256)})


@pytest.mark.parametrize("S,T", SHAPES)
def test_pass_offsets_affine(S, T):
    P = S // T
    NS = 1
    while NS < S:
        R = radix(S, T, NS)
        NB = P // R
        written = set()
        for t in range(T):
            for b in range(NB):
                j = t + T * b
                base = (j // NS) * NS * R + (j & (NS - 1))
                for r in range(R):
                    idx = base + r * NS
                    assert pad(idx) == pad(base) + r * NS + ((r * NS) >> 5), (S, T, NS, t, b, r)
                    assert idx not in written
                    written.add(idx)
        assert len(written) == S
        if NS * R < S:
            R2 = radix(S, T, NS * R)
            Q = S // R2
            for t in range(T):
                for b in range(P // R2):
                    jp = t + T * b
                    for r in range(R2):
                        assert pad(jp + r * Q) == pad(jp) + r * Q + ((r * Q) >> 5), (S, T, NS, t, b, r)
        NS *= R


def mirror_slot(S, T, ts, i, q):
    """The kernels' LDS slot of the real-spectrum partner (fft.hpp, mirror_*)."""
    x = ts + q
    base = -x - ((x + 31) >> 5)
    C = S - T * i
    slot = base + C + (C >> 5)
    return 0 if (i == 0 and q == 0 and ts == 0) else slot


# (S, T) of the kernels that read the partner through mirror_slot:
# fftconv.hip (every S, 4 to 16 points per thread)
MIRROR_SHAPES = [(256, 64), (512, 64), (1024, 128), (2048, 256), (4096, 256), (8192, 512),
                 (16384, 1024)]


@pytest.mark.parametrize("S,T", MIRROR_SHAPES)
def test_mirror_slot(S, T):
    """mirror_slot equals lds_pad of the partner index for every thread, point
    and parity half: kk = (S - k) mod S (even half), S - 1 - k (odd half)."""
    for q in (0, 1):
        seen = set()
        for ts in range(T):
            for i in range(S // T):
                k = ts + T * i
                kk = (S - k) % S if q == 0 else S - 1 - k
                assert mirror_slot(S, T, ts, i, q) == pad(kk), (S, T, q, ts, i)
                seen.add(kk)
        assert len(seen) == S


# ---------------------------------------------------------------- matrix-core h
# fftconv.hip (modal_pairs_mfma) forms lane l's h pairs (h[2m], h[2m + 1]),
# m = t + T i, t = 64 w + l, from one 32x32x16 product per 16 modes.  The
# model below takes the product's documented lane layout (A: lane l holds row
# l % 32, K slots 8 (l / 32) .. + 7; B: lane l holds K slots 8 (l / 32) ..
# + 7 of column l % 32; result register r of lane l: row 8 (r / 4) +
# 4 (l / 32) + r % 4, column l % 32) and the kernel's exponent formulas, and
# checks that every lane and register gets the h value of its point.
def _mfma_h_model(T, w, lam, R, odd):
    import numpy as np
    N = lam.shape[0]
    A = np.zeros((32, 16))
    B = np.zeros((16, 32))
    for lane in range(64):
        hf, rho = lane >> 5, lane & 31
        xe = 64 * ((rho >> 2) & 1) + 2 * T * (4 * (rho >> 3) + (rho & 3))
        ye = 2 * ((64 * w) + rho)
        for j in range(8):
            n = 8 * hf + j
            if n < N:
                A[rho, n] = R[n] * np.exp(lam[n] * (xe + odd))
                B[n, rho] = np.exp(lam[n] * ye)
    D = A @ B
    out = np.zeros((64, 16))
    for lane in range(64):
        for r in range(16):
            out[lane, r] = D[8 * (r >> 2) + 4 * (lane >> 5) + (r & 3), lane & 31]
    return out


@pytest.mark.parametrize("T", [256, 512, 1024])
def test_mfma_h_layout(T):
    import numpy as np
    rng = np.random.default_rng(T)
    N = 16
    lam = -rng.uniform(1e-3, 1e-2, N)
    R = rng.normal(0, 0.25, N)
    for w in (0, 1, T // 64 - 1):
        for odd in (0, 1):
            got = _mfma_h_model(T, w, lam, R, odd)
            for lane in range(64):
                t = 64 * w + lane
                for i in range(16):
                    tok = 2 * (t + T * i) + odd
                    ref = float(np.sum(R * np.exp(lam * tok)))
                    assert abs(got[lane, i] - ref) <= 1e-12 * max(1.0, abs(ref)), (T, w, lane, i, odd)


def _mfma_h_model_cpx(T, w, lam, R, odd):
    """modal_pairs_mfma_cpx: K slot 8 hf + j of a lane holds mode 4 hf + j/2,
    (Re, -Im) of R p^(row exponent) in A and (Re, Im) of p^(column exponent)
    in B, so the product over slots is Re sum_n R_n p_n^(row + column)."""
    import numpy as np
    N = lam.shape[0]
    A = np.zeros((32, 16))
    B = np.zeros((16, 32))
    for lane in range(64):
        hf, rho = lane >> 5, lane & 31
        xe = 64 * ((rho >> 2) & 1) + 2 * T * (4 * (rho >> 3) + (rho & 3)) + odd
        ye = 2 * ((64 * w) + rho)
        for jj in range(4):
            n = 4 * hf + jj
            if n < N:
                x = R[n] * np.exp(lam[n] * xe)
                y = np.exp(lam[n] * ye)
                A[rho, 8 * hf + 2 * jj], A[rho, 8 * hf + 2 * jj + 1] = x.real, -x.imag
                B[8 * hf + 2 * jj, rho], B[8 * hf + 2 * jj + 1, rho] = y.real, y.imag
    D = A @ B
    out = np.zeros((64, 16))
    for lane in range(64):
        for r in range(16):
            out[lane, r] = D[8 * (r >> 2) + 4 * (lane >> 5) + (r & 3), lane & 31]
    return out


@pytest.mark.parametrize("T", [256, 1024])
def test_mfma_h_layout_cpx(T):
    import numpy as np
    rng = np.random.default_rng(T + 1)
    N = 8
    lam = -rng.uniform(1e-3, 1e-2, N) + 1j * rng.uniform(-np.pi, np.pi, N)
    R = rng.normal(0, 0.25, N) + 1j * rng.normal(0, 0.25, N)
    for w in (0, T // 64 - 1):
        for odd in (0, 1):
            got = _mfma_h_model_cpx(T, w, lam, R, odd)
            for lane in range(64):
                t = 64 * w + lane
                for i in range(16):
                    tok = 2 * (t + T * i) + odd
                    ref = float(np.sum(R * np.exp(lam * tok)).real)
                    assert abs(got[lane, i] - ref) <= 1e-12 * max(1.0, abs(ref)), (T, w, lane, i, odd)
