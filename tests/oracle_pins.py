"""Pins of the fp64 oracle against facts other than itself.

Each pin takes the oracle module (or a stand-in with the same functions) and
raises AssertionError when the oracle disagrees with:

* hand-worked values (tests/golden/hand_worked.json);
* exact rational brute force (fractions.Fraction) on tiny inputs;
* closed forms: the geometric-series DFT of the modal filter, the per-mode
  recurrence s(t) = p s(t-1) + u(t), the impulse response;
* invariants: linearity, time invariance, scale equivariance, chunked == full;
* a textbook routine: numpy.convolve.

The same pins are run against oracles with a planted mistake to show that each
plausible mistake is caught (tests/test_oracle_pins.py).
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _rng(seed):
    return np.random.default_rng(seed)


def _params(rng, D, N, lam_lo=1e-3):
    lam = -np.exp(rng.uniform(math.log(lam_lo), 0.0, (D, N)))
    R = rng.normal(0, 0.25, (D, N))
    return lam, R


# ---------------------------------------------------------------- golden
def pin_golden(O):
    with open(GOLDEN) as f:
        g = json.load(f)
    for c in g["modal_cases"]:
        lam = np.log(np.array(c["poles"]))[None, :]
        R = np.array(c["residues"])[None, :]
        sh = lambda a: np.array(a, dtype=np.float64)[None, None, :]
        x1, v, x2 = sh(c["x1"]), sh(c["v"]), sh(c["x2"])
        skip = np.array([c["skip"]])
        y = O.hyena_fwd(x1, x2, v, lam, R, skip)
        assert np.allclose(y[0, 0], c["y"], rtol=0, atol=1e-13), (c["name"], y, c["y"])
        s = O.modal_state(x1 * v, lam)
        assert np.allclose(s[0, 0], c["state"], rtol=0, atol=1e-13), (c["name"], s)
        L = len(c["x1"])
        for C in (1, L, c.get("chunk", 2)):
            yc, sc = O.chunk_fwd(x1, x2, v, lam, R, skip, C)
            assert np.allclose(yc[0, 0], c["y"], rtol=0, atol=1e-13), (c["name"], C, yc)
            assert np.allclose(sc[0, 0], c["state"], rtol=0, atol=1e-13), (c["name"], C, sc)
        if "chunk" in c:
            half = c["chunk"]
            _, s1 = O.chunk_fwd(x1[..., :half], x2[..., :half], v[..., :half],
                                lam, R, skip, half)
            assert np.allclose(s1[0, 0], c["state_after_first_chunk"], rtol=0, atol=1e-13)
    for c in g["fir_cases"]:
        sh = lambda a: np.array(a, dtype=np.float64)[None, None, :]
        y = O.fir_fwd(sh(c["x1"]), sh(c["x2"]), sh(c["v"]),
                      np.array(c["taps"], dtype=np.float64)[None, :],
                      np.array([c["skip"]]))
        assert np.allclose(y[0, 0], c["y"], rtol=0, atol=1e-13), (c["name"], y)


# ---------------------------------------------------------------- filter
def pin_filter_rational(O):
    """h = sum_n R_n p_n^t with rational p_n, R_n, against exact fractions."""
    poles = [Fraction(1, 2), Fraction(3, 4), Fraction(7, 8), Fraction(1, 16)]
    res = [Fraction(1), Fraction(-3, 2), Fraction(5, 4), Fraction(2)]
    L = 40
    lam = np.log(np.array([float(p) for p in poles]))[None, :]
    R = np.array([float(r) for r in res])[None, :]
    h = O.modal_filter(lam, R, L)[0]
    for t in range(L):
        exact = sum(r * p ** t for r, p in zip(res, poles))
        scale = sum(abs(r) * p ** t for r, p in zip(res, poles))
        assert abs(h[t] - float(exact)) <= 1e-13 * float(scale), (t, h[t], float(exact))
    assert h[0] == float(sum(res))


def pin_filter_dft(O):
    """Geometric series: DFT_2L of h[0:L] = sum_n R_n (1 - p^L w^(kL)) / (1 - p w^k)."""
    rng = _rng(11)
    D, N, L = 3, 16, 512
    lam, R = _params(rng, D, N)
    h = O.modal_filter(lam, R, L)
    n = 2 * L
    H = np.fft.rfft(h, n=n, axis=-1)
    k = np.arange(n // 2 + 1)
    w = np.exp(-2j * np.pi * k / n)
    p = np.exp(lam)
    closed = np.zeros((D, k.size), dtype=complex)
    for m in range(N):
        pm = p[:, m:m + 1]
        closed += R[:, m:m + 1] * (1 - pm ** L * (-1.0) ** k) / (1 - pm * w[None])
    err = np.linalg.norm(H - closed) / np.linalg.norm(closed)
    assert err < 1e-11, err


def pin_recurrence(O):
    """Per-mode recurrence s(t) = p s(t-1) + u(t) and z(t) = sum_n R_n s_n(t)."""
    rng = _rng(12)
    B, D, N, L = 2, 3, 5, 300
    lam, R = _params(rng, D, N)
    x1 = rng.normal(size=(B, D, L))
    v = rng.normal(size=(B, D, L))
    u = x1 * v
    p = np.exp(lam)
    s = np.zeros((B, D, N))
    z = np.zeros((B, D, L))
    for t in range(L):
        s = p[None] * s + u[:, :, t:t + 1]
        z[:, :, t] = np.sum(R[None] * s, axis=-1)
    y = O.hyena_fwd(x1, np.ones_like(x1), v, lam, R, np.zeros(D))
    assert np.max(np.abs(y - z)) <= 1e-11 * np.max(np.abs(z)), np.max(np.abs(y - z))
    s_or = O.modal_state(u, lam)
    assert np.max(np.abs(s_or - s)) <= 1e-11 * np.max(np.abs(s))


# ---------------------------------------------------------------- conv
def pin_impulse(O):
    rng = _rng(13)
    D, N, L = 4, 16, 700
    lam, R = _params(rng, D, N)
    h = O.modal_filter(lam, R, L)
    for t0 in (0, 1, 333, L - 1):
        x1 = np.zeros((1, D, L))
        x1[..., t0] = 1.0
        y = O.hyena_fwd(x1, np.ones_like(x1), np.ones_like(x1), lam, R, np.zeros(D))
        assert np.all(y[..., :t0] == 0.0), t0
        assert np.allclose(y[0, :, t0:], h[:, :L - t0], rtol=1e-12, atol=1e-14), t0
        taps = rng.normal(size=(D, 9))
        yf = O.fir_fwd(x1, np.ones_like(x1), np.ones_like(x1), taps, np.zeros(D))
        assert np.all(yf[..., :t0] == 0.0)
        m = min(9, L - t0)
        assert np.array_equal(yf[0, :, t0:t0 + m], taps[:, :m])


def pin_linearity_time_invariance(O):
    rng = _rng(14)
    D, N, L = 3, 16, 1500
    lam, R = _params(rng, D, N)
    skip = rng.normal(size=D)
    x1a, x1b = rng.normal(size=(2, 1, D, L))
    x2 = rng.normal(size=(1, D, L))
    v = rng.normal(size=(1, D, L))
    a, b = 0.7, -1.9
    f = lambda x: O.hyena_fwd(x, x2, v, lam, R, skip)
    lhs = f(a * x1a + b * x1b)
    rhs = a * f(x1a) + b * f(x1b)
    assert np.max(np.abs(lhs - rhs)) <= 1e-12 * np.max(np.abs(rhs))
    # time invariance of the filter part (x2 = 1, v = 1): shifting u shifts z
    sh = 57
    g = lambda x: O.hyena_fwd(x, np.ones_like(x), np.ones_like(x), lam, R, np.zeros(D))
    xs = np.zeros_like(x1a)
    xs[..., sh:] = x1a[..., :L - sh]
    assert np.allclose(g(xs)[..., sh:], g(x1a)[..., :L - sh], rtol=1e-11, atol=1e-11)
    assert np.all(g(xs)[..., :sh] == 0)


def pin_numpy_convolve(O):
    rng = _rng(15)
    D, N = 2, 16
    for L in (1, 2, 17, 999, 5000):
        lam, R = _params(rng, D, N)
        x1 = rng.normal(size=(1, D, L))
        y = O.hyena_fwd(x1, np.ones_like(x1), np.ones_like(x1), lam, R, np.zeros(D))
        h = O.modal_filter(lam, R, L)
        for c in range(D):
            ref = np.convolve(x1[0, c], h[c])[:L]
            assert np.allclose(y[0, c], ref, rtol=1e-10, atol=1e-10 * np.max(np.abs(ref))), (L, c)
        for K in (1, 7, 128):
            taps = rng.normal(size=(D, K))
            yf = O.fir_fwd(x1, np.ones_like(x1), np.ones_like(x1), taps, np.zeros(D))
            for c in range(D):
                ref = np.convolve(x1[0, c], taps[c])[:L]
                assert np.allclose(yf[0, c], ref, rtol=1e-12, atol=1e-12), (L, K, c)


def pin_direct_vs_fft(O):
    rng = _rng(16)
    u = rng.normal(size=(2, 3, 3000))
    h = rng.normal(size=(3, 3000)) * np.exp(-np.arange(3000) / 500.0)
    a = O.conv_direct(u, h[None])
    b = O.conv_fft(u, h[None])
    assert np.max(np.abs(a - b)) <= 1e-12 * np.max(np.abs(a))
    hs = rng.normal(size=(3, 7))
    assert np.max(np.abs(O.conv_direct(u, hs[None]) - O.conv_fft(u, hs[None]))) < 1e-12


def pin_fraction_bruteforce(O):
    """Exact rational evaluation of the gated FIR operator on a tiny input."""
    rng = _rng(17)
    L, K = 9, 4
    q = lambda: Fraction(int(rng.integers(-8, 9)), int(rng.integers(1, 5)))
    x1 = [q() for _ in range(L)]
    v = [q() for _ in range(L)]
    x2 = [q() for _ in range(L)]
    w = [q() for _ in range(K)]
    sk = q()
    u = [a * b for a, b in zip(x1, v)]
    y = []
    for t in range(L):
        z = sum((w[k] * u[t - k] for k in range(K) if t - k >= 0), Fraction(0))
        y.append(x2[t] * z + sk * u[t])
    f = lambda a: np.array([float(x) for x in a])[None, None, :]
    yo = O.fir_fwd(f(x1), f(x2), f(v), np.array([float(x) for x in w])[None], np.array([float(sk)]))
    assert np.allclose(yo[0, 0], [float(x) for x in y], rtol=1e-15, atol=1e-15)


# ---------------------------------------------------------------- gate
def pin_gate_special(O):
    rng = _rng(18)
    D, N, L = 3, 16, 200
    lam, _ = _params(rng, D, N)
    x1, x2, v = rng.normal(size=(3, 2, D, L))
    skip = rng.normal(size=D)
    y = O.hyena_fwd(x1, x2, v, lam, np.zeros((D, N)), skip)
    assert np.array_equal(y, skip[None, :, None] * (x1 * v))
    _, R = _params(rng, D, N)
    y0 = O.hyena_fwd(x1, np.zeros_like(x2), v, lam, R, skip)
    assert np.array_equal(y0, skip[None, :, None] * (x1 * v))


def pin_fir_delta(O):
    rng = _rng(19)
    D, L = 3, 300
    x1, x2, v = rng.normal(size=(3, 1, D, L))
    skip = rng.normal(size=D)
    u = x1 * v
    for K, lag in ((1, 0), (7, 3), (128, 127), (128, 5)):
        taps = np.zeros((D, K))
        taps[:, lag] = 1.0
        y = O.fir_fwd(x1, x2, v, taps, skip)
        us = np.zeros_like(u)
        us[..., lag:] = u[..., :L - lag]
        assert np.array_equal(y, x2 * us + skip[None, :, None] * u), (K, lag)


# ---------------------------------------------------------------- chunked
def pin_chunk_equals_full(O):
    rng = _rng(20)
    B, D, N, L = 2, 3, 16, 777
    lam, R = _params(rng, D, N)
    x1, x2, v = rng.normal(size=(3, B, D, L))
    skip = rng.normal(size=D)
    yf = O.hyena_fwd(x1, x2, v, lam, R, skip)
    sf = O.modal_state(x1 * v, lam)
    for C in (1, 2, 64, 100, 256, L, 1000):
        yc, sc = O.chunk_fwd(x1, x2, v, lam, R, skip, C)
        assert np.max(np.abs(yc - yf)) <= 1e-10 * np.max(np.abs(yf)), C
        assert np.max(np.abs(sc - sf)) <= 1e-10 * np.max(np.abs(sf)), C


def pin_chunk_resume(O):
    """Split anywhere, hand the state over, continue: equals the single call."""
    rng = _rng(21)
    B, D, N, L = 1, 3, 16, 600
    lam, R = _params(rng, D, N)
    x1, x2, v = rng.normal(size=(3, B, D, L))
    skip = rng.normal(size=D)
    s0 = rng.normal(size=(B, D, N))
    y_all, s_all = O.chunk_fwd(x1, x2, v, lam, R, skip, 128, state_in=s0)
    for cut in (128, 256, 301):
        ya, sa = O.chunk_fwd(x1[..., :cut], x2[..., :cut], v[..., :cut], lam, R, skip, 128, state_in=s0)
        yb, sb = O.chunk_fwd(x1[..., cut:], x2[..., cut:], v[..., cut:], lam, R, skip, 128, state_in=sa)
        y = np.concatenate([ya, yb], axis=-1)
        assert np.max(np.abs(y - y_all)) <= 1e-10 * np.max(np.abs(y_all)), cut
        assert np.max(np.abs(sb - s_all)) <= 1e-10 * np.max(np.abs(s_all)), cut
    # a non-zero initial state adds sum_n R_n p_n^(t+1) s0_n to z
    y_zero, _ = O.chunk_fwd(x1, x2, v, lam, R, skip, 128)
    t = np.arange(L)
    extra = np.einsum("dn,bdn,dnt->bdt", R, s0, np.exp(lam[:, :, None] * (t + 1)))
    assert np.allclose(y_all - y_zero, x2 * extra, rtol=1e-9, atol=1e-9)


def pin_chunk_state_rational(O):
    """state_out = p^L s_in + sum_k p^(L-1-k) u[k], exactly, with rational p."""
    poles = [Fraction(1, 2), Fraction(3, 4), Fraction(5, 8)]
    L, C = 11, 4
    rng = _rng(22)
    u = [Fraction(int(rng.integers(-5, 6)), int(rng.integers(1, 4))) for _ in range(L)]
    s0 = [Fraction(1, 3), Fraction(-2), Fraction(3, 2)]
    exact = [p ** L * s + sum(p ** (L - 1 - k) * u[k] for k in range(L)) for p, s in zip(poles, s0)]
    lam = np.log(np.array([float(p) for p in poles]))[None]
    x1 = np.array([float(x) for x in u])[None, None]
    ones = np.ones_like(x1)
    _, s = O.chunk_fwd(x1, ones, ones, lam, np.ones((1, 3)), None, C,
                       state_in=np.array([float(x) for x in s0])[None, None])
    assert np.allclose(s[0, 0], [float(e) for e in exact], rtol=1e-13, atol=1e-13), (s, exact)


def pin_scale_equivariance(O):
    rng = _rng(23)
    D, N, L = 4, 16, 512
    lam, R = _params(rng, D, N)
    x1, x2, v = rng.normal(size=(3, 1, D, L))
    skip = rng.normal(size=D)
    sc = np.exp(rng.uniform(0, math.log(1e12), D))
    y = O.hyena_fwd(x1, x2, v, lam, R, skip)
    ys = O.hyena_fwd(x1 * sc[None, :, None], x2, v, lam, R, skip)
    ref = y * sc[None, :, None]
    err = np.max(np.abs(ys - ref), axis=-1) / np.max(np.abs(ref), axis=-1)
    assert np.all(err <= 1e-12), err


# ---------------------------------------------------------------- decode / caches
def pin_decode_after_prefill(O):
    """Prefill L tokens, then decode T more one at a time from the cached
    state: equals the single-pass operator over all L + T tokens (computed by
    the convolution, not the recurrence)."""
    rng = _rng(30)
    B, D, N, L, T = 2, 3, 16, 300, 40
    lam, R = _params(rng, D, N)
    x1, x2, v = rng.normal(size=(3, B, D, L + T))
    skip = rng.normal(size=D)
    y_full = O.hyena_fwd(x1, x2, v, lam, R, skip)
    y_pre, s = O.chunk_fwd(x1[..., :L], x2[..., :L], v[..., :L], lam, R, skip, 128)
    ys = [y_pre]
    for t in range(L, L + T):
        yt, s = O.modal_decode(x1[..., t], x2[..., t], v[..., t], lam, R, skip, state_in=s)
        ys.append(yt[..., None])
    y = np.concatenate(ys, axis=-1)
    assert np.max(np.abs(y - y_full)) <= 1e-10 * np.max(np.abs(y_full))
    # decoding from an empty prefix
    s = None
    for t in range(T):
        yt, s = O.modal_decode(x1[..., t], x2[..., t], v[..., t], lam, R, skip, state_in=s)
        ref = O.hyena_fwd(x1[..., :t + 1], x2[..., :t + 1], v[..., :t + 1], lam, R, skip)[..., t]
        assert np.max(np.abs(yt - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref))), t


def pin_decode_impulse_rational(O):
    """A unit impulse decoded step by step gives h[t] = sum_n R_n p_n^t exactly
    (rational poles and residues, fractions.Fraction)."""
    poles = [Fraction(1, 2), Fraction(3, 4), Fraction(5, 8)]      # p = exp(lam) > 0
    res = [Fraction(1), Fraction(-2, 3), Fraction(5, 4)]
    lam = np.log(np.array([float(p) for p in poles]))[None]
    R = np.array([float(r) for r in res])[None]
    s = None
    for t in range(12):
        one = np.array([[1.0 if t == 0 else 0.0]])
        yt, s = O.modal_decode(one, np.ones((1, 1)), np.ones((1, 1)), lam, R, None, state_in=s)
        exact = sum(r * p ** t for r, p in zip(res, poles))
        assert abs(yt[0, 0] - float(exact)) <= 1e-14, (t, yt, exact)


def pin_fir_window_pieces(O):
    """An FIR sequence cut into pieces of any length (shorter than K-1 too,
    single tokens too), the window handed over between calls, equals one call
    over the whole sequence; the final window is the last K-1 values of u."""
    rng = _rng(31)
    B, D, L = 2, 3, 300
    x1, x2, v = rng.normal(size=(3, B, D, L))
    skip = rng.normal(size=D)
    for K in (1, 2, 7, 33):
        w = rng.normal(size=(D, K))
        y_full = O.fir_fwd(x1, x2, v, w, skip)
        for cuts in ([0, 100, L], [0, 1, 2, 3, 5, 40, 41, 200, L], list(range(0, L + 1, 7)) + [L]):
            cuts = sorted(set(cuts))
            win, ys = None, []
            for a, b in zip(cuts[:-1], cuts[1:]):
                yp, win = O.fir_fwd_window(x1[..., a:b], x2[..., a:b], v[..., a:b], w, skip,
                                           window_in=win)
                ys.append(yp)
            y = np.concatenate(ys, axis=-1)
            assert np.max(np.abs(y - y_full)) <= 1e-12 * np.max(np.abs(y_full)), (K, cuts[:4])
            assert win.shape == (B, D, K - 1)
            assert np.array_equal(win, (x1 * v)[..., L - (K - 1):]), K


# ---------------------------------------------------------------- complex poles
def _cparams(rng, D, N, lam_lo=1e-3):
    a = -np.exp(rng.uniform(math.log(lam_lo), 0.0, (D, N)))
    b = rng.uniform(-math.pi, math.pi, (D, N))
    R = rng.normal(0, 0.25, (D, N)) + 1j * rng.normal(0, 0.25, (D, N))
    return a + 1j * b, R


def _gmul(x, y):
    return (x[0] * y[0] - x[1] * y[1], x[0] * y[1] + x[1] * y[0])


def pin_cpx_filter_rational(O):
    """h[t] = Re sum_n R_n p_n^t with Gaussian-rational poles and residues,
    computed exactly with fractions.Fraction pairs."""
    poles = [(Fraction(1, 2), Fraction(1, 3)), (Fraction(-3, 4), Fraction(1, 8)),
             (Fraction(2, 5), Fraction(-3, 5))]
    res = [(Fraction(1), Fraction(-1, 2)), (Fraction(2, 3), Fraction(1, 4)),
           (Fraction(-5, 4), Fraction(3, 2))]
    lam = np.log(np.array([complex(float(a), float(b)) for a, b in poles]))[None]
    R = np.array([complex(float(a), float(b)) for a, b in res])[None]
    h = O.modal_filter_cpx(lam, R, 14)
    for t in range(14):
        tot = Fraction(0)
        for p, r in zip(poles, res):
            pt = (Fraction(1), Fraction(0))
            for _ in range(t):
                pt = _gmul(pt, p)
            tot += _gmul(r, pt)[0]
        assert abs(h[0, t] - float(tot)) <= 1e-14 * max(1.0, abs(float(tot))), (t, h[0, t], tot)


def pin_cpx_second_order_recurrence(O):
    """One complex mode p = r e^(i th) gives a real filter obeying
    h[t] = 2 r cos(th) h[t-1] - r^2 h[t-2]."""
    rng = _rng(40)
    lam, R = _cparams(rng, 3, 1)
    h = O.modal_filter_cpx(lam, R, 300)
    r = np.exp(lam.real)[:, 0]
    th = lam.imag[:, 0]
    pred = 2 * r[:, None] * np.cos(th)[:, None] * h[:, 1:-1] - (r ** 2)[:, None] * h[:, :-2]
    assert np.max(np.abs(pred - h[:, 2:])) <= 1e-12 * np.max(np.abs(h))


def pin_cpx_real_special_case(O):
    """Complex modes with zero imaginary parts give the real-mode operator,
    state and decode step."""
    rng = _rng(41)
    B, D, N, L = 2, 3, 16, 400
    lam, R = _params(rng, D, N)
    x1, x2, v = rng.normal(size=(3, B, D, L))
    skip = rng.normal(size=D)
    y_r = O.hyena_fwd(x1, x2, v, lam, R, skip)
    y_c = O.hyena_fwd_cpx(x1, x2, v, lam + 0j, R + 0j, skip)
    assert np.max(np.abs(y_c - y_r)) <= 1e-12 * np.max(np.abs(y_r))
    yc_r, s_r = O.chunk_fwd(x1, x2, v, lam, R, skip, 128)
    yc_c, s_c = O.chunk_fwd_cpx(x1, x2, v, lam + 0j, R + 0j, skip, 128)
    assert np.max(np.abs(yc_c - yc_r)) <= 1e-12 * np.max(np.abs(yc_r))
    assert np.max(np.abs(s_c.imag)) == 0.0
    assert np.max(np.abs(s_c.real - s_r)) <= 1e-12 * np.max(np.abs(s_r))
    yd_r, sd_r = O.modal_decode(x1[..., 0], x2[..., 0], v[..., 0], lam, R, skip, state_in=s_r)
    yd_c, sd_c = O.modal_decode_cpx(x1[..., 0], x2[..., 0], v[..., 0], lam + 0j, R + 0j, skip,
                                    state_in=s_c)
    assert np.max(np.abs(yd_c - yd_r)) <= 1e-12 * np.max(np.abs(yd_r))


def pin_cpx_chunk_and_decode_equal_full(O):
    """Complex modes: chunked prefill (any C) and decode steps after it give
    the single pass over the whole sequence; the state is its definition."""
    rng = _rng(42)
    B, D, N, L, T = 2, 3, 8, 500, 12
    lam, R = _cparams(rng, D, N)
    x1, x2, v = rng.normal(size=(3, B, D, L + T))
    skip = rng.normal(size=D)
    y_full = O.hyena_fwd_cpx(x1, x2, v, lam, R, skip)
    s_full = O.modal_state_cpx((x1 * v)[..., :L], lam)
    for C in (1, 64, 100, L):
        yc, sc = O.chunk_fwd_cpx(x1[..., :L], x2[..., :L], v[..., :L], lam, R, skip, C)
        assert np.max(np.abs(yc - y_full[..., :L])) <= 1e-10 * np.max(np.abs(y_full)), C
        assert np.max(np.abs(sc - s_full)) <= 1e-10 * np.max(np.abs(s_full)), C
    s = sc
    for t in range(L, L + T):
        yt, s = O.modal_decode_cpx(x1[..., t], x2[..., t], v[..., t], lam, R, skip, state_in=s)
        assert np.max(np.abs(yt - y_full[..., t])) <= 1e-10 * np.max(np.abs(y_full)), t


# ---------------------------------------------------------------- token-major layout
def pin_tokmajor_layout_literal(O):
    """in_proj's token-major layout written out by hand: B = 1, L = 2, D = 2,
    element (t, 3c + j) = 100 t + 10 c + j, with x1, x2, v at triple
    positions 2, 0, 1."""
    xin = np.array([[[0, 1, 2, 10, 11, 12],
                     [100, 101, 102, 110, 111, 112]]], dtype=np.float64)
    x1, x2, v = O.tokmajor_streams(xin, (2, 0, 1))
    assert np.array_equal(x1, [[[2, 102], [12, 112]]]), x1
    assert np.array_equal(x2, [[[0, 100], [10, 110]]]), x2
    assert np.array_equal(v, [[[1, 101], [11, 111]]]), v


def pin_tokmajor_impulse(O):
    """An impulse in x1 of channel c0 at token t0, v = x2 = 1, skip = 0: y
    (B, L, D) holds channel c0's filter from t0 on in column c0 and zeros
    elsewhere; poles 1/2 and 1/4 make every value exact."""
    D, L, t0, c0 = 3, 12, 4, 1
    pos = (1, 2, 0)
    lam = np.log(np.array([[0.5, 0.25]] * D))
    R = np.array([[1.0, -2.0], [3.0, 0.5], [-1.0, 1.0]])
    xin = np.zeros((1, L, 3 * D))
    xin[0, :, 3 * np.arange(D) + pos[1]] = 1.0          # x2
    xin[0, :, 3 * np.arange(D) + pos[2]] = 1.0          # v
    xin[0, t0, 3 * c0 + pos[0]] = 1.0                   # x1
    y, s = O.chunk_fwd_tokmajor(xin, lam, R, np.zeros(D), pos)
    want = np.zeros((1, L, D))
    for t in range(t0, L):
        k = t - t0
        want[0, t, c0] = R[c0, 0] * 0.5 ** k + R[c0, 1] * 0.25 ** k
    assert y.shape == (1, L, D) and np.allclose(y, want, rtol=0, atol=1e-15), (y, want)
    want_s = np.zeros((1, D, 2))
    want_s[0, c0] = [0.5 ** (L - 1 - t0), 0.25 ** (L - 1 - t0)]
    assert np.allclose(s, want_s, rtol=0, atol=1e-15), s


def pin_tokmajor_fir_impulse(O):
    """FIR on the token-major layout: an impulse in x1 of channel c0 at token
    t0 gives that channel's taps, lag by lag, in column c0 from t0 on; the
    window handed out holds u of the last K-1 tokens, here [0, 1, 0] in c0."""
    D, L, K, t0, c0 = 3, 10, 4, 8, 2
    pos = (2, 0, 1)
    taps = np.array([[0.5, -1.0, 2.0, 0.25], [1.0, 0.0, 0.0, 3.0], [-2.0, 0.75, 1.5, -0.125]])
    xin = np.zeros((1, L, 3 * D))
    xin[0, :, 3 * np.arange(D) + pos[1]] = 1.0          # x2
    xin[0, :, 3 * np.arange(D) + pos[2]] = 1.0          # v
    xin[0, t0, 3 * c0 + pos[0]] = 1.0                   # x1
    y, win = O.fir_fwd_tokmajor(xin, taps, np.zeros(D), pos)
    want = np.zeros((1, L, D))
    want[0, 8, c0] = taps[c0, 0]
    want[0, 9, c0] = taps[c0, 1]
    assert y.shape == (1, L, D) and np.array_equal(y, want), (y, want)
    want_w = np.zeros((1, D, K - 1))
    want_w[0, c0] = [0.0, 1.0, 0.0]                     # tokens 7, 8, 9
    assert np.array_equal(win, want_w), win


ALL_PINS = [
    pin_golden, pin_filter_rational, pin_filter_dft, pin_recurrence,
    pin_impulse, pin_linearity_time_invariance, pin_numpy_convolve,
    pin_direct_vs_fft, pin_fraction_bruteforce, pin_gate_special,
    pin_fir_delta, pin_chunk_equals_full, pin_chunk_resume,
    pin_chunk_state_rational, pin_scale_equivariance,
    pin_decode_after_prefill, pin_decode_impulse_rational, pin_fir_window_pieces,
    pin_cpx_filter_rational, pin_cpx_second_order_recurrence, pin_cpx_real_special_case,
    pin_cpx_chunk_and_decode_equal_full,
    pin_tokmajor_layout_literal, pin_tokmajor_impulse, pin_tokmajor_fir_impulse,
]
