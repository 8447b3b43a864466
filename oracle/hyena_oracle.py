"""fp64 CPU oracle for the Hyena operator -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this module.  The product path (the HIP library and its Python
binding) never calls it, and it shares no code with that path.

What it computes (plain definitions, written out, in fp64):

* Modal long filter (hcl blocks): h[c,t] = sum_n R[c,n] * exp(lam[c,n] * t),
  lam = log_poles, R = residues, both stored in fp32.  The pages describe the
  hcl block as a modal-form IIR filter whose log_poles / residues stay in fp32
  (Evo2-7B-262K model card, §Architecture 'Training dtype' and §Implementation
  Notes 'log_poles / residues kept in fp32'; Evo1-1.5-7B-8K model card,
  §Architecture).  t = 0 is lag 0; there is no window or normalisation.
* Hyena gate: y = x2 * z + skip * u with u = x1 * v and z the causal
  convolution of u with h over the sequence, u[t<0] = 0.  The three streams
  come from the 3H input projection and the gated result feeds out_proj
  (evo2_flash README, layer_names table: 'blocks.N.projections' and
  'blocks.N.filter').  The skip term sits outside the x2 gate.
* Long convolution by a zero-padded FFT of length >= 2L ('modal-form IIR via
  FFT': Evo2-7B-262K model card, §Implementation Notes 'Block dispatch';
  'FFT-based long convolution': Evo1-1.5-7B-8K model card, §Implementation
  Notes 'Hyena engine').
* Explicit FIR blocks, inner length 7 (hcs) and 128 (hcm): the same gate with
  z[t] = sum_{k<K} w[c,k] * u[t-k]  (Evo2-7B-262K model card, §Implementation
  Notes 'Block dispatch').  w[c,k] is the coefficient of lag k.
* Chunked prefill with the modal state carried between chunks.  The state of
  mode n after token t is s_n(t) = sum_{k<=t} p_n^(t-k) u[k], p_n = exp(lam_n).
  Within a chunk starting at t0 the output is the in-chunk convolution plus
  sum_n R_n p_n^(t-t0+1) s_n(t0-1); after the chunk the state becomes
  p_n^C' s_n + sum_j p_n^(C'-1-j) u[t0+j].  The chunked output must equal the
  single-pass output (TurboQuant-Bio int4 Evo 2 checkpoints, §'Important: a
  correctness fix comes with this' and §Chunk size 'Fidelity is independent
  of chunk size'; the IIR modal state is the per-layer cache: Evo2-7B-262K
  model card, §Implementation Notes 'Custom cache', and Evo1-1.5-7B-8K model
  card, §Implementation Notes 'Cache subclass').

* Decode from the per-layer caches.  The hcl cache is the modal state
  (Evo2-7B-262K model card, §Implementation Notes 'Custom cache': IIR inference
  params for hcl, FIR inference params for hcm / hcs; Evo1-1.5-7B-8K model
  card, §Implementation Notes 'Cache subclass': the Hyena params hold the FIR
  window and the IIR modal state).  One modal step is the state recurrence
  s_n <- p_n s_n + u followed by z = sum_n R_n s_n (the same z as the
  convolution, since z[t] = sum_n R_n s_n(t)).  The FIR cache is the window of
  the last K-1 values of u; a call continuing a sequence convolves over the
  window followed by its own u, and leaves the last K-1 values of that
  concatenation as the new window.

* Complex-pole modal filters (Evo 1: the Hyena filter is given by modal-form
  poles / residues with a state size of 8, Evo1-1.5-7B-8K model card,
  §Architecture).  The pages give no formula; the reading taken here is the
  real part of a sum of complex exponentials,
      h[c,t] = Re sum_n R[c,n] * exp(lam[c,n] * t),  lam, R complex,
  with the poles given in log form like Evo 2's log_poles (p = exp(lam); a
  pole p enters as lam = log|p| + i arg p).  Real modes are the case
  Im lam = 0 = Im R.  The modal state is complex, s_n(t) = sum_{k<=t}
  p_n^(t-k) u[k], and z[t] = Re sum_n R_n s_n(t).

* Token-major layout of the mixer's projections.  in_proj's 3H output holds
  every channel's three streams side by side (Hyena channels are interleaved
  per triple: evo2_flash README, §Limitations), one row per token, and the
  gated output feeds out_proj token by token (evo2_flash README, layer_names
  table).  The reading taken here: xin is (B, L, 3D) with channel c's x1, x2,
  v at columns 3c + pos[0], 3c + pos[1], 3c + pos[2] -- the order inside a
  triple is not given on the pages, so it is a parameter -- and y is
  (B, L, D).  The operator itself is unchanged: the streams are split out and
  the chunked oracle above runs on them as one chunk.

Arrays are channel-major unless named token-major: activations (B, D, L), parameters (D, N) / (D,) /
(D, K), state (B, D, N), FIR window (B, D, K-1) oldest first; complex
parameters and states are numpy complex arrays.  Everything is upcast to
fp64 (complex128) first.
"""
from __future__ import annotations

import numpy as np
import scipy.fft

__all__ = [
    "modal_filter", "conv_direct", "conv_fft", "causal_conv",
    "hyena_fwd", "fir_fwd", "modal_state", "chunk_fwd", "next_pow2",
    "modal_decode", "fir_fwd_window",
    "modal_filter_cpx", "hyena_fwd_cpx", "modal_state_cpx", "chunk_fwd_cpx", "modal_decode_cpx",
    "tokmajor_streams", "chunk_fwd_tokmajor", "fir_fwd_tokmajor",
]

DIRECT_MAX_L = 4096      # direct O(L^2) sum up to this length, FFT above


def next_pow2(n: int) -> int:
    return 1 << max(0, int(n - 1).bit_length())


def modal_filter(log_poles, residues, L: int) -> np.ndarray:
    """h[c, t] = sum_n R[c, n] exp(lam[c, n] t) for t in [0, L); fp64 (D, L)."""
    lam = np.asarray(log_poles, dtype=np.float64)
    R = np.asarray(residues, dtype=np.float64)
    t = np.arange(L, dtype=np.float64)
    h = np.zeros((lam.shape[0], L))
    for n in range(lam.shape[1]):                   # one mode at a time
        h += R[:, n:n + 1] * np.exp(lam[:, n:n + 1] * t[None, :])
    return h


def conv_direct(u, h) -> np.ndarray:
    """Causal convolution by its definition: z[.., t] = sum_{k<=t} h[.., t-k] u[.., k].

    u is (..., L); h is (..., Lh) (Lh may be shorter than L: an FIR).  Loops
    over the lag, vectorised over the other axes: O(L * Lh).
    """
    u = np.asarray(u, dtype=np.float64)
    h = np.asarray(h, dtype=np.float64)
    L = u.shape[-1]
    z = np.zeros_like(u)
    for lag in range(min(L, h.shape[-1])):
        z[..., lag:] += h[..., lag:lag + 1] * u[..., :L - lag]
    return z


def conv_fft(u, h) -> np.ndarray:
    """Causal convolution as a zero-padded real FFT product, fp64.

    Length n = next power of two >= L + Lh - 1, so there is no circular wrap;
    only the first L outputs are kept.
    """
    u = np.asarray(u, dtype=np.float64)
    h = np.asarray(h, dtype=np.float64)
    L = u.shape[-1]
    hl = min(L, h.shape[-1])
    n = next_pow2(L + hl - 1)
    U = scipy.fft.rfft(u, n=n, axis=-1)
    H = scipy.fft.rfft(h[..., :hl], n=n, axis=-1)
    return scipy.fft.irfft(U * H, n=n, axis=-1)[..., :L]


def causal_conv(u, h) -> np.ndarray:
    """Direct sum for short sequences, FFT otherwise (same result to ~1e-15)."""
    if u.shape[-1] <= DIRECT_MAX_L or h.shape[-1] <= 64:
        return conv_direct(u, h)
    return conv_fft(u, h)


def _gate(x1, x2, v, z_of_u, skip):
    x1 = np.asarray(x1, dtype=np.float64)
    x2 = np.asarray(x2, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    u = x1 * v
    z = z_of_u(u)
    sk = np.zeros(x1.shape[-2]) if skip is None else np.asarray(skip, dtype=np.float64)
    return x2 * z + sk[:, None] * u


def hyena_fwd(x1, x2, v, log_poles, residues, skip, conv=causal_conv) -> np.ndarray:
    """Single-pass modal Hyena operator: y = x2 * (h conv u) + skip * u, fp64."""
    L = np.asarray(x1).shape[-1]
    h = modal_filter(log_poles, residues, L)
    return _gate(x1, x2, v, lambda u: conv(u, h[None]), skip)


def fir_fwd(x1, x2, v, taps, skip, conv=conv_direct) -> np.ndarray:
    """Explicit-FIR Hyena operator with taps[c, k] = coefficient of lag k."""
    w = np.asarray(taps, dtype=np.float64)
    return _gate(x1, x2, v, lambda u: conv(u, w[None]), skip)


def modal_state(u, log_poles, state_in=None) -> np.ndarray:
    """s_n(L-1) = p^L s_in + sum_k p^(L-1-k) u[k]; u (B, D, L) -> (B, D, N)."""
    u = np.asarray(u, dtype=np.float64)
    lam = np.asarray(log_poles, dtype=np.float64)
    L = u.shape[-1]
    k = np.arange(L, dtype=np.float64)
    w = np.exp(lam[:, :, None] * (L - 1 - k)[None, None, :])       # (D, N, L)
    s = np.einsum("bdl,dnl->bdn", u, w)
    if state_in is not None:
        s += np.exp(lam * L)[None] * np.asarray(state_in, dtype=np.float64)
    return s


def chunk_fwd(x1, x2, v, log_poles, residues, skip, C: int, state_in=None,
              return_states=False):
    """Chunked prefill with the modal state carried across chunks, fp64.

    Chunks are [t0, t0 + C'), C' = min(C, L - t0).  Within each chunk:
      1. in-chunk causal convolution of u with h[0:C'];
      2. plus the carried term sum_n R_n p_n^(t - t0 + 1) s_n;
      3. then the state update s_n <- p_n^C' s_n + sum_j p_n^(C'-1-j) u[t0+j].
    Returns y (B, D, L) and the final state (B, D, N); with return_states also
    the list of states after every chunk.
    """
    x1 = np.asarray(x1, dtype=np.float64)
    x2 = np.asarray(x2, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lam = np.asarray(log_poles, dtype=np.float64)
    R = np.asarray(residues, dtype=np.float64)
    B, D, L = x1.shape
    N = lam.shape[1]
    s = (np.zeros((B, D, N)) if state_in is None
         else np.asarray(state_in, dtype=np.float64).copy())
    u = x1 * v
    z = np.zeros_like(u)
    h = modal_filter(lam, R, min(C, L))
    states = []
    for t0 in range(0, L, C):
        Cp = min(C, L - t0)
        uc = u[..., t0:t0 + Cp]
        zc = causal_conv(uc, h[None, :, :Cp])
        j = np.arange(Cp, dtype=np.float64)
        carry = np.exp(lam[:, :, None] * (j + 1)[None, None, :])        # (D, N, C')
        zc += np.einsum("dn,bdn,dnj->bdj", R, s, carry)
        z[..., t0:t0 + Cp] = zc
        decay_in = np.exp(lam[:, :, None] * (Cp - 1 - j)[None, None, :])  # (D, N, C')
        s = np.exp(lam * Cp)[None] * s + np.einsum("bdj,dnj->bdn", uc, decay_in)
        if return_states:
            states.append(s.copy())
    sk = np.zeros(D) if skip is None else np.asarray(skip, dtype=np.float64)
    y = x2 * z + sk[:, None] * u
    if return_states:
        return y, s, states
    return y, s


def modal_decode(x1, x2, v, log_poles, residues, skip, state_in=None):
    """One decode step of the modal operator from its cached state, fp64.

    x1, x2, v are the token's three streams, (B, D).  The cache holds
    s_n = s_n(t-1) (zero for an empty prefix); the step updates it to
    s_n(t) = p_n s_n(t-1) + u_t, p_n = exp(lam_n), and outputs
    y_t = x2_t * sum_n R_n s_n(t) + skip * u_t.
    Returns y (B, D) and the new state (B, D, N).
    """
    x1 = np.asarray(x1, dtype=np.float64)
    x2 = np.asarray(x2, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lam = np.asarray(log_poles, dtype=np.float64)
    R = np.asarray(residues, dtype=np.float64)
    B, D = x1.shape
    s = (np.zeros((B, D, lam.shape[1])) if state_in is None
         else np.asarray(state_in, dtype=np.float64))
    u = x1 * v
    s = np.exp(lam)[None] * s + u[:, :, None]
    z = np.einsum("dn,bdn->bd", R, s)
    sk = np.zeros(D) if skip is None else np.asarray(skip, dtype=np.float64)
    return x2 * z + sk[None, :] * u, s


def fir_fwd_window(x1, x2, v, taps, skip, window_in=None):
    """Explicit-FIR operator continuing a sequence from its cached window, fp64.

    window_in (B, D, K-1) holds u of the K-1 tokens before this call, oldest
    first (zeros, or None, for a fresh sequence).  With e the window followed
    by this call's u, z[t] = sum_{k<K} w[c,k] e[K-1+t-k].  Returns y (B, D, L)
    and the new window: the last K-1 entries of e.
    """
    x1 = np.asarray(x1, dtype=np.float64)
    x2 = np.asarray(x2, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    w = np.asarray(taps, dtype=np.float64)
    B, D, L = x1.shape
    K = w.shape[1]
    win = (np.zeros((B, D, K - 1)) if window_in is None
           else np.asarray(window_in, dtype=np.float64))
    u = x1 * v
    e = np.concatenate([win, u], axis=-1)
    z = np.zeros_like(u)
    for k in range(K):
        z += w[None, :, k:k + 1] * e[..., K - 1 - k:K - 1 - k + L]
    sk = np.zeros(D) if skip is None else np.asarray(skip, dtype=np.float64)
    return x2 * z + sk[None, :, None] * u, e[..., e.shape[-1] - (K - 1):]


# ---------------------------------------------------------------- complex poles
def _cpx(a):
    return np.asarray(a, dtype=np.complex128)


def modal_filter_cpx(log_poles, residues, L: int) -> np.ndarray:
    """h[c, t] = Re sum_n R[c, n] exp(lam[c, n] t), t in [0, L); fp64 (D, L)."""
    lam = _cpx(log_poles)
    R = _cpx(residues)
    t = np.arange(L, dtype=np.float64)
    return np.real(np.einsum("dn,dnt->dt", R, np.exp(lam[:, :, None] * t[None, None, :])))


def hyena_fwd_cpx(x1, x2, v, log_poles, residues, skip, conv=causal_conv) -> np.ndarray:
    """The Hyena operator with a complex-pole modal filter, single pass."""
    L = np.asarray(x1).shape[-1]
    h = modal_filter_cpx(log_poles, residues, L)
    return _gate(x1, x2, v, lambda u: conv(u, h[None]), skip)


def modal_state_cpx(u, log_poles, state_in=None) -> np.ndarray:
    """s_n(L-1) = p^L s_in + sum_k p^(L-1-k) u[k], complex (B, D, N)."""
    u = np.asarray(u, dtype=np.float64)
    lam = _cpx(log_poles)
    L = u.shape[-1]
    k = np.arange(L, dtype=np.float64)
    w = np.exp(lam[:, :, None] * (L - 1 - k)[None, None, :])
    s = np.einsum("bdl,dnl->bdn", u, w)
    if state_in is not None:
        s = s + np.exp(lam * L)[None] * _cpx(state_in)
    return s


def chunk_fwd_cpx(x1, x2, v, log_poles, residues, skip, C: int, state_in=None):
    """Chunked prefill with a complex modal state, fp64.

    Within the chunk [t0, t0 + C'): the in-chunk convolution plus
    Re sum_n R_n p_n^(t-t0+1) s_n; then s_n <- p_n^C' s_n + sum_j
    p_n^(C'-1-j) u[t0+j].  Returns y (B, D, L) and the state (B, D, N).
    """
    x1 = np.asarray(x1, dtype=np.float64)
    x2 = np.asarray(x2, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lam = _cpx(log_poles)
    R = _cpx(residues)
    B, D, L = x1.shape
    N = lam.shape[1]
    s = np.zeros((B, D, N), np.complex128) if state_in is None else _cpx(state_in).copy()
    u = x1 * v
    z = np.zeros_like(u)
    h = modal_filter_cpx(lam, R, min(C, L))
    for t0 in range(0, L, C):
        Cp = min(C, L - t0)
        uc = u[..., t0:t0 + Cp]
        zc = causal_conv(uc, h[None, :, :Cp])
        j = np.arange(Cp, dtype=np.float64)
        carry = np.exp(lam[:, :, None] * (j + 1)[None, None, :])
        zc = zc + np.real(np.einsum("dn,bdn,dnj->bdj", R, s, carry))
        z[..., t0:t0 + Cp] = zc
        decay_in = np.exp(lam[:, :, None] * (Cp - 1 - j)[None, None, :])
        s = np.exp(lam * Cp)[None] * s + np.einsum("bdj,dnj->bdn", uc, decay_in)
    sk = np.zeros(D) if skip is None else np.asarray(skip, dtype=np.float64)
    return x2 * z + sk[:, None] * u, s


def modal_decode_cpx(x1, x2, v, log_poles, residues, skip, state_in=None):
    """One decode step with a complex modal state: s <- p s + u,
    y = x2 Re sum_n R_n s_n + skip u.  Returns y (B, D) and the state."""
    x1 = np.asarray(x1, dtype=np.float64)
    x2 = np.asarray(x2, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    lam = _cpx(log_poles)
    R = _cpx(residues)
    B, D = x1.shape
    s = np.zeros((B, D, lam.shape[1]), np.complex128) if state_in is None else _cpx(state_in)
    u = x1 * v
    s = np.exp(lam)[None] * s + u[:, :, None]
    z = np.real(np.einsum("dn,bdn->bd", R, s))
    sk = np.zeros(D) if skip is None else np.asarray(skip, dtype=np.float64)
    return x2 * z + sk[None, :] * u, s


# ---------------------------------------------------------------- token-major layout
def tokmajor_streams(xin, pos=(0, 1, 2)):
    """Split in_proj's token-major output into the three channel-major streams.

    xin (B, L, 3D): channel c's x1, x2, v at columns 3c + pos[0], 3c + pos[1],
    3c + pos[2] (channels interleaved per triple: evo2_flash README,
    §Limitations).  Returns x1, x2, v as (B, D, L) arrays.
    """
    xin = np.asarray(xin)
    B, L, D3 = xin.shape
    per_channel = xin.reshape(B, L, D3 // 3, 3)          # [b, t, c, position in triple]
    return tuple(np.ascontiguousarray(np.moveaxis(per_channel[..., p], 1, 2)) for p in pos)


def chunk_fwd_tokmajor(xin, log_poles, residues, skip, pos=(0, 1, 2), state_in=None):
    """The modal operator on the token-major layout, fp64: the streams of xin
    (see tokmajor_streams), the sequence continued from state_in (zero state
    when None) as one chunk of chunk_fwd.  Returns y as (B, L, D), the layout
    out_proj reads (evo2_flash README, layer_names table: 'blocks.N.filter'),
    and the final state (B, D, N)."""
    x1, x2, v = tokmajor_streams(xin, pos)
    L = x1.shape[-1]
    y, s = chunk_fwd(x1, x2, v, log_poles, residues, skip, max(L, 1), state_in=state_in)
    return np.ascontiguousarray(np.moveaxis(y, 1, 2)), s


def fir_fwd_tokmajor(xin, taps, skip, pos=(0, 1, 2), window_in=None):
    """The explicit-FIR operator on the token-major layout, fp64: the streams
    of xin (see tokmajor_streams) through fir_fwd_window.  Returns y as
    (B, L, D) and the new window (B, D, K-1)."""
    x1, x2, v = tokmajor_streams(xin, pos)
    y, win = fir_fwd_window(x1, x2, v, taps, skip, window_in=window_in)
    return np.ascontiguousarray(np.moveaxis(y, 1, 2)), win
