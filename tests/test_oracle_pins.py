"""The fp64 oracle against its pins, and the pins against planted mistakes.

A planted mistake lives in a copy of an oracle function, on the CPU; each must
make at least one pin fail.
"""
import types

import numpy as np
import pytest

import oracle.hyena_oracle as HO
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(HO)


# ------------------------------------------------------------ planted mistakes
def _mutant(**over):
    """A namespace with the oracle's functions, some replaced, re-bound so the
    replaced helpers are used by the functions that call them."""
    ns = {k: getattr(HO, k) for k in dir(HO) if not k.startswith("__")}
    ns.update(over)
    mod = types.SimpleNamespace(**ns)
    # rebuild the composite functions over the (possibly replaced) helpers
    def hyena_fwd(x1, x2, v, log_poles, residues, skip, conv=None):
        L = np.asarray(x1).shape[-1]
        h = mod.modal_filter(log_poles, residues, L)
        cv = conv or mod.causal_conv
        return mod._gate(x1, x2, v, lambda u: cv(u, h[None]), skip)

    def fir_fwd(x1, x2, v, taps, skip, conv=None):
        w = np.asarray(taps, dtype=np.float64)
        cv = conv or mod.conv_direct
        return mod._gate(x1, x2, v, lambda u: cv(u, w[None]), skip)

    def causal_conv(u, h):
        if u.shape[-1] <= HO.DIRECT_MAX_L or h.shape[-1] <= 64:
            return mod.conv_direct(u, h)
        return mod.conv_fft(u, h)

    def hyena_fwd_cpx(x1, x2, v, log_poles, residues, skip, conv=None):
        L = np.asarray(x1).shape[-1]
        h = mod.modal_filter_cpx(log_poles, residues, L)
        cv = conv or mod.causal_conv
        return mod._gate(x1, x2, v, lambda u: cv(u, h[None]), skip)

    def chunk_fwd_tokmajor(xin, log_poles, residues, skip, pos=(0, 1, 2), state_in=None):
        x1, x2, v = mod.tokmajor_streams(xin, pos)
        L = x1.shape[-1]
        y, s = mod.chunk_fwd(x1, x2, v, log_poles, residues, skip, max(L, 1), state_in=state_in)
        return mod.tokmajor_out(y), s

    def fir_fwd_tokmajor(xin, taps, skip, pos=(0, 1, 2), window_in=None):
        x1, x2, v = mod.tokmajor_streams(xin, pos)
        y, win = mod.fir_fwd_window(x1, x2, v, taps, skip, window_in=window_in)
        return mod.tokmajor_out(y), win

    mod.tokmajor_out = over.get("tokmajor_out", lambda y: np.moveaxis(y, 1, 2))
    if "fir_fwd_tokmajor" not in over:
        mod.fir_fwd_tokmajor = fir_fwd_tokmajor
    if "chunk_fwd_tokmajor" not in over:
        mod.chunk_fwd_tokmajor = chunk_fwd_tokmajor
    if "hyena_fwd" not in over:
        mod.hyena_fwd = hyena_fwd
    if "hyena_fwd_cpx" not in over:
        mod.hyena_fwd_cpx = hyena_fwd_cpx
    if "fir_fwd" not in over:
        mod.fir_fwd = fir_fwd
    if "causal_conv" not in over:
        mod.causal_conv = causal_conv
    return mod


def _filter_shifted(log_poles, residues, L):          # time origin off by one
    lam = np.asarray(log_poles, float)
    R = np.asarray(residues, float)
    t = np.arange(L) + 1.0
    return np.einsum("dn,dnt->dt", R, np.exp(lam[:, :, None] * t))


def _filter_dropped_mode(log_poles, residues, L):     # last mode dropped
    lam = np.asarray(log_poles, float)[:, :-1]
    R = np.asarray(residues, float)[:, :-1]
    t = np.arange(L, dtype=float)
    if lam.shape[1] == 0:
        return np.zeros((np.asarray(log_poles).shape[0], L))
    return np.einsum("dn,dnt->dt", R, np.exp(lam[:, :, None] * t))


def _conv_anticausal(u, h):                           # transposed operand
    u = np.asarray(u, float)
    h = np.asarray(h, float)
    L = u.shape[-1]
    z = np.zeros_like(u)
    for lag in range(min(L, h.shape[-1])):
        z[..., :L - lag] += h[..., lag:lag + 1] * u[..., lag:]
    return z


def _conv_fft_circular(u, h):                         # no zero padding
    import scipy.fft
    u = np.asarray(u, float)
    h = np.asarray(h, float)
    L = u.shape[-1]
    return scipy.fft.irfft(scipy.fft.rfft(u, n=L) * scipy.fft.rfft(h[..., :L], n=L), n=L)


def _gate_skip_inside(x1, x2, v, z_of_u, skip):       # skip inside the x2 gate
    x1, x2, v = (np.asarray(a, float) for a in (x1, x2, v))
    u = x1 * v
    sk = np.zeros(x1.shape[-2]) if skip is None else np.asarray(skip, float)
    return x2 * (z_of_u(u) + sk[:, None] * u)


def _chunk_variant(carry_off=1, decay_off=1, last_len_full=False):
    """chunk_fwd with a planted mistake in the carried term or state update."""
    def chunk_fwd(x1, x2, v, log_poles, residues, skip, C, state_in=None, return_states=False):
        x1, x2, v = (np.asarray(a, float) for a in (x1, x2, v))
        lam = np.asarray(log_poles, float)
        R = np.asarray(residues, float)
        B, D, L = x1.shape
        s = np.zeros((B, D, lam.shape[1])) if state_in is None else np.array(state_in, float)
        u = x1 * v
        z = np.zeros_like(u)
        h = HO.modal_filter(lam, R, min(C, L))
        for t0 in range(0, L, C):
            Cp = min(C, L - t0)
            uc = u[..., t0:t0 + Cp]
            zc = HO.conv_direct(uc, h[None, :, :Cp])
            j = np.arange(Cp, dtype=float)
            zc += np.einsum("dn,bdn,dnj->bdj", R, s, np.exp(lam[:, :, None] * (j + carry_off)))
            z[..., t0:t0 + Cp] = zc
            Cs = C if last_len_full else Cp
            dec = np.exp(lam[:, :, None] * (Cp - decay_off - j))
            s = np.exp(lam * Cs)[None] * s + np.einsum("bdj,dnj->bdn", uc, dec)
        sk = np.zeros(D) if skip is None else np.asarray(skip, float)
        return x2 * z + sk[:, None] * u, s
    return chunk_fwd


def _decode_variant(forget_input=False, output_before_update=False):
    """modal_decode with a planted mistake in the state step."""
    def modal_decode(x1, x2, v, log_poles, residues, skip, state_in=None):
        x1, x2, v = (np.asarray(a, float) for a in (x1, x2, v))
        lam = np.asarray(log_poles, float)
        R = np.asarray(residues, float)
        B, D = x1.shape
        s0 = np.zeros((B, D, lam.shape[1])) if state_in is None else np.asarray(state_in, float)
        u = x1 * v
        s = np.exp(lam)[None] * s0 + (0.0 if forget_input else u[:, :, None])
        z = np.einsum("dn,bdn->bd", R, s0 if output_before_update else s)
        sk = np.zeros(D) if skip is None else np.asarray(skip, float)
        return x2 * z + sk[None, :] * u, s
    return modal_decode


def _fir_window_variant(first_values=False, reversed_taps=False):
    """fir_fwd_window with a planted mistake in the window or the taps."""
    def fir_fwd_window(x1, x2, v, taps, skip, window_in=None):
        x1, x2, v = (np.asarray(a, float) for a in (x1, x2, v))
        w = np.asarray(taps, float)
        if reversed_taps:
            w = w[:, ::-1]
        B, D, L = x1.shape
        K = w.shape[1]
        win = np.zeros((B, D, K - 1)) if window_in is None else np.asarray(window_in, float)
        u = x1 * v
        e = np.concatenate([win, u], axis=-1)
        z = np.zeros_like(u)
        for k in range(K):
            z += w[None, :, k:k + 1] * e[..., K - 1 - k:K - 1 - k + L]
        sk = np.zeros(D) if skip is None else np.asarray(skip, float)
        out_win = e[..., :K - 1] if first_values else e[..., e.shape[-1] - (K - 1):]
        return x2 * z + sk[None, :, None] * u, out_win
    return fir_fwd_window


def _filter_cpx_imag(log_poles, residues, L):        # imaginary part taken
    lam = np.asarray(log_poles, complex)
    R = np.asarray(residues, complex)
    t = np.arange(L, dtype=float)
    return np.imag(np.einsum("dn,dnt->dt", R, np.exp(lam[:, :, None] * t)))


def _filter_cpx_conj_pole(log_poles, residues, L):   # pole conjugated
    lam = np.conj(np.asarray(log_poles, complex))
    R = np.asarray(residues, complex)
    t = np.arange(L, dtype=float)
    return np.real(np.einsum("dn,dnt->dt", R, np.exp(lam[:, :, None] * t)))


def _chunk_cpx_carry_conj(x1, x2, v, log_poles, residues, skip, C, state_in=None):
    """chunk_fwd_cpx with the carried state conjugated."""
    x1, x2, v = (np.asarray(a, float) for a in (x1, x2, v))
    lam = np.asarray(log_poles, complex)
    R = np.asarray(residues, complex)
    B, D, L = x1.shape
    s = np.zeros((B, D, lam.shape[1]), complex) if state_in is None else np.array(state_in, complex)
    u = x1 * v
    z = np.zeros_like(u)
    h = HO.modal_filter_cpx(lam, R, min(C, L))
    for t0 in range(0, L, C):
        Cp = min(C, L - t0)
        uc = u[..., t0:t0 + Cp]
        zc = HO.causal_conv(uc, h[None, :, :Cp])
        j = np.arange(Cp, dtype=float)
        zc = zc + np.real(np.einsum("dn,bdn,dnj->bdj", R, np.conj(s), np.exp(lam[:, :, None] * (j + 1))))
        z[..., t0:t0 + Cp] = zc
        s = np.exp(lam * Cp)[None] * s + np.einsum("bdj,dnj->bdn", uc, np.exp(lam[:, :, None] * (Cp - 1 - j)))
    sk = np.zeros(D) if skip is None else np.asarray(skip, float)
    return x2 * z + sk[:, None] * u, s


def _streams_fixed_order(xin, pos=(0, 1, 2)):         # triple order ignored
    return HO.tokmajor_streams(xin, (0, 1, 2))


def _streams_blocked(xin, pos=(0, 1, 2)):             # [x1 | x2 | v] blocks, not triples
    xin = np.asarray(xin)
    B, L, D3 = xin.shape
    D = D3 // 3
    return tuple(np.ascontiguousarray(np.moveaxis(xin[..., p * D:(p + 1) * D], 1, 2)) for p in pos)


def _out_reshaped(y):                                 # y reshaped instead of transposed
    B, D, L = y.shape
    return y.reshape(B, L, D)


MUTANTS = {
    "filter_time_origin": dict(modal_filter=_filter_shifted),
    "filter_dropped_mode": dict(modal_filter=_filter_dropped_mode),
    "conv_anticausal": dict(conv_direct=_conv_anticausal),
    "conv_fft_circular": dict(conv_fft=_conv_fft_circular),
    "gate_skip_inside": dict(_gate=_gate_skip_inside),
    "chunk_carry_exponent": dict(chunk_fwd=_chunk_variant(carry_off=0)),
    "chunk_decay_exponent": dict(chunk_fwd=_chunk_variant(decay_off=0)),
    "chunk_last_length": dict(chunk_fwd=_chunk_variant(last_len_full=True)),
    "decode_forgets_input": dict(modal_decode=_decode_variant(forget_input=True)),
    "decode_output_before_update": dict(modal_decode=_decode_variant(output_before_update=True)),
    "fir_window_first_values": dict(fir_fwd_window=_fir_window_variant(first_values=True)),
    "fir_window_reversed_taps": dict(fir_fwd_window=_fir_window_variant(reversed_taps=True)),
    "cpx_filter_imag_part": dict(modal_filter_cpx=_filter_cpx_imag),
    "cpx_filter_conj_pole": dict(modal_filter_cpx=_filter_cpx_conj_pole),
    "cpx_chunk_carry_conj": dict(chunk_fwd_cpx=_chunk_cpx_carry_conj),
    "tokmajor_order_ignored": dict(tokmajor_streams=_streams_fixed_order),
    "tokmajor_blocked_streams": dict(tokmajor_streams=_streams_blocked),
    "tokmajor_output_reshaped": dict(tokmajor_out=_out_reshaped),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    mod = _mutant(**MUTANTS[name])
    failed = []
    for pin in P.ALL_PINS:
        try:
            pin(mod)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {name}"
