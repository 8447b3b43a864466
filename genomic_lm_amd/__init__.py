"""genomic_lm_amd -- MI355X (gfx950) Hyena operator, Python binding of libhyena.so.

A thin ctypes layer over the C ABI in include/hyena.h: it checks dtype,
device and contiguity of torch tensors, passes their device pointers and the
current HIP stream, and turns status codes into exceptions.  Every step of the
operator runs in the HIP kernels of libhyena.so; there is no fallback path.
If the library is not built the functions raise HyenaNotBuilt.

Entry points (names follow the C ABI):
  modal_filter(log_poles, residues, L)                      -> h (D, L) fp32
  fir_fwd(x1, x2, v, taps, skip=None)                       -> y
  fftconv_fwd(x1, x2, v, log_poles, residues, skip=None)    -> y
  chunk_fwd(x1, x2, v, log_poles, residues, C, skip=None,
            state_in=None, algo="auto")                      -> (y, state_out)
            (algo "auto" calls hyena_chunk_fwd, "fft" / "mfma" hyena_chunk_fwd_algo)
  modal_decode(x1, x2, v, log_poles, residues, skip=None,
               state_in=None)       (x of shape (B, D))       -> (y, state_out)
  fir_fwd_window(x1, x2, v, taps, skip=None, window_in=None) -> (y, window_out)
  chunk_fwd_tokmajor(xin, log_poles, residues, skip=None, state_in=None,
                     pos=(0, 1, 2))  (xin (B, L, 3D))   -> (y (B, L, D), state_out)
  fir_fwd_tokmajor(xin, taps, skip=None, window_in=None, pos=(0, 1, 2))
                                                         -> (y (B, L, D), window_out)
Complex-pole variants (log_poles / residues complex64 (D, N), states
complex64 (B, D, N)): modal_filter_cpx, fftconv_fwd_cpx, chunk_fwd_cpx,
modal_decode_cpx.

Every function is also available under the C name (hyena_fftconv_fwd, ...),
and the submodule hyena_op gives the four core calls the short names
fftconv, fir, chunk and modal_filter.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "HyenaError", "HyenaNotBuilt", "lib", "LIB_PATH", "abi_version",
    "modal_filter", "fir_fwd", "fftconv_fwd", "fftconv_workspace_size", "fftconv_fwd_noalloc",
    "chunk_fwd",
    "modal_decode", "fir_fwd_window",
    "modal_filter_cpx", "fftconv_fwd_cpx", "chunk_fwd_cpx", "modal_decode_cpx",
    "chunk_fwd_tokmajor", "chunk_tokmajor_workspace_size", "fir_fwd_tokmajor",
    "OK", "ERR_INVALID_ARG", "ERR_UNSUPPORTED", "ERR_WORKSPACE", "ERR_LAUNCH",
    "F32", "BF16", "ALGOS", "EXPORTS",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhyena.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_LAUNCH = 0, 1, 2, 3, 4
F32, BF16 = 0, 1
ALGOS = {"auto": 0, "fft": 1, "mfma": 2}
TOKMAJOR_ALGOS = {"auto": 0, "mfma": 2, "recurrence": 3}

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_size = ctypes.c_size_t

# name -> (restype, argtypes); the full set of symbols include/hyena.h declares
EXPORTS = {
    "hyena_abi_version": (_int, []),
    "hyena_status_string": (ctypes.c_char_p, [_int]),
    "hyena_modal_filter": (_int, [_p, _p, _i64, _i64, _i64, _p, _p]),
    "hyena_fir_fwd": (_int, [_p, _p, _p, _p, _i64, _p, _p, _i64, _i64, _i64, _int, _p]),
    "hyena_fftconv_fwd": (_int, [_p, _p, _p, _p, _p, _i64, _p, _p, _i64, _i64, _i64, _int,
                                 _p, _size, _p]),
    "hyena_fftconv_workspace_size": (_size, [_i64, _i64, _i64, _i64, _int]),
    "hyena_fftconv_fwd_noalloc": (_int, [_p, _p, _p, _p, _p, _i64, _p, _p, _i64, _i64, _i64, _int,
                                         _p]),
    "hyena_chunk_fwd": (_int, [_p, _p, _p, _p, _p, _i64, _p, _p, _p, _p, _i64, _i64, _i64,
                               _i64, _int, _p]),
    "hyena_chunk_fwd_algo": (_int, [_p, _p, _p, _p, _p, _i64, _p, _p, _p, _p, _i64, _i64, _i64,
                                    _i64, _int, _int, _p]),
    "hyena_modal_decode": (_int, [_p, _p, _p, _p, _p, _i64, _p, _p, _p, _p, _i64, _i64, _int,
                                  _p]),
    "hyena_fir_fwd_window": (_int, [_p, _p, _p, _p, _i64, _p, _p, _p, _p, _i64, _i64, _i64,
                                    _int, _p]),
    "hyena_modal_filter_cpx": (_int, [_p, _p, _i64, _i64, _i64, _p, _p]),
    "hyena_fftconv_fwd_cpx": (_int, [_p, _p, _p, _p, _p, _i64, _p, _p, _i64, _i64, _i64, _int,
                                     _p, _size, _p]),
    "hyena_chunk_fwd_cpx": (_int, [_p, _p, _p, _p, _p, _i64, _p, _p, _p, _p, _i64, _i64, _i64,
                                   _i64, _int, _p]),
    "hyena_chunk_fwd_cpx_algo": (_int, [_p, _p, _p, _p, _p, _i64, _p, _p, _p, _p, _i64, _i64,
                                        _i64, _i64, _int, _int, _p]),
    "hyena_modal_decode_cpx": (_int, [_p, _p, _p, _p, _p, _i64, _p, _p, _p, _p, _i64, _i64,
                                      _int, _p]),
    "hyena_chunk_fwd_tokmajor": (_int, [_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _p,
                                        _p, _i64, _p, _p, _p, _p, _i64, _i64, _i64, _int, _p,
                                        _size, _p]),
    "hyena_chunk_fwd_tokmajor_algo": (_int, [_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                             _p, _p, _i64, _p, _p, _p, _p, _i64, _i64, _i64, _int,
                                             _int, _p, _size, _p]),
    "hyena_chunk_tokmajor_workspace_size": (_size, [_i64, _i64, _i64, _i64, _int]),
    "hyena_fir_fwd_tokmajor": (_int, [_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _p,
                                      _i64, _p, _p, _p, _p, _i64, _i64, _i64, _int, _p]),
}


class HyenaNotBuilt(RuntimeError):
    pass


class HyenaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libhyena.so, with argument types declared."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise HyenaNotBuilt(
                f"{LIB_PATH} is missing: build it with `python -m genomic_lm_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib


def abi_version() -> int:
    return lib().hyena_abi_version()


def status_string(status: int) -> str:
    return lib().hyena_status_string(status).decode()


def _check(fn: str, status: int):
    if status != OK:
        raise HyenaError(fn, status)


# The per-call host work is a fixed cost in front of every launch (a
# 1024-token chunk per call at D = 4096 is ~10 us of GPU time): the current
# stream is read as a raw handle without building a Stream object, pointers
# go to ctypes as plain integers, and valid arguments pass each check in one
# expression (the detailed checks below run only to name what is wrong).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
_ACT_DTYPES = (torch.bfloat16, torch.float32)


def _stream(t: torch.Tensor):
    if _raw_stream is not None:
        return _raw_stream(t.get_device())
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _act(name, t, like=None, dims=3):
    if (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype in _ACT_DTYPES and t.dim() == dims
            and t.is_contiguous() and (like is None or (t.shape == like.shape
                                                        and t.dtype == like.dtype
                                                        and t.get_device() == like.get_device()))):
        return t
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU device")
    if t.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"{name} must be bfloat16 or float32, got {t.dtype}")
    if t.dim() != dims:
        want = "(B, D, L)" if dims == 3 else "(B, D)"
        raise ValueError(f"{name} must be {want}, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if like is not None:
        if t.shape != like.shape or t.dtype != like.dtype or t.device != like.device:
            raise ValueError(f"{name} must match x1 in shape, dtype and device")
    return t


def _param(name, t, shape, dev, optional=False):
    # (the device is compared by index: a tensor's .device builds a new object)
    if (isinstance(t, torch.Tensor) and t.dtype == torch.float32 and t.get_device() == dev.index
            and t.shape == shape and t.is_contiguous()):
        return t
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32:
        raise TypeError(f"{name} must be a float32 tensor")
    if t.device != dev:
        raise ValueError(f"{name} must be on {dev}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _io(t):
    return BF16 if t.dtype == torch.bfloat16 else F32


def modal_filter(log_poles: torch.Tensor, residues: torch.Tensor, L: int) -> torch.Tensor:
    """h[c, t] = sum_n residues[c, n] * exp(log_poles[c, n] * t), fp32 (D, L)."""
    if not log_poles.is_cuda:
        raise ValueError("log_poles must be on a GPU device")
    D, N = log_poles.shape
    _param("log_poles", log_poles, (D, N), log_poles.device)
    _param("residues", residues, (D, N), log_poles.device)
    h = torch.empty((D, L), dtype=torch.float32, device=log_poles.device)
    _check("hyena_modal_filter", lib().hyena_modal_filter(
        _ptr(log_poles), _ptr(residues), D, N, L, _ptr(h), _stream(h)))
    return h


def fir_fwd(x1, x2, v, taps, skip=None, out=None) -> torch.Tensor:
    """Gated explicit FIR: y = x2 * (taps conv x1*v) + skip * x1*v."""
    _act("x1", x1)
    _act("x2", x2, x1)
    _act("v", v, x1)
    B, D, L = x1.shape
    K = taps.shape[-1] if isinstance(taps, torch.Tensor) and taps.dim() == 2 else -1
    _param("taps", taps, (D, K), x1.device)
    _param("skip", skip, (D,), x1.device, optional=True)
    y = torch.empty_like(x1) if out is None else _act("out", out, x1)
    _check("hyena_fir_fwd", lib().hyena_fir_fwd(
        _ptr(x1), _ptr(x2), _ptr(v), _ptr(taps), K, _ptr(skip), _ptr(y), B, D, L,
        _io(x1), _stream(x1)))
    return y


def fftconv_workspace_size(B: int, D: int, L: int, N: int, dtype=torch.bfloat16) -> int:
    return int(lib().hyena_fftconv_workspace_size(B, D, L, N, BF16 if dtype == torch.bfloat16 else F32))


def fftconv_fwd(x1, x2, v, log_poles, residues, skip=None, out=None, workspace=None) -> torch.Tensor:
    """Single-pass modal Hyena operator with a zero-padded FFT convolution."""
    _act("x1", x1)
    _act("x2", x2, x1)
    _act("v", v, x1)
    B, D, L = x1.shape
    N = log_poles.shape[-1] if isinstance(log_poles, torch.Tensor) and log_poles.dim() == 2 else -1
    _param("log_poles", log_poles, (D, N), x1.device)
    _param("residues", residues, (D, N), x1.device)
    _param("skip", skip, (D,), x1.device, optional=True)
    y = torch.empty_like(x1) if out is None else _act("out", out, x1)
    need = fftconv_workspace_size(B, D, L, N, x1.dtype)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x1.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("hyena_fftconv_fwd", lib().hyena_fftconv_fwd(
        _ptr(x1), _ptr(x2), _ptr(v), _ptr(log_poles), _ptr(residues), N, _ptr(skip), _ptr(y),
        B, D, L, _io(x1), _ptr(workspace), ws_bytes, _stream(x1)))
    return y


def fftconv_fwd_noalloc(x1, x2, v, log_poles, residues, skip=None, out=None) -> torch.Tensor:
    """fftconv_fwd through the library's device scratch instead of a
    workspace (hyena_fftconv_fwd_noalloc): no device memory is allocated
    when `out` is given."""
    _act("x1", x1)
    _act("x2", x2, x1)
    _act("v", v, x1)
    B, D, L = x1.shape
    N = log_poles.shape[-1] if isinstance(log_poles, torch.Tensor) and log_poles.dim() == 2 else -1
    _param("log_poles", log_poles, (D, N), x1.device)
    _param("residues", residues, (D, N), x1.device)
    _param("skip", skip, (D,), x1.device, optional=True)
    y = torch.empty_like(x1) if out is None else _act("out", out, x1)
    _check("hyena_fftconv_fwd_noalloc", lib().hyena_fftconv_fwd_noalloc(
        _ptr(x1), _ptr(x2), _ptr(v), _ptr(log_poles), _ptr(residues), N, _ptr(skip), _ptr(y),
        B, D, L, _io(x1), _stream(x1)))
    return y


def chunk_fwd(x1, x2, v, log_poles, residues, C: int, skip=None, state_in=None,
              algo: str = "auto", out=None, state_out=None):
    """Chunked prefill with the modal state carried in and out; returns (y, state_out)."""
    _act("x1", x1)
    _act("x2", x2, x1)
    _act("v", v, x1)
    B, D, L = x1.shape
    N = log_poles.shape[-1] if isinstance(log_poles, torch.Tensor) and log_poles.dim() == 2 else -1
    dev = x1.device
    _param("log_poles", log_poles, (D, N), dev)
    _param("residues", residues, (D, N), dev)
    _param("skip", skip, (D,), dev, optional=True)
    _param("state_in", state_in, (B, D, N), dev, optional=True)
    if algo not in ALGOS:
        raise ValueError(f"algo must be one of {sorted(ALGOS)}")
    y = torch.empty_like(x1) if out is None else _act("out", out, x1)
    if state_out is None:
        state_out = torch.empty((B, D, N), dtype=torch.float32, device=dev)
    else:
        _param("state_out", state_out, (B, D, N), dev)
    args = (_ptr(x1), _ptr(x2), _ptr(v), _ptr(log_poles), _ptr(residues), N, _ptr(skip),
            _ptr(state_in), _ptr(state_out), _ptr(y), B, D, L, int(C), _io(x1))
    h = lib()
    if algo == "auto":
        _check("hyena_chunk_fwd", h.hyena_chunk_fwd(*args, _stream(x1)))
    else:
        _check("hyena_chunk_fwd_algo", h.hyena_chunk_fwd_algo(*args, ALGOS[algo], _stream(x1)))
    return y, state_out


def modal_decode(x1, x2, v, log_poles, residues, skip=None, state_in=None, out=None,
                 state_out=None):
    """One decode step from the modal state: x1, x2, v are (B, D), one token each.

    Returns (y (B, D), state_out (B, D, N)); state_out may be state_in.
    """
    _act("x1", x1, dims=2)
    _act("x2", x2, x1, dims=2)
    _act("v", v, x1, dims=2)
    B, D = x1.shape
    N = log_poles.shape[-1] if isinstance(log_poles, torch.Tensor) and log_poles.dim() == 2 else -1
    _param("log_poles", log_poles, (D, N), x1.device)
    _param("residues", residues, (D, N), x1.device)
    _param("skip", skip, (D,), x1.device, optional=True)
    _param("state_in", state_in, (B, D, N), x1.device, optional=True)
    y = torch.empty_like(x1) if out is None else _act("out", out, x1, dims=2)
    if state_out is None:
        state_out = torch.empty((B, D, N), dtype=torch.float32, device=x1.device)
    else:
        _param("state_out", state_out, (B, D, N), x1.device)
    _check("hyena_modal_decode", lib().hyena_modal_decode(
        _ptr(x1), _ptr(x2), _ptr(v), _ptr(log_poles), _ptr(residues), N, _ptr(skip),
        _ptr(state_in), _ptr(state_out), _ptr(y), B, D, _io(x1), _stream(x1)))
    return y, state_out


def fir_fwd_window(x1, x2, v, taps, skip=None, window_in=None, out=None, window_out=None):
    """Gated explicit FIR continuing from the window of the last K-1 inputs.

    Returns (y, window_out (B, D, K-1) fp32); window_out may be window_in.
    """
    _act("x1", x1)
    _act("x2", x2, x1)
    _act("v", v, x1)
    B, D, L = x1.shape
    K = taps.shape[-1] if isinstance(taps, torch.Tensor) and taps.dim() == 2 else -1
    _param("taps", taps, (D, K), x1.device)
    _param("skip", skip, (D,), x1.device, optional=True)
    _param("window_in", window_in, (B, D, K - 1), x1.device, optional=True)
    y = torch.empty_like(x1) if out is None else _act("out", out, x1)
    if window_out is None:
        window_out = torch.empty((B, D, K - 1), dtype=torch.float32, device=x1.device)
    else:
        _param("window_out", window_out, (B, D, K - 1), x1.device)
    _check("hyena_fir_fwd_window", lib().hyena_fir_fwd_window(
        _ptr(x1), _ptr(x2), _ptr(v), _ptr(taps), K, _ptr(skip), _ptr(window_in),
        _ptr(window_out), _ptr(y), B, D, L, _io(x1), _stream(x1)))
    return y, window_out


# ------------------------------------------------------------------ complex poles
def _cparam(name, t, D, dev, optional=False):
    """A complex (D, N) parameter: complex64, or float32 with a trailing (re, im)
    axis.  Returns (tensor viewed as float32 pairs, N)."""
    if t is None:
        if optional:
            return None, None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype == torch.complex64:
        t = torch.view_as_real(t)
    if t.dtype != torch.float32 or t.dim() != 3 or t.shape[0] != D or t.shape[2] != 2:
        raise ValueError(f"{name} must be complex64 (D, N) or float32 (D, N, 2)")
    if t.device != dev or not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous on {dev}")
    return t, t.shape[1]


def _cstate(name, t, shape, dev, optional=False):
    """A complex state (B, D, N): complex64 or float32 (B, D, N, 2)."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if t.dtype == torch.complex64:
        t = torch.view_as_real(t)
    _param(name, t, tuple(shape) + (2,), dev)
    return t


def modal_filter_cpx(log_poles, residues, L: int) -> torch.Tensor:
    """h[c, t] = Re sum_n residues[c, n] exp(log_poles[c, n] t), fp32 (D, L)."""
    D = log_poles.shape[0]
    lp, N = _cparam("log_poles", log_poles, D, log_poles.device)
    rs, N2 = _cparam("residues", residues, D, log_poles.device)
    if N2 != N:
        raise ValueError("log_poles and residues must have the same number of modes")
    h = torch.empty((D, L), dtype=torch.float32, device=lp.device)
    _check("hyena_modal_filter_cpx", lib().hyena_modal_filter_cpx(
        _ptr(lp), _ptr(rs), D, N, L, _ptr(h), _stream(h)))
    return h


def _cmodal(x1, log_poles, residues):
    B, D = x1.shape[0], x1.shape[1]
    lp, N = _cparam("log_poles", log_poles, D, x1.device)
    rs, N2 = _cparam("residues", residues, D, x1.device)
    if N2 != N:
        raise ValueError("log_poles and residues must have the same number of modes")
    return lp, rs, N


def fftconv_fwd_cpx(x1, x2, v, log_poles, residues, skip=None, out=None,
                    workspace=None) -> torch.Tensor:
    """Single pass with a complex-pole modal filter."""
    _act("x1", x1)
    _act("x2", x2, x1)
    _act("v", v, x1)
    B, D, L = x1.shape
    lp, rs, N = _cmodal(x1, log_poles, residues)
    _param("skip", skip, (D,), x1.device, optional=True)
    y = torch.empty_like(x1) if out is None else _act("out", out, x1)
    need = fftconv_workspace_size(B, D, L, N, x1.dtype)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x1.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("hyena_fftconv_fwd_cpx", lib().hyena_fftconv_fwd_cpx(
        _ptr(x1), _ptr(x2), _ptr(v), _ptr(lp), _ptr(rs), N, _ptr(skip), _ptr(y),
        B, D, L, _io(x1), _ptr(workspace), ws_bytes, _stream(x1)))
    return y


def chunk_fwd_cpx(x1, x2, v, log_poles, residues, C: int, skip=None, state_in=None,
                  algo: str = "auto", out=None, state_out=None):
    """Chunked prefill with a complex modal state; returns (y, state_out complex64)."""
    if algo not in ALGOS:
        raise ValueError(f"algo must be one of {sorted(ALGOS)}")
    _act("x1", x1)
    _act("x2", x2, x1)
    _act("v", v, x1)
    B, D, L = x1.shape
    lp, rs, N = _cmodal(x1, log_poles, residues)
    _param("skip", skip, (D,), x1.device, optional=True)
    si = _cstate("state_in", state_in, (B, D, N), x1.device, optional=True)
    y = torch.empty_like(x1) if out is None else _act("out", out, x1)
    if state_out is None:
        state_out = torch.empty((B, D, N), dtype=torch.complex64, device=x1.device)
    so = _cstate("state_out", state_out, (B, D, N), x1.device)
    args = (_ptr(x1), _ptr(x2), _ptr(v), _ptr(lp), _ptr(rs), N, _ptr(skip), _ptr(si), _ptr(so),
            _ptr(y), B, D, L, int(C), _io(x1))
    if algo == "auto":
        _check("hyena_chunk_fwd_cpx", lib().hyena_chunk_fwd_cpx(*args, _stream(x1)))
    else:
        _check("hyena_chunk_fwd_cpx_algo",
               lib().hyena_chunk_fwd_cpx_algo(*args, ALGOS[algo], _stream(x1)))
    return y, state_out


def modal_decode_cpx(x1, x2, v, log_poles, residues, skip=None, state_in=None, out=None,
                     state_out=None):
    """One decode step from a complex modal state: x1, x2, v are (B, D)."""
    _act("x1", x1, dims=2)
    _act("x2", x2, x1, dims=2)
    _act("v", v, x1, dims=2)
    B, D = x1.shape
    lp, rs, N = _cmodal(x1, log_poles, residues)
    _param("skip", skip, (D,), x1.device, optional=True)
    si = _cstate("state_in", state_in, (B, D, N), x1.device, optional=True)
    y = torch.empty_like(x1) if out is None else _act("out", out, x1, dims=2)
    if state_out is None:
        state_out = torch.empty((B, D, N), dtype=torch.complex64, device=x1.device)
    so = _cstate("state_out", state_out, (B, D, N), x1.device)
    _check("hyena_modal_decode_cpx", lib().hyena_modal_decode_cpx(
        _ptr(x1), _ptr(x2), _ptr(v), _ptr(lp), _ptr(rs), N, _ptr(skip), _ptr(si), _ptr(so),
        _ptr(y), B, D, _io(x1), _stream(x1)))
    return y, state_out


def chunk_tokmajor_workspace_size(B: int, D: int, L: int, N: int, dtype=torch.bfloat16) -> int:
    return int(lib().hyena_chunk_tokmajor_workspace_size(
        B, D, L, N, BF16 if dtype == torch.bfloat16 else F32))


def chunk_fwd_tokmajor(xin, log_poles, residues, skip=None, state_in=None, pos=(0, 1, 2),
                       out=None, state_out=None, workspace=None, algo: str = "auto"):
    """The modal operator on in_proj's token-major layout: xin (B, L, 3D) with
    channel c's x1, x2, v at columns 3c + pos[0], 3c + pos[1], 3c + pos[2];
    returns (y (B, L, D), state_out (B, D, N)).  algo "auto" calls
    hyena_chunk_fwd_tokmajor, "mfma" / "recurrence" hyena_chunk_fwd_tokmajor_algo."""
    if algo not in TOKMAJOR_ALGOS:
        raise ValueError(f"algo must be one of {sorted(TOKMAJOR_ALGOS)}")
    _act("xin", xin)
    B, L, D3 = xin.shape
    if D3 % 3:
        raise ValueError(f"xin must be (B, L, 3D), got shape {tuple(xin.shape)}")
    D = D3 // 3
    if sorted(int(p) for p in pos) != [0, 1, 2]:
        raise ValueError("pos must be a permutation of (0, 1, 2)")
    N = log_poles.shape[-1] if isinstance(log_poles, torch.Tensor) and log_poles.dim() == 2 else -1
    _param("log_poles", log_poles, (D, N), xin.device)
    _param("residues", residues, (D, N), xin.device)
    _param("skip", skip, (D,), xin.device, optional=True)
    _param("state_in", state_in, (B, D, N), xin.device, optional=True)
    if out is None:
        y = torch.empty((B, L, D), dtype=xin.dtype, device=xin.device)
    else:
        y = _act("out", out)
        if tuple(y.shape) != (B, L, D) or y.dtype != xin.dtype or y.device != xin.device:
            raise ValueError("out must be (B, L, D) with the dtype and device of xin")
    if state_out is None:
        state_out = torch.empty((B, D, N), dtype=torch.float32, device=xin.device)
    else:
        _param("state_out", state_out, (B, D, N), xin.device)
    need = chunk_tokmajor_workspace_size(B, D, L, N, xin.dtype)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=xin.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(xin), int(pos[0]), int(pos[1]), int(pos[2]), _ptr(log_poles), _ptr(residues), N,
            _ptr(skip), _ptr(state_in), _ptr(state_out), _ptr(y), B, D, L, _io(xin))
    if algo == "auto":
        _check("hyena_chunk_fwd_tokmajor", lib().hyena_chunk_fwd_tokmajor(
            *args, _ptr(workspace), ws_bytes, _stream(xin)))
    else:
        _check("hyena_chunk_fwd_tokmajor_algo", lib().hyena_chunk_fwd_tokmajor_algo(
            *args, TOKMAJOR_ALGOS[algo], _ptr(workspace), ws_bytes, _stream(xin)))
    return y, state_out


def fir_fwd_tokmajor(xin, taps, skip=None, window_in=None, pos=(0, 1, 2), out=None,
                     window_out=None):
    """Explicit FIR on in_proj's token-major layout, continuing from a window:
    xin (B, L, 3D) as chunk_fwd_tokmajor; returns (y (B, L, D), window_out
    (B, D, K-1), None when K = 1)."""
    _act("xin", xin)
    B, L, D3 = xin.shape
    if D3 % 3:
        raise ValueError(f"xin must be (B, L, 3D), got shape {tuple(xin.shape)}")
    D = D3 // 3
    if sorted(int(p) for p in pos) != [0, 1, 2]:
        raise ValueError("pos must be a permutation of (0, 1, 2)")
    K = taps.shape[-1] if isinstance(taps, torch.Tensor) and taps.dim() == 2 else -1
    _param("taps", taps, (D, K), xin.device)
    _param("skip", skip, (D,), xin.device, optional=True)
    _param("window_in", window_in, (B, D, K - 1), xin.device, optional=True)
    if out is None:
        y = torch.empty((B, L, D), dtype=xin.dtype, device=xin.device)
    else:
        y = _act("out", out)
        if tuple(y.shape) != (B, L, D) or y.dtype != xin.dtype or y.device != xin.device:
            raise ValueError("out must be (B, L, D) with the dtype and device of xin")
    if K > 1 and window_out is None:
        window_out = torch.empty((B, D, K - 1), dtype=torch.float32, device=xin.device)
    elif window_out is not None:
        _param("window_out", window_out, (B, D, K - 1), xin.device)
    _check("hyena_fir_fwd_tokmajor", lib().hyena_fir_fwd_tokmajor(
        _ptr(xin), int(pos[0]), int(pos[1]), int(pos[2]), _ptr(taps), K, _ptr(skip),
        _ptr(window_in), _ptr(window_out), _ptr(y), B, D, L, _io(xin), _stream(xin)))
    return y, window_out


# The same functions under the names of the C entry points they call
# (chunk_fwd / chunk_fwd_cpx call the *_algo entry point when algo is not
# "auto").
hyena_modal_filter = modal_filter
hyena_fir_fwd = fir_fwd
hyena_fftconv_fwd = fftconv_fwd
hyena_fftconv_workspace_size = fftconv_workspace_size
hyena_fftconv_fwd_noalloc = fftconv_fwd_noalloc
hyena_chunk_fwd = chunk_fwd
hyena_modal_decode = modal_decode
hyena_fir_fwd_window = fir_fwd_window
hyena_modal_filter_cpx = modal_filter_cpx
hyena_fftconv_fwd_cpx = fftconv_fwd_cpx
hyena_chunk_fwd_cpx = chunk_fwd_cpx
hyena_modal_decode_cpx = modal_decode_cpx
hyena_chunk_fwd_tokmajor = chunk_fwd_tokmajor
hyena_chunk_tokmajor_workspace_size = chunk_tokmajor_workspace_size
hyena_fir_fwd_tokmajor = fir_fwd_tokmajor
__all__ += [n for n in list(globals()) if n.startswith("hyena_") and callable(globals()[n])]

from . import hyena_op  # noqa: E402,F401  (short names of the four core calls)
