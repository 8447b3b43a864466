"""Helpers of the GPU tests: move seeded workloads to the device, run the oracle
on sampled channels, compare with the gates."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

import oracle
import workloads as W

# fp32 I/O has no output rounding; the HIP path's own error (fp32 FFT
# rounding, three-part bf16 products) is ~1e-6 relative.  The relative-L2
# gate is tightened to 1e-4; the per-element gate stays at 2e-2.
F32_REL_L2_MAX = 1e-4
F32_ELEM_MAX = 2e-2


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def act_to_dev(a: np.ndarray, io: str) -> torch.Tensor:
    if io == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a)).view(torch.bfloat16).to(dev())
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def par_to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev())


def offset_copy(t: torch.Tensor) -> torch.Tensor:
    """A contiguous copy of t whose data starts one element into its buffer
    (2 or 4 bytes: no 16-byte alignment), for the kernels' unaligned paths."""
    buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
    out = buf[1:].view(t.shape)
    out.copy_(t)
    return out


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


class DevWorkload:
    """Device copies of a workload's tensors."""

    def __init__(self, w: W.Workload):
        self.w = w
        self.x1 = act_to_dev(w.x1, w.io)
        self.x2 = act_to_dev(w.x2, w.io)
        self.v = act_to_dev(w.v, w.io)
        self.lam = par_to_dev(w.log_poles)
        self.res = par_to_dev(w.residues)
        self.skip = par_to_dev(w.skip)
        self.taps = {K: par_to_dev(t) for K, t in w.taps.items()}


def sample_rows(D: int, k: int = 8, seed: int = 0) -> np.ndarray:
    """k channel indices spread over [0, D), always including 0 and D-1."""
    if D <= k:
        return np.arange(D)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, D - 1), size=k - 2, replace=False)
    return np.sort(np.concatenate([[0, D - 1], mid]))


def oracle_modal(w: W.Workload, rows=None, C=None, state_in=None):
    """Oracle of the modal operator on channel subset `rows` (all batch items)."""
    rows = np.arange(w.D) if rows is None else np.asarray(rows)
    x1, x2, v = (w.f64(k, rows) for k in ("x1", "x2", "v"))
    lam = w.log_poles[rows].astype(np.float64)
    R = w.residues[rows].astype(np.float64)
    sk = w.skip[rows].astype(np.float64)
    if C is None and state_in is None:
        return oracle.hyena_fwd(x1, x2, v, lam, R, sk), oracle.modal_state(x1 * v, lam)
    s0 = None if state_in is None else state_in[:, rows]
    if C is not None and w.L <= 4096:
        return oracle.chunk_fwd(x1, x2, v, lam, R, sk, C, state_in=s0)
    # chunked == single pass (pinned in fp64); the state term of a non-zero
    # initial state adds x2 * sum_n R_n p_n^(t+1) s0_n
    y = oracle.hyena_fwd(x1, x2, v, lam, R, sk)
    if s0 is not None:
        t = np.arange(w.L, dtype=np.float64)
        for n in range(lam.shape[1]):
            y += x2 * (R[None, :, n:n + 1] * s0[:, :, n:n + 1]
                       * np.exp(lam[None, :, n:n + 1] * (t + 1)))
    return y, oracle.modal_state(x1 * v, lam, state_in=s0)


def oracle_fir(w: W.Workload, K: int, rows=None, taps=None):
    rows = np.arange(w.D) if rows is None else np.asarray(rows)
    x1, x2, v = (w.f64(k, rows) for k in ("x1", "x2", "v"))
    tp = (w.taps[K] if taps is None else taps)[rows].astype(np.float64)
    return oracle.fir_fwd(x1, x2, v, tp, w.skip[rows].astype(np.float64))


def gate(y_dev: torch.Tensor, ref: np.ndarray, io: str, rows=None, label: str = ""):
    y = to_f64(y_dev if rows is None else y_dev[:, torch.as_tensor(rows, device=y_dev.device)])
    m = oracle.compare(y, ref)
    log(f"  {label}: {m}")
    if io == "bf16":
        ok = oracle.passes(m)
    else:
        ok = oracle.passes(m, F32_REL_L2_MAX, F32_ELEM_MAX)
    assert ok, (label, m)
    return m


def state_gate(s_dev: torch.Tensor, ref: np.ndarray, rows=None, label: str = "", tol=1e-4):
    s = to_f64(s_dev if rows is None else s_dev[:, torch.as_tensor(rows, device=s_dev.device)])
    num = np.sqrt(np.sum((s - ref) ** 2, axis=-1))
    den = np.sqrt(np.sum(ref ** 2, axis=-1))
    rel = float(np.sqrt(np.mean((num / np.where(den > 0, den, 1)) ** 2)))
    log(f"  {label} state rel_l2_ch={rel:.3e}")
    assert np.all(np.isfinite(s)) and rel <= tol, (label, rel)
    return rel
