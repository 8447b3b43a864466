"""Helpers of the GPU tests: move seeded workloads to the device, run the oracle
on sampled channels, compare with the gates."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

import oracle
import workloads as W

# fp32 I/O has no output rounding.  The HIP paths compute in fp32: a length-N
# FFT convolution leaves ~log2(N) * 2^-24 * (a few) of the row's rms in every
# output, the matrix-core path ~2^-24 per three-part product, and the carried
# state one fp32 rounding per step.  At a zero crossing of the output the
# per-element metric divides by its floor, 1e-3 of the row's rms, so an
# absolute error of 1e-5 rms (about 100 fp32 ulps of the rms) reads as 1e-2.
# Gates: relative L2 <= 1e-4 and per-element <= 1e-2.
F32_REL_L2_MAX = 1e-4
F32_ELEM_MAX = 1e-2
STATE_TOL = 1e-4


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
    """Oracle of the modal operator on channel subset `rows` (all batch items).

    Without a chunk length or an initial state: the single-pass definition
    (oracle.hyena_fwd) and the final state (oracle.modal_state).  With either:
    the chunk recurrence itself (oracle.chunk_fwd, one chunk of the whole
    sequence when C is None), whatever the length."""
    rows = np.arange(w.D) if rows is None else np.asarray(rows)
    x1, x2, v = (w.f64(k, rows) for k in ("x1", "x2", "v"))
    lam = w.log_poles[rows].astype(np.float64)
    R = w.residues[rows].astype(np.float64)
    sk = w.skip[rows].astype(np.float64)
    if C is None and state_in is None:
        return oracle.hyena_fwd(x1, x2, v, lam, R, sk), oracle.modal_state(x1 * v, lam)
    s0 = None if state_in is None else state_in[:, rows]
    return oracle.chunk_fwd(x1, x2, v, lam, R, sk, max(1, w.L) if C is None else C,
                            state_in=s0)


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


def state_gate(s_dev: torch.Tensor, ref: np.ndarray, rows=None, label: str = "",
               tol=STATE_TOL):
    s = to_f64(s_dev if rows is None else s_dev[:, torch.as_tensor(rows, device=s_dev.device)])
    num = np.sqrt(np.sum((s - ref) ** 2, axis=-1))
    den = np.sqrt(np.sum(ref ** 2, axis=-1))
    rel = float(np.sqrt(np.mean((num / np.where(den > 0, den, 1)) ** 2)))
    log(f"  {label} state rel_l2_ch={rel:.3e}")
    assert np.all(np.isfinite(s)) and rel <= tol, (label, rel)
    return rel


# ------------------------------------------------------------------ full-size checks
def poisoned(like: torch.Tensor) -> torch.Tensor:
    """An output buffer filled with NaN, so an element a kernel never writes
    shows up as non-finite."""
    return torch.full_like(like, float("nan"))


def all_finite(t: torch.Tensor, label: str):
    n_bad = int((~torch.isfinite(t.float())).sum().item())
    log(f"  {label}: non-finite outputs {n_bad} of {t.numel()}")
    assert n_bad == 0, (label, n_bad)


def host(t: torch.Tensor) -> np.ndarray:
    """A device result as host bits: bf16 as uint16 patterns, fp32 as float32."""
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.float().cpu().numpy()


def pool_gate(name: str, jobs, channels, io: str, overrides=None, block=64):
    """Every job of `jobs` (tests.oracle_pool) over `channels` of workload
    `name`, checked against the gates: outputs as gate(), states as
    state_gate()."""
    from tests import oracle_pool
    res = oracle_pool.check(name, jobs, channels, overrides=overrides, block=block)
    n = len(np.unique(np.asarray(list(channels))))
    for label, r in res.items():
        if "y" in r:
            m = r["y"]
            log(f"  {label} ({n} channels): {m}")
            ok = oracle.passes(m) if io == "bf16" else oracle.passes(m, F32_REL_L2_MAX, F32_ELEM_MAX)
            assert ok, (label, m)
        if "state" in r:
            log(f"  {label} state rel_l2_ch={r['state']:.3e}")
            assert r["state"] <= STATE_TOL, (label, r["state"])
    return res


def compare_dev(y: torch.Tensor, ref: torch.Tensor, scale: float = 1.0, block: int = 256) -> dict:
    """oracle.compare of two device results (ref multiplied by `scale`), in
    blocks of channels copied to the host and compared on host threads."""
    from concurrent.futures import ThreadPoolExecutor
    y2 = y.reshape(-1, y.shape[-1])
    r2 = ref.reshape(-1, ref.shape[-1])

    def one(a):
        yy = y2[a:a + block].double().cpu().numpy()
        rr = r2[a:a + block].double().cpu().numpy() * scale
        return oracle.channel_stats(yy, rr)

    with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        parts = list(ex.map(one, range(0, y2.shape[0], block)))
    return oracle.from_stats(parts)
