"""Seeded synthetic inputs for the Hyena operator.

This module is shared by the tests, the benchmark and the oracle-side checks.
It draws random numbers, rounds them to the storage formats the operator
consumes (fp32, bf16) and decodes those formats back to fp64.  It holds none
of the operator's arithmetic: no filter, no convolution, no gate.

Shapes and distributions follow the workloads the pages describe:

* D=4096 channels, 8K and 262K contexts: Evo2-7B-262K model card,
  §Architecture (hidden size, max sequence length) and §Related Models.
* 32 kb scoring with chunk 1024 (chunk 4096 also discussed): TurboQuant-Bio
  int4 Evo 2 checkpoints, §Measured and §Chunk size.
* residual-stream values up to ~1e12, hence bf16 and never fp16: evo2_flash
  README, §Requirements and install.
* modal-form filter parameters (log_poles, residues) kept in fp32:
  Evo2-7B-262K model card, §Usage 'Note on dtype'.

Real Evo 2 activations need trained checkpoints and DNA inputs that are not
available; these synthetic tensors stand in for them with the same shapes.

Every array is drawn in fp64 from numpy's PCG64 and rounded once to fp32
(round-to-nearest-even, numpy's cast); bf16 configs then round that fp32 value
to bf16 (round-to-nearest-even on the bit pattern).  Both the GPU path and the
oracle consume the identical rounded bits.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Config", "CONFIGS", "Workload", "make",
    "f32_to_bf16_bits", "bf16_bits_to_f32", "to_f64",
]

# Order in which child seeds are spawned from a config's SeedSequence.
_STREAMS = ("x1", "x2", "v", "log_poles", "residues", "skip",
            "taps7", "taps128", "scale")
_ROW_BLOCK = 64          # rows drawn per independent grandchild stream


@dataclass(frozen=True)
class Config:
    name: str
    seed: int
    B: int
    D: int
    L: int
    io: str                      # "f32" or "bf16"
    N: int = 16                  # modes per channel
    lam_lo: float = 1e-3         # |log_pole| drawn log-uniform in [lam_lo, 1]
    chunks: tuple = ()           # chunk sizes this workload is run with
    fir_taps: tuple = ()         # explicit FIR lengths run on the same input
    x1_scale_max: float = 1.0    # per-channel x1 scale, log-uniform in [1, max]
    desc: str = ""


CONFIGS = {
    "tiny": Config(
        "tiny", 1001, 1, 64, 1024, "f32", chunks=(128,),
        desc="B=1 D=64 L=1024 fp32 I/O, modal N=16, full-sequence long conv"),
    "7b_layer_set": Config(
        "7b_layer_set", 1002, 1, 4096, 8192, "bf16", fir_taps=(7, 128),
        desc="B=1 D=4096 L=8192 bf16: FIR-7, FIR-128 and the modal long filter"),
    "32k_chunked": Config(
        "32k_chunked", 1003, 1, 4096, 32768, "bf16", chunks=(1024,),
        desc="B=1 D=4096 L=32768 bf16, modal N=16, chunk 1024 with carried state"),
    "40b_shaped": Config(
        "40b_shaped", 1004, 1, 8192, 32768, "bf16", chunks=(1024,),
        x1_scale_max=1e12,
        desc="B=1 D=8192 L=32768 bf16, per-channel x1 scale log-uniform in [1,1e12]"),
    "262k": Config(
        "262k", 1005, 1, 4096, 262144, "bf16", lam_lo=1e-5, chunks=(4096,),
        desc="B=1 D=4096 L=262144 bf16, slow decays |log_pole| in [1e-5,1]"),
}


# ---------------------------------------------------------------- formats
def f32_to_bf16_bits(a) -> np.ndarray:
    """fp32 -> bf16 bit pattern (uint16), round to nearest even; NaN -> quiet NaN."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = a.view(np.uint32)
    r = ((b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))
         >> np.uint32(16)).astype(np.uint16)
    nan = (b & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    if nan.any():
        r[nan] = ((b[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return r


def bf16_bits_to_f32(bits) -> np.ndarray:
    """bf16 bit pattern (uint16) -> fp32 (exact)."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(a, io: str) -> np.ndarray:
    """Decode a stored activation array to fp64 (exact)."""
    if io == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def _round_param(a64: np.ndarray, bf16: bool) -> np.ndarray:
    """fp64 draw -> fp32; for bf16 configs also snapped to a bf16 value."""
    a32 = a64.astype(np.float32)
    if bf16:
        a32 = bf16_bits_to_f32(f32_to_bf16_bits(a32))
    return a32


# ---------------------------------------------------------------- workload
@dataclass
class Workload:
    cfg: Config
    B: int
    D: int
    L: int
    io: str
    x1: np.ndarray = field(repr=False)
    x2: np.ndarray = field(repr=False)
    v: np.ndarray = field(repr=False)
    log_poles: np.ndarray = field(repr=False)
    residues: np.ndarray = field(repr=False)
    skip: np.ndarray = field(repr=False)
    taps: dict = field(repr=False, default_factory=dict)
    scale: np.ndarray | None = field(repr=False, default=None)

    @property
    def N(self) -> int:
        return self.log_poles.shape[1]

    def f64(self, name: str, rows=None) -> np.ndarray:
        """fp64 view of an activation ('x1', 'x2', 'v'); rows = channel index list."""
        a = getattr(self, name)
        if rows is not None:
            a = a[:, rows, :]
        return to_f64(a, self.io)


def _seqs(cfg: Config):
    return dict(zip(_STREAMS, np.random.SeedSequence(cfg.seed).spawn(len(_STREAMS))))


def _draw_rows(ss: np.random.SeedSequence, rows: int, L: int, scale=None,
               io="bf16", threads=None, keep=None) -> np.ndarray:
    """Draw a (rows, L) N(0,1) activation, row block by row block.

    Block i of _ROW_BLOCK rows comes from the i-th grandchild of `ss`, so blocks
    are independent streams and can be drawn in parallel.  `keep`, a list of
    (start, stop) row ranges, draws only the blocks those ranges touch and
    returns their rows stacked in order: the same values as those rows of
    the full draw.  `scale` is indexed by the full row number.
    """
    nblk = (rows + _ROW_BLOCK - 1) // _ROW_BLOCK
    kids = ss.spawn(nblk)
    ranges = [(0, rows)] if keep is None else list(keep)
    n_out = sum(b - a for a, b in ranges)
    out = np.empty((n_out, L), dtype=np.uint16 if io == "bf16" else np.float32)
    jobs = []                    # (block, first row of the block kept, rows kept, output row)
    o = 0
    for a, b in ranges:
        r = a
        while r < b:
            i = r // _ROW_BLOCK
            r_end = min(b, (i + 1) * _ROW_BLOCK)
            jobs.append((i, r, r_end, o))
            o += r_end - r
            r = r_end

    def one(job):
        i, ra, rb, o = job
        r0 = i * _ROW_BLOCK
        r1 = min(rows, r0 + _ROW_BLOCK)
        g = np.random.Generator(np.random.PCG64(kids[i]))
        a = g.standard_normal((r1 - r0, L))[ra - r0:rb - r0]
        if scale is not None:
            a *= scale[ra:rb, None]
        a32 = a.astype(np.float32)
        out[o:o + rb - ra] = f32_to_bf16_bits(a32) if io == "bf16" else a32

    nt = threads or min(16, os.cpu_count() or 1)
    if len(jobs) == 1 or nt == 1:
        for j in jobs:
            one(j)
    else:
        with ThreadPoolExecutor(nt) as ex:
            list(ex.map(one, jobs))
    return out


def make(name: str, *, B: int | None = None, D: int | None = None,
         L: int | None = None, N: int | None = None,
         lam_lo: float | None = None, channels: tuple | None = None) -> Workload:
    """Build a seeded workload; overrides shrink it for fast tests.

    channels=(c0, c1) keeps only channels c0 <= c < c1 of the workload (every
    batch item), drawing only those rows: the arrays equal the same channels
    of the whole workload, and D is then c1 - c0."""
    cfg = CONFIGS[name]
    B = cfg.B if B is None else B
    D = cfg.D if D is None else D
    L = cfg.L if L is None else L
    N = cfg.N if N is None else N
    lam_lo = cfg.lam_lo if lam_lo is None else lam_lo
    bf16 = cfg.io == "bf16"
    ss = _seqs(cfg)

    def param_rng(key):
        return np.random.Generator(np.random.PCG64(ss[key]))

    scale = None
    if cfg.x1_scale_max > 1.0:
        # s_c = exp(U(0, ln max)), one per channel (shared over the batch)
        scale = np.exp(param_rng("scale").uniform(0.0, math.log(cfg.x1_scale_max), D))
    # |lambda| log-uniform in [lam_lo, 1]; poles are real and negative
    lam = -np.exp(param_rng("log_poles").uniform(math.log(lam_lo), 0.0, (D, N)))
    res = param_rng("residues").normal(0.0, math.sqrt(1.0 / 16.0), (D, N))
    skip = param_rng("skip").normal(0.0, 1.0, D)
    taps = {}
    for K, key in ((7, "taps7"), (128, "taps128")):
        taps[K] = _round_param(param_rng(key).normal(0.0, math.sqrt(1.0 / K), (D, K)), bf16)

    c0, c1 = (0, D) if channels is None else (int(channels[0]), int(channels[1]))
    assert 0 <= c0 <= c1 <= D, (channels, D)
    keep = None if channels is None else [(b * D + c0, b * D + c1) for b in range(B)]
    acts = {}
    for key in ("x1", "x2", "v"):
        sc = None
        if key == "x1" and scale is not None:
            sc = np.tile(scale, B)
        acts[key] = _draw_rows(ss[key], B * D, L, scale=sc, io=cfg.io,
                               keep=keep).reshape(B, c1 - c0, L)

    return Workload(
        cfg=cfg, B=B, D=c1 - c0, L=L, io=cfg.io,
        x1=acts["x1"], x2=acts["x2"], v=acts["v"],
        log_poles=lam.astype(np.float32)[c0:c1],
        residues=res.astype(np.float32)[c0:c1],
        skip=_round_param(skip, bf16)[c0:c1],
        taps={K: t[c0:c1] for K, t in taps.items()},
        scale=None if scale is None else scale[c0:c1],
    )


def random_taps(K: int, D: int, seed: int, bf16: bool) -> np.ndarray:
    """Extra FIR taps ~ N(0, 1/K) for lengths outside a config's own set."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, K])))
    return _round_param(g.normal(0.0, math.sqrt(1.0 / K), (D, K)), bf16)


def random_state(B: int, D: int, N: int, seed: int) -> np.ndarray:
    """A (B, D, N) fp32 modal state ~ N(0, 1) for resume tests."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7])))
    return g.normal(0.0, 1.0, (B, D, N)).astype(np.float32)


def complex_modes(D: int, N: int, seed: int, lam_lo: float = 1e-3):
    """Complex log-poles and residues (D, N) complex64, the parameters of a
    complex-pole modal filter (Evo 1: state size 8):
    Re lam = -exp(U(ln lam_lo, 0)) (decay as the real log_poles),
    Im lam ~ U(-pi, pi) (oscillation per token),
    R ~ N(0, 1/16) + i N(0, 1/16)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 11])))
    a = -np.exp(g.uniform(np.log(lam_lo), 0.0, (D, N)))
    b = g.uniform(-np.pi, np.pi, (D, N))
    R = g.normal(0.0, 0.25, (D, N)) + 1j * g.normal(0.0, 0.25, (D, N))
    return (a + 1j * b).astype(np.complex64), R.astype(np.complex64)


def random_complex_state(B: int, D: int, N: int, seed: int) -> np.ndarray:
    """A (B, D, N) complex64 modal state ~ N(0, 1) + i N(0, 1) for resume tests."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 13])))
    return (g.normal(0.0, 1.0, (B, D, N)) + 1j * g.normal(0.0, 1.0, (B, D, N))).astype(np.complex64)


def interleave_triples(x1, x2, v, pos=(0, 1, 2)) -> np.ndarray:
    """The same streams in in_proj's token-major layout: (B, D, L) arrays
    (stored bf16 bits or fp32) -> (B, L, 3D) with channel c's x1, x2, v at
    columns 3c + pos[0], 3c + pos[1], 3c + pos[2].  Layout only: elements are
    copied bit for bit."""
    B, D, L = x1.shape
    out = np.empty((B, L, D, 3), dtype=x1.dtype)
    for a, p in zip((x1, x2, v), pos):
        out[..., p] = np.moveaxis(a, 1, 2)
    return out.reshape(B, L, 3 * D)
