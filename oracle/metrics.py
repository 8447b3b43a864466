"""Error metrics used to compare a result with the fp64 oracle -- TEST INFRASTRUCTURE.

* rel_l2     = ||y - ref||_2 / ||ref||_2 over the whole array;
* rel_l2_ch  = sqrt(mean_c ||y_c - ref_c||^2 / ||ref_c||^2), channel-equalised,
               so channels of very different magnitude weigh the same;
* elem_rel   = max |y - ref| / (|ref| + tau * rms_c(ref)), tau = 1e-3: a
               per-element relative error with a per-channel floor, since the
               bare ratio is unbounded where ref crosses zero;
* nonfinite  = number of non-finite entries of y where ref is finite.

All four are functions of per-channel sums (channel_stats), so a large array
can be compared block of channels by block (from_stats) with the same result.

Channels are every axis but the last; the last axis is time.
"""
from __future__ import annotations

import numpy as np

TAU = 1e-3
# Gates for bf16 I/O with fp32 compute against the fp64 oracle.
REL_L2_MAX = 2e-3
ELEM_REL_MAX = 2e-2


def channel_stats(y, ref, tau: float = TAU) -> dict:
    """Per-channel sums behind compare(): squared error, squared reference,
    the largest per-element ratio and the count of non-finite outputs where
    the reference is finite.  Channels are every axis but the last, flattened.
    Stats of disjoint channel sets combine with from_stats() into exactly the
    metrics compare() gives for all of them at once."""
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    L = ref.shape[-1]
    y2 = y.reshape(-1, L)
    r2 = ref.reshape(-1, L)
    fin_ref = np.isfinite(r2)
    nonfinite = np.count_nonzero(~np.isfinite(y2) & fin_ref, axis=1)
    d = np.where(fin_ref, y2 - r2, 0.0)
    d = np.where(np.isfinite(d), d, np.inf)
    e_ch = np.sum(d * d, axis=1)
    n_ch = np.sum(np.where(fin_ref, r2 * r2, 0.0), axis=1)
    rms = np.sqrt(n_ch / L) if L else n_ch
    den = np.abs(r2) + tau * rms[:, None]
    den = np.where(den > 0, den, 1.0)
    elem = np.max(np.abs(d) / den, axis=1) if L else np.zeros(r2.shape[0])
    return {"e_ch": e_ch, "n_ch": n_ch, "elem_ch": elem, "nonfinite_ch": nonfinite}


def from_stats(parts) -> dict:
    """The compare() metrics of the union of the channel sets in `parts`
    (a list of channel_stats() results)."""
    e_ch = np.concatenate([p["e_ch"] for p in parts])
    n_ch = np.concatenate([p["n_ch"] for p in parts])
    elem = np.concatenate([p["elem_ch"] for p in parts])
    nonfinite = int(sum(int(np.sum(p["nonfinite_ch"])) for p in parts))
    tot_n = float(np.sum(n_ch))
    rel_l2 = float(np.sqrt(np.sum(e_ch) / tot_n)) if tot_n > 0 else float(np.sqrt(np.sum(e_ch)))
    safe = np.where(n_ch > 0, n_ch, 1.0)
    ch = np.where(n_ch > 0, e_ch / safe, e_ch)
    rel_l2_ch = float(np.sqrt(np.mean(ch))) if ch.size else 0.0
    return {
        "rel_l2": rel_l2,
        "rel_l2_ch": rel_l2_ch,
        "rel_l2_ch_max": float(np.sqrt(np.max(ch))) if ch.size else 0.0,
        "elem_rel": float(np.max(elem)) if elem.size else 0.0,
        "nonfinite": nonfinite,
    }


def compare(y, ref, tau: float = TAU) -> dict:
    return from_stats([channel_stats(y, ref, tau)])


def passes(m: dict, rel_l2_max: float = REL_L2_MAX, elem_max: float = ELEM_REL_MAX) -> bool:
    return (m["nonfinite"] == 0 and m["rel_l2"] <= rel_l2_max
            and m["rel_l2_ch"] <= rel_l2_max and m["elem_rel"] <= elem_max)
