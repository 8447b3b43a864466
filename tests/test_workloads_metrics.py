"""Host-side checks of the input generators and the comparison metrics."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import metrics as M


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(0)
    a = np.concatenate([
        rng.normal(size=20000).astype(np.float32),
        (rng.normal(size=2000) * 1e30).astype(np.float32),
        (rng.normal(size=2000) * 1e-30).astype(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, 1.0 + 2 ** -8,
                  1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20], dtype=np.float32),
    ])
    ours = W.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = W.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(a).to(torch.bfloat16).float().numpy())
    nan = W.f32_to_bf16_bits(np.array([np.nan], dtype=np.float32))
    assert np.isnan(W.bf16_bits_to_f32(nan)[0])


def test_workload_deterministic_and_shaped():
    a = W.make("tiny")
    b = W.make("tiny")
    for k in ("x1", "x2", "v", "log_poles", "residues", "skip"):
        assert np.array_equal(getattr(a, k), getattr(b, k)), k
    assert a.x1.shape == (1, 64, 1024) and a.x1.dtype == np.float32
    assert a.log_poles.shape == (64, 16) and a.log_poles.dtype == np.float32
    assert np.all(a.log_poles < 0) and np.all(a.log_poles >= -1.0)
    assert np.all(a.log_poles <= -1e-3 * (1 - 1e-6))
    c = W.make("7b_layer_set", D=8, L=256)
    assert c.x1.dtype == np.uint16 and c.x1.shape == (1, 8, 256)
    # bf16 configs: skip and taps are bf16-representable fp32
    for arr in (c.skip, c.taps[7], c.taps[128]):
        assert np.array_equal(W.bf16_bits_to_f32(W.f32_to_bf16_bits(arr)), arr)
    assert c.taps[7].shape == (8, 7) and c.taps[128].shape == (8, 128)


def test_workload_distributions():
    w = W.make("32k_chunked", D=64, L=4096)
    x = w.f64("x1")
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    assert abs(w.residues.std() - 0.25) < 0.02
    w5 = W.make("262k", D=256, L=64)
    lo = np.log(-w5.log_poles.astype(np.float64))
    assert lo.min() >= math.log(1e-5) - 1e-6 and lo.max() <= 1e-6
    assert lo.min() < math.log(1e-4)          # slow decays present
    w4 = W.make("40b_shaped", D=64, L=512)
    assert w4.scale.min() >= 1.0 and w4.scale.max() <= 1e12
    ch = np.sqrt(np.mean(w4.f64("x1") ** 2, axis=-1))[0]
    assert np.allclose(ch / w4.scale, 1.0, rtol=0.15)


def test_row_blocks_are_independent_of_threading():
    a = W._draw_rows(np.random.SeedSequence(5), 200, 100, threads=1)
    b = W._draw_rows(np.random.SeedSequence(5), 200, 100, threads=4)
    assert np.array_equal(a, b)


def test_metrics_constructed():
    rng = np.random.default_rng(1)
    ref = rng.normal(size=(3, 4, 500))
    m = M.compare(ref, ref)
    assert m["rel_l2"] == 0 and m["elem_rel"] == 0 and m["nonfinite"] == 0
    eps = 1e-3
    m = M.compare(ref * (1 + eps), ref)
    assert abs(m["rel_l2"] - eps) < 1e-12 and abs(m["rel_l2_ch"] - eps) < 1e-12
    assert m["elem_rel"] <= eps * (1 + 1e-9)
    y = ref.copy()
    y[1, 2, 3] = np.nan
    y[0, 0, 0] = np.inf
    assert M.compare(y, ref)["nonfinite"] == 2
    assert not M.passes(M.compare(y, ref))
    # channel equalisation: a tiny channel with a large relative error shows up
    ref2 = ref.copy()
    ref2[0, 0] *= 1e-9
    y2 = ref2.copy()
    y2[0, 0] *= 1.1
    m2 = M.compare(y2, ref2)
    assert m2["rel_l2"] < 1e-9 and m2["rel_l2_ch"] > 0.1 / math.sqrt(12) * 0.99
    # the floor: an error of 1e-4 * rms at a zero crossing stays bounded
    ref3 = np.ones((1, 100))
    ref3[0, 50] = 0.0
    y3 = ref3.copy()
    y3[0, 50] = 1e-4
    assert abs(M.compare(y3, ref3)["elem_rel"] - 1e-4 / (1e-3 * math.sqrt(0.99))) < 1e-6


def test_bf16_rounding_floor_within_gate():
    """Rounding the exact answer to bf16 alone must pass the gates with margin."""
    rng = np.random.default_rng(2)
    ref = rng.normal(size=(64, 4096)) * np.exp(rng.uniform(0, 20, 64))[:, None]
    y = W.bf16_bits_to_f32(W.f32_to_bf16_bits(ref.astype(np.float32))).astype(np.float64)
    m = M.compare(y, ref)
    assert 1.2e-3 < m["rel_l2_ch"] < 1.8e-3, m
    assert M.passes(m)
