"""The oracle process pool used by the full-size GPU checks: comparing block
of channels by block, in worker processes that regenerate their channels,
gives the metrics oracle.compare gives on the whole array (no GPU needed)."""
import numpy as np
import pytest

import oracle
import workloads as W
from tests import oracle_pool


@pytest.fixture(scope="module", autouse=True)
def stop_pool():
    yield
    oracle_pool.shutdown()


def test_channel_subset_draw_equals_full_draw():
    w = W.make("40b_shaped", B=2, D=300, L=100)
    for c0, c1 in [(0, 300), (5, 70), (64, 128), (299, 300), (130, 257)]:
        p = W.make("40b_shaped", B=2, D=300, L=100, channels=(c0, c1))
        for k in ("x1", "x2", "v"):
            assert np.array_equal(getattr(p, k), getattr(w, k)[:, c0:c1]), (k, c0, c1)
        assert np.array_equal(p.log_poles, w.log_poles[c0:c1])
        assert np.array_equal(p.residues, w.residues[c0:c1])
        assert np.array_equal(p.taps[7], w.taps[7][c0:c1])
        assert np.array_equal(p.scale, w.scale[c0:c1]) and p.D == c1 - c0


def _close(a, b):
    for k in ("rel_l2", "rel_l2_ch", "rel_l2_ch_max", "elem_rel"):
        assert a[k] == pytest.approx(b[k], rel=1e-12, abs=0), k
    assert a["nonfinite"] == b["nonfinite"]


def test_pool_blocks_equal_whole_array_metrics():
    ov = dict(B=2, D=130, L=300)
    w = W.make("7b_layer_set", **ov)
    x1, x2, v = w.f64("x1"), w.f64("x2"), w.f64("v")
    lam, R, sk = (a.astype(np.float64) for a in (w.log_poles, w.residues, w.skip))
    rng = np.random.default_rng(5)
    ref = oracle.hyena_fwd(x1, x2, v, lam, R, sk)
    # results with errors of known size, one non-finite element, stored as
    # the kernels store them
    y = W.f32_to_bf16_bits((ref * (1 + 3e-3 * rng.standard_normal(ref.shape))).astype(np.float32))
    y[1, 77, 5] = 0x7FC0                                      # NaN
    s_ref = oracle.modal_state(x1 * v, lam)
    s = (s_ref * (1 + 1e-5 * rng.standard_normal(s_ref.shape))).astype(np.float32)
    yc_ref, sc_ref = oracle.chunk_fwd(x1, x2, v, lam, R, sk, 100)
    yc = W.f32_to_bf16_bits(yc_ref.astype(np.float32))
    yf_ref = oracle.fir_fwd(x1, x2, v, w.taps[7].astype(np.float64), sk)
    yf = (yf_ref * (1 + 1e-4 * rng.standard_normal(yf_ref.shape))).astype(np.float32)
    jobs = [("modal", "m", y), ("modal_state", "s", s), ("chunk", "c", 100, yc, sc_ref.astype(np.float32)),
            ("fir", "f", 7, yf)]
    got = oracle_pool.check("7b_layer_set", jobs, range(w.D), overrides=ov, block=64)
    _close(got["m"]["y"], oracle.compare(W.to_f64(y, "bf16"), ref))
    assert got["m"]["y"]["nonfinite"] == 1
    _close(got["c"]["y"], oracle.compare(W.to_f64(yc, "bf16"), yc_ref))
    _close(got["f"]["y"], oracle.compare(yf.astype(np.float64), yf_ref))
    num = np.sum((s.astype(np.float64) - s_ref) ** 2, -1)
    den = np.sum(s_ref ** 2, -1)
    assert got["s"]["state"] == pytest.approx(float(np.sqrt(np.mean(num / den))), rel=1e-12)
    assert got["c"]["state"] < 1e-6
    # a scattered channel subset: the metrics of those channels alone
    rows = [0, 5, 63, 64, 65, 129]
    sub = oracle_pool.check("7b_layer_set", [("modal", "m", y)], rows, overrides=ov)
    _close(sub["m"]["y"], oracle.compare(W.to_f64(y[:, rows], "bf16"), ref[:, rows]))
