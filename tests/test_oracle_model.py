"""Pins of the oracle's symbol model (a conditional model of the E8 lattice coordinates, EntroPack
paper, Abstract) and of its sampled rate search (the step size picked from a storage estimate on
a sample, same passage). Pins: normalization invariants, closed forms for a Gaussian source, monotonicity of
the estimate, and the target being met by the coded payload."""
import numpy as np
import pytest

import oracle
from decode_tile_interleaved_rans_amd import workloads as W


@pytest.mark.parametrize("n", [10, 11, 12])
def test_normalize_invariants(n):
    rng = np.random.default_rng(n)
    M = 1 << n
    cases = [
        rng.integers(0, 1000, 256),                                   # dense
        np.r_[10 ** 7, np.ones(255, np.int64)],                       # one huge + many singletons
        np.r_[np.zeros(100, np.int64), 5, np.zeros(155, np.int64)],   # single present symbol
        (rng.pareto(1.2, 256) * 10).astype(np.int64) * (rng.random(256) < 0.5),
    ]
    for c in cases:
        f = oracle.normalize(c, n)
        assert int(f.sum()) == M
        assert np.all((f > 0) == (np.asarray(c) > 0)), "f >= 1 exactly where the symbol occurs"
    f = oracle.normalize(np.zeros(256, np.int64), n)
    assert f[0] == M and f[1:].sum() == 0, "an empty table codes nothing and is all mass on 0"


def test_normalize_rules_closed_form():
    n = 12
    # floor(c M / T) already sums to M: unchanged
    f = oracle.normalize([1, 1, 2], n)
    assert list(f[:3]) == [1024, 1024, 2048]
    # shortfall of 1 goes to the largest count (lowest index on ties)
    f = oracle.normalize([1, 1, 1], n)
    assert list(f[:3]) == [1366, 1365, 1365]
    # excess from bumping singletons to 1 is taken from the largest frequency
    c = np.r_[10 ** 9, np.ones(200, np.int64)]
    f = oracle.normalize(c, n)
    assert f[0] == 4096 - 200 and np.all(f[1:201] == 1)


def gaussian_rows(R=512, C=2048, seed=0):
    rng = np.random.default_rng(seed)
    return rng.normal(0, 1, (R, C)).astype(np.float32)


def test_estimate_gaussian_closed_form():
    """High-resolution E8 coding of unit-RMS Gaussian rows: the entropy per weight is
    h(N(0,1)) - log2(step) = 2.0471 - log2(step) bits for the joint lattice point (E8 has unit
    volume); coding the coset bit plus per-position marginals gives up at most the coordinate
    parity (1 bit per 8-block, 0.125 bit per weight)."""
    w = gaussian_rows()
    for step in (0.05, 0.1, 0.2):
        est = oracle.estimate_bpp(w, step)
        ideal = 0.5 * np.log2(2 * np.pi * np.e) - np.log2(step)
        assert ideal - 0.02 <= est <= ideal + 0.125 + 0.03, (step, est, ideal)


@pytest.mark.parametrize("maker", ["gauss", "t5"])
def test_estimate_non_increasing_in_step(maker):
    w = W.gaussian_with_outliers(512, 1024, seed=3) if maker == "gauss" else \
        W.bf16_bits_to_f32(W.student_t(512, 1024, 4)).copy()
    steps = np.geomspace(0.02, 8.0, 40)
    est = np.array([oracle.estimate_bpp(w, s) for s in steps])
    assert np.all(np.diff(est) <= 1e-9), est


@pytest.mark.parametrize("target", [2.5, 4.0, 6.0])
def test_select_step_meets_target(target):
    w = W.gaussian_with_outliers(1024, 1024, seed=1)
    step = oracle.select_step(w, target)
    assert oracle.estimate_bpp(w, step) <= target + 1e-3
    assert oracle.estimate_bpp(w, step * 0.99) > target - 0.05   # not far from the boundary


def test_gaussian_quality_closed_form():
    """Per-row RMS error of the normalized rows ~ sqrt(G(E8)) * step = 0.26774 * step at high
    resolution (G(E8) = 0.0716821)."""
    w = gaussian_rows(256, 2048, 1)
    s, _ = oracle.compress(w, 5.0)
    d = oracle.info(s)
    q, _ = oracle.decode_symbols(s)
    scale = np.sqrt((w.astype(np.float64) ** 2).mean(1))
    rec = q * (d["step"] / 2) * scale[:, None]
    err = np.sqrt(((rec - w) ** 2).mean(1)) / scale
    assert err.mean() == pytest.approx(np.sqrt(0.0716821) * d["step"], rel=0.05)


def test_row_scale_closed_form():
    w = np.zeros((3, 40), np.float32)
    w[0] = 3.0
    w[1, ::2] = -2.0
    assert oracle.row_scale(w, 0) == np.float32(3.0)
    assert oracle.row_scale(w, 1) == np.float32(np.sqrt(2.0))
    assert oracle.row_scale(w, 2) == 0.0
