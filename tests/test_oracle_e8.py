"""Pins of the oracle's nearest-E8 quantizer against brute force, lattice invariants and the
lattice's known second moment (normalized rows quantized on the E8 lattice, EntroPack paper,
Abstract). The oracle is reached through its C library; nothing here shares its code."""
import itertools

import numpy as np
import pytest

import oracle

OFFS = np.array(list(itertools.product((-1.0, 0.0, 1.0), repeat=8)))      # 3^8 neighbours


def brute_min_dist(y: np.ndarray) -> np.ndarray:
    """Smallest squared distance from each y (n, 8) to E8 = D8 u (D8 + 1/2), by enumeration.
    A nearest point of either coset lies within 1 of y in every coordinate (else moving that
    coordinate by 2 keeps the parity and gets strictly closer), so the coset's nearest point is
    among round(y - shift) + shift + {-1, 0, 1}^8."""
    best = np.full(len(y), np.inf)
    for shift in (0.0, 0.5):
        base = np.round(y - shift)
        for lo in range(0, len(y), 200):
            cand = base[lo:lo + 200, None, :] + OFFS[None]                 # integer part
            ok = (cand.sum(-1) % 2) == 0                                   # D8: even sum
            d = ((y[lo:lo + 200, None, :] - (cand + shift)) ** 2).sum(-1)
            d = np.where(ok, d, np.inf)
            best[lo:lo + 200] = np.minimum(best[lo:lo + 200], d.min(1))
    return best


def check_lattice(q: np.ndarray, b: np.ndarray):
    par = q & 1
    assert np.all(par == b[:, None]), "all coordinates share the coset parity"
    assert np.all(q.sum(1) % 4 == 0), "doubled E8 points have coordinate sum = 0 mod 4"


def test_e8_matches_brute_force_random():
    rng = np.random.default_rng(11)
    y = np.concatenate([rng.uniform(-4, 4, (2500, 8)), rng.normal(0, 3, (1000, 8))])
    q, b = oracle.e8_nearest(y)
    check_lattice(q, b)
    d = ((y - q / 2.0) ** 2).sum(1)
    assert np.all(d <= brute_min_dist(y) + 1e-12)
    assert np.all(d <= 1.0 + 1e-12), "covering radius of E8 is 1"


def test_e8_matches_brute_force_ties():
    rng = np.random.default_rng(12)
    half = rng.integers(-6, 7, (600, 8)) / 2.0                  # half-integer grid: rounding ties
    quarter = rng.integers(-12, 13, (600, 8)) / 4.0             # coset-distance ties
    odd = rng.integers(-5, 6, (300, 8)).astype(float)
    odd[:, 0] += (odd.sum(1) % 2 == 0)                          # integer vectors with odd sum
    y = np.concatenate([half, quarter, odd])
    q, b = oracle.e8_nearest(y)
    check_lattice(q, b)
    d = ((y - q / 2.0) ** 2).sum(1)
    assert np.all(d <= brute_min_dist(y) + 1e-12)


def test_e8_tie_rules():
    # equal distance to both cosets -> integer coset
    q, b = oracle.e8_nearest(np.full((1, 8), 0.25))
    assert b[0] == 0 and np.all(q == 0)
    # odd rounding sum, three equal rounding errors: the lowest index moves back towards y
    q, b = oracle.e8_nearest(np.array([[0.6, 0.6, 0.6, 0, 0, 0, 0, 0]]))
    assert b[0] == 0 and list(q[0]) == [0, 2, 2, 0, 0, 0, 0, 0]
    # an integer vector with odd sum: all errors are zero -> coordinate 0 moves up
    q, b = oracle.e8_nearest(np.array([[1.0, 0, 0, 0, 0, 0, 0, 0]]))
    assert b[0] == 0 and list(q[0]) == [4, 0, 0, 0, 0, 0, 0, 0]
    # a half-integer point is its own nearest point, in coset 1
    q, b = oracle.e8_nearest(np.array([[0.5, -0.5, 0.5, -0.5, 0.5, -0.5, 0.5, 1.5]]))
    assert b[0] == 1 and list(q[0]) == [1, -1, 1, -1, 1, -1, 1, 3]


def test_e8_idempotent_on_lattice_points():
    rng = np.random.default_rng(13)
    a = rng.integers(-5, 6, (2000, 8)).astype(float)
    a[:, 7] += a.sum(1) % 2                                     # D8 points
    pts = np.concatenate([a, a + 0.5])                          # and D8 + 1/2
    q, b = oracle.e8_nearest(pts)
    assert np.array_equal(q / 2.0, pts)
    assert np.array_equal(b, np.r_[np.zeros(2000), np.ones(2000)].astype(np.int32))


def test_e8_second_moment():
    """Uniform input over a large box: mean squared error per dimension -> G(E8) = 0.0716821...
    (Conway & Sloane's normalized second moment; unimodular E8 has volume 1). The cubic lattice
    Z^8 would give 1/12 = 0.0833."""
    rng = np.random.default_rng(14)
    y = rng.uniform(-50, 50, (200000, 8))
    q, _ = oracle.e8_nearest(y)
    mse = ((y - q / 2.0) ** 2).sum(1).mean() / 8.0
    assert mse == pytest.approx(0.0716821, rel=0.01)
