"""Pins for the oracle's Lloyd-Max codebook (Hub, technical principle steps
1-2; Roadmap §6.3 distortion factor ~2.7)."""

import math
import os

import numpy as np
import pytest
from scipy import integrate

from oracle import codebook

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "gaussian_lloyd_max.txt")


def _max_table():
    rows = {}
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if not line:
            continue
        parts = line.split()
        b = int(parts[0])
        vals = [float(v) for v in parts[1:]]
        rows[b] = (np.array(vals[:-1]), vals[-1])
    return rows


def test_density_integrates_to_one_and_has_variance_1_over_d():
    for d in (128, 256):
        f = lambda u: codebook.density(u, d)
        m0, _ = integrate.quad(f, -1, 1, epsabs=1e-14, limit=200)
        m2, _ = integrate.quad(lambda u: u * u * f(u), -1, 1, epsabs=1e-15, limit=200)
        assert abs(m0 - 1.0) < 1e-12
        assert abs(m2 - 1.0 / d) < 1e-12


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("b", [2, 3, 4, 8])
def test_fixed_point_by_independent_quadrature(d, b):
    """Each centroid equals its cell's conditional mean and each threshold is
    the midpoint — the mean computed by adaptive quadrature of the density,
    not by the closed forms the solver uses."""
    c, t, it = codebook.lloyd_max(d, b)
    assert it < 200000
    assert np.allclose(t, 0.5 * (c[:-1] + c[1:]), atol=0, rtol=0)
    edges = np.concatenate(([-1.0], t, [1.0]))
    for k in range(len(c)):
        a, bb = edges[k], edges[k + 1]
        pts = [x for x in (-0.5, 0.0, 0.5) if a < x < bb]
        mass, _ = integrate.quad(lambda u: codebook.density(u, d), a, bb, epsabs=1e-15, epsrel=1e-13, limit=400, points=pts or None)
        m1, _ = integrate.quad(lambda u: u * codebook.density(u, d), a, bb, epsabs=1e-16, epsrel=1e-13, limit=400, points=pts or None)
        assert abs(m1 / mass - c[k]) < 1e-11 * max(1.0, abs(c[k])) + 1e-13


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("b", [1, 2, 3, 4, 8])
def test_symmetry_and_zero_middle_threshold(d, b):
    c, t, _ = codebook.lloyd_max(d, b)
    assert np.array_equal(c, -c[::-1])
    assert np.all(np.diff(c) > 0)
    assert t[len(t) // 2] == 0.0
    c32, t32 = codebook.tables_fp32(d, b)
    assert t32[len(t32) // 2] == 0.0 and np.array_equal(c32, -c32[::-1])


@pytest.mark.parametrize("d", [16, 128, 256])
def test_one_bit_closed_form(d):
    # E|U| = Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2)); the 1-bit optimum is +-E|U|.
    c, t, _ = codebook.lloyd_max(d, 1)
    ref = math.exp(math.lgamma(d / 2) - math.lgamma((d + 1) / 2)) / math.sqrt(math.pi)
    assert abs(c[1] - ref) < 1e-14 and t[0] == 0.0
    assert abs(ref - 0.0706616) < 5e-7 if d == 128 else True


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_large_d_limit_is_gaussian_lloyd_max(b):
    """sqrt(d) c tends to the N(0, 1) Lloyd-Max levels (Max 1960)."""
    levels, mse = _max_table()[b]
    d = 4096
    c, t, _ = codebook.lloyd_max(d, b, tol=1e-9)
    pos = np.sqrt(d) * c[len(c) // 2:]
    assert np.allclose(pos, levels, atol=2e-3)
    assert abs(codebook.distortion(d, c, t) - mse) < 3e-4


@pytest.mark.parametrize("d,b,ref", [(128, 2, 0.1160), (128, 3, 0.03397), (128, 4, 0.00932)])
def test_distortion_values_and_page_bound(d, b, ref):
    c, t, _ = codebook.lloyd_max(d, b)
    D = codebook.distortion(d, c, t)
    assert abs(D - ref) < 2e-4
    # within the ~2.7x factor of the 4^-b lower bound (Roadmap §6.3)
    assert 1.0 < D * 4 ** b <= 2.7


@pytest.mark.parametrize("b", [2, 3, 4])
def test_distortion_matches_monte_carlo_on_random_unit_vectors(b):
    """Empirical d * mean squared coordinate error of random unit vectors,
    quantised by nearest centroid, matches the closed-form distortion."""
    d = 128
    c, t, _ = codebook.lloyd_max(d, b)
    rng = np.random.default_rng(7)
    x = rng.standard_normal((20000, d))
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    q = c[np.argmin(np.abs(u[..., None] - c), axis=-1)]
    emp = np.mean(np.sum((u - q) ** 2, axis=1))
    D = codebook.distortion(d, c, t)
    se = np.std(np.sum((u - q) ** 2, axis=1)) / np.sqrt(len(u))
    assert abs(emp - D) < 4 * se


def test_mass_and_moment_closed_forms_against_quadrature():
    d = 128
    for a, b in [(-1.0, -0.2), (-0.05, 0.03), (0.1, 0.3), (0.25, 1.0)]:
        m, _ = integrate.quad(lambda u: codebook.density(u, d), a, b, epsabs=1e-15)
        m1, _ = integrate.quad(lambda u: u * codebook.density(u, d), a, b, epsabs=1e-16)
        assert abs(codebook.cell_mass(a, b, d) - m) < 1e-12
        assert abs(codebook.cell_first_moment(a, b, d) - m1) < 1e-13


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("b", [3, 4])
def test_newton_finish_leaves_a_converged_lloyd_codebook_in_place(d, b):
    """Where Lloyd's iteration converges (few levels), Newton's method on the
    same conditions starts at its fixed point and stays there."""
    c, _, _ = codebook.lloyd_max(d, b)
    assert np.max(np.abs(codebook._newton_refine(d, c) - c)) < 1e-12


@pytest.mark.parametrize("d", [128, 256])
def test_eight_bit_distortion_approaches_the_high_resolution_limit(d):
    """Many-level quantisers approach the Panter-Dite asymptote
    D ~ d (int f^(1/3))^3 / (12 L^2) of an optimal quantiser with L levels
    (a result independent of Lloyd's conditions): within 1 % at 256 levels,
    and the gap shrinks from 64 to 256 levels."""
    k, _ = integrate.quad(lambda u: codebook.density(u, d) ** (1.0 / 3.0), -1, 1, epsabs=1e-14, limit=400,
                          points=[-0.3, 0.0, 0.3])
    gaps = []
    for b in (6, 8):
        c, t, _ = codebook.lloyd_max(d, b)
        D = codebook.distortion(d, c, t)
        pd = d * k ** 3 / (12.0 * (1 << b) ** 2)
        gaps.append(abs(D / pd - 1.0))
    assert gaps[1] < 0.01 and gaps[1] < gaps[0]


def test_eight_bit_distortion_matches_monte_carlo_on_random_unit_vectors():
    d = 128
    c, t, _ = codebook.lloyd_max(d, 8)
    rng = np.random.default_rng(8)
    x = rng.standard_normal((4000, d))
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    # nearest centroid from the two centroids around each value (no thresholds)
    j = np.clip(np.searchsorted(c, u), 1, len(c) - 1)
    lo, hi = c[j - 1], c[j]
    q = np.where(np.abs(u - lo) <= np.abs(hi - u), lo, hi)
    err = np.sum((u - q) ** 2, axis=1)
    D = codebook.distortion(d, c, t)
    assert abs(np.mean(err) - D) < 4 * np.std(err) / np.sqrt(len(u))
