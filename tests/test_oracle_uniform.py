"""Pins for the equally spaced key codebook (Roadmap §4.3, the "tq4u" mode:
dequantisation idx * step + c0 instead of a Lloyd-Max lookup).

The step is the reading "least mean squared error for the rotated-coordinate
law" (the page fixes only the equal spacing).  Pinned by:
* minimality of the distortion, evaluated by numerical quadrature of the
  density (independent of the closed-form cell moments the solver uses);
* the large-d limit sqrt(d) * step -> Max's optimum uniform Gaussian step
  (tests/golden/gaussian_uniform_quantizer.txt, Max 1960 Table II), and the
  same limit for the distortion;
* equal spacing, odd symmetry and a zero middle threshold;
* its distortion above the Lloyd-Max codebook's, as optimality of the latter
  requires, and the empirical MSE of random unit vectors.
"""

import os

import numpy as np
import pytest
from scipy import integrate

from oracle import codebook, rotation

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "gaussian_uniform_quantizer.txt")


def _golden():
    rows = {}
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        b, step, mse = line.split()
        rows[int(b)] = (float(step), float(mse))
    return rows


def _quad_distortion(d, step, bits):
    """d * E[(U - Q(U))^2] by adaptive quadrature of the density."""
    L = 1 << bits
    a = np.arange(L) - 0.5 * (L - 1)
    edges = np.concatenate(([-1.0], np.clip((a[:-1] + 0.5) * step, -1, 1), [1.0]))
    tot = 0.0
    for k in range(L):
        ck = a[k] * step
        val, _ = integrate.quad(lambda u: (u - ck) ** 2 * codebook.density(u, d), edges[k], edges[k + 1],
                                epsabs=1e-16, epsrel=1e-13, limit=200)
        tot += val
    return d * tot


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_step_minimises_the_distortion(bits):
    d = 128
    _, _, step = codebook.uniform(d, bits)
    d0 = _quad_distortion(d, step, bits)
    for rel in (1e-3, 1e-2, 5e-2):
        assert _quad_distortion(d, step * (1 + rel), bits) > d0
        assert _quad_distortion(d, step * (1 - rel), bits) > d0
    # the closed form agrees with the quadrature
    c, t, _ = codebook.uniform(d, bits)
    assert abs(codebook.distortion(d, c, t) - d0) < 1e-9 * d0


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_large_d_limit_is_the_gaussian_optimum_uniform_quantiser(bits):
    step_g, mse_g = _golden()[bits]
    d = 1 << 16
    c, t, step = codebook.uniform(d, bits)
    assert abs(step * np.sqrt(d) - step_g) < 1.5e-3
    assert abs(codebook.distortion(d, c, t) - mse_g) < 1.5e-3 * mse_g + 5e-5


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_equal_spacing_symmetry_and_tables(d, bits):
    c, t, step = codebook.uniform(d, bits)
    L = 1 << bits
    assert np.allclose(np.diff(c), step, rtol=1e-14, atol=0)
    assert np.array_equal(c, -c[::-1])
    assert t[L // 2 - 1] == 0.0
    c32, t32 = codebook.tables_fp32(d, bits, uniform_codebook=True)
    assert np.array_equal(c32, -c32[::-1]) and np.array_equal(t32, -t32[::-1])
    assert np.all(np.diff(c32) > 0) and np.all((t32 > c32[:-1]) & (t32 < c32[1:]))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_uniform_is_worse_than_lloyd_max_and_matches_empirical_mse(bits):
    d = 128
    cu, tu, _ = codebook.uniform(d, bits)
    cl, tl, _ = codebook.lloyd_max(d, bits)
    Du, Dl = codebook.distortion(d, cu, tu), codebook.distortion(d, cl, tl)
    assert Du > Dl
    # Gaussian-limit ratio of the two (Max's tables: 1.011, 1.084, 1.215)
    assert Du / Dl < {2: 1.03, 3: 1.10, 4: 1.25}[bits]
    rng = np.random.default_rng(101 + bits)
    X = rng.standard_normal((20000, d))
    U = X / np.linalg.norm(X, axis=1, keepdims=True)
    d1 = rng.choice([-1.0, 1.0], d)
    d2 = rng.choice([-1.0, 1.0], d)
    U = rotation.rotate(U, d1, d2)
    c32, t32 = codebook.tables_fp32(d, bits, uniform_codebook=True)
    idx = np.sum(U[:, :, None] > t32.astype(np.float64)[None, None, :], axis=2)
    mse = np.mean(np.sum((U - c32.astype(np.float64)[idx]) ** 2, axis=1))
    assert abs(mse - Du) < 0.02 * Du
