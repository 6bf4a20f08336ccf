"""Pins for the oracle's random-sign Hadamard rotation (Roadmap §1, §4.2;
iThome "the core idea of TurboQuant": norms and geometry are preserved)."""

import numpy as np
import pytest
import scipy.linalg

from oracle import rotation


def _butterfly(x):
    """Independent fast Walsh-Hadamard transform (in-place butterflies)."""
    y = np.array(x, dtype=np.float64, copy=True)
    d = y.shape[-1]
    h = 1
    while h < d:
        y = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(y.shape[:-3] + (d,))
        h *= 2
    return y


@pytest.mark.parametrize("d", [2, 8, 128, 256])
def test_hadamard_is_sylvester_library_matrix(d):
    # scipy.linalg.hadamard builds the Sylvester construction H_2n = [[H, H], [H, -H]].
    assert np.array_equal(rotation.hadamard(d), scipy.linalg.hadamard(d).astype(np.float64))


@pytest.mark.parametrize("d", [128, 256])
def test_scaled_hadamard_is_an_involution(d):
    H = rotation.hadamard(d) / np.sqrt(d)
    assert np.allclose(H @ H, np.eye(d), atol=1e-12)


@pytest.mark.parametrize("d", [128, 256])
def test_rotation_orthogonal_and_norm_preserving(d):
    rng = np.random.default_rng(1)
    d1 = rng.choice([-1.0, 1.0], d)
    d2 = rng.choice([-1.0, 1.0], d)
    P = rotation.rotation_matrix(d1, d2)
    assert np.allclose(P @ P.T, np.eye(d), atol=1e-12)
    x = rng.standard_normal((50, d)) * 7.0
    y = rotation.rotate(x, d1, d2)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)
    # inner products (geometry) are preserved too
    assert np.allclose(y @ y.T, x @ x.T, atol=1e-9)


@pytest.mark.parametrize("d", [128, 256])
def test_rotation_equals_signed_butterfly(d):
    # forward = D2 H D1 x / sqrt(d): signs d1 applied first, d2 last (Roadmap §4.2)
    rng = np.random.default_rng(2)
    d1 = rng.choice([-1.0, 1.0], d)
    d2 = rng.choice([-1.0, 1.0], d)
    x = rng.standard_normal((20, d))
    fast = d2 * _butterfly(d1 * x) / np.sqrt(d)
    assert np.allclose(rotation.rotate(x, d1, d2), fast, atol=1e-12)
    # the swapped order is a different map (catches an order mix-up)
    swapped = d1 * _butterfly(d2 * x) / np.sqrt(d)
    assert not np.allclose(rotation.rotate(x, d1, d2), swapped, atol=1e-6)


def test_inverse_is_d1_h_d2():
    d = 128
    rng = np.random.default_rng(3)
    d1 = rng.choice([-1.0, 1.0], d)
    d2 = rng.choice([-1.0, 1.0], d)
    P = rotation.rotation_matrix(d1, d2)
    Pinv = rotation.inverse_rotation_matrix(d1, d2)
    assert np.allclose(Pinv @ P, np.eye(d), atol=1e-12)
    # applying the forward order twice is not the inverse (the review's bug)
    assert not np.allclose(P @ P, np.eye(d), atol=1e-3)


def test_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        rotation.hadamard(96)
