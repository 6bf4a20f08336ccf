"""Random-sign Walsh-Hadamard rotation, as a dense matrix.

Roadmap §1: the first stage rotates each vector with a (random) Walsh-Hadamard
transform so that the coordinates become nearly independent and concentrated.
Roadmap §4.2: the forward rotation is D2 @ H @ D1 applied to the vector, and
its inverse is D1 @ H @ D2 (the sign-vector order the SGLang review caught).
iThome, "the core idea of TurboQuant": the rotation (a fast Hadamard
transform) preserves norms and geometry.

Reading: H is the Sylvester-ordered Hadamard matrix H[i, j] =
(-1)^popcount(i & j), scaled by 1/sqrt(d) so that it is orthogonal; D1 and D2
are diagonal +-1 matrices.  The oracle builds Pi = D2 (H / sqrt d) D1 and
multiplies by it; it never uses a fast transform.
"""

from __future__ import annotations

import functools

import numpy as np

__all__ = ["hadamard", "rotation_matrix", "inverse_rotation_matrix", "rotate"]


def hadamard(d: int) -> np.ndarray:
    """Unnormalised Sylvester Hadamard matrix, H[i, j] = (-1)^popcount(i & j)."""
    return _hadamard(d).copy()


@functools.lru_cache(maxsize=None)
def _hadamard(d: int) -> np.ndarray:
    if d <= 0 or d & (d - 1):
        raise ValueError("d must be a power of two")
    i = np.arange(d, dtype=np.int64)
    both = i[:, None] & i[None, :]
    pop = np.zeros_like(both)
    x = both.copy()
    while np.any(x):
        pop += x & 1
        x >>= 1
    return np.where(pop % 2 == 0, 1.0, -1.0)


def rotation_matrix(d1, d2) -> np.ndarray:
    """Pi = D2 (H / sqrt d) D1 with D1 = diag(d1), D2 = diag(d2)."""
    d1 = np.asarray(d1, dtype=np.float64)
    d2 = np.asarray(d2, dtype=np.float64)
    d = d1.shape[0]
    return np.diag(d2) @ (hadamard(d) / np.sqrt(d)) @ np.diag(d1)


def inverse_rotation_matrix(d1, d2) -> np.ndarray:
    """Pi^-1 = D1 (H / sqrt d) D2 (Roadmap §4.2)."""
    d1 = np.asarray(d1, dtype=np.float64)
    d2 = np.asarray(d2, dtype=np.float64)
    d = d1.shape[0]
    return np.diag(d1) @ (hadamard(d) / np.sqrt(d)) @ np.diag(d2)


def rotate(x, d1, d2) -> np.ndarray:
    """Pi x for each row of x (shape [..., d])."""
    x = np.asarray(x, dtype=np.float64)
    return x @ rotation_matrix(d1, d2).T
