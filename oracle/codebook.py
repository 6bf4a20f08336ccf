"""Lloyd-Max codebook for one coordinate of a randomly rotated unit vector.

Hub, "technical principle", steps 1-2: after the random orthogonal rotation
each coordinate of the (unit) key direction follows a Beta-type law, and the
method precomputes optimal (Lloyd-Max) scalar codebooks (here of 2, 3, 4 and,
for MSE-only keys, 8 bits) for head_dim 128 and 256; quantising a coordinate means finding its nearest
codeword.  iThome, "the core idea of TurboQuant": for MSE, each rotated
coordinate is given its closest optimal centroid.

The law of one coordinate U of a uniform point on the sphere S^(d-1) has
density  f(u) = (1-u^2)^((d-3)/2) / B(1/2, (d-1)/2)  on [-1, 1]; equivalently
(U+1)/2 ~ Beta(a, a) with a = (d-1)/2, which is the pages' "Beta distribution".

Lloyd's conditions (the textbook definition of a Lloyd-Max quantiser):
thresholds are midpoints of neighbouring centroids, and each centroid is the
conditional mean of U over its cell.  Both are evaluated here in closed form:

* cell mass  P(a < U <= b) = I_{(b+1)/2}(a, a) - I_{(a+1)/2}(a, a)
  (regularised incomplete beta);
* first moment  E[U 1{a<U<=b}] = ((1-a^2)^((d-1)/2) - (1-b^2)^((d-1)/2))
  / ((d-1) B(1/2, (d-1)/2))  (the antiderivative of u (1-u^2)^((d-3)/2)).

The density is even, so the optimal quantiser is odd-symmetric; each iterate
is averaged with its reflection so that symmetry (and a middle threshold of
exactly 0 for even level counts) holds to the last bit.
"""

from __future__ import annotations

import math

import numpy as np
from scipy import optimize, special

__all__ = [
    "beta_half",
    "density",
    "cell_mass",
    "cell_first_moment",
    "lloyd_max",
    "tables_fp32",
    "distortion",
]


def beta_half(d: int) -> float:
    """B(1/2, (d-1)/2), the normaliser of the coordinate density."""
    return math.exp(special.betaln(0.5, (d - 1) / 2.0))


def density(u, d: int):
    """f(u) = (1-u^2)^((d-3)/2) / B(1/2, (d-1)/2) on [-1, 1]."""
    u = np.asarray(u, dtype=np.float64)
    return np.power(np.clip(1.0 - u * u, 0.0, None), (d - 3) / 2.0) / beta_half(d)


def _cdf(x, d: int):
    """P(U <= x) through the Beta(a, a) law of (U+1)/2; upper tail when x > 0."""
    a = (d - 1) / 2.0
    x = np.asarray(x, dtype=np.float64)
    y = (x + 1.0) / 2.0
    lo = special.betainc(a, a, np.clip(y, 0.0, 1.0))
    hi = 1.0 - special.betaincc(a, a, np.clip(y, 0.0, 1.0))
    return np.where(x <= 0.0, lo, hi)


def _sf(x, d: int):
    """P(U > x)."""
    a = (d - 1) / 2.0
    x = np.asarray(x, dtype=np.float64)
    y = (x + 1.0) / 2.0
    return special.betaincc(a, a, np.clip(y, 0.0, 1.0))


def cell_mass(a, b, d: int):
    """P(a < U <= b).  Upper-tail differences are used right of 0 to keep
    relative accuracy in the outer cells."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    left = _cdf(b, d) - _cdf(a, d)
    right = _sf(a, d) - _sf(b, d)
    return np.where(a >= 0.0, right, left)


def cell_first_moment(a, b, d: int):
    """E[U 1{a < U <= b}] in closed form."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    e = (d - 1) / 2.0
    pa = np.power(np.clip(1.0 - a * a, 0.0, None), e)
    pb = np.power(np.clip(1.0 - b * b, 0.0, None), e)
    return (pa - pb) / ((d - 1) * beta_half(d))


def _initial_centroids(d: int, levels: int) -> np.ndarray:
    """Start from the conditional means of equal-mass cells (quantiles of the
    law), which never underflow the density."""
    a = (d - 1) / 2.0
    probs = np.arange(levels + 1, dtype=np.float64) / levels
    y = special.betaincinv(a, a, probs)
    edges = 2.0 * y - 1.0
    edges[0], edges[-1] = -1.0, 1.0
    return cell_first_moment(edges[:-1], edges[1:], d) / cell_mass(edges[:-1], edges[1:], d)


_SOLVED = {}  # (d, bits, tol, max_iter) -> (centroids, thresholds, iterations); the solve is deterministic


def lloyd_max(d: int, bits: int, tol: float = 1e-14, max_iter: int = 100000):
    """Lloyd-Max codebook (see _lloyd_max); solved once per argument set and
    returned as fresh copies."""
    key = (int(d), int(bits), float(tol), int(max_iter))
    if key not in _SOLVED:
        _SOLVED[key] = _lloyd_max(d, bits, tol, max_iter)
    c, t, it = _SOLVED[key]
    return c.copy(), t.copy(), it


def _lloyd_max(d: int, bits: int, tol: float, max_iter: int):
    """Run Lloyd's iteration to a fixed point.

    Stops when no centroid moves by more than ``tol`` times the largest
    centroid magnitude.  Returns ``(centroids, thresholds, iterations)`` in
    fp64, centroids ascending (index 0 the most negative), ``2**bits`` of
    them, and ``2**bits - 1`` thresholds (midpoints)."""
    levels = 1 << bits
    c = _initial_centroids(d, levels)
    c = 0.5 * (c - c[::-1])
    it = 0
    # beyond 4 bits Lloyd's iteration only brings the codebook near the fixed
    # point, which Newton's method then solves (see _newton_refine)
    for it in range(1, (max_iter if bits <= 4 else 200) + 1):
        t = 0.5 * (c[:-1] + c[1:])
        lo = np.concatenate(([-1.0], t))
        hi = np.concatenate((t, [1.0]))
        c_new = cell_first_moment(lo, hi, d) / cell_mass(lo, hi, d)
        c_new = 0.5 * (c_new - c_new[::-1])
        delta = float(np.max(np.abs(c_new - c)))
        c = c_new
        if delta <= tol * float(np.max(np.abs(c))):
            break
    if bits > 4:  # many levels: finish the fixed point by Newton's method
        c = _newton_refine(d, c)
    t = 0.5 * (c[:-1] + c[1:])
    return c, t, it


def _newton_refine(d: int, c: np.ndarray, tol: float = 1e-15, max_iter: int = 200) -> np.ndarray:
    """Solve Lloyd's conditions with Newton's method on the thresholds.

    Lloyd's iteration (above) converges slowly when there are many levels:
    its error shrinks by a factor ~1 - O(1/L^2) per step, so at 6-8 bits it
    stops far from the fixed point.  The fixed point is the same set of
    equations, F_j(t) = t_j - (c_j(t) + c_{j+1}(t)) / 2 = 0 for the L - 1
    thresholds, where c_k(t) is the conditional mean of cell k (bounded by
    t_{k-1} and t_k).  A cell's mean moves with its edges as
    dc_k/dt_k = f(t_k) (t_k - c_k) / P_k and dc_k/dt_{k-1} = f(t_{k-1})
    (c_k - t_{k-1}) / P_k (Leibniz's rule on E[U 1]/P), so the Jacobian is
    tridiagonal and each Newton step is one banded solve.  Steps are halved
    until the thresholds stay ordered inside (-1, 1) and the residual drops;
    the iterate is kept odd-symmetric.  Starts from the centroids ``c`` and
    returns the centroids of the solution."""
    from scipy.linalg import solve_banded

    L = len(c)
    t = 0.5 * (c[:-1] + c[1:])

    def cells(t):
        lo = np.concatenate(([-1.0], t))
        hi = np.concatenate((t, [1.0]))
        m = cell_mass(lo, hi, d)
        return m, cell_first_moment(lo, hi, d) / m

    def resid(t):
        m, cc = cells(t)
        return t - 0.5 * (cc[:-1] + cc[1:]), m, cc

    F, m, cc = resid(t)
    for _ in range(max_iter):
        if float(np.max(np.abs(F))) <= tol * float(np.max(np.abs(cc))):
            break
        ft = density(t, d)
        up = ft * (t - cc[:-1]) / m[:-1]    # dc_k / dt_k, cells k = 0 .. L-2
        lo = ft * (cc[1:] - t) / m[1:]      # dc_{k+1} / dt_k
        ab = np.zeros((3, L - 1))
        ab[0, 1:] = -0.5 * up[1:]           # dF_j / dt_{j+1} = -dc_{j+1}/dt_{j+1} / 2
        ab[1, :] = 1.0 - 0.5 * (up + lo)    # dF_j / dt_j
        ab[2, :-1] = -0.5 * lo[:-1]         # dF_{j+1} / dt_j = -dc_{j+1}/dt_j / 2
        delta = solve_banded((1, 1), ab, -F)
        lam = 1.0
        f0 = float(np.max(np.abs(F)))
        while True:
            tn = t + lam * delta
            tn = 0.5 * (tn - tn[::-1])
            if np.all(np.diff(tn) > 0.0) and tn[0] > -1.0 and tn[-1] < 1.0:
                Fn, mn, ccn = resid(tn)
                if float(np.max(np.abs(Fn))) < f0 or lam < 1e-6:
                    break
            lam *= 0.5
            if lam < 1e-12:
                return cc
        t, F, m, cc = tn, Fn, mn, ccn
    return 0.5 * (cc - cc[::-1])


def uniform(d: int, bits: int):
    """Equally spaced codebook (Roadmap §4.3, the "tq4u" mode: centroids
    idx * step + c0).  The page does not say how the step is chosen; the
    reading here is the step of least mean squared error for the rotated
    coordinate law, with c0 = -(L - 1) step / 2 (a symmetric codebook) and
    thresholds at the midpoints.

    With c_k = a_k step, a_k = k - (L - 1)/2, the distortion
    D(step) = sum_k E[(U - a_k step)^2 1{U in cell k}] has
    dD/dstep = -2 sum_k a_k (E[U 1{cell k}] - a_k step P(cell k)) (the moving
    midpoints contribute nothing: both neighbouring centroids are equally far
    from them), so the optimum is the root of that sum, found by Brent's
    method.  Returns ``(centroids, thresholds, step)`` in fp64."""
    levels = 1 << bits
    a = np.arange(levels, dtype=np.float64) - 0.5 * (levels - 1)

    def dist_slope(step):
        mids = np.clip((a[:-1] + 0.5) * step, -1.0, 1.0)  # cell edges cut to the support
        lo = np.concatenate(([-1.0], mids))
        hi = np.concatenate((mids, [1.0]))
        return float(np.sum(a * (cell_first_moment(lo, hi, d) - a * step * cell_mass(lo, hi, d))))

    step = optimize.brentq(dist_slope, 1e-4 / np.sqrt(d), 8.0 / np.sqrt(d), xtol=1e-300, rtol=8.9e-16, maxiter=500)
    c = a * step
    t = 0.5 * (c[:-1] + c[1:])
    return c, t, step


def tables_fp32(d: int, bits: int, uniform_codebook: bool = False):
    """The stored tables: fp32 centroids and fp32 thresholds, where each
    threshold is the fp32 rounding of the fp64 midpoint (of the Lloyd-Max
    codebook, or of the equally spaced one)."""
    c, t, _ = uniform(d, bits) if uniform_codebook else lloyd_max(d, bits)
    return c.astype(np.float32), t.astype(np.float32)


def distortion(d: int, centroids, thresholds) -> float:
    """Total distortion d * E[(U - Q(U))^2] of the quantiser, in closed form.

    Per cell (a, b] with centroid c it is  E[U^2 1] - 2 c E[U 1] + c^2 P.
    Integrating u * u (1-u^2)^((d-3)/2) by parts gives
    E[U^2 1{a<U<=b}] = (a (1-a^2)^((d-1)/2) - b (1-b^2)^((d-1)/2)) / (d B)
    + P(a<U<=b) / d, with B = B(1/2, (d-1)/2); over [-1, 1] this is 1/d."""
    c = np.asarray(centroids, dtype=np.float64)
    t = np.asarray(thresholds, dtype=np.float64)
    lo = np.concatenate(([-1.0], t))
    hi = np.concatenate((t, [1.0]))
    e = (d - 1) / 2.0
    bh = beta_half(d)
    mass = cell_mass(lo, hi, d)
    m1 = cell_first_moment(lo, hi, d)
    pa = np.power(np.clip(1.0 - lo * lo, 0.0, None), e)
    pb = np.power(np.clip(1.0 - hi * hi, 0.0, None), e)
    m2 = (lo * pa - hi * pb) / (d * bh) + mass / d
    per_coord = float(np.sum(m2 - 2.0 * c * m1 + c * c * mass))
    return d * per_coord
