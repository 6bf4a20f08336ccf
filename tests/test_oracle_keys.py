"""Pins for the oracle's key encoding and score estimator: nearest codeword
by brute force, the norm/direction split, QJL unbiasedness over many draws of
S (Roadmap §1; Hub "unbiased estimator"), and the bias of the MSE-only score
(Roadmap §1; Yage "step 3")."""

import math

import numpy as np
import pytest

from oracle import bits, codebook, keys, rotation


@pytest.fixture(scope="module")
def ctx128():
    rng = np.random.default_rng(11)
    d = 128
    d1 = rng.choice([-1.0, 1.0], d)
    d2 = rng.choice([-1.0, 1.0], d)
    S = rng.standard_normal((d, d)).astype(np.float32)
    c32, t32 = codebook.tables_fp32(d, 3)
    return d, d1, d2, S, c32, t32


def test_threshold_search_equals_brute_force_nearest(ctx128):
    d, d1, d2, S, c32, t32 = ctx128
    rng = np.random.default_rng(12)
    K = rng.standard_normal((4000, d))
    K[:, 5] *= 10.0
    enc = keys.encode_keys(K, d1, d2, S, c32, t32)
    u = enc["u"]
    c = c32.astype(np.float64)
    brute = np.argmin(np.abs(u[..., None] - c), axis=-1)  # lowest index on ties
    # away from the (fp32-rounded) midpoints the two must agree exactly
    near = np.min(np.abs(u[..., None] - t32.astype(np.float64)), axis=-1) < 1e-7
    assert np.array_equal(enc["idx"][~near], brute[~near])
    assert near.mean() < 1e-4


def test_exact_threshold_ties_go_to_lower_index():
    d = 8
    c32, t32 = codebook.tables_fp32(d, 2)
    d1 = np.ones(d)
    d2 = np.ones(d)
    S = np.eye(d, dtype=np.float32)
    # build a key whose rotated, normalised coordinates hit thresholds exactly:
    # u = Pi k / |k|; choose u first then k = Pi^T u * 3 (scale cancels).
    P = rotation.rotation_matrix(d1, d2)
    t = t32.astype(np.float64)
    u = np.array([t[0], t[1], t[2], -0.3, 0.3, 0.1, -0.1, 0.0])
    u /= np.linalg.norm(u)
    enc = keys.encode_keys((P.T @ u * 3.0)[None, :], d1, d2, S, c32, t32)
    expect = np.sum(enc["u"][0][:, None] > t[None, :], axis=1)
    assert np.array_equal(enc["idx"][0], expect)
    # a coordinate exactly on a threshold is not counted as above it
    k2 = np.zeros(d)
    k2[0] = 1.0  # u = d2 * H[:,0]/sqrt(d) * d1[0] -> all +-1/sqrt(8), none equal to a threshold
    enc2 = keys.encode_keys(k2[None, :], d1, d2, S, c32, t32)
    assert np.all(enc2["idx"][0] == np.sum(enc2["u"][0][:, None] > t[None, :], axis=1))


def test_norm_direction_split_and_fp16_metadata(ctx128):
    d, d1, d2, S, c32, t32 = ctx128
    rng = np.random.default_rng(13)
    K = rng.standard_normal((100, d)) * 3.0
    enc = keys.encode_keys(K, d1, d2, S, c32, t32)
    assert np.allclose(enc["n"], np.linalg.norm(K, axis=1), rtol=1e-14)
    assert np.allclose(np.linalg.norm(enc["u"], axis=1), 1.0, atol=1e-13)
    r = enc["u"] - c32.astype(np.float64)[enc["idx"]]
    assert np.allclose(enc["gamma"], np.linalg.norm(r, axis=1), rtol=1e-14)
    assert np.array_equal(enc["n16"], np.float16(enc["n"]).view(np.uint16))
    assert np.all(np.abs(bits.from_fp16_bits(enc["n16"]) / enc["n"] - 1) <= 2 ** -11)
    # sign bit is 1 exactly where S r >= 0
    z = r @ S.astype(np.float64).T
    assert np.array_equal(enc["sign"], (z >= 0).astype(np.uint8))


def test_zero_key_stores_zero_record(ctx128):
    d, d1, d2, S, c32, t32 = ctx128
    enc = keys.encode_keys(np.zeros((2, d)), d1, d2, S, c32, t32)
    assert not enc["idx"].any() and not enc["sign"].any()
    assert not enc["n16"].any() and not enc["g16"].any()
    est = keys.estimate_scores(np.ones(d), enc["idx"], enc["sign"], enc["n16"], enc["g16"], d1, d2, S, c32)
    assert np.all(est == 0.0)


def _qjl_term_variance(n, gamma, qt, r, d):
    # Var over S of n * sqrt(pi/2)/d * gamma * sum_i <S_i,qt> sign<S_i,r>:
    # each row contributes E[(<s,qt> sign<s,r>)^2] = |qt|^2 and mean
    # sqrt(2/pi) <qt,r>/|r|, so per draw Var = (n^2/d) ((pi/2) g^2 |qt|^2 - <qt,r>^2).
    return (n * n / d) * ((math.pi / 2) * gamma ** 2 * qt @ qt - (qt @ r) ** 2)


def test_qjl_estimator_is_unbiased_over_S():
    """Fix q, k and the rotation; draw S many times.  The full estimate
    (with fp64 n, gamma) averages to <q, k>; the MSE-only part does not."""
    d = 128
    rng = np.random.default_rng(21)
    d1 = rng.choice([-1.0, 1.0], d)
    d2 = rng.choice([-1.0, 1.0], d)
    c32, t32 = codebook.tables_fp32(d, 2)
    k = rng.standard_normal(d)
    q = 0.6 * k + rng.standard_normal(d)
    exact = q @ k
    N = 20000
    ests = np.empty(N)
    for i in range(N):
        S = rng.standard_normal((d, d)).astype(np.float32)
        enc = keys.encode_keys(k[None, :], d1, d2, S, c32, t32)
        qt, p = keys.query_tables(q, d1, d2, S)
        c = c32.astype(np.float64)
        mse = qt @ c[enc["idx"][0]]
        qjl = keys.QJL_SCALE(d) * enc["gamma"][0] * ((2.0 * enc["sign"][0] - 1.0) @ p)
        ests[i] = enc["n"][0] * (mse + qjl)
    enc = keys.encode_keys(k[None, :], d1, d2, S, c32, t32)
    qt = rotation.rotate(q, d1, d2)
    r = enc["u"][0] - c32.astype(np.float64)[enc["idx"][0]]
    sd = math.sqrt(_qjl_term_variance(enc["n"][0], enc["gamma"][0], qt, r, d))
    assert abs(ests.mean() - exact) < 4 * sd / math.sqrt(N)
    assert abs(ests.std() / sd - 1.0) < 0.05
    mse_only = enc["n"][0] * (qt @ c32.astype(np.float64)[enc["idx"][0]])
    assert abs(mse_only - exact) > 10 * sd / math.sqrt(N)


def test_mse_only_score_is_biased_towards_zero_over_rotations():
    """Averaged over random rotations the MSE-only inner product shrinks by
    about (1 - D) where D is the codebook's total distortion; adding the QJL
    term removes the shrinkage."""
    d = 128
    rng = np.random.default_rng(22)
    c32, t32 = codebook.tables_fp32(d, 3)
    c, t, _ = codebook.lloyd_max(d, 3)
    D = codebook.distortion(d, c, t)
    k = rng.standard_normal(d)
    q = k + 0.3 * rng.standard_normal(d)
    ratios_mse, ratios_full = [], []
    for _ in range(3000):
        d1 = rng.choice([-1.0, 1.0], d)
        d2 = rng.choice([-1.0, 1.0], d)
        S = rng.standard_normal((d, d)).astype(np.float32)
        enc = keys.encode_keys(k[None, :], d1, d2, S, c32, t32)
        qt, p = keys.query_tables(q, d1, d2, S)
        mse = enc["n"][0] * (qt @ c32.astype(np.float64)[enc["idx"][0]])
        full = mse + enc["n"][0] * keys.QJL_SCALE(d) * enc["gamma"][0] * ((2.0 * enc["sign"][0] - 1.0) @ p)
        ratios_mse.append(mse / (q @ k))
        ratios_full.append(full / (q @ k))
    assert abs(np.mean(ratios_mse) - (1 - D)) < 0.01
    assert abs(np.mean(ratios_full) - 1.0) < 0.01


def test_estimate_scores_uses_stored_fp16_metadata(ctx128):
    d, d1, d2, S, c32, t32 = ctx128
    rng = np.random.default_rng(23)
    K = rng.standard_normal((8, d))
    q = rng.standard_normal(d)
    enc = keys.encode_keys(K, d1, d2, S, c32, t32)
    est = keys.estimate_scores(q, enc["idx"], enc["sign"], enc["n16"], enc["g16"], d1, d2, S, c32)
    qt, p = keys.query_tables(q, d1, d2, S)
    n16 = bits.from_fp16_bits(enc["n16"])
    g16 = bits.from_fp16_bits(enc["g16"])
    for i in range(8):
        mse = sum(qt[j] * float(c32[enc["idx"][i, j]]) for j in range(d))
        pm = sum(p[j] * (1.0 if enc["sign"][i, j] else -1.0) for j in range(d))
        ref = n16[i] * (mse + math.sqrt(math.pi / 2) / d * g16[i] * pm)
        assert abs(est[i] - ref) < 1e-10 * max(1.0, abs(ref))
