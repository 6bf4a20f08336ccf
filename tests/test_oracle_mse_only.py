"""Pins for MSE-only keys (iThome, "which path vLLM actually takes": presets
that keep the Hadamard rotation and MSE-quantised keys and leave QJL out;
iThome, "the core idea": the MSE stage alone versus MSE plus the 1-bit QJL
residual for the inner product).

* the MSE-only score equals <q, k^> for the key reconstructed by the inverse
  rotation (Roadmap §4.2's D1 H D2 form), an independent route to the same
  number;
* its shrinkage towards zero over random rotations is (1 - D) at 3 and at 4
  bits, D the codebook's total distortion, while the QJL estimate of the
  same keys is unbiased;
* the record drops exactly the d/8 sign bytes and the 2-byte residual norm
  per token-head; a written record reads back field by field.
"""

import numpy as np
import pytest

from oracle import attention, bits, codebook, keys, paged, rotation, values


def test_mse_only_score_is_the_inner_product_with_the_reconstructed_key():
    d = 128
    rng = np.random.default_rng(61)
    d1 = rng.choice([-1.0, 1.0], d)
    d2 = rng.choice([-1.0, 1.0], d)
    S = rng.standard_normal((d, d)).astype(np.float32)
    c32, t32 = codebook.tables_fp32(d, 3)
    K = rng.standard_normal((16, d))
    K[:, 3] *= 10.0
    q = rng.standard_normal(d)
    enc = keys.encode_keys(K, d1, d2, S, c32, t32, qjl=False)
    assert not enc["sign"].any() and not enc["g16"].any()
    est = keys.estimate_scores(q, enc["idx"], enc["sign"], enc["n16"], enc["g16"], d1, d2, S, c32, qjl=False)
    Pinv = rotation.inverse_rotation_matrix(d1, d2)
    n16 = bits.from_fp16_bits(enc["n16"])
    khat = n16[:, None] * (c32.astype(np.float64)[enc["idx"]] @ Pinv.T)
    ref = khat @ q
    assert np.max(np.abs(est - ref)) < 1e-10 * np.max(np.abs(ref))
    # the codes are those of the full preset: QJL only adds fields
    full = keys.encode_keys(K, d1, d2, S, c32, t32)
    assert np.array_equal(full["idx"], enc["idx"]) and np.array_equal(full["n16"], enc["n16"])


@pytest.mark.parametrize("b", [3, 4])
def test_mse_only_shrinks_by_one_minus_distortion_qjl_does_not(b):
    d = 128
    rng = np.random.default_rng(62 + b)
    c32, t32 = codebook.tables_fp32(d, b)
    c, t, _ = codebook.lloyd_max(d, b)
    D = codebook.distortion(d, c, t)
    k = rng.standard_normal(d)
    q = k + 0.3 * rng.standard_normal(d)
    exact = q @ k
    r_mse, r_qjl = [], []
    for _ in range(2000):
        d1 = rng.choice([-1.0, 1.0], d)
        d2 = rng.choice([-1.0, 1.0], d)
        S = rng.standard_normal((d, d)).astype(np.float32)
        em = keys.encode_keys(k[None, :], d1, d2, S, c32, t32, qjl=False)
        ef = keys.encode_keys(k[None, :], d1, d2, S, c32, t32)
        sm = keys.estimate_scores(q, em["idx"], em["sign"], em["n16"], em["g16"], d1, d2, S, c32, qjl=False)[0]
        sf = keys.estimate_scores(q, ef["idx"], ef["sign"], ef["n16"], ef["g16"], d1, d2, S, c32)[0]
        r_mse.append(sm / exact)
        r_qjl.append(sf / exact)
    assert abs(np.mean(r_mse) - (1 - D)) < 0.004
    assert abs(np.mean(r_qjl) - 1.0) < 0.01
    # the shrinkage is large against its own spread
    assert (1 - np.mean(r_mse)) > 5 * np.std(r_mse) / np.sqrt(len(r_mse))


@pytest.mark.parametrize("bk,bv", [(3, 4), (4, 4), (3, 2), (2, 2)])
def test_mse_only_record_drops_the_sign_bits_and_residual_norm(bk, bv):
    for d in (128, 256):
        full = paged.layout(d, bk, bv)
        mse = paged.layout(d, bk, bv, qjl=False)
        assert full["bytes"] - mse["bytes"] == paged.BLOCK * (d // 8 + 2)
        per = mse["bytes"] // paged.BLOCK
        assert per == (bk + bv) * d // 8 + 2 + (d // 32) * 4
        for name in ("kcodes", "kmeta", "vcodes", "vmeta"):
            assert mse[name][0] % 16 == 0
    assert paged.layout(128, 3, 4, qjl=False)["bytes"] // paged.BLOCK == 130


def test_mse_only_record_round_trip_and_byte_placement():
    d, bk, bv, L = 128, 3, 4, 37
    rng = np.random.default_rng(64)
    d1 = rng.choice([-1.0, 1.0], d)
    d2 = rng.choice([-1.0, 1.0], d)
    S = rng.standard_normal((d, d)).astype(np.float32)
    c32, t32 = codebook.tables_fp32(d, bk)
    K = rng.standard_normal((L, d))
    V = rng.standard_normal((L, d)).astype(np.float32)
    lay = paged.layout(d, bk, bv, qjl=False)
    pool = paged.new_pool(8, 2, lay)
    bt = np.array([5, 2, 7], dtype=np.int64)
    t = np.arange(L)
    slots = bt[t // 16] * 16 + t % 16
    ke = keys.encode_keys(K, d1, d2, S, c32, t32, qjl=False)
    ve = values.encode_values(V, bv)
    paged.write_tokens(pool, slots, 1, ke, ve, lay)
    back = paged.read_tokens(pool, bt, L, 1, lay)
    assert np.array_equal(back["idx"], ke["idx"]) and np.array_equal(back["n16"], ke["n16"])
    assert np.array_equal(back["q"], ve["q"]) and np.array_equal(back["s16"], ve["s16"])
    assert not back["sign"].any() and not back["g16"].any()
    # n of token 20 (block bt[1], slot 4) sits at kmeta + 2 * 4, little-endian
    o = lay["kmeta"][0] + 2 * 4
    assert int(pool[2, 1, o]) | (int(pool[2, 1, o + 1]) << 8) == int(ke["n16"][20])
    # head 0 untouched
    assert not pool[:, 0].any()
    # decode through the layout equals decode straight from the encodings
    ctx = {"d1": d1, "d2": d2, "S": S, "c32": c32, "qjl": False}
    q = rng.standard_normal((4, d))
    fields = {k2: ke[k2] for k2 in ("idx", "sign", "n16", "g16")} | {k2: ve[k2] for k2 in ("q", "s16", "z16")}
    o1, s1 = attention.decode_one_sequence(q, [fields], ctx)
    o2, s2 = attention.decode_one_sequence(q, [back], ctx)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)
