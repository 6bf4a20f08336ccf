"""Pins for rotated values with the inverse rotation folded into the output
projection (Roadmap §4.2, W_O weight absorption, and the sign-vector order
its code review caught: forward D2 H D1, inverse D1 H D2).

* the folded projection applied to rotated head outputs equals the original
  projection applied to the unrotated outputs (forward rotation built
  independently of the fold's inverse), for several heads;
* folding with the forward sign order instead (the bug the page describes)
  breaks that identity;
* on data with 0.5 % x20 outliers the rotated values quantise with a lower
  error than the plain ones (the reason to rotate them), at 2 and 4 bits;
* decode over a rotated-value cache followed by the folded projection equals
  the plain projection of the attention over the de-rotated values.
"""

import numpy as np
import pytest

import synth
from oracle import attention, codebook, keys, rotation, values


def _params(seed, d):
    rng = np.random.default_rng(seed)
    return rng.choice([-1.0, 1.0], d), rng.choice([-1.0, 1.0], d), rng


def test_folded_projection_restores_the_unrotated_output():
    d, H, rows = 128, 4, 64
    d1, d2, rng = _params(121, d)
    W = rng.standard_normal((rows, H * d))
    o = rng.standard_normal((H, d))
    P = rotation.rotation_matrix(d1, d2)
    o_rot = o @ P.T  # each head's output rotated forward
    Wf = attention.fold_output_projection(W, d1, d2, H)
    assert np.max(np.abs(Wf @ o_rot.reshape(-1) - W @ o.reshape(-1))) < 1e-10 * np.max(np.abs(W @ o.reshape(-1)))


def test_folding_with_the_forward_sign_order_is_wrong():
    d, H, rows = 128, 2, 16
    d1, d2, rng = _params(122, d)
    assert not np.array_equal(d1, d2)
    W = rng.standard_normal((rows, H * d))
    o = rng.standard_normal((H, d))
    o_rot = rotation.rotate(o, d1, d2)
    # the buggy fold: the forward matrix D2 H D1 where the inverse belongs
    wrong = np.concatenate([W[:, h * d:(h + 1) * d] @ rotation.rotation_matrix(d1, d2) for h in range(H)], axis=1)
    ref = W @ o.reshape(-1)
    assert np.max(np.abs(wrong @ o_rot.reshape(-1) - ref)) > 0.1 * np.max(np.abs(ref))
    right = attention.fold_output_projection(W, d1, d2, H)
    assert np.max(np.abs(right @ o_rot.reshape(-1) - ref)) < 1e-10 * np.max(np.abs(ref))


@pytest.mark.parametrize("b", [2, 4])
def test_rotated_values_quantise_better_with_outliers(b):
    d = 128
    d1, d2, rng = _params(123, d)
    V = synth.normal_with_outliers(rng, (3000, d), 0.005, 20.0)
    e = values.encode_values(V, b)
    plain = values.dequantize_values(e["q"], e["s16"], e["z16"])
    Vr = values.rotate_values(V, d1, d2)
    assert Vr.dtype == np.float32
    er = values.encode_values(Vr, b)
    back = values.dequantize_values(er["q"], er["s16"], er["z16"]) @ rotation.inverse_rotation_matrix(d1, d2).T
    assert np.mean((back - V) ** 2) < 0.7 * np.mean((plain - V) ** 2)


def test_decode_over_rotated_values_then_folded_projection():
    d, Hq, Hkv, L = 128, 4, 2, 300
    d1, d2, rng = _params(124, d)
    S = rng.standard_normal((d, d)).astype(np.float32)
    c32, t32 = codebook.tables_fp32(d, 3)
    ctx = {"d1": d1, "d2": d2, "S": S, "c32": c32}
    fields = []
    for h in range(Hkv):
        K = rng.standard_normal((L, d))
        V = synth.normal_with_outliers(rng, (L, d), 0.005, 20.0)
        ke = keys.encode_keys(K, d1, d2, S, c32, t32)
        ve = values.encode_values(values.rotate_values(V, d1, d2), 4)
        fields.append({k2: ke[k2] for k2 in ("idx", "sign", "n16", "g16")} | {k2: ve[k2] for k2 in ("q", "s16", "z16")})
    q = rng.standard_normal((Hq, d))
    out_rot, scores = attention.decode_one_sequence(q, fields, ctx)
    W = rng.standard_normal((32, Hq * d))
    y = attention.fold_output_projection(W, d1, d2, Hq) @ out_rot.reshape(-1)
    # reference: softmax weights of the same scores over the de-rotated values
    inv = rotation.inverse_rotation_matrix(d1, d2)
    ref_heads = []
    for h in range(Hq):
        f = fields[h // (Hq // Hkv)]
        vhat = values.dequantize_values(f["q"], f["s16"], f["z16"]) @ inv.T
        ref_heads.append(attention.softmax_attend(scores[h] / np.sqrt(d), vhat))
    ref = W @ np.concatenate(ref_heads)
    assert np.max(np.abs(y - ref)) < 1e-10 * np.max(np.abs(ref))
