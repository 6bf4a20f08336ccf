"""Pins of the extend (chunked prefill) oracle, oracle.attention.extend_one_sequence.

* With no prefix it is textbook causal scaled-dot-product attention over the
  chunk (dense matrices, an upper-triangular -inf mask and scipy's softmax,
  written here independently).
* Every row equals the decode oracle of that query with the prefix as the
  compressed cache and the chunk's tokens up to and including its own as the
  recent full-precision window, so a chunk of one token is exactly decode.
* Causality: changing a later chunk token changes no earlier row.
"""

import numpy as np
import pytest
from scipy.special import softmax

import synth
from oracle import attention, codebook, keys, paged, values


def _prefix_fields(rng, prm, d, kb, vb, P, Hkv):
    lay = paged.layout(d, kb, vb)
    nb = max(1, (P + 15) // 16)
    pool = paged.new_pool(nb, Hkv, lay)
    bt = np.arange(nb)
    fields = []
    for h in range(Hkv):
        K = synth.bf16_round(rng.standard_normal((P, d)).astype(np.float32))
        V = synth.bf16_round(rng.standard_normal((P, d)).astype(np.float32))
        if P:
            ke = keys.encode_keys(K.astype(np.float64), prm["d1"], prm["d2"], prm["S"], prm["c32"], prm["t32"])
            ve = values.encode_values(V, vb)
            paged.write_tokens(pool, np.arange(P), h, ke, ve, lay)
        fields.append(paged.read_tokens(pool, bt, P, h, lay))
    return fields


def _params(seed, d, kb):
    d1, d2, S = synth.method_params(seed, d)
    c32, t32 = codebook.tables_fp32(d, kb)
    return {"d1": d1.astype(np.float64), "d2": d2.astype(np.float64), "S": S, "c32": c32, "t32": t32}


@pytest.mark.parametrize("G", [1, 4])
def test_no_prefix_is_textbook_causal_attention(G):
    rng = np.random.default_rng(5 + G)
    d, kb, vb, C, Hkv = 64, 3, 4, 23, 2
    Hq = G * Hkv
    prm = _params(11, d, kb)
    fields = _prefix_fields(rng, prm, d, kb, vb, 0, Hkv)
    q = synth.bf16_round(rng.standard_normal((C, Hq, d)).astype(np.float32))
    k = synth.bf16_round(rng.standard_normal((C, Hkv, d)).astype(np.float32))
    v = synth.bf16_round(rng.standard_normal((C, Hkv, d)).astype(np.float32))
    got = attention.extend_one_sequence(q, fields, k, v, prm)
    scale = 1.0 / np.sqrt(d)
    mask = np.triu(np.full((C, C), -np.inf), k=1)  # key j > query i is hidden
    for hq in range(Hq):
        hk = hq // G
        logits = (q[:, hq].astype(np.float64) @ k[:, hk].astype(np.float64).T) * scale + mask
        ref = softmax(logits, axis=1) @ v[:, hk].astype(np.float64)
        assert np.allclose(got[:, hq], ref, rtol=1e-12, atol=1e-13), hq


def test_every_row_is_decode_with_the_chunk_as_recent_window():
    rng = np.random.default_rng(21)
    d, kb, vb, P, C, Hkv, G = 128, 3, 4, 70, 9, 2, 4
    Hq = G * Hkv
    prm = _params(12, d, kb)
    fields = _prefix_fields(rng, prm, d, kb, vb, P, Hkv)
    q = synth.bf16_round(rng.standard_normal((C, Hq, d)).astype(np.float32))
    k = synth.bf16_round(rng.standard_normal((C, Hkv, d)).astype(np.float32))
    v = synth.bf16_round(rng.standard_normal((C, Hkv, d)).astype(np.float32))
    got = attention.extend_one_sequence(q, fields, k, v, prm)
    for i in range(C):
        rk = np.transpose(k[:i + 1], (1, 0, 2)).astype(np.float64)  # [Hkv, i+1, d]
        rv = np.transpose(v[:i + 1], (1, 0, 2)).astype(np.float64)
        ref, _ = attention.decode_one_sequence(q[i].astype(np.float64), fields, prm, rk, rv)
        assert np.allclose(got[i], ref, rtol=1e-12, atol=1e-14), i


def test_chunk_of_one_token_is_decode():
    rng = np.random.default_rng(22)
    d, kb, vb, P, Hkv, G = 128, 4, 2, 33, 1, 8
    prm = _params(13, d, kb)
    fields = _prefix_fields(rng, prm, d, kb, vb, P, Hkv)
    q = synth.bf16_round(rng.standard_normal((1, G * Hkv, d)).astype(np.float32))
    k = synth.bf16_round(rng.standard_normal((1, Hkv, d)).astype(np.float32))
    v = synth.bf16_round(rng.standard_normal((1, Hkv, d)).astype(np.float32))
    got = attention.extend_one_sequence(q, fields, k, v, prm)
    ref, _ = attention.decode_one_sequence(q[0].astype(np.float64), fields, prm,
                                           np.transpose(k, (1, 0, 2)).astype(np.float64),
                                           np.transpose(v, (1, 0, 2)).astype(np.float64))
    assert np.allclose(got[0], ref, rtol=1e-12, atol=1e-14)


def test_later_chunk_tokens_do_not_change_earlier_rows():
    rng = np.random.default_rng(23)
    d, kb, vb, P, C, Hkv, G = 128, 3, 4, 40, 12, 1, 2
    prm = _params(14, d, kb)
    fields = _prefix_fields(rng, prm, d, kb, vb, P, Hkv)
    q = synth.bf16_round(rng.standard_normal((C, G, d)).astype(np.float32))
    k = synth.bf16_round(rng.standard_normal((C, Hkv, d)).astype(np.float32))
    v = synth.bf16_round(rng.standard_normal((C, Hkv, d)).astype(np.float32))
    a = attention.extend_one_sequence(q, fields, k, v, prm)
    k2, v2 = k.copy(), v.copy()
    k2[7:] *= -3.0
    v2[7:] += 5.0
    b = attention.extend_one_sequence(q, fields, k2, v2, prm)
    assert np.array_equal(a[:7], b[:7])
    assert not np.allclose(a[7:], b[7:])
