"""Pins for the oracle's decode attention (iThome "why not just round":
softmax(Q.K) V; Roadmap §3.2 exp2 online softmax and split-KV; Hub hybrid
recent window) and the pages' byte-budget arithmetic (iThome "first compute
how much can be saved"; Roadmap §4 and §7)."""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention, codebook, keys, paged, values

PAGE = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")))


def _blockwise_online(logits, vals, splits):
    """Independent split-KV online softmax in the exp2 domain: per split a
    running (max, sum, acc); then a log-sum-exp merge that ignores empty
    splits (max = -inf, sum = 0)."""
    LOG2E = 1.0 / math.log(2.0)
    parts = []
    for idx in splits:
        m, l, acc = -np.inf, 0.0, np.zeros(vals.shape[1])
        for start in range(0, len(idx), 5):
            blk = idx[start:start + 5]
            x = logits[blk] * LOG2E
            m_new = max(m, x.max())
            alpha = 2.0 ** (m - m_new) if m > -np.inf else 0.0
            p = 2.0 ** (x - m_new)
            l = l * alpha + p.sum()
            acc = acc * alpha + p @ vals[blk]
            m = m_new
        parts.append((m, l, acc))
    M = max(p[0] for p in parts)
    L = sum(l * 2.0 ** (m - M) for m, l, _ in parts if l > 0)
    out = sum(acc * 2.0 ** (m - M) for m, l, acc in parts if l > 0)
    return out / L


@pytest.fixture(scope="module")
def small_ctx():
    rng = np.random.default_rng(41)
    d = 128
    ctx = {"d1": rng.choice([-1.0, 1.0], d), "d2": rng.choice([-1.0, 1.0], d),
           "S": rng.standard_normal((d, d)).astype(np.float32)}
    ctx["c32"], ctx["t32"] = codebook.tables_fp32(d, 3)
    return ctx


def _encode_fields(K, V, ctx, bv=4):
    ke = keys.encode_keys(K, ctx["d1"], ctx["d2"], ctx["S"], ctx["c32"], ctx["t32"])
    ve = values.encode_values(V, bv)
    return {"idx": ke["idx"], "sign": ke["sign"], "n16": ke["n16"], "g16": ke["g16"],
            "q": ve["q"], "s16": ve["s16"], "z16": ve["z16"]}


def test_direct_softmax_equals_split_online_softmax(small_ctx):
    rng = np.random.default_rng(42)
    T, d = 333, 128
    K = rng.standard_normal((T, d)).astype(np.float32)
    V = rng.standard_normal((T, d)).astype(np.float32)
    q = rng.standard_normal((4, d))
    f = _encode_fields(K, V, small_ctx)
    out, sc = attention.decode_one_sequence(q, [f], small_ctx)
    vhat = values.dequantize_values(f["q"], f["s16"], f["z16"])
    cuts = [0, 0, 50, 51, 200, 333, 333]
    splits = [np.arange(a, b) for a, b in zip(cuts[:-1], cuts[1:])]
    for h in range(4):
        ref = _blockwise_online(sc[h] / np.sqrt(d), vhat, splits)
        assert np.allclose(out[h], ref, rtol=1e-12, atol=1e-12)


def test_identical_keys_give_mean_value_and_dominant_logit_selects(small_ctx):
    rng = np.random.default_rng(43)
    T, d = 40, 128
    K = np.tile(rng.standard_normal((1, d)).astype(np.float32), (T, 1))
    V = rng.standard_normal((T, d)).astype(np.float32)
    f = _encode_fields(K, V, small_ctx)
    vhat = values.dequantize_values(f["q"], f["s16"], f["z16"])
    out, _ = attention.decode_one_sequence(rng.standard_normal((1, d)), [f], small_ctx)
    assert np.allclose(out[0], vhat.mean(axis=0), atol=1e-12)
    # one key far more aligned with q than the rest dominates the softmax
    K2 = rng.standard_normal((T, d)).astype(np.float32) * 0.01
    qv = rng.standard_normal(d)
    K2[7] = (qv * 50).astype(np.float32)
    f2 = _encode_fields(K2, V, small_ctx)
    vhat2 = values.dequantize_values(f2["q"], f2["s16"], f2["z16"])
    out2, _ = attention.decode_one_sequence(qv[None, :], [f2], small_ctx)
    assert np.allclose(out2[0], vhat2[7], atol=1e-9)


def test_recent_only_reduces_to_textbook_attention(small_ctx):
    rng = np.random.default_rng(44)
    d, R, Hkv, Hq = 128, 128, 2, 8
    rk = rng.standard_normal((Hkv, R, d))
    rv = rng.standard_normal((Hkv, R, d))
    q = rng.standard_normal((Hq, d))
    empty = {"idx": np.zeros((0, d), np.int64), "sign": np.zeros((0, d), np.uint8), "n16": np.zeros(0, np.uint16),
             "g16": np.zeros(0, np.uint16), "q": np.zeros((0, d), np.int64), "s16": np.zeros((0, 4), np.uint16),
             "z16": np.zeros((0, 4), np.uint16)}
    out, _ = attention.decode_one_sequence(q, [empty] * Hkv, small_ctx, rk, rv)
    G = Hq // Hkv
    qt = torch.tensor(q).view(Hq, 1, d)
    kt = torch.tensor(rk).repeat_interleave(G, 0)
    vt = torch.tensor(rv).repeat_interleave(G, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt).view(Hq, d).numpy()
    assert np.allclose(out, ref, atol=1e-12)


def test_gqa_uses_consecutive_grouping(small_ctx):
    rng = np.random.default_rng(45)
    d, T = 128, 20
    fa = _encode_fields(rng.standard_normal((T, d)).astype(np.float32), np.ones((T, d), np.float32), small_ctx)
    fb = _encode_fields(rng.standard_normal((T, d)).astype(np.float32), -np.ones((T, d), np.float32), small_ctx)
    out, _ = attention.decode_one_sequence(rng.standard_normal((4, d)), [fa, fb], small_ctx)
    assert np.allclose(out[:2], 1.0) and np.allclose(out[2:], -1.0)


def test_empty_sequence_gives_zero_output():
    assert np.array_equal(attention.softmax_attend(np.zeros(0), np.zeros((0, 8))), np.zeros(8))


# ---------------------------------------------------------------- byte budget
def test_sglang_bytes_per_token_arithmetic():
    # 32 layers x 8 KV heads x d=128: bf16 K+V = 131072 B; 4-bit K + 4-bit V
    # + 4 B of metadata per token-head = 33792 B, a 3.88x reduction.
    layers, heads, d = 32, 8, 128
    bf16 = layers * heads * d * 2 * 2
    tq4 = layers * heads * (d * 4 // 8 + d * 4 // 8 + 4)
    assert bf16 == PAGE["sglang_bytes_per_token_bf16"]["value"]
    assert tq4 == PAGE["sglang_bytes_per_token_tq4u"]["value"]
    assert round(bf16 / tq4, 2) == PAGE["sglang_compression"]["value"]


def test_llama_1b_kv_is_one_gib():
    layers, kv_heads, d, ctx = 16, 8, 64, 32768
    assert layers * kv_heads * d * 2 * 2 * ctx == PAGE["llama32_1b_32k_bf16_kv_bytes"]["value"]


@pytest.mark.parametrize("bk,bv", [(3, 4), (3, 2), (4, 4), (4, 2)])
def test_bit_budget_of_the_record_layout(bk, bv):
    d = 128
    lay = paged.layout(d, bk, bv)
    per_token_head = lay["bytes"] // paged.BLOCK
    payload = (bk * d + bv * d) // 8
    qjl = d // 8
    meta = 4 + (d // 32) * 4
    assert per_token_head == payload + qjl + meta
    # the page's ideal ratio (K bits + V bits)/(16 + 16) counts payload only
    assert payload / (2 * d * 2) == (bk + bv) / 32
    if (bk, bv) == (3, 4):
        assert abs((bk + bv) / 32 - 0.21875) < 1e-12
        assert abs((payload + qjl) / 512 - 0.25) < 1e-12
        assert per_token_head == 148 and abs(per_token_head / 512 - 0.289) < 1e-3


def test_k4v2_is_a_quarter_smaller_than_k4v4():
    assert 1 - (4 + 2) / (4 + 4) == PAGE["k4v2_saving_vs_k4v4"]["value"]
