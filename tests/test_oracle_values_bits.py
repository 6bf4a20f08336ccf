"""Pins for value group quantisation (Hub, technical principle step 4; Hub
quality table), bit packing (Hub, step 5) and the paged record layout."""

import json
import os

import numpy as np
import pytest

from oracle import bits, paged, values

PAGE = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")))


# ---------------------------------------------------------------- values
@pytest.mark.parametrize("b", [2, 4])
def test_value_codes_are_the_nearest_level(b):
    rng = np.random.default_rng(31)
    V = rng.standard_normal((500, 128)).astype(np.float32) * 3
    enc = values.encode_values(V, b)
    s = bits.from_fp16_bits(enc["s16"]).repeat(32, axis=1)
    z = bits.from_fp16_bits(enc["z16"]).repeat(32, axis=1)
    levels = np.arange(1 << b)[None, None, :] * s[..., None] + z[..., None]
    brute = np.argmin(np.abs(V.astype(np.float64)[..., None] - levels), axis=-1)
    x = enc["x"]
    near_tie = np.abs(x - np.floor(x) - 0.5) < 1e-4
    assert np.array_equal(enc["q"][~near_tie], brute[~near_tie])


@pytest.mark.parametrize("b", [2, 4])
def test_value_roundtrip_error_bound(b):
    rng = np.random.default_rng(32)
    V = rng.standard_normal((500, 128)).astype(np.float32)
    enc = values.encode_values(V, b)
    vh = values.dequantize_values(enc["q"], enc["s16"], enc["z16"])
    s = bits.from_fp16_bits(enc["s16"]).repeat(32, axis=1)
    z = bits.from_fp16_bits(enc["z16"]).repeat(32, axis=1)
    mn = V.reshape(500, 4, 32).min(axis=2).repeat(32, axis=1)
    err = np.abs(vh - V)
    # half a step, plus what the fp16 zero-point and scale roundings can shift
    bound = s / 2 + np.abs(z - mn) + (1 << b) * np.abs(s - (V.reshape(500, 4, 32).max(2) - V.reshape(500, 4, 32).min(2)).repeat(32, axis=1) / ((1 << b) - 1)) + 1e-6
    assert np.all(err <= bound)


def test_constant_group_stores_zero_scale():
    V = np.full((3, 128), 1.25, np.float32)
    V[1, 40:64] = -2.0  # group 1 of row 1 is not constant
    enc = values.encode_values(V, 4)
    assert enc["s16"][0].tolist() == [0, 0, 0, 0]
    assert not enc["q"][0].any()
    vh = values.dequantize_values(enc["q"], enc["s16"], enc["z16"])
    assert np.all(vh[0] == 1.25) and enc["s16"][1, 1] != 0


def test_value_cos_sim_close_to_page_audit():
    """N(0, 1) values at 2 / 4 bits give cos-sim near the Hub table's
    0.940 / 0.997 (a loose check: the page measured model KV, not N(0, 1))."""
    rng = np.random.default_rng(33)
    V = rng.standard_normal((4000, 128)).astype(np.float32)
    for b, key in ((2, "value_cos_sim_2bit"), (4, "value_cos_sim_4bit")):
        enc = values.encode_values(V, b)
        vh = values.dequantize_values(enc["q"], enc["s16"], enc["z16"])
        cs = np.sum(vh * V, axis=1) / np.linalg.norm(vh, axis=1) / np.linalg.norm(V, axis=1)
        assert abs(cs.mean() - PAGE[key]["value"]) < 0.01


# ---------------------------------------------------------------- bits
def test_pack_golden_bytes():
    # LSB-first: element 0 in the lowest bits of byte 0
    assert bits.pack(np.array([[1, 2, 3, 0]]), 2).tolist() == [[0b00111001]]
    assert bits.pack(np.array([[0xA, 0x5]]), 4).tolist() == [[0x5A]]
    # 3-bit stream of 1..7,0: bits 001 010 011 100 101 110 111 000 (LSB first)
    # byte0 = 1 | 2<<3 | (3&3)<<6 = 0xD1; byte1 = 3>>2 | 4<<1 | 5<<4 | (6&1)<<7 = 0x58; byte2 = 6>>1 | 7<<2 | 0 = 0x1F
    assert bits.pack(np.array([[1, 2, 3, 4, 5, 6, 7, 0]]), 3).tolist() == [[0xD1, 0x58, 0x1F]]
    # sign bits: bit i of the stream is element i
    assert bits.pack(np.array([[1, 0, 0, 0, 0, 0, 0, 1, 1, 1, 0, 0, 0, 0, 0, 0]]), 1).tolist() == [[0x81, 0x03]]


@pytest.mark.parametrize("b", [1, 2, 3, 4])
def test_pack_roundtrip_and_density(b):
    rng = np.random.default_rng(34)
    v = rng.integers(0, 1 << b, size=(10, 128))
    p = bits.pack(v, b)
    assert p.shape == (10, 128 * b // 8)
    assert np.array_equal(bits.unpack(p, b, 128), v)
    if b in (2, 4):
        key = "codes_per_byte_%dbit" % b
        assert 128 // p.shape[1] == PAGE[key]["value"]


def test_fp16_helpers_round_to_nearest_even():
    # 2049 lies exactly between 2048 and 2050 in fp16 -> ties to even (2048)
    assert bits.from_fp16_bits(bits.to_fp16_bits(2049.0)) == 2048.0
    assert bits.from_fp16_bits(bits.to_fp16_bits(2051.0)) == 2052.0
    assert bits.to_fp16_bits(1.0) == 0x3C00


# ---------------------------------------------------------------- layout
@pytest.mark.parametrize("d,bk,bv,expect", [(128, 3, 4, 2368), (128, 3, 2, 1856), (128, 4, 4, 2624), (256, 4, 4, 5184)])
def test_record_sizes(d, bk, bv, expect):
    lay = paged.layout(d, bk, bv)
    assert lay["bytes"] == expect
    for name in ("kcodes", "kqjl", "kmeta", "vcodes", "vmeta"):
        off, size = lay[name]
        assert off % 16 == 0 and size % 16 == 0
    # per token-head: payload codes + QJL + 2 fp16 key scalars + per-group fp16 pairs
    per_tok = (bk * d + d + bv * d) // 8 + 4 + (d // 32) * 4
    assert expect == 16 * per_tok


def test_layout_roundtrip_with_random_slots():
    rng = np.random.default_rng(35)
    d, bk, bv = 128, 3, 2
    lay = paged.layout(d, bk, bv)
    pool = paged.new_pool(12, 3, lay)
    N = 100
    slots = rng.permutation(12 * 16)[:N]
    kenc = {"idx": rng.integers(0, 8, (N, d)), "sign": rng.integers(0, 2, (N, d)).astype(np.uint8),
            "n16": rng.integers(0, 1 << 15, N).astype(np.uint16), "g16": rng.integers(0, 1 << 15, N).astype(np.uint16)}
    venc = {"q": rng.integers(0, 4, (N, d)), "s16": rng.integers(0, 1 << 15, (N, 4)).astype(np.uint16),
            "z16": rng.integers(0, 1 << 16, (N, 4)).astype(np.uint16)}
    paged.write_tokens(pool, slots, 2, kenc, venc, lay)
    bt = np.arange(12)
    f = paged.read_tokens(pool, bt, 12 * 16, 2, lay)
    for key, src in (("idx", kenc), ("sign", kenc), ("n16", kenc), ("g16", kenc), ("q", venc), ("s16", venc), ("z16", venc)):
        assert np.array_equal(f[key][slots], src[key]), key
    assert not pool[:, :2].any()  # other heads untouched


def test_value_bytes_are_stored_in_dword_columns():
    d, bk, bv = 128, 3, 4
    lay = paged.layout(d, bk, bv)
    pool = paged.new_pool(1, 1, lay)
    q = np.zeros((16, d), np.int64)
    q[3, 0], q[3, 1] = 0x7, 0xA  # slot 3, channels 0 and 1 -> byte 0 = 0xA7
    q[5, 12], q[5, 13] = 0x3, 0x1  # slot 5, channels 12, 13 -> byte 6 = 0x13 (dword 1, byte 2)
    venc = {"q": q, "s16": np.zeros((16, 4), np.uint16), "z16": np.zeros((16, 4), np.uint16)}
    kenc = {"idx": np.zeros((16, d), np.int64), "sign": np.zeros((16, d), np.uint8),
            "n16": np.zeros(16, np.uint16), "g16": np.zeros(16, np.uint16)}
    paged.write_tokens(pool, np.arange(16), 0, kenc, venc, lay)
    off, _ = lay["vcodes"]
    assert pool[0, 0, off + (0 * 16 + 3) * 4 + 0] == 0xA7
    assert pool[0, 0, off + (1 * 16 + 5) * 4 + 2] == 0x13
    assert np.count_nonzero(pool[0, 0, off:off + lay["vcodes"][1]]) == 2


@pytest.mark.parametrize("d,bk,bv,qjl", [(128, 3, 4, True), (128, 4, 2, False), (256, 4, 4, True)])
def test_reader_follows_the_block_table_and_stops_at_the_length(d, bk, bv, qjl):
    """Tokens written through a permuted block table with a ragged length come
    back in token order from read_tokens, and nothing of other heads or of
    the unused slots of the last block leaks into the fields."""
    rng = np.random.default_rng(77 + d + bk)
    lay = paged.layout(d, bk, bv, qjl=qjl)
    nb, Hkv, L = 9, 2, 37  # 3 blocks, the last one partial
    pool = paged.new_pool(nb, Hkv, lay)
    pool[:] = rng.integers(0, 256, pool.shape, dtype=np.uint8)  # garbage everywhere else
    bt = rng.permutation(nb)[:3]
    t = np.arange(L)
    slots = bt[t // 16].astype(np.int64) * 16 + t % 16
    ng = d // 32
    kenc = {"idx": rng.integers(0, 1 << bk, (L, d)), "sign": rng.integers(0, 2, (L, d)).astype(np.uint8),
            "n16": rng.integers(0, 1 << 15, L).astype(np.uint16), "g16": rng.integers(0, 1 << 15, L).astype(np.uint16)}
    venc = {"q": rng.integers(0, 1 << bv, (L, d)), "s16": rng.integers(0, 1 << 15, (L, ng)).astype(np.uint16),
            "z16": rng.integers(0, 1 << 16, (L, ng)).astype(np.uint16)}
    paged.write_tokens(pool, slots, 1, kenc, venc, lay)
    f = paged.read_tokens(pool, bt, L, 1, lay)
    keys_ = ("idx", "sign", "n16", "g16") if qjl else ("idx", "n16")
    for key in keys_:
        assert f[key].shape[0] == L and np.array_equal(f[key], kenc[key]), key
    for key in ("q", "s16", "z16"):
        assert f[key].shape[0] == L and np.array_equal(f[key], venc[key]), key
    if not qjl:
        assert not f["sign"].any() and not f["g16"].any()
