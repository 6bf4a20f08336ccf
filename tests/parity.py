"""Helpers for the GPU parity tests (not collected by pytest).

Expected values and exemption masks come only from the oracle and the seeded
inputs; the HIP path's outputs are only ever compared against them.
"""

from __future__ import annotations

import numpy as np

import synth
from oracle import bits, codebook, keys, paged, values

BAND = 1e-6


def fp16_midpoint_distance(x):
    """Relative distance of fp64 values to the nearest binary16 rounding
    midpoint (where fp32 vs fp64 rounding could disagree)."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    h = x.astype(np.float16).astype(np.float64)
    up = np.nextafter(h.astype(np.float16), np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(h.astype(np.float16), np.float16(0)).astype(np.float64)
    mid = np.minimum(np.abs(x - (h + up) / 2), np.abs(x - (h + dn) / 2))
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.where(x > 0, mid / x, np.inf)


def oracle_params(seed: int, d: int, k_bits: int, uniform: bool = False):
    d1, d2, S = synth.method_params(seed, d)
    c32, t32 = codebook.tables_fp32(d, k_bits, uniform_codebook=uniform)
    return {"d1": d1.astype(np.float64), "d2": d2.astype(np.float64), "S": S, "c32": c32, "t32": t32,
            "signs": np.stack([d1, d2]).astype(np.int8)}


def expected_records(K, V, slots, head, prm, d, kb, vb, pool, mask, qjl=True):
    """Encode K, V [N, d] of one KV head with the oracle, write them into the
    expected ``pool`` and mark every bit the comparison must exempt in
    ``mask`` (same layout).  Returns a dict of exemption counts.  ``qjl=False``:
    MSE-only keys (no sign bits or residual norm to compare)."""
    ke = keys.encode_keys(K, prm["d1"], prm["d2"], prm["S"], prm["c32"], prm["t32"], qjl=qjl)
    ve = values.encode_values(V, vb)
    lay = paged.layout(d, kb, vb, qjl=qjl)
    paged.write_tokens(pool, slots, head, ke, ve, lay)

    t = prm["t32"].astype(np.float64)
    code_band = np.min(np.abs(ke["u"][..., None] - t), axis=-1) <= BAND
    code_band &= ~ke["zero"][:, None]
    vec_hit = code_band.any(axis=1)
    if qjl:
        qjl_band = (np.abs(ke["z"]) <= BAND) & ~ke["zero"][:, None]
        qjl_band |= vec_hit[:, None]
    else:
        qjl_band = np.zeros_like(code_band)
    n_band = (fp16_midpoint_distance(ke["n"]) <= BAND) & ~ke["zero"]
    g_band = ((fp16_midpoint_distance(ke["gamma"]) <= BAND) | vec_hit) & ~ke["zero"] & qjl
    x = ve["x"]
    v_band = np.abs(x - np.floor(x) - 0.5) <= BAND
    v_band = np.where(np.isnan(x), False, v_band)
    s_band = fp16_midpoint_distance(ve["s_pre"]) <= BAND

    full = (1 << kb) - 1
    kmask = {"idx": np.where(code_band, full, 0), "sign": qjl_band.astype(np.uint8),
             "n16": np.where(n_band, 0xFFFF, 0).astype(np.uint16), "g16": np.where(g_band, 0xFFFF, 0).astype(np.uint16)}
    vmask = {"q": np.where(v_band | s_band.repeat(32, axis=1), (1 << vb) - 1, 0),
             "s16": np.where(s_band, 0xFFFF, 0).astype(np.uint16), "z16": np.zeros_like(ve["z16"])}
    paged.write_tokens(mask, slots, head, kmask, vmask, lay)
    return {"codes": int(code_band.sum()), "vectors": int(vec_hit.sum()), "qjl": int(qjl_band.sum()),
            "norms": int(n_band.sum()), "gammas": int(g_band.sum()), "values": int(v_band.sum()),
            "scales": int(s_band.sum())}


def compare_pools(gpu, expected, mask, select=None):
    """Number of differing bits outside the exemption mask, and inside it."""
    g = np.asarray(gpu, dtype=np.uint8)
    e = np.asarray(expected, dtype=np.uint8)
    m = np.asarray(mask, dtype=np.uint8)
    if select is not None:
        g, e, m = g[select], e[select], m[select]
    diff = g ^ e
    outside = np.bitwise_count(diff & ~m).sum(dtype=np.int64)
    inside = np.bitwise_count(diff & m).sum(dtype=np.int64)
    return int(outside), int(inside)


def oracle_cache(prm, d, kb, vb, lengths, Hkv, block_table, pool, seed, p=0.0, factor=20.0, seqs=None, kv=None,
                 qjl=True):
    """Encode seeded keys/values of every (sequence, KV head) with the oracle
    and write them into ``pool`` through ``block_table``.  ``kv(b, h, L)``
    overrides the generator.  Returns the fields per sequence (list over KV
    heads) for the oracle's decode.  ``qjl=False``: MSE-only keys."""
    lay = paged.layout(d, kb, vb, qjl=qjl)
    fields = {}
    for b in (range(len(lengths)) if seqs is None else seqs):
        L = int(lengths[b])
        per_head = []
        for h in range(Hkv):
            K, V = kv(b, h, L) if kv is not None else synth.seq_kv(seed, b, h, L, d, p, factor)
            ke = keys.encode_keys(K.astype(np.float64), prm["d1"], prm["d2"], prm["S"], prm["c32"], prm["t32"], qjl=qjl)
            ve = values.encode_values(V, vb)
            t = np.arange(L)
            slots = block_table[b][t // 16].astype(np.int64) * 16 + t % 16
            paged.write_tokens(pool, slots, h, ke, ve, lay)
            per_head.append({"idx": ke["idx"], "sign": ke["sign"], "n16": ke["n16"], "g16": ke["g16"],
                             "q": ve["q"], "s16": ve["s16"], "z16": ve["z16"]})
        fields[b] = per_head
    return fields


def score_errors(got, ref):
    """max |got - ref| / max(|ref|, rms(ref row)) over a [rows, T] pair."""
    rms = np.sqrt(np.mean(ref ** 2, axis=-1, keepdims=True))
    return float(np.max(np.abs(got - ref) / np.maximum(np.maximum(np.abs(ref), rms), 1e-30)))


def output_errors(got, ref):
    """max over rows of ||got - ref|| / ||ref|| (rows with a zero reference
    compare absolutely)."""
    num = np.linalg.norm(got - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    return float(np.max(np.where(den > 0, num / np.where(den > 0, den, 1), num)))
