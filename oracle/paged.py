"""Paged KV-cache record layout.

iThome (introduction, and "which path vLLM actually takes"): the cache is cut
into fixed-size blocks located through a block table; the store kernel
quantises and packs new K/V and writes them into the paged cache, and the
decode kernel reads the compressed K/V back through the block table.

Reading (the pages fix no byte layout): the pool is
``pool[num_blocks][num_kv_heads][record]`` with 16 token slots per block.  A
record holds the 16 slots of one (block, KV head) as consecutive regions, each
a multiple of 16 bytes:

  Kcodes  [16][b_k*d/8]   slot-major: the LSB-first code stream of each slot
  Kqjl    [16][d/8]       slot-major: the QJL sign bits of each slot
  Kmeta   [16][2] fp16    (n, gamma) of each slot
  Vcodes  [b_v*d/32][16][4]  dword-column-major: dword w (bytes 4w..4w+3)
                          of every slot's value-code stream together, i.e.
                          byte f of slot s at ((f // 4) * 16 + s) * 4 + f % 4
  Vmeta   [d/32][16][2]   fp16 (scale, zero) per (group, slot)

MSE-only presets (keys without the QJL sketch) have no Kqjl region and a
Kmeta region of [16] fp16 n (32 bytes); the other regions are unchanged.

Token t of sequence s lives in block ``block_table[s][t // 16]``, slot
``t % 16``; the writer addresses slot ``slot_mapping[i]`` of token i as block
``slot_mapping[i] // 16``, slot ``slot_mapping[i] % 16``.
"""

from __future__ import annotations

import numpy as np

from . import bits as _bits

__all__ = ["BLOCK", "layout", "write_tokens", "read_tokens", "new_pool"]

BLOCK = 16


def layout(d: int, b_k: int, b_v: int, qjl: bool = True) -> dict:
    kc = BLOCK * (b_k * d // 8)
    kq = BLOCK * (d // 8) if qjl else 0
    km = BLOCK * (4 if qjl else 2)
    vc = (b_v * d // 8) * BLOCK
    vm = (d // 32) * BLOCK * 4
    off = {}
    o = 0
    for name, size in (("kcodes", kc), ("kqjl", kq), ("kmeta", km), ("vcodes", vc), ("vmeta", vm)):
        off[name] = (o, size)
        o += size
    off["bytes"] = o
    off["d"], off["b_k"], off["b_v"], off["qjl"] = d, b_k, b_v, qjl
    return off


def new_pool(num_blocks: int, num_kv_heads: int, lay: dict) -> np.ndarray:
    return np.zeros((num_blocks, num_kv_heads, lay["bytes"]), dtype=np.uint8)


def _region_index(lay: dict, name: str, slots, width: int, slot_major: bool):
    """Byte offsets inside a record of ``width`` bytes per slot for each slot:
    slot-major regions hold a slot's bytes contiguously; dword-column regions
    hold dword w of every slot contiguously (byte f of slot s at
    ((f // 4) * 16 + s) * 4 + f % 4)."""
    o, _ = lay[name]
    s = np.asarray(slots, dtype=np.int64)[:, None]
    f = np.arange(width, dtype=np.int64)[None, :]
    return o + (s * width + f if slot_major else ((f // 4) * BLOCK + s) * 4 + f % 4)


def write_tokens(pool, slot_mapping, head: int, kenc: dict, venc: dict, lay: dict) -> None:
    """Write encoded tokens (rows of ``kenc``/``venc``) of one KV head into the
    slots named by ``slot_mapping``."""
    d, b_k, b_v = lay["d"], lay["b_k"], lay["b_v"]
    ng = d // 32
    sm = np.asarray(slot_mapping, dtype=np.int64)
    blk = (sm // BLOCK)[:, None]
    slot = sm % BLOCK
    qjl = lay["qjl"]
    kcodes = _bits.pack(kenc["idx"], b_k)
    if qjl:
        kmeta = np.stack([kenc["n16"], kenc["g16"]], axis=1).astype(np.uint16).view(np.uint8)
    else:
        kmeta = np.asarray(kenc["n16"], dtype=np.uint16)[:, None].view(np.uint8)
    vcodes = _bits.pack(venc["q"], b_v)
    pool[blk, head, _region_index(lay, "kcodes", slot, b_k * d // 8, True)] = kcodes
    if qjl:
        pool[blk, head, _region_index(lay, "kqjl", slot, d // 8, True)] = _bits.pack(kenc["sign"], 1)
    pool[blk, head, _region_index(lay, "kmeta", slot, kmeta.shape[1], True)] = kmeta
    pool[blk, head, _region_index(lay, "vcodes", slot, b_v * d // 8, False)] = vcodes
    o, _ = lay["vmeta"]
    for g in range(ng):
        pair = np.stack([venc["s16"][:, g], venc["z16"][:, g]], axis=1).astype(np.uint16).view(np.uint8)
        idx = o + (g * BLOCK + slot[:, None]) * 4 + np.arange(4)[None, :]
        pool[blk, head, idx] = pair


def read_tokens(pool, block_table_row, length: int, head: int, lay: dict) -> dict:
    """Read the first ``length`` tokens of one sequence and KV head back into
    fields: idx [L, d], sign [L, d], n16, g16 [L], q [L, d], s16, z16 [L, d/32]
    (sign and g16 are zeros for MSE-only keys).

    The records of the sequence's blocks are gathered whole, then each region
    is cut out of them as the layout above describes: slot-major regions are
    [16][width] per record, the value codes are [width/4][16][4] (dword
    columns), the value metadata [d/32][16] pairs of fp16."""
    d, b_k, b_v = lay["d"], lay["b_k"], lay["b_v"]
    ng = d // 32
    nblk = (length + BLOCK - 1) // BLOCK
    recs = pool[np.asarray(block_table_row, dtype=np.int64)[:nblk], head]  # [nblk, record bytes]
    qjl = lay["qjl"]

    def region(name, width):
        o, size = lay[name]
        assert size == BLOCK * width
        return recs[:, o:o + size]

    def slot_major(name, width):
        return region(name, width).reshape(nblk * BLOCK, width)[:length]

    def dword_columns(name, width):
        r = region(name, width).reshape(nblk, width // 4, BLOCK, 4)  # [block, dword, slot, byte]
        return r.transpose(0, 2, 1, 3).reshape(nblk * BLOCK, width)[:length]

    kcodes = slot_major("kcodes", b_k * d // 8)
    if qjl:
        sign = _bits.unpack(slot_major("kqjl", d // 8), 1, d).astype(np.uint8)
    else:
        sign = np.zeros((length, d), dtype=np.uint8)
    kmeta = np.ascontiguousarray(slot_major("kmeta", 4 if qjl else 2)).view(np.uint16)
    vcodes = dword_columns("vcodes", b_v * d // 8)
    o, size = lay["vmeta"]
    vm = np.ascontiguousarray(recs[:, o:o + size]).view(np.uint16).reshape(nblk, ng, BLOCK, 2)
    vm = vm.transpose(0, 2, 1, 3).reshape(nblk * BLOCK, ng, 2)[:length]  # [token, group, (s, z)]
    return {
        "idx": _bits.unpack(kcodes, b_k, d),
        "sign": sign,
        "n16": kmeta[:, 0].copy(),
        "g16": kmeta[:, 1].copy() if qjl else np.zeros(length, dtype=np.uint16),
        "q": _bits.unpack(vcodes, b_v, d),
        "s16": np.ascontiguousarray(vm[:, :, 0]),
        "z16": np.ascontiguousarray(vm[:, :, 1]),
    }
