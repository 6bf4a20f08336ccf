"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds no arithmetic of the method: it only draws random tensors
(keys, values, queries, block tables, lengths) and the random parameters the
method itself draws (the rotation signs D1, D2 and the QJL matrix S), which
are passed to both the HIP library and the CPU oracle as inputs.

Shapes follow the workloads the pages discuss: a Llama-3.1-8B attention layer
(32 query / 8 KV heads, head_dim 128; Roadmap §2.3 figure), 131K-token
contexts (Hub, opening section), K3V2 / K4V4 / K4V2 presets (Hub; Roadmap §4.5)
— no public dataset is used.  Every generator is a pure function of its seed
(NumPy ``default_rng``), and bf16 tensors are produced by round-to-nearest-even
from fp32, so the same values can be regenerated on the CPU for any subset of
sequences and heads.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_round",
    "bf16_bits",
    "method_params",
    "normal_with_outliers",
    "config1",
    "seq_kv",
    "queries",
    "block_table",
    "ragged_lengths",
    "CONFIGS",
]


def bf16_round(x) -> np.ndarray:
    """fp32 array of the bf16 round-to-nearest-even of ``x``."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    out = rounded.astype(np.uint32).view(np.float32)
    return np.where(np.isnan(f), f, out)


def bf16_bits(x) -> np.ndarray:
    """uint16 bf16 bit patterns of values that are already bf16-exact."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def method_params(seed: int, d: int):
    """The method's random draws for one context: D1, D2 Rademacher (int8 +-1)
    and S i.i.d. N(0, 1) (fp32, [d, d] row-major)."""
    rng = np.random.default_rng([0x5EED, seed, d])
    signs = rng.integers(0, 2, size=(2, d)).astype(np.int8) * 2 - 1
    S = rng.standard_normal((d, d), dtype=np.float32)
    return signs[0].copy(), signs[1].copy(), S


def normal_with_outliers(rng, shape, p=0.005, factor=20.0) -> np.ndarray:
    """N(0, 1) fp32 with each coordinate multiplied by ``factor`` with
    probability ``p`` (i.i.d. mask); bf16-rounded."""
    x = rng.standard_normal(shape, dtype=np.float32)
    if p > 0:
        mask = rng.random(shape, dtype=np.float32) < p
        x = np.where(mask, x * np.float32(factor), x)
    return bf16_round(x)


def config1(seed: int = 0):
    """Tiny case: one KV head, d = 128, 4096 fp32 keys and values ~N(0, 1) with
    two outlier channels (chosen from the seed) scaled by 10, and 8 fp32
    queries ~N(0, 1)."""
    rng = np.random.default_rng(seed)
    d, T = 128, 4096
    ch = rng.choice(d, size=2, replace=False)
    K = rng.standard_normal((T, d), dtype=np.float32)
    V = rng.standard_normal((T, d), dtype=np.float32)
    K[:, ch] *= np.float32(10.0)
    V[:, ch] *= np.float32(10.0)
    Q = rng.standard_normal((8, d), dtype=np.float32)
    return K, V, Q, ch


def seq_kv(seed: int, seq: int, head: int, length: int, d: int, p=0.0, factor=20.0):
    """bf16-exact fp32 keys and values [length, d] of one (sequence, KV head),
    drawn from their own stream so that any subset can be regenerated."""
    rng = np.random.default_rng([seed, seq, head])
    K = normal_with_outliers(rng, (length, d), p, factor)
    V = normal_with_outliers(rng, (length, d), p, factor)
    return K, V


def queries(seed: int, batch: int, num_q_heads: int, d: int) -> np.ndarray:
    """bf16-exact fp32 queries [batch, Hq, d] ~N(0, 1)."""
    rng = np.random.default_rng([seed, 0xA11])
    return bf16_round(rng.standard_normal((batch, num_q_heads, d), dtype=np.float32))


def block_table(seed: int, batch: int, blocks_per_seq: int, pool_blocks: int) -> np.ndarray:
    """int32 [batch, blocks_per_seq]: a random permutation of the pool, cut
    into consecutive rows (no block shared)."""
    rng = np.random.default_rng([seed, 0xB10C])
    need = batch * blocks_per_seq
    if need > pool_blocks:
        raise ValueError("pool too small")
    perm = rng.permutation(pool_blocks)[:need].astype(np.int32)
    return perm.reshape(batch, blocks_per_seq)


def ragged_lengths(seed: int, batch: int, lo: int = 1024, hi: int = 131072, median: float = 16384.0, sigma: float = 1.0):
    """Lognormal lengths round(exp(N(ln median, sigma))) clipped to [lo, hi]."""
    rng = np.random.default_rng([seed, 0x1E6])
    L = np.rint(np.exp(rng.normal(np.log(median), sigma, size=batch)))
    return np.clip(L, lo, hi).astype(np.int64)


# The five workloads (shape parameters only).
CONFIGS = {
    1: dict(name="tiny-d128-k3v4-fp32", d=128, Hq=8, Hkv=1, B=1, L=4096, b_k=3, b_v=4, seed=0),
    2: dict(name="quantize-llama8b-layer-65536tok", d=128, Hkv=8, T=65536, b_k=3, b_v=(4, 2),
            pool_blocks=4096, seed=2, p=0.005, factor=20.0),
    3: dict(name="decode-b32-hq32-hkv8-d128-ctx8192-k3v4", d=128, Hq=32, Hkv=8, B=32, L=8192,
            b_k=3, b_v=4, pool_blocks=16384, seed=3, p=0.0),
    4: dict(name="decode-b8-hq16-hkv4-d256-ctx131072-k4v4", d=256, Hq=16, Hkv=4, B=8, L=131072,
            b_k=4, b_v=4, pool_blocks=65536, seed=4, p=0.0),
    5: dict(name="decode-ragged-b64-hq32-hkv8-d128-k3v2|k4v4-recent128", d=128, Hq=32, Hkv=8, B=64,
            presets=((3, 2), (4, 4)), recent=128, seed=5, p=0.005, factor=20.0),
}


def torch_normal_bf16(shape, seed: int, device="cuda", p: float = 0.0, factor: float = 20.0):
    """Seeded N(0, 1) bf16 tensor generated on the device (for the bench's
    large inputs), each element scaled by ``factor`` with probability ``p``."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if p > 0:
        mask = torch.rand(shape, generator=g, device=device) < p
        x = torch.where(mask, x * factor, x)
    return x.to(torch.bfloat16)
