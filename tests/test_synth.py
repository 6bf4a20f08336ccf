"""The seeded input generators: bf16 rounding agrees with torch's, and every
generator is a pure function of its seed."""

import numpy as np
import torch

import synth


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 100,
                        np.array([0.0, -0.0, 1e-40, 65504.0, 3.3895314e38, np.inf, -np.inf], np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(synth.bf16_round(x), ref)
    assert np.array_equal(synth.bf16_bits(ref), torch.from_numpy(ref).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def test_generators_are_deterministic_and_shaped():
    a = synth.seq_kv(3, 5, 2, 64, 128, p=0.005)
    b = synth.seq_kv(3, 5, 2, 64, 128, p=0.005)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert a[0].shape == (64, 128) and np.array_equal(synth.bf16_round(a[0]), a[0])
    d1, d2, S = synth.method_params(7, 128)
    assert set(np.unique(d1)) <= {-1, 1} and S.shape == (128, 128) and S.dtype == np.float32
    bt = synth.block_table(3, 32, 512, 16384)
    assert len(np.unique(bt)) == bt.size
    L = synth.ragged_lengths(5, 64)
    assert L.min() >= 1024 and L.max() <= 131072
    K, V, Q, ch = synth.config1()
    assert K.shape == (4096, 128) and Q.shape == (8, 128) and len(set(ch)) == 2
