"""CPU-only checks of the C-ABI library: it loads, exports every symbol the
header declares, its host math agrees with the oracle, and its argument
validation returns the documented codes.  No compute call touches a GPU."""

import ctypes
import os
import re

import numpy as np
import pytest

import kv_cache_vector_03_amd as tq
from oracle import attention, codebook, paged

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tq_api.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = tq.load()
    declared = _declared_functions()
    assert declared, "no declarations found"
    for name in declared:
        assert hasattr(lib, name), name
    assert sorted(tq.EXPORTED_SYMBOLS) == declared


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("b", [2, 3, 4, 8])
def test_lloyd_max_agrees_with_oracle(d, b):
    c, t = tq.tq_lloyd_max(d, b)
    c2, t2, _ = codebook.lloyd_max(d, b)
    # two independent solvers (the host's Lloyd / Newton and the oracle's)
    assert np.max(np.abs(c - c2)) < (1e-12 if b <= 4 else 2e-11) and np.max(np.abs(t - t2)) < (1e-12 if b <= 4 else 2e-11)
    # the stored fp32 tables are identical on both sides
    assert np.array_equal(c.astype(np.float32), c2.astype(np.float32))
    assert np.array_equal(t.astype(np.float32), t2.astype(np.float32))
    assert t[len(t) // 2] == 0.0 and np.array_equal(c, -c[::-1])


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("b", [2, 3, 4])
def test_uniform_codebook_agrees_with_oracle(d, b):
    c, t = tq.tq_uniform_codebook(d, b)
    c2, t2, step = codebook.uniform(d, b)
    assert np.max(np.abs(c - c2)) < 1e-12 * step * (1 << b)
    assert np.array_equal(c.astype(np.float32), c2.astype(np.float32))
    assert np.array_equal(t.astype(np.float32), t2.astype(np.float32))


@pytest.mark.parametrize("d", [128, 256])
def test_fold_output_projection_agrees_with_oracle(d):
    rng = np.random.default_rng(131)
    signs = np.stack([rng.choice([-1, 1], d), rng.choice([-1, 1], d)]).astype(np.int8)
    H, rows = 3, 40
    W = rng.standard_normal((rows, H * d)).astype(np.float32)
    got = tq.tq_fold_output_projection(signs, W, H)
    ref = attention.fold_output_projection(W, signs[0].astype(np.float64), signs[1].astype(np.float64), H)
    assert got.dtype == np.float32
    assert np.max(np.abs(got - ref)) <= 1e-6 * np.max(np.abs(ref))
    # in place gives the same
    lib = tq.load()
    W2 = W.copy()
    assert lib.tq_fold_output_projection(d, signs.ctypes.data, W2.ctypes.data, rows, H, W2.ctypes.data) == tq.TQ_OK
    assert np.array_equal(W2, got)
    bad = signs.copy()
    bad[1, 3] = 0
    assert lib.tq_fold_output_projection(d, bad.ctypes.data, W.ctypes.data, rows, H, W2.ctypes.data) == tq.TQ_EINVAL
    assert lib.tq_fold_output_projection(96, signs.ctypes.data, W.ctypes.data, rows, H, W2.ctypes.data) == tq.TQ_EINVAL


@pytest.mark.parametrize("mse_only", [False, True])
@pytest.mark.parametrize("d,bk,bv", [(128, 3, 4), (128, 3, 2), (128, 4, 4), (128, 2, 2), (256, 4, 4), (256, 3, 2),
                                     (128, 8, 4), (256, 8, 2)])
def test_record_layout_matches_oracle(d, bk, bv, mse_only):
    if bk == 8 and not mse_only:
        pytest.skip("8-bit keys exist only as MSE-only presets")
    lib_lay = tq.tq_record_layout(d, bk, bv, mse_only=mse_only)
    o = paged.layout(d, bk, bv, qjl=not mse_only)
    for name in ("kcodes", "kqjl", "kmeta", "vcodes", "vmeta"):
        assert lib_lay[name] == o[name][0]
    assert lib_lay["record_bytes"] == o["bytes"]


def test_seeded_draw_statistics():
    sg, S = tq.tq_draw_params(12345, 256)
    assert set(np.unique(sg)) == {-1, 1}
    assert abs(sg.mean()) < 4 / np.sqrt(sg.size)
    x = S.astype(np.float64).ravel()
    n = x.size
    assert abs(x.mean()) < 4 / np.sqrt(n)
    assert abs(x.var() - 1) < 4 * np.sqrt(2 / n)
    assert abs(np.mean(x ** 4) - 3) < 0.05  # Gaussian kurtosis
    sg2, S2 = tq.tq_draw_params(12345, 256)
    assert np.array_equal(sg, sg2) and np.array_equal(S, S2)
    sg3, S3 = tq.tq_draw_params(12346, 256)
    assert not np.array_equal(S, S3)


def test_unsupported_presets_are_rejected():
    lib = tq.load()
    lay = tq.tq_layout()
    for d, bk, bv in ((64, 3, 4), (128, 5, 4), (128, 3, 3), (512, 3, 4), (128, 1, 4)):
        p = tq.tq_preset(d, bk, bv, 32, 16, 0, 0)
        assert lib.tq_record_layout(ctypes.byref(p), ctypes.byref(lay)) == tq.TQ_EUNSUPPORTED
        assert "unsupported preset" in tq.tq_last_error()
    p = tq.tq_preset(128, 3, 4, 16, 16, 0, 0)
    assert lib.tq_record_layout(ctypes.byref(p), ctypes.byref(lay)) == tq.TQ_EUNSUPPORTED
    for flags in (8, 9, -1):  # TQ_PRESET_MSE_ONLY, _UNIFORM and _ROTATE_V are the known flags
        p = tq.tq_preset(128, 3, 4, 32, 16, flags, 0)
        assert lib.tq_record_layout(ctypes.byref(p), ctypes.byref(lay)) == tq.TQ_EUNSUPPORTED
    p = tq.tq_preset(128, 3, 4, 32, 16, tq.TQ_PRESET_MSE_ONLY, 0)
    assert lib.tq_record_layout(ctypes.byref(p), ctypes.byref(lay)) == tq.TQ_OK
    assert lib.tq_record_layout(None, ctypes.byref(lay)) == tq.TQ_EINVAL
    # 8-bit keys: MSE-only presets only (the vLLM K8V4 preset)
    for d in (128, 256):
        p = tq.tq_preset(d, 8, 4, 32, 16, 0, 0)
        assert lib.tq_record_layout(ctypes.byref(p), ctypes.byref(lay)) == tq.TQ_EUNSUPPORTED
        for flags in (tq.TQ_PRESET_MSE_ONLY, tq.TQ_PRESET_MSE_ONLY | tq.TQ_PRESET_UNIFORM):
            p = tq.tq_preset(d, 8, 4, 32, 16, flags, 0)
            assert lib.tq_record_layout(ctypes.byref(p), ctypes.byref(lay)) == tq.TQ_OK
            assert lay.record_bytes == 16 * d + 32 + 16 * d // 2 + d // 32 * 64


def test_host_helpers_validate_arguments():
    lib = tq.load()
    buf = np.zeros(16, np.float64)
    assert lib.tq_lloyd_max(7, 3, buf.ctypes.data, buf.ctypes.data) == tq.TQ_EINVAL
    assert lib.tq_lloyd_max(128, 0, buf.ctypes.data, buf.ctypes.data) == tq.TQ_EINVAL
    assert lib.tq_lloyd_max(128, 3, None, buf.ctypes.data) == tq.TQ_EINVAL
    assert lib.tq_draw_params(1, 0, None, None) == tq.TQ_EINVAL
    assert lib.tq_block_bytes(None) == 0
    assert lib.tq_ctx_destroy(None) == tq.TQ_OK


def test_entry_points_reject_bad_arguments_before_touching_a_device():
    lib = tq.load()
    # NULL context / bad sizes fail in host validation
    assert lib.tq_quantize_store(None, None, None, 1, 1, 1, None, None, 1, None) == tq.TQ_EINVAL
    a = tq.tq_decode_args()
    assert lib.tq_decode_attention(ctypes.byref(a), None) == tq.TQ_EINVAL
    assert lib.tq_decode_workspace_bytes(ctypes.byref(a)) == 0
    assert lib.tq_decode_attention(None, None) == tq.TQ_EINVAL
    p = tq.tq_preset(128, 3, 4, 32, 16, 0, 0)
    out = ctypes.c_void_p()
    bad = np.full((2, 128), 2, np.int8)
    assert lib.tq_codebook_init(ctypes.byref(p), bad.ctypes.data, None, ctypes.byref(out)) == tq.TQ_EINVAL
    assert "not +-1" in tq.tq_last_error()
    S = np.full((128, 128), np.nan, np.float32)
    assert lib.tq_codebook_init(ctypes.byref(p), None, S.ctypes.data, ctypes.byref(out)) == tq.TQ_EINVAL
    p.k_bits = 7
    assert lib.tq_codebook_init(ctypes.byref(p), None, None, ctypes.byref(out)) == tq.TQ_EUNSUPPORTED
