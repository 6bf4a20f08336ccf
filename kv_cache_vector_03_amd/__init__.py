"""MI355X (gfx950) TurboQuant KV-cache hot path — thin Python binding.

Every function here marshals arguments to the C ABI declared in
``include/tq_api.h`` and calls ``libtq_mi355x.so``; all work of the path runs
in the library's HIP kernels.  PyTorch supplies device memory and streams
only.  There is no fallback: if the library is missing, importing the
binding's entry points raises.
"""

from __future__ import annotations

import ctypes
import os

__all__ = [
    "TQ_OK", "TQ_EINVAL", "TQ_EUNSUPPORTED", "TQ_EHIP", "TQ_ENOMEM", "TQ_DTYPE_F32", "TQ_DTYPE_BF16", "TQ_PRESET_MSE_ONLY",
    "TQ_PRESET_UNIFORM", "TQ_PRESET_ROTATE_V", "TQ_DECODE_DETERMINISTIC", "tq_uniform_codebook", "tq_fold_output_projection",
    "TqError", "Context", "library_path", "load", "tq_codebook_init", "tq_ctx_destroy", "tq_ctx_tables",
    "tq_lloyd_max", "tq_record_layout", "tq_draw_params", "tq_block_bytes", "tq_quantize_store",
    "tq_decode_workspace_bytes", "tq_decode_attention", "tq_decode_attention_noalloc", "NOALLOC_SCRATCH_BYTES",
    "PreparedDecode", "PreparedQuantize", "PreparedExtend", "tq_extend_attention",
    "tq_last_error", "EXPORTED_SYMBOLS",
]

TQ_OK, TQ_EINVAL, TQ_EUNSUPPORTED, TQ_EHIP, TQ_ENOMEM = 0, -1, -2, -3, -4
TQ_DTYPE_F32, TQ_DTYPE_BF16 = 0, 1
TQ_PRESET_MSE_ONLY = 1
TQ_PRESET_UNIFORM = 2
TQ_PRESET_ROTATE_V = 4
TQ_DECODE_DETERMINISTIC = 1
NOALLOC_SCRATCH_BYTES = 32 << 20  # TQ_NOALLOC_SCRATCH_BYTES of include/tq_api.h

EXPORTED_SYMBOLS = [
    "tq_codebook_init", "tq_ctx_destroy", "tq_ctx_tables", "tq_ctx_preset", "tq_lloyd_max", "tq_uniform_codebook",
    "tq_record_layout", "tq_fold_output_projection",
    "tq_draw_params", "tq_block_bytes", "tq_quantize_store", "tq_decode_workspace_bytes", "tq_decode_attention",
    "tq_decode_attention_noalloc", "tq_extend_attention", "tq_last_error",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


def library_path() -> str:
    return os.path.join(_HERE, "libtq_mi355x.so")


class TqError(RuntimeError):
    def __init__(self, code, where):
        super().__init__(f"{where} failed with {code}: {tq_last_error()}")
        self.code = code


class tq_preset(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("k_bits", ctypes.c_int32), ("v_bits", ctypes.c_int32),
                ("v_group", ctypes.c_int32), ("block_size", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("seed", ctypes.c_uint64)]


class tq_layout(ctypes.Structure):
    _fields_ = [("kcodes", ctypes.c_int64), ("kqjl", ctypes.c_int64), ("kmeta", ctypes.c_int64),
                ("vcodes", ctypes.c_int64), ("vmeta", ctypes.c_int64), ("record_bytes", ctypes.c_int64)]


class tq_decode_args(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("q_dtype", ctypes.c_int32), ("batch", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("num_presets", ctypes.c_int32),
        ("ctx", ctypes.c_void_p * 2), ("pool", ctypes.c_void_p * 2), ("pool_blocks", ctypes.c_int64 * 2),
        ("seq_preset", ctypes.c_void_p), ("block_tables", ctypes.c_void_p), ("max_blocks_per_seq", ctypes.c_int32),
        ("seq_lens", ctypes.c_void_p), ("recent_k", ctypes.c_void_p), ("recent_v", ctypes.c_void_p),
        ("recent_lens", ctypes.c_void_p), ("recent_window", ctypes.c_int32), ("sm_scale", ctypes.c_float),
        ("chunk_tokens", ctypes.c_int32), ("max_seq_len", ctypes.c_int32), ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t), ("out", ctypes.c_void_p), ("scores_out", ctypes.c_void_p),
        ("scores_stride", ctypes.c_int32), ("flags", ctypes.c_int32),
    ]


class tq_extend_args(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("cu_chunk", ctypes.c_void_p),
        ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("max_chunk", ctypes.c_int32), ("ctx", ctypes.c_void_p), ("pool", ctypes.c_void_p),
        ("pool_blocks", ctypes.c_int64), ("block_tables", ctypes.c_void_p), ("max_blocks_per_seq", ctypes.c_int32),
        ("prefix_lens", ctypes.c_void_p), ("max_prefix_len", ctypes.c_int32), ("sm_scale", ctypes.c_float),
        ("out", ctypes.c_void_p),
    ]


def load(path: str | None = None):
    """Load the library once; raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = path or library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m kv_cache_vector_03_amd.build`")
    lib = ctypes.CDLL(path)
    c = ctypes
    P = c.c_void_p
    sig = {
        "tq_codebook_init": (c.c_int, [c.POINTER(tq_preset), P, P, c.POINTER(P)]),
        "tq_ctx_destroy": (c.c_int, [P]),
        "tq_ctx_tables": (c.c_int, [P, P, P, P, P]),
        "tq_ctx_preset": (c.c_int, [P, c.POINTER(tq_preset)]),
        "tq_lloyd_max": (c.c_int, [c.c_int32, c.c_int32, P, P]),
        "tq_uniform_codebook": (c.c_int, [c.c_int32, c.c_int32, P, P]),
        "tq_fold_output_projection": (c.c_int, [c.c_int32, P, P, c.c_int64, c.c_int32, P]),
        "tq_record_layout": (c.c_int, [c.POINTER(tq_preset), c.POINTER(tq_layout)]),
        "tq_draw_params": (c.c_int, [c.c_uint64, c.c_int32, P, P]),
        "tq_block_bytes": (c.c_size_t, [P]),
        "tq_quantize_store": (c.c_int, [P, P, P, c.c_int32, c.c_int64, c.c_int32, P, P, c.c_int64, P]),
        "tq_decode_workspace_bytes": (c.c_size_t, [c.POINTER(tq_decode_args)]),
        "tq_decode_attention": (c.c_int, [c.POINTER(tq_decode_args), P]),
        "tq_decode_attention_noalloc": (c.c_int, [c.POINTER(tq_decode_args), P]),
        "tq_extend_attention": (c.c_int, [c.POINTER(tq_extend_args), P]),
        "tq_last_error": (c.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _LIB = lib
    return lib


def tq_last_error() -> str:
    if _LIB is None:
        return ""
    return _LIB.tq_last_error().decode()


def _check(code, where):
    if code != TQ_OK:
        raise TqError(code, where)


def _ptr(arr) -> int:
    """Address of a numpy array or torch tensor (None -> NULL)."""
    if arr is None:
        return None
    if hasattr(arr, "data_ptr"):
        return arr.data_ptr()
    return arr.ctypes.data


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return TQ_DTYPE_BF16
    if t.dtype == torch.float32:
        return TQ_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


class Context:
    """Owner of a ``tq_ctx*`` (freed on ``close()`` or garbage collection)."""

    def __init__(self, handle: int, head_dim: int, k_bits: int, v_bits: int, mse_only: bool = False,
                 uniform: bool = False, rotate_v: bool = False):
        self.handle = handle
        self.head_dim, self.k_bits, self.v_bits = head_dim, k_bits, v_bits
        self.mse_only, self.uniform, self.rotate_v = mse_only, uniform, rotate_v

    @property
    def block_bytes(self) -> int:
        return tq_block_bytes(self)

    def close(self):
        if self.handle:
            load().tq_ctx_destroy(ctypes.c_void_p(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def tq_codebook_init(head_dim: int, k_bits: int, v_bits: int, seed: int = 0, signs=None, S=None,
                     mse_only: bool = False, uniform: bool = False, rotate_v: bool = False) -> Context:
    """Create a context.  ``signs`` (int8 [2, d]) and ``S`` (float32 [d, d])
    are host numpy arrays or None (then drawn from ``seed``); ``mse_only``
    selects keys without the QJL sketch (TQ_PRESET_MSE_ONLY), ``uniform`` the
    equally spaced key codebook (TQ_PRESET_UNIFORM), ``rotate_v`` rotated
    values (TQ_PRESET_ROTATE_V)."""
    lib = load()
    flags = ((TQ_PRESET_MSE_ONLY if mse_only else 0) | (TQ_PRESET_UNIFORM if uniform else 0)
             | (TQ_PRESET_ROTATE_V if rotate_v else 0))
    p = tq_preset(head_dim, k_bits, v_bits, 32, 16, flags, seed)
    h = ctypes.c_void_p()
    if signs is not None:
        import numpy as np
        signs = np.ascontiguousarray(signs, dtype=np.int8)
    if S is not None:
        import numpy as np
        S = np.ascontiguousarray(S, dtype=np.float32)
    _check(lib.tq_codebook_init(ctypes.byref(p), _ptr(signs), _ptr(S), ctypes.byref(h)), "tq_codebook_init")
    return Context(h.value, head_dim, k_bits, v_bits, mse_only, uniform, rotate_v)


def tq_ctx_destroy(ctx: Context) -> None:
    ctx.close()


def tq_ctx_tables(ctx: Context):
    """(centroids, thresholds, signs, S) host copies as numpy arrays."""
    import numpy as np
    L = 1 << ctx.k_bits
    d = ctx.head_dim
    c = np.zeros(L, np.float32)
    t = np.zeros(L - 1, np.float32)
    sg = np.zeros((2, d), np.int8)
    S = np.zeros((d, d), np.float32)
    _check(load().tq_ctx_tables(ctx.handle, _ptr(c), _ptr(t), _ptr(sg), _ptr(S)), "tq_ctx_tables")
    return c, t, sg, S


def tq_lloyd_max(head_dim: int, bits: int):
    import numpy as np
    c = np.zeros(1 << bits, np.float64)
    t = np.zeros((1 << bits) - 1, np.float64)
    _check(load().tq_lloyd_max(head_dim, bits, _ptr(c), _ptr(t)), "tq_lloyd_max")
    return c, t


def tq_uniform_codebook(head_dim: int, bits: int):
    import numpy as np
    c = np.zeros(1 << bits, np.float64)
    t = np.zeros((1 << bits) - 1, np.float64)
    _check(load().tq_uniform_codebook(head_dim, bits, _ptr(c), _ptr(t)), "tq_uniform_codebook")
    return c, t


def tq_fold_output_projection(signs, w_o, num_q_heads: int):
    """W_o [rows, num_q_heads * d] (host fp32) with the inverse value rotation
    absorbed, for the context whose rotation signs are ``signs`` (int8 [2, d]);
    returns a new fp32 numpy array."""
    import numpy as np
    sg = np.ascontiguousarray(signs, dtype=np.int8)
    w = np.ascontiguousarray(w_o, dtype=np.float32)
    out = np.empty_like(w)
    _check(load().tq_fold_output_projection(sg.shape[1], _ptr(sg), _ptr(w), w.shape[0], num_q_heads, _ptr(out)),
           "tq_fold_output_projection")
    return out


def tq_record_layout(head_dim: int, k_bits: int, v_bits: int, mse_only: bool = False, flags=None) -> dict:
    p = tq_preset(head_dim, k_bits, v_bits, 32, 16, (TQ_PRESET_MSE_ONLY if mse_only else 0) if flags is None else flags, 0)
    out = tq_layout()
    _check(load().tq_record_layout(ctypes.byref(p), ctypes.byref(out)), "tq_record_layout")
    return {f: getattr(out, f) for f, _ in tq_layout._fields_}


def tq_draw_params(seed: int, head_dim: int):
    import numpy as np
    sg = np.zeros((2, head_dim), np.int8)
    S = np.zeros((head_dim, head_dim), np.float32)
    _check(load().tq_draw_params(seed, head_dim, _ptr(sg), _ptr(S)), "tq_draw_params")
    return sg, S


def tq_block_bytes(ctx: Context) -> int:
    return int(load().tq_block_bytes(ctx.handle))


def tq_quantize_store(ctx: Context, k, v, slot_mapping, pool, stream=None) -> None:
    """k, v: device tensors [T, Hkv, d] (bf16 or f32, same dtype);
    slot_mapping: device int32 [T]; pool: device uint8 [num_blocks, Hkv, record]."""
    _check(load().tq_quantize_store(*_quantize_args(ctx, k, v, slot_mapping, pool), _stream(stream)),
           "tq_quantize_store")


def _quantize_args(ctx, k, v, slot_mapping, pool):
    import torch
    _check_dev("k", k)
    _check_dev("v", v)
    _check_dev("slot_mapping", slot_mapping)
    _check_dev("pool", pool)
    if k.shape != v.shape or k.dtype != v.dtype or k.dim() != 3:
        raise ValueError("k and v must be [T, Hkv, d] tensors of one dtype")
    if slot_mapping.dtype != torch.int32 or pool.dtype != torch.uint8:
        raise TypeError("slot_mapping must be int32 and pool uint8")
    if not (k.is_contiguous() and v.is_contiguous() and slot_mapping.is_contiguous() and pool.is_contiguous()):
        raise ValueError("tensors must be contiguous")
    T, Hkv, d = k.shape
    if d != ctx.head_dim or pool.dim() != 3 or pool.shape[1] != Hkv or pool.shape[2] != ctx.block_bytes:
        raise ValueError("shape mismatch between k/v, pool and context")
    if slot_mapping.numel() != T:
        raise ValueError("slot_mapping must have one entry per token")
    return (ctx.handle, _ptr(k), _ptr(v), _dtype_code(k), T, Hkv, _ptr(slot_mapping), _ptr(pool), pool.shape[0])


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _on_device(t) -> bool:
    return t.is_cuda


def _check_dev(name, t, dtype=None, shape=None, dim=None):
    """A CUDA tensor, contiguous, of the given dtype and (prefix of) shape."""
    import torch
    _need(isinstance(t, torch.Tensor), f"{name} must be a torch tensor")
    _need(_on_device(t), f"{name} must be a device (CUDA) tensor")
    _need(t.is_contiguous(), f"{name} must be contiguous")
    if dtype is not None:
        _need(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    if dim is not None:
        _need(t.dim() == dim, f"{name} must have {dim} dimensions, got shape {tuple(t.shape)}")
    if shape is not None:
        for i, n in enumerate(shape):
            if n is not None:
                _need(t.dim() > i and t.shape[i] == n, f"{name} has shape {tuple(t.shape)}, expected {shape}")


def _decode_args(q, ctxs, pools, block_tables, seq_lens, out, workspace=None, seq_preset=None, recent_k=None,
                 recent_v=None, recent_lens=None, sm_scale=0.0, chunk_tokens=512, max_seq_len=None,
                 scores_out=None, deterministic=False, check_workspace=True):
    """Marshal the decode arguments after checking every tensor's device,
    dtype, layout and shape against the others (the library trusts device
    pointers, so a mismatch here would otherwise address memory out of
    bounds)."""
    import torch
    _need(1 <= len(ctxs) <= 2 and len(ctxs) == len(pools), "one or two contexts, one pool per context")
    _check_dev("q", q, dim=3)
    _need(q.dtype in (torch.bfloat16, torch.float32), "q must be bfloat16 or float32")
    B, Hq, d = q.shape
    for i, (c, p) in enumerate(zip(ctxs, pools)):
        _need(c.handle, f"context {i} is closed")
        _need(c.head_dim == d, f"q has head_dim {d} but context {i} has {c.head_dim}")
        _check_dev(f"pools[{i}]", p, torch.uint8, dim=3)
        _need(p.shape[2] == c.block_bytes, f"pools[{i}] records are {p.shape[2]} bytes, context {i} needs {c.block_bytes}")
    Hkv = pools[0].shape[1]
    _need(all(p.shape[1] == Hkv for p in pools), "every pool must have the same number of KV heads")
    _need(Hkv > 0 and Hq % Hkv == 0, f"num_q_heads {Hq} must be a multiple of num_kv_heads {Hkv}")
    _check_dev("block_tables", block_tables, torch.int32, (B, None), dim=2)
    _check_dev("seq_lens", seq_lens, torch.int32, (B,), dim=1)
    _check_dev("out", out, torch.float32, (B, Hq, d), dim=3)
    if len(ctxs) == 2:
        _need(seq_preset is not None, "two presets need seq_preset")
    if seq_preset is not None:
        _check_dev("seq_preset", seq_preset, torch.int8, (B,), dim=1)
    has_recent = recent_k is not None
    _need(has_recent == (recent_v is not None) == (recent_lens is not None),
          "recent_k, recent_v and recent_lens go together")
    if has_recent:
        _check_dev("recent_k", recent_k, torch.bfloat16, (B, Hkv, None, d), dim=4)
        _check_dev("recent_v", recent_v, torch.bfloat16, tuple(recent_k.shape), dim=4)
        _check_dev("recent_lens", recent_lens, torch.int32, (B,), dim=1)
    W = recent_k.shape[2] if has_recent else 0
    msl = block_tables.shape[1] * 16 if max_seq_len is None else int(max_seq_len)
    if scores_out is not None:
        _check_dev("scores_out", scores_out, torch.float32, (B, Hq, None), dim=3)
        _need(scores_out.shape[2] >= msl + W, f"scores_out needs >= {msl + W} columns")
    if check_workspace:
        _check_dev("workspace", workspace, torch.uint8)
    a = tq_decode_args()
    a.q = _ptr(q)
    a.q_dtype = _dtype_code(q)
    a.batch, a.num_q_heads = B, Hq
    a.num_kv_heads = Hkv
    a.num_presets = len(ctxs)
    for i, (c, p) in enumerate(zip(ctxs, pools)):
        a.ctx[i] = c.handle
        a.pool[i] = _ptr(p)
        a.pool_blocks[i] = p.shape[0]
    a.seq_preset = _ptr(seq_preset)
    a.block_tables = _ptr(block_tables)
    a.max_blocks_per_seq = block_tables.shape[1]
    a.seq_lens = _ptr(seq_lens)
    a.recent_k, a.recent_v, a.recent_lens = _ptr(recent_k), _ptr(recent_v), _ptr(recent_lens)
    a.recent_window = W
    a.sm_scale = sm_scale
    a.chunk_tokens = chunk_tokens
    a.max_seq_len = msl
    a.workspace = _ptr(workspace)
    a.workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    a.out = _ptr(out)
    a.scores_out = _ptr(scores_out)
    a.scores_stride = scores_out.shape[-1] if scores_out is not None else 0
    a.flags = TQ_DECODE_DETERMINISTIC if deterministic else 0
    return a


def tq_decode_workspace_bytes(q, ctxs, pools, block_tables, seq_lens, out, **kw) -> int:
    a = _decode_args(q, ctxs, pools, block_tables, seq_lens, out, check_workspace=False, **kw)
    n = load().tq_decode_workspace_bytes(ctypes.byref(a))
    if n == 0:
        raise TqError(TQ_EINVAL, "tq_decode_workspace_bytes")
    return int(n)


def tq_decode_attention(q, ctxs, pools, block_tables, seq_lens, out, workspace, stream=None, **kw) -> None:
    """q: device [B, Hq, d] bf16/f32; ctxs/pools: one or two presets;
    block_tables int32 [B, max_blocks]; seq_lens int32 [B]; out float32 [B, Hq, d];
    workspace: device uint8 tensor of tq_decode_workspace_bytes(...) bytes.
    Keyword arguments: seq_preset (int8 [B]), recent_k / recent_v (bf16
    [B, Hkv, W, d]) with recent_lens (int32 [B]), sm_scale, chunk_tokens,
    max_seq_len, scores_out (float32 [B, Hq, stride]), deterministic (sets
    TQ_DECODE_DETERMINISTIC, which changes nothing: every call takes the
    steps in a fixed order per wave, so outputs are bit-identical run to run)."""
    a = _decode_args(q, ctxs, pools, block_tables, seq_lens, out, workspace, **kw)
    _check(load().tq_decode_attention(ctypes.byref(a), _stream(stream)), "tq_decode_attention")


def tq_decode_attention_noalloc(q, ctxs, pools, block_tables, seq_lens, out, stream=None, **kw) -> None:
    """tq_decode_attention without a workspace argument: the split partials go
    to the library's static device scratch (NOALLOC_SCRATCH_BYTES per GPU),
    so the call allocates nothing.  Calls on one GPU share that scratch:
    keep them on one stream."""
    a = _decode_args(q, ctxs, pools, block_tables, seq_lens, out, None, check_workspace=False, **kw)
    _check(load().tq_decode_attention_noalloc(ctypes.byref(a), _stream(stream)), "tq_decode_attention_noalloc")


class PreparedDecode:
    """A decode call validated and marshalled once, launched many times (the
    serving loop's form of tq_decode_attention: the per-launch host cost is
    one ctypes call).  The tensors' storage is captured, so their contents may
    change between launches but they must stay allocated and in place; ``ctxs``
    must stay open.  ``noalloc=True`` launches tq_decode_attention_noalloc
    (then no workspace is passed)."""

    def __init__(self, q, ctxs, pools, block_tables, seq_lens, out, workspace=None, stream=None, noalloc=False, **kw):
        self._args = _decode_args(q, ctxs, pools, block_tables, seq_lens, out, workspace,
                                  check_workspace=not noalloc, **kw)
        self._keep = (q, list(ctxs), list(pools), block_tables, seq_lens, out, workspace, dict(kw))
        self._stream = _stream(stream)
        lib = load()
        self._fn = lib.tq_decode_attention_noalloc if noalloc else lib.tq_decode_attention
        self._name = "tq_decode_attention_noalloc" if noalloc else "tq_decode_attention"
        self._ref = ctypes.byref(self._args)

    def __call__(self) -> None:
        _check(self._fn(self._ref, self._stream), self._name)


class PreparedQuantize:
    """A tq_quantize_store call validated and marshalled once, launched many
    times (same storage rules as PreparedDecode)."""

    def __init__(self, ctx: Context, k, v, slot_mapping, pool, stream=None):
        self._a = _quantize_args(ctx, k, v, slot_mapping, pool)
        self._keep = (ctx, k, v, slot_mapping, pool)
        self._stream = _stream(stream)
        self._fn = load().tq_quantize_store

    def __call__(self) -> None:
        _check(self._fn(*self._a, self._stream), "tq_quantize_store")


def _extend_args(q, k, v, cu_chunk, ctx, pool, block_tables, prefix_lens, out, max_chunk, max_prefix_len=None,
                 sm_scale=0.0):
    """Marshal the extend arguments after checking every tensor against the
    others (device, dtype, layout, shape)."""
    import torch
    _check_dev("q", q, torch.bfloat16, dim=3)
    T, Hq, d = q.shape
    _need(ctx.handle, "context is closed")
    _need(ctx.head_dim == d, f"q has head_dim {d} but the context has {ctx.head_dim}")
    _check_dev("pool", pool, torch.uint8, dim=3)
    _need(pool.shape[2] == ctx.block_bytes, f"pool records are {pool.shape[2]} bytes, the context needs {ctx.block_bytes}")
    Hkv = pool.shape[1]
    _need(Hkv > 0 and Hq % Hkv == 0, f"num_q_heads {Hq} must be a multiple of num_kv_heads {Hkv}")
    _check_dev("k", k, torch.bfloat16, (T, Hkv, d), dim=3)
    _check_dev("v", v, torch.bfloat16, (T, Hkv, d), dim=3)
    _check_dev("cu_chunk", cu_chunk, torch.int32, dim=1)
    B = cu_chunk.shape[0] - 1
    _need(B >= 0, "cu_chunk needs batch + 1 entries")
    _check_dev("prefix_lens", prefix_lens, torch.int32, (B,), dim=1)
    _check_dev("block_tables", block_tables, torch.int32, (B, None), dim=2)
    _check_dev("out", out, torch.float32, (T, Hq, d), dim=3)
    _need(int(max_chunk) >= 0, "max_chunk must be >= 0")
    a = tq_extend_args()
    a.q, a.k, a.v, a.cu_chunk = _ptr(q), _ptr(k), _ptr(v), _ptr(cu_chunk)
    a.batch, a.num_q_heads, a.num_kv_heads, a.max_chunk = B, Hq, Hkv, int(max_chunk)
    a.ctx = ctx.handle
    a.pool, a.pool_blocks = _ptr(pool), pool.shape[0]
    a.block_tables, a.max_blocks_per_seq = _ptr(block_tables), block_tables.shape[1]
    a.prefix_lens = _ptr(prefix_lens)
    a.max_prefix_len = block_tables.shape[1] * 16 if max_prefix_len is None else int(max_prefix_len)
    a.sm_scale = sm_scale
    a.out = _ptr(out)
    return a


def tq_extend_attention(q, k, v, cu_chunk, ctx, pool, block_tables, prefix_lens, out, max_chunk, stream=None,
                        **kw) -> None:
    """Extend (chunked prefill) attention: the chunks' queries q (bf16
    [T, Hq, 128], sequence after sequence as cu_chunk (int32 [B + 1]) says)
    attend to each sequence's compressed prefix (prefix_lens int32 [B] tokens
    through block_tables into pool) and causally to the chunk's own bf16 keys
    and values k, v [T, Hkv, 128]; out float32 [T, Hq, 128].  ``max_chunk``
    bounds every chunk length; keyword arguments: max_prefix_len, sm_scale."""
    a = _extend_args(q, k, v, cu_chunk, ctx, pool, block_tables, prefix_lens, out, max_chunk, **kw)
    _check(load().tq_extend_attention(ctypes.byref(a), _stream(stream)), "tq_extend_attention")


class PreparedExtend:
    """tq_extend_attention validated and marshalled once, launched many times
    (same storage rules as PreparedDecode)."""

    def __init__(self, q, k, v, cu_chunk, ctx, pool, block_tables, prefix_lens, out, max_chunk, stream=None, **kw):
        self._args = _extend_args(q, k, v, cu_chunk, ctx, pool, block_tables, prefix_lens, out, max_chunk, **kw)
        self._keep = (q, k, v, cu_chunk, ctx, pool, block_tables, prefix_lens, out)
        self._stream = _stream(stream)
        self._fn = load().tq_extend_attention
        self._ref = ctypes.byref(self._args)

    def __call__(self) -> None:
        _check(self._fn(self._ref, self._stream), "tq_extend_attention")
