"""Decode attention over the compressed cache (plus an optional window of
recent full-precision tokens).

iThome, "why not just round": score = Q . K, output = softmax(score) . V.
Roadmap §3.2: decode scores keys straight from the codes (rotate q once, look
the codebook up per query) and runs the softmax in the exp2 domain; the
oracle computes the same quantities directly in fp64, with no splitting.
Hub, "vLLM integration" (hybrid mode): the most recent 128 tokens (configurable)
stay in full precision and join the same attention.

Readings: logits are sm_scale * score with sm_scale = 1/sqrt(d) by default
(the iThome formula writes score = Q . K without a scale); query head h uses KV
head h // G with G = num_q_heads / num_kv_heads (consecutive grouping); every
cached token is attended; recent tokens are scored exactly, <q, k> with the
bf16 key and unrotated query.
"""

from __future__ import annotations

import numpy as np

from . import keys as _keys
from . import rotation as _rot
from . import values as _values

__all__ = ["decode_one_sequence", "extend_one_sequence", "softmax_attend", "fold_output_projection"]


def softmax_attend(logits, values) -> np.ndarray:
    """Textbook softmax(logits) @ values in fp64 (logits [T], values [T, d]).
    An empty set of tokens gives a zero vector."""
    logits = np.asarray(logits, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    if logits.size == 0:
        return np.zeros(values.shape[-1])
    w = np.exp(logits - logits.max())
    return (w / w.sum()) @ values


def decode_one_sequence(q, fields_per_head, ctx, recent_k=None, recent_v=None, sm_scale=None):
    """Attention output and raw scores for one sequence.

    ``q``: [Hq, d] query (fp32-exact values).
    ``fields_per_head``: list over KV heads of the dicts returned by
    ``oracle.paged.read_tokens`` (quantised tokens, all the same length L).
    ``ctx``: dict with d1, d2, S, c32 and optionally ``qjl`` (False for
    MSE-only keys; default True).
    ``recent_k``/``recent_v``: [Hkv, R, d] full-precision window or None.

    Returns (out [Hq, d], scores [Hq, L + R]) where scores are the unscaled
    estimates for the quantised tokens followed by exact <q, k> for the
    recent ones."""
    q = np.asarray(q, dtype=np.float64)
    Hq, d = q.shape
    Hkv = len(fields_per_head)
    G = Hq // Hkv
    scale = (1.0 / np.sqrt(d)) if sm_scale is None else float(sm_scale)
    outs, scores = [], []
    for hk in range(Hkv):
        f = fields_per_head[hk]
        heads = q[hk * G:(hk + 1) * G]  # the query heads that read KV head hk
        est = _keys.estimate_scores(heads, f["idx"], f["sign"], f["n16"], f["g16"],
                                    ctx["d1"], ctx["d2"], ctx["S"], ctx["c32"], qjl=ctx.get("qjl", True))
        vhat = _values.dequantize_values(f["q"], f["s16"], f["z16"])
        if recent_k is not None:
            rk = np.asarray(recent_k[hk], dtype=np.float64)
            rv = np.asarray(recent_v[hk], dtype=np.float64)
            v_all = np.concatenate([vhat, rv], axis=0)
        else:
            v_all = vhat
        for g in range(G):
            s_all = np.concatenate([est[g], rk @ heads[g]]) if recent_k is not None else est[g]
            outs.append(softmax_attend(scale * s_all, v_all))
            scores.append(s_all)
    return np.stack(outs), np.stack(scores)


def extend_one_sequence(q, fields_per_head, k_chunk, v_chunk, ctx, sm_scale=None):
    """Extend (chunked prefill) attention for one sequence: a chunk of C new
    tokens attends to the sequence's compressed prefix and, causally, to the
    chunk itself.

    Roadmap §4.1: SGLang's extend (prefill) stage is a fused kernel over the
    compressed pool, like its decode kernel; Roadmap §4.4: prefill is where
    the rotation / quantisation cost shows.  Reading (the pages give no
    formula for it): query token i of the chunk (position P + i) scores the P
    prefix tokens with the same estimator as decode (rotated query, codes,
    QJL correction, stored fp16 n and gamma) and the chunk tokens j <= i
    exactly, <q_i, k_j> with the bf16 key and unrotated query; its values are
    the dequantised q s + z of the prefix and the bf16 values of the chunk;
    one softmax runs over all P + i + 1 logits.  The chunk's own keys and
    values are stored compressed by the store path (tq_quantize_store), not
    read back from the cache here.

    ``q``: [C, Hq, d]; ``fields_per_head``: list over KV heads of the
    ``paged.read_tokens`` fields of the prefix (all of length P);
    ``k_chunk``, ``v_chunk``: [C, Hkv, d]; ``ctx`` as for
    ``decode_one_sequence``.  Returns out [C, Hq, d] in fp64."""
    q = np.asarray(q, dtype=np.float64)
    C, Hq, d = q.shape
    Hkv = len(fields_per_head)
    G = Hq // Hkv
    scale = (1.0 / np.sqrt(d)) if sm_scale is None else float(sm_scale)
    out = np.zeros((C, Hq, d))
    for hk in range(Hkv):
        f = fields_per_head[hk]
        kc = np.asarray(k_chunk[:, hk], dtype=np.float64)
        vc = np.asarray(v_chunk[:, hk], dtype=np.float64)
        vhat = _values.dequantize_values(f["q"], f["s16"], f["z16"])
        for g in range(G):
            hq = hk * G + g
            est = _keys.estimate_scores(q[:, hq], f["idx"], f["sign"], f["n16"], f["g16"],
                                        ctx["d1"], ctx["d2"], ctx["S"], ctx["c32"], qjl=ctx.get("qjl", True))
            exact = q[:, hq] @ kc.T   # [C, C]: <q_i, k_j>
            for i in range(C):
                logits = np.concatenate([est[i], exact[i, :i + 1]])
                vals = np.concatenate([vhat, vc[:i + 1]], axis=0)
                out[i, hq] = softmax_attend(scale * logits, vals)
    return out


def fold_output_projection(w_o, d1, d2, num_heads: int) -> np.ndarray:
    """Output projection with the inverse value rotation absorbed (Roadmap
    §4.2, W_O weight absorption): when the cached values are rotated, the
    attention output of head h is (approximately) Pi o_h, and
    W_o [.., h d:(h+1) d] Pi^-1 restores W_o o.  Pi^-1 = D1 (H / sqrt d) D2:
    the sign vectors in the reverse order of the forward rotation (the order
    the page's code review caught).  Returns W_o blockdiag(Pi^-1, ...) in
    fp64."""
    w = np.asarray(w_o, dtype=np.float64)
    d = np.asarray(d1).shape[0]
    inv = _rot.inverse_rotation_matrix(d1, d2)
    out = np.empty_like(w)
    for h in range(num_heads):
        out[:, h * d:(h + 1) * d] = w[:, h * d:(h + 1) * d] @ inv
    return out
