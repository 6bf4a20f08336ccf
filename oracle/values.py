"""Value group quantisation.

Hub, "technical principle", step 4: values are not rotated; they are
quantised in groups (32 elements by default) with a recorded scale and
zero-point, then stored at 2 or 4 bits.

Reading: the page calls this quantisation "symmetric" yet records a
zero-point; asymmetric min-max is the only reading that uses a zero-point, so:

  per group of 32 consecutive channels:  mn = min v, mx = max v,
  s = fp16( fp32( fp32(mx - mn) / fp32(2^b - 1) ) ),   z = fp16(mn),
  q = clamp( rint_half_even( fp32( fp32(v - z) / s ) ), 0, 2^b - 1 )
  (q = 0 for the whole group when s == 0),
  dequantised value  v^ = q s + z.

The code decision is taken in fp32 with IEEE (correctly rounded) division —
the same precision the GPU kernel decides in — so both sides round the same
number; the inputs are fp32 (bf16 inputs are exact in fp32).
"""

from __future__ import annotations

import numpy as np

from . import bits as _bits
from . import rotation as _rot

__all__ = ["encode_values", "dequantize_values", "rotate_values", "GROUP"]

GROUP = 32


def encode_values(v, b: int):
    """Encode values ``v`` [N, d] (fp32 exact) at ``b`` bits.

    Returns dict with ``q`` int64 [N, d], ``s16``, ``z16`` uint16 [N, d/32]
    and, for boundary accounting, ``x`` fp32 [N, d] (the rounded quotient,
    NaN where s == 0) and ``s_mid``/``z_mid`` fp64 inputs of the fp16
    roundings."""
    v = np.asarray(v, dtype=np.float32)
    N, d = v.shape
    G = d // GROUP
    vg = v.reshape(N, G, GROUP)
    mn = vg.min(axis=2)
    mx = vg.max(axis=2)
    levels = np.float32((1 << b) - 1)
    s_f32 = (mx - mn).astype(np.float32) / levels
    s16 = s_f32.astype(np.float16)
    z16 = mn.astype(np.float16)
    s32 = s16.astype(np.float32)
    z32 = z16.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        x = (vg - z32[:, :, None]).astype(np.float32) / s32[:, :, None]
    x = x.astype(np.float32)
    q = np.clip(np.rint(x), 0, (1 << b) - 1)
    live = s32 != 0
    q = np.where(live[:, :, None], q, 0).astype(np.int64)
    x = np.where(live[:, :, None], x, np.nan)
    return {
        "q": q.reshape(N, d),
        "s16": s16.view(np.uint16),
        "z16": z16.view(np.uint16),
        "x": x.reshape(N, d),
        "s_pre": s_f32.astype(np.float64),
        "z_pre": mn.astype(np.float64),
    }


def dequantize_values(q, s16, z16) -> np.ndarray:
    """v^ = q s + z in fp64, from codes [N, d] and fp16 scale / zero [N, d/32]."""
    q = np.asarray(q, dtype=np.float64)
    N, d = q.shape
    s = _bits.from_fp16_bits(s16).reshape(N, d // GROUP, 1)
    z = _bits.from_fp16_bits(z16).reshape(N, d // GROUP, 1)
    return (q.reshape(N, d // GROUP, GROUP) * s + z).reshape(N, d)


def rotate_values(v, d1, d2) -> np.ndarray:
    """Rotated values for the weight-absorption variant (Roadmap §4.2: the
    value vectors are rotated with the same D2 H D1 / sqrt(d) as the keys when
    they are written, and the inverse rotation is folded into the output
    projection instead of being applied at read time).

    Reading: the rotation is taken exactly (fp64) and rounded once to fp32;
    the group quantisation then runs on those fp32 values unchanged."""
    return _rot.rotate(np.asarray(v, dtype=np.float64), d1, d2).astype(np.float32)
