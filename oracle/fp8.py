"""fp64 CPU oracle of per-tensor FP8 (E4M3) quantization and the FP8 linear map.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no
code with the HIP path.

The pages list FP8 among the precisions Megatron Core trains in (page
"Megatron-LM / Megatron Core README digest", §2, and the precision flags of
page "Megatron-LM 3D parallelism guide", §5.3) and give no recipe.  Reading
taken: the OCP E4M3 format without infinities (1 sign bit, 4 exponent bits
with bias 7, 3 mantissa bits; largest finite value 448, smallest subnormal
2^-9) and one fp32 scale per tensor, s = amax / 448, so the largest
magnitude maps to 448:

    q(x) = RNE_E4M3(clamp(fl32(x / s), -448, 448)),   x = q(x) * s
    y    = (q(A) q(B)^T) * (s_A s_B)                    (+ bias)

where fl32 is the fp32-rounded quotient and RNE_E4M3 rounds to the nearest
E4M3 value, ties to the even mantissa.  A tensor of zeros gets s = 1.
"""
from __future__ import annotations

import numpy as np

__all__ = ["E4M3_MAX", "e4m3_round", "e4m3_encode", "e4m3_decode", "quantize_per_tensor",
           "fp8_linear"]

E4M3_MAX = 448.0
_MIN_NORMAL_EXP = -6      # smallest normal: 2^-6
_MANT_BITS = 3


def e4m3_round(v: np.ndarray) -> np.ndarray:
    """Nearest E4M3 value (ties to even mantissa) of each |v| <= 448, in fp64.

    A normal value with exponent e lies on a grid of spacing 2^(e-3); the
    subnormals (below 2^-6) on a grid of spacing 2^-9.  Rounding to the grid
    with numpy's round-half-to-even picks the even mantissa on ties; a value
    that rounds up to the next power of two is that power (representable)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, _MIN_NORMAL_EXP)
    # guard the floor(log2) against representation error at exact powers of two
    e = np.where(2.0 ** e > a, e - 1, e)
    e = np.where(2.0 ** (e + 1) <= a, e + 1, e)
    e = np.maximum(e, _MIN_NORMAL_EXP)
    spacing = 2.0 ** (e - _MANT_BITS)
    r = np.round(a / spacing) * spacing
    return np.copysign(r, v)


def e4m3_encode(q: np.ndarray) -> np.ndarray:
    """Bit patterns (uint8) of E4M3 values: sign << 7 | exponent << 3 | mantissa."""
    q = np.asarray(q, dtype=np.float64)
    sign = (np.signbit(q)).astype(np.uint8) << 7
    a = np.abs(q)
    sub = a < 2.0 ** _MIN_NORMAL_EXP
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0))).astype(np.int64)
    mant_n = np.round(a / 2.0 ** e * 8 - 8).astype(np.int64)
    mant_s = np.round(a / 2.0 ** -9).astype(np.int64)
    exp_field = np.where(sub, 0, e + 7)
    mant = np.where(sub, mant_s, mant_n)
    return (sign | (exp_field.astype(np.uint8) << 3) | mant.astype(np.uint8)).astype(np.uint8)


def e4m3_decode(code: np.ndarray) -> np.ndarray:
    """fp64 values of E4M3 bit patterns (0x7f / 0xff, the NaN codes, give NaN)."""
    c = np.asarray(code, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    m = c & 7
    val = np.where(ef == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (ef - 7))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return s * val


def quantize_per_tensor(x):
    """(q, s): q the E4M3 values (fp64) of x / s, s = amax / 448 in fp32."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0)
    s = np.float32(amax / np.float32(E4M3_MAX)) if amax > 0 else np.float32(1.0)
    v = (x32 / s).astype(np.float32)                 # fp32 quotient
    v = np.clip(v.astype(np.float64), -E4M3_MAX, E4M3_MAX)
    return e4m3_round(v), s


def fp8_linear(qa, sa, qb, sb, bias=None):
    """y = (qa qb^T) * (sa sb) (+ bias) in fp64."""
    y = np.asarray(qa, np.float64) @ np.asarray(qb, np.float64).T * (float(sa) * float(sb))
    if bias is not None:
        y = y + np.asarray(bias, np.float64)
    return y
