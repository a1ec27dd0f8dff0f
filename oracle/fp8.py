"""fp64 CPU oracle of per-tensor FP8 quantization (E4M3 and E5M2) and the
FP8 linear maps of the layer, forward and backward.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no
code with the HIP path.

The pages list FP8 among the precisions Megatron Core trains in (page
"Megatron-LM / Megatron Core README digest", §0, and the ``--enable-fp8``
flag of page "Megatron-LM 3D parallelism guide", §5.1) and give no recipe.
Reading taken:

* two OCP 8-bit formats without infinities in use: E4M3 (1 sign bit, 4
  exponent bits with bias 7, 3 mantissa bits; largest finite value 448,
  smallest subnormal 2^-9) for activations and weights, and E5M2 (5 exponent
  bits with bias 15, 2 mantissa bits; largest finite 57344, smallest
  subnormal 2^-16) for gradients, whose range matters more than their
  precision;
* one fp32 scale per tensor, s = amax / max_format, so the largest magnitude
  maps to the format's largest value (a tensor of zeros gets s = 1); the
  scale belongs to the whole (unsharded) tensor, so tensor-parallel ranks
  agree on it and the column/row split stays exact:

      q(x) = RNE_fmt(clamp(fl32(x / s), -max, max)),   x ~ q(x) * s

  where fl32 is the fp32-rounded quotient and RNE_fmt rounds to the nearest
  value of the format, ties to the even mantissa;
* the forward linear map y = x W^T (+ b) is (q(x) q(W)^T) s_x s_W in fp32
  (+ b), both operands E4M3; the data gradient dx = dy W is
  (q(dy) q(W)) s_dy s_W with dy in E5M2 and the forward's E4M3 codes of W;
  the weight gradient dW = dy^T x is (q(dy)^T q(x)) s_dy s_x with the same
  E5M2 codes of dy and the forward's E4M3 codes of x.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = ["E4M3", "E5M2", "E4M3_MAX", "E5M2_MAX", "fp8_round", "fp8_encode", "fp8_decode",
           "e4m3_round", "e4m3_encode", "e4m3_decode", "quantize_per_tensor", "dequantize",
           "fp8_linear", "fp8_dgrad", "fp8_wgrad"]


@dataclass(frozen=True)
class Fmt:
    name: str
    exp_bits: int
    mant_bits: int
    bias: int
    max: float

    @property
    def min_normal_exp(self) -> int:
        return 1 - self.bias

    @property
    def sub_spacing(self) -> float:
        return 2.0 ** (self.min_normal_exp - self.mant_bits)


E4M3 = Fmt("e4m3", 4, 3, 7, 448.0)
E5M2 = Fmt("e5m2", 5, 2, 15, 57344.0)
E4M3_MAX = E4M3.max
E5M2_MAX = E5M2.max


def _fmt(fmt) -> Fmt:
    if isinstance(fmt, Fmt):
        return fmt
    return {"e4m3": E4M3, "e5m2": E5M2}[fmt]


def _binade(a: np.ndarray, fmt: Fmt) -> np.ndarray:
    """Exponent e with 2^e <= a < 2^(e+1), at least the smallest normal one."""
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, fmt.min_normal_exp)
    # guard the floor(log2) against representation error at exact powers of two
    e = np.where(2.0 ** e > a, e - 1, e)
    e = np.where(2.0 ** (e + 1) <= a, e + 1, e)
    return np.maximum(e, fmt.min_normal_exp)


def fp8_round(v: np.ndarray, fmt="e4m3") -> np.ndarray:
    """Nearest value of the format (ties to even mantissa) of each |v| <= max, in fp64.

    A normal value with exponent e lies on a grid of spacing 2^(e - mant_bits);
    the subnormals (below the smallest normal power of two) on the grid of
    the smallest normal binade.  Rounding to the grid with numpy's
    round-half-to-even picks the even mantissa on ties; a value that rounds up
    to the next power of two is that power (representable)."""
    f = _fmt(fmt)
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    spacing = 2.0 ** (_binade(a, f) - f.mant_bits)
    r = np.round(a / spacing) * spacing
    return np.copysign(r, v)


def fp8_encode(q: np.ndarray, fmt="e4m3") -> np.ndarray:
    """Bit patterns (uint8) of values of the format:
    sign << 7 | exponent field << mant_bits | mantissa."""
    f = _fmt(fmt)
    q = np.asarray(q, dtype=np.float64)
    sign = (np.signbit(q)).astype(np.uint8) << 7
    a = np.abs(q)
    sub = a < 2.0 ** f.min_normal_exp
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0))).astype(np.int64)
    one = 1 << f.mant_bits
    mant_n = np.round(a / 2.0 ** e * one - one).astype(np.int64)
    mant_s = np.round(a / f.sub_spacing).astype(np.int64)
    exp_field = np.where(sub, 0, e + f.bias)
    mant = np.where(sub, mant_s, mant_n)
    return (sign | (exp_field.astype(np.uint8) << f.mant_bits) | mant.astype(np.uint8)).astype(np.uint8)


def fp8_decode(code: np.ndarray, fmt="e4m3") -> np.ndarray:
    """fp64 values of bit patterns of the format.  E4M3: 0x7f / 0xff are NaN;
    E5M2: the all-ones exponent field is infinity (mantissa 0) or NaN."""
    f = _fmt(fmt)
    c = np.asarray(code, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> f.mant_bits) & ((1 << f.exp_bits) - 1)
    m = c & ((1 << f.mant_bits) - 1)
    one = float(1 << f.mant_bits)
    val = np.where(ef == 0, m * f.sub_spacing, (1.0 + m / one) * 2.0 ** (ef - f.bias))
    if f is E4M3:
        val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    else:
        top = ef == (1 << f.exp_bits) - 1
        val = np.where(top & (m == 0), np.inf, np.where(top, np.nan, val))
    return s * val


def e4m3_round(v):
    return fp8_round(v, E4M3)


def e4m3_encode(q):
    return fp8_encode(q, E4M3)


def e4m3_decode(code):
    return fp8_decode(code, E4M3)


def quantize_per_tensor(x, fmt="e4m3"):
    """(q, s): q the format's values (fp64) of x / s, s = amax / max in fp32.
    x is taken in fp32 (the precision the quotient is formed in)."""
    f = _fmt(fmt)
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0)
    s = np.float32(amax / np.float32(f.max)) if amax > 0 else np.float32(1.0)
    v = (x32 / s).astype(np.float32)                 # fp32 quotient
    v = np.clip(v.astype(np.float64), -f.max, f.max)
    return fp8_round(v, f), s


def dequantize(q, s) -> np.ndarray:
    return np.asarray(q, np.float64) * float(s)


def fp8_linear(qa, sa, qb, sb, bias=None):
    """y = (qa qb^T) * (sa sb) (+ bias) in fp64."""
    y = np.asarray(qa, np.float64) @ np.asarray(qb, np.float64).T * (float(sa) * float(sb))
    if bias is not None:
        y = y + np.asarray(bias, np.float64)
    return y


def fp8_dgrad(qdy, sdy, qw, sw):
    """dx = (qdy qw) * (sdy sw): the data gradient through y = x W^T."""
    return np.asarray(qdy, np.float64) @ np.asarray(qw, np.float64) * (float(sdy) * float(sw))


def fp8_wgrad(qdy, sdy, qx, sx):
    """dW = (qdy^T qx) * (sdy sx): the weight gradient of y = x W^T."""
    return np.asarray(qdy, np.float64).T @ np.asarray(qx, np.float64) * (float(sdy) * float(sx))
