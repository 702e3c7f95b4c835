"""Per-tensor 8-bit quantization, written out from the format definition
(test infrastructure only).

The pages quantize each tensor as a whole with scale = FP8max / (Amax + eps),
Amax the largest magnitude in the tensor, one scale per tensor and no finer
blocks (OSP-Next summary, 方法步骤详情 method steps).  Their 8-bit format is
Huawei's HiF8, which is proprietary and not bit-defined on the pages
(局限与改进 limitations); the MI355X build uses OCP FP8 E4M3 (the "fn"
variant) in its place, with FP8max = 448.

OCP E4M3: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits.
  exponent field 0      -> subnormal  m * 2^-9
  exponent field 1..15  -> (1 + m/8) * 2^(e-7)
  exponent 15, m = 7    -> NaN (no infinities); largest finite value 448.

Encoding used here: round to nearest, ties to even, saturating to +-448 for
magnitudes at or above 464 (the midpoint past 448, infinities included); the
sign of zero is kept.  NaN has two codes in the format (either sign); this
build writes every NaN as 0xFF (S.1111.111 with the sign bit set), the code
gfx950's fp32 -> e4m3 conversion instruction produces for a NaN.

Non-finite tensors: Amax is the largest magnitude, so a NaN anywhere makes
Amax and the scale NaN and every product NaN (all codes 0xFF); an infinity
makes the scale 0, finite elements become signed zeros and the infinities
themselves (inf * 0) NaN.  A diverging tensor therefore shows up in its codes
instead of being hidden behind finite values.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode_table() -> np.ndarray:
    """float64 value of each of the 256 codes (NaN for the two NaN codes)."""
    vals = np.empty(256, np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = sign * m * 2.0 ** -9
        else:
            vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


_TABLE = e4m3_decode_table()
_POS = _TABLE[:127]  # codes 0x00..0x7E, non-negative finite, increasing


NAN_CODE = 0xFF


def e4m3_encode(x) -> np.ndarray:
    """Encode values (float64/float32 array) to E4M3 codes (uint8); NaN gives
    0xFF, infinities saturate."""
    xd = np.asarray(x, np.float64)
    nan = np.isnan(xd)
    a = np.abs(np.where(nan, 0.0, xd))
    neg = np.signbit(xd)
    hi = np.searchsorted(_POS, a, side="left")          # first value >= a
    hi = np.clip(hi, 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    dlo = a - _POS[lo]
    dhi = _POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(a >= _POS[hi], hi, np.where(pick_hi, hi, lo))
    code = np.where(a >= 464.0, 126, code)              # saturate
    code = code | np.where(neg, 0x80, 0)
    return np.where(nan, NAN_CODE, code).astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    return _TABLE[np.asarray(codes, np.uint8)]


def per_tensor_scale(amax: np.float32, fp8_max=E4M3_MAX, eps=1e-12) -> np.float32:
    """scale = fp8_max / (amax + eps), every step in IEEE fp32."""
    den = np.float32(amax) + np.float32(eps)
    return np.float32(np.float32(fp8_max) / den)


def quantize_per_tensor(x, fp8_max=E4M3_MAX, eps=1e-12):
    """Quantize one whole tensor: returns (codes uint8, scale fp32, amax fp32).

    x holds the values as given to the device (bf16 or fp32, widened to fp32
    exactly).  Each element is multiplied by the scale in fp32 and the product
    is encoded with :func:`e4m3_encode`.
    """
    xf = np.asarray(x, np.float32)
    # np.max propagates NaN: one NaN element makes Amax NaN
    amax = np.float32(np.max(np.abs(xf))) if xf.size else np.float32(0.0)
    with np.errstate(invalid="ignore", divide="ignore", over="ignore"):
        scale = per_tensor_scale(amax, fp8_max, eps)
        prod = (xf * scale).astype(np.float32)
    return e4m3_encode(prod), scale, amax


def dequantize(codes, scale) -> np.ndarray:
    """float64 values code / scale."""
    return e4m3_decode(codes) / np.float64(scale)
