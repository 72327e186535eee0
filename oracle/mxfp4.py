"""MXFP4 expert weights for the oracle: quantise and dequantise (numpy, float64).

TEST INFRASTRUCTURE ONLY, like the rest of this package.

The released model stores its experts in a block-scaled 4-bit format (QA: the
NVFP4 storage of the experts). The CDNA4-native 4-bit analogue built here is
the OCP Microscaling (MX) format with FP4 E2M1 elements, as the OCP
"Microscaling Formats (MX) Specification v1.0" defines it:
  * an E2M1 element has a sign, a 2-bit exponent (bias 1) and one mantissa
    bit; its magnitudes are 0, 0.5 (the one subnormal), 1, 1.5, 2, 3, 4, 6
    (no infinities or NaN);
  * a block is 32 consecutive elements along a row (the reduction dimension of
    an [out, in] weight) with a shared scale X = 2^e, e = floor(log2(max |v|))
    - 2 (2 is the exponent of E2M1's largest normal), stored as the E8M0 code
    e + 127; a block of zeros takes e = -127;
  * each element is v / X rounded to the nearest E2M1 value, ties to even
    (the value with mantissa bit 0), magnitudes above 6 saturating to 6;
  * two elements share a byte, the even-indexed one in the low nibble.
The dequantised weights are bf16 values for these exponent ranges, so the
layer's maths is unchanged.
"""
from __future__ import annotations

import numpy as np

__all__ = ["E2M1_VALUES", "e2m1_encode", "e2m1_decode", "quantize_mxfp4", "dequantize_mxfp4"]

MX_BLOCK = 32
E2M1_MAX = 6.0
E2M1_EMAX = 2
# magnitude of code c (c = 0..7): exponent field c >> 1, mantissa bit c & 1
E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(codes) -> np.ndarray:
    """E2M1 codes (0..15) -> float64 values."""
    c = np.asarray(codes).astype(np.int64)
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.exp2(e - 1.0))
    return np.where(c & 8, -mag, mag)


def e2m1_encode(v) -> np.ndarray:
    """float64 values -> E2M1 codes (uint8, 0..15): nearest value, ties to the
    even code (mantissa bit 0), magnitudes above 6 saturating to 6."""
    v = np.asarray(v, dtype=np.float64)
    assert np.all(np.isfinite(v))
    sign = np.signbit(v).astype(np.int64) << 3
    a = np.minimum(np.abs(v), E2M1_MAX)
    # the grid step in the binade of a: 0.5 below 2 (subnormal and e = 1), 1 in [2, 4), 2 in [4, 6]
    step = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    q = np.rint(a / step) * step                     # ties to even multiple of the step
    q = np.minimum(q, E2M1_MAX)
    mag_code = np.searchsorted(E2M1_VALUES, q)       # q is one of the grid values
    assert np.all(E2M1_VALUES[mag_code] == q)
    return (sign | mag_code).astype(np.uint8)


def quantize_mxfp4(w) -> tuple:
    """w [..., C] (C a multiple of 32) -> (packed codes uint8 [..., C/2], scales uint8 [..., C/32])."""
    w = np.asarray(w, dtype=np.float64)
    C = w.shape[-1]
    assert C % MX_BLOCK == 0
    blocks = w.reshape(w.shape[:-1] + (C // MX_BLOCK, MX_BLOCK))
    amax = np.max(np.abs(blocks), axis=-1)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - E2M1_EMAX, -127.0)
    e = np.clip(e, -127, 127)
    codes = e2m1_encode(blocks / np.exp2(e)[..., None]).reshape(w.shape)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, (e + 127).astype(np.uint8)


def dequantize_mxfp4(packed, scales) -> np.ndarray:
    """(packed codes [..., C/2], scales [..., C/32]) -> float64 [..., C]."""
    packed = np.asarray(packed, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    codes = np.stack([packed & 0xF, packed >> 4], axis=-1).reshape(packed.shape[:-1] + (2 * packed.shape[-1],))
    C = codes.shape[-1]
    vals = e2m1_decode(codes).reshape(codes.shape[:-1] + (C // MX_BLOCK, MX_BLOCK))
    e = scales.astype(np.float64) - 127.0
    return (vals * np.exp2(e)[..., None]).reshape(codes.shape)
