"""MXFP8 expert weights for the oracle: quantise and dequantise (numpy, float64).

TEST INFRASTRUCTURE ONLY, like the rest of this package.

The pages store the released model's experts in a 4-bit block-scaled format
(QA: the NVFP4 storage of the experts; WT: the weights are released in that
format) and run bf16 otherwise. The CDNA4-native analogue built here is the OCP
Microscaling (MX) format with FP8 E4M3 elements, as the OCP "Microscaling
Formats (MX) Specification v1.0" defines it:
  * a block is 32 consecutive elements along a row (the reduction dimension of
    an [out, in] weight);
  * its shared scale is X = 2^e, e = floor(log2(max |v|)) - 8 (8 is the largest
    exponent of an E4M3 normal; E4M3's largest finite value is 448 = 1.75 * 2^8),
    stored as the E8M0 code e + 127; a block of zeros takes e = -127;
  * each element is v / X rounded to the nearest E4M3 value, ties to even,
    magnitudes above 448 saturating to 448 (E4M3 "fn": no infinities; the codes
    0x7F and 0xFF are NaN and never produced);
  * the value of a stored element is e4m3(code) * 2^e; for the exponent ranges
    of these weights it is exactly representable in bf16, so the dequantised
    weights are bf16 values and the layer's maths is unchanged.
"""
from __future__ import annotations

import numpy as np

__all__ = ["MX_BLOCK", "e4m3_encode", "e4m3_decode", "quantize_mxfp8", "dequantize_mxfp8"]

MX_BLOCK = 32
E4M3_MAX = 448.0
E4M3_EMAX = 8          # exponent of the largest normal
E4M3_EMIN = -6         # exponent of the smallest normal
E4M3_MBITS = 3


def e4m3_decode(codes) -> np.ndarray:
    """E4M3fn codes (uint8) -> float64 values (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** (E4M3_EMIN - E4M3_MBITS),
                   (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(v) -> np.ndarray:
    """float64 values -> E4M3fn codes, round to nearest (ties to even), saturating at 448."""
    v = np.asarray(v, dtype=np.float64)
    assert np.all(np.isfinite(v))
    sign = (np.signbit(v)).astype(np.int64) << 7
    a = np.minimum(np.abs(v), E4M3_MAX)
    # grid spacing of the binade of a: subnormals share the spacing of the lowest binade
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.clip(e, E4M3_EMIN, E4M3_EMAX)
    step = np.exp2(e - E4M3_MBITS)
    q = np.rint(a / step) * step                 # np.rint: ties to even
    q = np.minimum(q, E4M3_MAX)                  # (rounding up may leave the binade; 448 is the top)
    # encode q exactly
    with np.errstate(divide="ignore"):
        eq = np.floor(np.log2(np.where(q > 0, q, 1.0)))
    normal = q >= 2.0 ** E4M3_EMIN
    exp_field = np.where(normal, eq + 7, 0).astype(np.int64)
    man = np.where(normal, q / np.exp2(eq) - 1.0, q / 2.0 ** (E4M3_EMIN - E4M3_MBITS) / 8.0) * 8.0
    man_field = np.rint(man).astype(np.int64)
    codes = sign | (exp_field << 3) | man_field
    return codes.astype(np.uint8)


def quantize_mxfp8(w) -> tuple:
    """w [..., C] (C a multiple of 32) -> (codes uint8 [..., C], scales uint8 [..., C/32])."""
    w = np.asarray(w, dtype=np.float64)
    C = w.shape[-1]
    assert C % MX_BLOCK == 0
    blocks = w.reshape(w.shape[:-1] + (C // MX_BLOCK, MX_BLOCK))
    amax = np.max(np.abs(blocks), axis=-1)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - E4M3_EMAX, -127.0)
    e = np.clip(e, -127, 127)
    codes = e4m3_encode(blocks / np.exp2(e)[..., None])
    scales = (e + 127).astype(np.uint8)
    return codes.reshape(w.shape), scales


def dequantize_mxfp8(codes, scales) -> np.ndarray:
    """(codes [..., C], scales [..., C/32]) -> float64 [..., C]."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    C = codes.shape[-1]
    vals = e4m3_decode(codes).reshape(codes.shape[:-1] + (C // MX_BLOCK, MX_BLOCK))
    e = scales.astype(np.float64) - 127.0
    return (vals * np.exp2(e)[..., None]).reshape(codes.shape)
