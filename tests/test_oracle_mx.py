"""Pins of the oracle's MXFP8 quantiser (oracle/mxfp8.py) against a library
routine (torch's float8_e4m3fn conversion) and closed forms of the OCP MX
definition."""
import numpy as np
import pytest
import torch

import oracle


def _torch_e4m3(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch_within_range():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.normal(0, 60, 200000), rng.normal(0, 0.01, 20000), rng.uniform(-448, 448, 20000),
                        # ties between neighbours, the subnormal range, the top of the range
                        (np.arange(-4000, 4000) + 0.5) * 2.0 ** -10, np.arange(0, 64) * 2.0 ** -12,
                        np.array([0.0, -0.0, 448.0, -448.0, 447.99, 432.0, 440.0, 2.0 ** -6, 2.0 ** -9])])
    v = v[np.abs(v) <= 448]
    assert np.array_equal(oracle.e4m3_encode(v), _torch_e4m3(v))


def test_e4m3_saturates_and_never_makes_nan():
    c = oracle.e4m3_encode(np.array([449.0, 464.0, 480.0, 1e6, -1e6]))
    assert list(c) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE]


def test_e4m3_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_decode(codes)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan) and list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(got[~nan], want[~nan])


@pytest.mark.parametrize("amax,e", [(1.0, -8), (1.5, -8), (1.75, -8), (2.0 ** -20, -28), (3.0 * 2.0 ** 7, 0), (3.0 * 2.0 ** 6, -1),
                                    (448.0, 0), (0.0, -127)])
def test_block_scale_closed_form(amax, e):
    w = np.zeros((1, 32))
    w[0, 5] = -amax
    w[0, 6] = amax / 3
    codes, scales = oracle.quantize_mxfp8(w)
    assert scales.shape == (1, 1) and int(scales[0, 0]) == e + 127
    if amax > 0:
        # the largest element becomes 2^(floor(log2 amax) - e) * mantissa, i.e. amax / 2^e exactly
        assert oracle.e4m3_decode(codes[0, 5]) * 2.0 ** e == -amax


def test_block_above_1p75_saturates_per_the_definition():
    w = np.full((1, 32), 0.1)
    w[0, 0] = 1.9                      # mantissa 1.9 > 1.75: 1.9 * 2^8 is beyond 448
    codes, scales = oracle.quantize_mxfp8(w)
    assert int(scales[0, 0]) == 127 - 8 and codes[0, 0] == 0x7E
    assert oracle.dequantize_mxfp8(codes, scales)[0, 0] == 1.75


def test_roundtrip_of_representable_weights_is_exact():
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 0x7E, size=(8, 128), dtype=np.uint8)        # finite positive codes
    codes[:, ::32] = 0x77                                               # 1.875 * 2^0 ... keep amax mantissa <= 1.75:
    codes[:, ::32] = 0x76                                               # 1.75 * 2^0, the largest of each block
    codes = np.where(oracle.e4m3_decode(codes) > 1.75, 0x76, codes).astype(np.uint8)
    sgn = rng.integers(0, 2, size=codes.shape).astype(np.uint8) << 7
    codes = codes | sgn
    e = rng.integers(-20, 4, size=(8, 4))
    w = oracle.e4m3_decode(codes).reshape(8, 4, 32) * np.exp2(e)[..., None]
    q, s = oracle.quantize_mxfp8(w.reshape(8, 128))
    assert np.array_equal(oracle.dequantize_mxfp8(q, s), w.reshape(8, 128))


def test_quantisation_error_bound():
    """Within a block whose amax mantissa is <= 1.75 every element is within half a
    step of the block's grid: |w - dq| <= 2^(e+floor(log2|w|)-3) / 2, and at most
    2^(e-9)/2 in the subnormal range."""
    rng = np.random.default_rng(2)
    w = rng.normal(0, 0.02, (256, 256))
    q, s = oracle.quantize_mxfp8(w)
    dq = oracle.dequantize_mxfp8(q, s)
    e = np.repeat(s.astype(np.float64) - 127, 32, axis=1)
    a = np.abs(w) / np.exp2(e)
    ok_block = np.repeat(np.max(a.reshape(256, 8, 32), axis=-1) <= 448, 32, axis=1)
    with np.errstate(divide="ignore"):
        step = np.exp2(np.maximum(np.floor(np.log2(np.where(a > 0, a, 1))), -6) - 3)
    assert np.all(np.abs(w - dq)[ok_block] <= 0.5 * step[ok_block] * np.exp2(e[ok_block]) * (1 + 1e-12))
