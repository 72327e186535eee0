"""Pins of the oracle's MXFP8 quantiser (oracle/mxfp8.py) against a library
routine (torch's float8_e4m3fn conversion) and closed forms of the OCP MX
definition."""
import os
import types

import numpy as np
import pytest
import torch

import oracle

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "mxfp8.py")


def _torch_e4m3(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch_within_range(m=oracle):
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.normal(0, 60, 200000), rng.normal(0, 0.01, 20000), rng.uniform(-448, 448, 20000),
                        # ties between neighbours, the subnormal range, the top of the range
                        (np.arange(-4000, 4000) + 0.5) * 2.0 ** -10, np.arange(0, 64) * 2.0 ** -12,
                        np.array([0.0, -0.0, 448.0, -448.0, 447.99, 432.0, 440.0, 2.0 ** -6, 2.0 ** -9])])
    v = v[np.abs(v) <= 448]
    assert np.array_equal(m.e4m3_encode(v), _torch_e4m3(v))


def test_e4m3_saturates_and_never_makes_nan(m=oracle):
    c = m.e4m3_encode(np.array([449.0, 464.0, 480.0, 1e6, -1e6]))
    assert list(c) == [0x7E, 0x7E, 0x7E, 0x7E, 0xFE]


def test_e4m3_decode_matches_torch_for_every_code(m=oracle):
    codes = np.arange(256, dtype=np.uint8)
    got = m.e4m3_decode(codes)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan) and list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(got[~nan], want[~nan])


@pytest.mark.parametrize("amax,e", [(1.0, -8), (1.5, -8), (1.75, -8), (2.0 ** -20, -28), (3.0 * 2.0 ** 7, 0), (3.0 * 2.0 ** 6, -1),
                                    (448.0, 0), (0.0, -127)])
def test_block_scale_closed_form(amax, e, m=oracle):
    w = np.zeros((1, 32))
    w[0, 5] = -amax
    w[0, 6] = amax / 3
    codes, scales = m.quantize_mxfp8(w)
    assert scales.shape == (1, 1) and int(scales[0, 0]) == e + 127
    if amax > 0:
        # the largest element becomes 2^(floor(log2 amax) - e) * mantissa, i.e. amax / 2^e exactly
        assert m.e4m3_decode(codes[0, 5]) * 2.0 ** e == -amax


def test_block_above_1p75_saturates_per_the_definition(m=oracle):
    w = np.full((1, 32), 0.1)
    w[0, 0] = 1.9                      # mantissa 1.9 > 1.75: 1.9 * 2^8 is beyond 448
    codes, scales = m.quantize_mxfp8(w)
    assert int(scales[0, 0]) == 127 - 8 and codes[0, 0] == 0x7E
    assert m.dequantize_mxfp8(codes, scales)[0, 0] == 1.75


def test_roundtrip_of_representable_weights_is_exact(m=oracle):
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 0x7E, size=(8, 128), dtype=np.uint8)        # finite positive codes
    codes[:, ::32] = 0x77                                               # 1.875 * 2^0 ... keep amax mantissa <= 1.75:
    codes[:, ::32] = 0x76                                               # 1.75 * 2^0, the largest of each block
    codes = np.where(m.e4m3_decode(codes) > 1.75, 0x76, codes).astype(np.uint8)
    sgn = rng.integers(0, 2, size=codes.shape).astype(np.uint8) << 7
    codes = codes | sgn
    e = rng.integers(-20, 4, size=(8, 4))
    w = m.e4m3_decode(codes).reshape(8, 4, 32) * np.exp2(e)[..., None]
    q, s = m.quantize_mxfp8(w.reshape(8, 128))
    assert np.array_equal(m.dequantize_mxfp8(q, s), w.reshape(8, 128))


def test_quantisation_error_bound(m=oracle):
    """Within a block whose amax mantissa is <= 1.75 every element is within half a
    step of the block's grid: |w - dq| <= 2^(e+floor(log2|w|)-3) / 2, and at most
    2^(e-9)/2 in the subnormal range."""
    rng = np.random.default_rng(2)
    w = rng.normal(0, 0.02, (256, 256))
    q, s = m.quantize_mxfp8(w)
    dq = m.dequantize_mxfp8(q, s)
    e = np.repeat(s.astype(np.float64) - 127, 32, axis=1)
    a = np.abs(w) / np.exp2(e)
    ok_block = np.repeat(np.max(a.reshape(256, 8, 32), axis=-1) <= 448, 32, axis=1)
    with np.errstate(divide="ignore"):
        step = np.exp2(np.maximum(np.floor(np.log2(np.where(a > 0, a, 1))), -6) - 3)
    assert np.all(np.abs(w - dq)[ok_block] <= 0.5 * step[ok_block] * np.exp2(e[ok_block]) * (1 + 1e-12))


MUTANTS = {
    "scale_exponent_minus_7": ("- E4M3_EMAX, -127.0)", "- (E4M3_EMAX - 1), -127.0)"),
    "scale_exponent_ceil": ("np.floor(np.log2(np.where(amax > 0", "np.ceil(np.log2(np.where(amax > 0"),
    "zero_block_scale_0": ("- E4M3_EMAX, -127.0)", "- E4M3_EMAX, 0.0)"),
    "encode_truncates": ("q = np.rint(a / step) * step", "q = np.trunc(a / step) * step"),
    "encode_half_up": ("q = np.rint(a / step) * step", "q = np.floor(a / step + 0.5) * step"),
    "no_saturation": [("a = np.minimum(np.abs(v), E4M3_MAX)", "a = np.abs(v)"),
                      ("q = np.minimum(q, E4M3_MAX)", "q = q")],
    "sign_dropped": ("sign = (np.signbit(v)).astype(np.int64) << 7", "sign = 0 * (np.signbit(v)).astype(np.int64)"),
    "decode_bias_8": ("np.exp2(e.astype(np.float64) - 7)", "np.exp2(e.astype(np.float64) - 8)"),
    "decode_subnormal_as_normal": ("np.where(e == 0, m * 2.0 ** (E4M3_EMIN - E4M3_MBITS),",
                                   "np.where(e == 0, (1.0 + m / 8.0) * 2.0 ** E4M3_EMIN,"),
    "dequant_scale_bias_128": ("scales.astype(np.float64) - 127.0", "scales.astype(np.float64) - 128.0"),
}

PINS = [test_e4m3_encode_matches_torch_within_range, test_e4m3_saturates_and_never_makes_nan,
        test_e4m3_decode_matches_torch_for_every_code, test_block_above_1p75_saturates_per_the_definition,
        test_roundtrip_of_representable_weights_is_exact, test_quantisation_error_bound] + \
    [(lambda a, e: (lambda m: test_block_scale_closed_form(a, e, m)))(a, e)
     for a, e in [(1.0, -8), (1.5, -8), (1.75, -8), (2.0 ** -20, -28), (3.0 * 2.0 ** 7, 0), (3.0 * 2.0 ** 6, -1),
                  (448.0, 0), (0.0, -127)]]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_every_quantiser_mutant_fails_a_pin(name):
    edits = MUTANTS[name]
    src = open(SRC, encoding="utf-8").read()
    for old, new in (edits if isinstance(edits, list) else [edits]):
        assert src.count(old) == 1, f"mutant {name}: snippet not found once in the oracle source"
        src = src.replace(old, new)
    mod = types.ModuleType(f"mxfp8_mutant_{name}")
    exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)
    failed = 0
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(m=mod)
        except Exception:
            failed += 1
    assert failed > 0, f"mutant {name} passes every pin"
