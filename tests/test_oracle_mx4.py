"""Pins of the oracle's MXFP4 quantiser (oracle/mxfp4.py): the E2M1 value table
of the OCP MX definition written out by hand, encoding against a brute-force
nearest-value search, the block scale's closed form, exact round trips, and
planted mistakes that must each fail a pin."""
import os
import types

import numpy as np
import pytest

import oracle
import oracle.mxfp4 as OX

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "mxfp4.py")

# E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0 is the subnormal 0.5 * m
TABLE = {0: 0.0, 1: 0.5, 2: 1.0, 3: 1.5, 4: 2.0, 5: 3.0, 6: 4.0, 7: 6.0}


def pin_decode_table(m=OX):
    got = m.e2m1_decode(np.arange(16))
    want = [TABLE[c] for c in range(8)] + [-TABLE[c] for c in range(8)]
    assert np.array_equal(got, want) and np.signbit(got[8])


def _brute_encode(v):
    """Nearest E2M1 value by search; ties to the code whose mantissa bit is 0."""
    out = []
    for x in np.ravel(v):
        a = min(abs(x), 6.0)
        best = None
        for c in range(8):
            d = abs(TABLE[c] - a)
            if best is None or d < best[0] - 1e-300 or (d == best[0] and (c & 1) == 0):
                best = (d, c)
        out.append(best[1] | (8 if np.signbit(x) else 0))
    return np.array(out, dtype=np.uint8).reshape(np.shape(v))


def pin_encode_matches_brute_force(m=OX):
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.uniform(-7, 7, 4000), np.arange(-28, 29) * 0.25,     # every tie of the grid
                        np.array([0.0, -0.0, 6.0, -6.0, 6.5, 100.0, -1e9, 0.2499, 0.2501, 5.0, 4.99, 5.01])])
    assert np.array_equal(m.e2m1_encode(v), _brute_encode(v))


def pin_block_scale_closed_form(m=OX):
    for amax, e in [(1.0, -2), (1.5, -2), (6.0, 0), (7.9, 0), (8.0, 1), (2.0 ** -30, -32), (0.0, -127),
                    (2.0 ** -126, -127), (3.0 * 2.0 ** 100, 99)]:
        w = np.zeros((1, 32))
        w[0, 3] = -amax
        w[0, 9] = amax / 5
        packed, scales = m.quantize_mxfp4(w)
        assert packed.shape == (1, 16) and scales.shape == (1, 1)
        assert int(scales[0, 0]) == e + 127, (amax, e, scales)


def pin_packing_order(m=OX):
    """Element 2i goes to the low nibble of byte i."""
    w = np.zeros((1, 32))
    w[0, 0], w[0, 1] = 4.0, -1.0            # amax 4 -> e = 0: codes 6 and 8|2
    packed, scales = m.quantize_mxfp4(w)
    assert int(scales[0, 0]) == 127 and int(packed[0, 0]) == (6 | (10 << 4))


def pin_roundtrip_of_representable_blocks(m=OX):
    rng = np.random.default_rng(1)
    vals = rng.choice([-6, -4, -3, -2, -1.5, -1, -0.5, 0, 0.5, 1, 1.5, 2, 3, 4, 6], size=(6, 4, 32))
    vals[:, :, 0] = 6.0                    # every block holds its largest magnitude 6 = 1.5 * 2^2
    e = rng.integers(-30, 10, size=(6, 4))
    w = (vals * np.exp2(e)[..., None]).reshape(6, 128)
    packed, scales = m.quantize_mxfp4(w)
    assert np.array_equal(m.dequantize_mxfp4(packed, scales), w)


def pin_error_bound(m=OX):
    """Within a block every element is within half a grid step of its value
    (steps 0.5 / 1 / 2 times the block scale), or saturated."""
    rng = np.random.default_rng(2)
    w = rng.normal(0, 0.02, (64, 256))
    packed, scales = m.quantize_mxfp4(w)
    dq = m.dequantize_mxfp4(packed, scales)
    X = np.repeat(np.exp2(scales.astype(np.float64) - 127), 32, axis=1)
    a = np.abs(w) / X
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0)) * X
    ok = a <= 6
    assert np.all(np.abs(w - dq)[ok] <= 0.5 * step[ok] * (1 + 1e-12))


PINS = [pin_decode_table, pin_encode_matches_brute_force, pin_block_scale_closed_form, pin_packing_order,
        pin_roundtrip_of_representable_blocks, pin_error_bound]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


MUTANTS = {
    "scale_exponent_minus_1": ("- E2M1_EMAX, -127.0)", "- (E2M1_EMAX - 1), -127.0)"),
    "scale_exponent_ceil": ("np.floor(np.log2(np.where(amax > 0", "np.ceil(np.log2(np.where(amax > 0"),
    "encode_truncates": ("q = np.rint(a / step) * step", "q = np.floor(a / step) * step"),
    "encode_half_up": ("q = np.rint(a / step) * step", "q = np.floor(a / step + 0.5) * step"),
    "subnormal_as_normal": ("np.where(e == 0, 0.5 * m,", "np.where(e == 0, 1.0 + 0.5 * m,"),
    "exponent_bias_2": ("np.exp2(e - 1.0))", "np.exp2(e - 2.0))"),
    "nibbles_swapped": ("(codes[..., 0::2] | (codes[..., 1::2] << 4))", "(codes[..., 1::2] | (codes[..., 0::2] << 4))"),
    "sign_dropped": ("sign = np.signbit(v).astype(np.int64) << 3", "sign = 0 * np.signbit(v).astype(np.int64)"),
    "dequant_scale_bias_128": ("scales.astype(np.float64) - 127.0", "scales.astype(np.float64) - 128.0"),
    "step_boundary_off": ("step = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))",
                          "step = np.where(a < 2.0, 0.5, np.where(a < 3.0, 1.0, 2.0))"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_every_mxfp4_mutant_fails_a_pin(name):
    old, new = MUTANTS[name]
    src = open(SRC, encoding="utf-8").read()
    assert src.count(old) == 1, f"mutant {name}: snippet not found once in the oracle source"
    mod = types.ModuleType(f"mxfp4_mutant_{name}")
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    failed = 0
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except Exception:
            failed += 1
    assert failed > 0, f"mutant {name} passes every pin"
