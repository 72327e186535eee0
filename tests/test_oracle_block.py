"""Pins of the oracle's block neighbours (oracle/block.py): the RMSNorm against
torch's own rms_norm and hand-derived closed forms, the block's residual and
norm structure through properties that hold exactly, and the bias update
against hand-computed cases and its invariants. Each planted mistake must fail
one of them."""
import os
import types

import numpy as np
import pytest
import torch

import oracle
import oracle.block as OB

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "block.py")


def _bits(v):
    return oracle.f64_to_bf16_bits(oracle.round_bf16(np.asarray(v, np.float64)))


def _rand_bits(shape, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return _bits(rng.normal(0, scale, shape))


# ----------------------------------------------------------------------------
# RMSNorm
# ----------------------------------------------------------------------------

def pin_rmsnorm_matches_torch_unrounded(m=OB):
    """Without the bf16 roundings the norm is torch.nn.functional.rms_norm in float64."""
    x = _rand_bits((16, 512), 0, 3.0)
    g = _rand_bits((512,), 1, 1.0)
    for eps in (1e-5, 0.0, 0.5):
        got = m.rmsnorm(x, g, eps, mirror=False)
        want = torch.nn.functional.rms_norm(torch.from_numpy(oracle.bf16_bits_to_f64(x)), (512,),
                                            torch.from_numpy(oracle.bf16_bits_to_f64(g)), eps).numpy()
        np.testing.assert_allclose(got, want, rtol=1e-13, atol=0)


def pin_rmsnorm_two_roundings_closed_form(m=OB):
    """x = [1, 1, 5], eps = 0: mean(x^2) = 9, so the scale is exactly 1/3 and the
    normed row is [1/3, 1/3, 5/3] before rounding. bf16(1/3) = 171/512 (the bits
    after the eighth significant one are 1010..., so it rounds up) and
    bf16(5/3) = 213/128 (rounds down). With gamma = 65/256:
    gamma * 171/512 = 11115/131072 = 173.67 * 2^-11 -> 174 * 2^-11 = 0.0849609375
    gamma * 213/128 = 13845/32768 = 216.33 * 2^-9 -> 216 * 2^-9 = 0.421875.
    Rounding gamma * (1/3) once instead would give 0.08447265625: the two
    roundings of the page's code (cast to bf16, then the bf16 product) matter."""
    x = _bits([[1.0, 1.0, 5.0]])
    g = _bits([65 / 256] * 3)
    y = m.rmsnorm(x, g, 0.0)
    assert y.tolist() == [[0.0849609375, 0.0849609375, 0.421875]]


def pin_rmsnorm_constant_row(m=OB):
    """A row of equal values c: mean = c^2, y = gamma * bf16(c / sqrt(c^2 + eps)).
    With eps = 0 the normed row is exactly sign(c); with eps = 1e-5 and |c| = 1
    it is 1/sqrt(1.00001) = 0.999995..., which rounds to 1 in bf16."""
    g = _bits(np.linspace(-2, 2, 64))
    for c in (1.0, -3.0, 0.0078125):
        x = _bits(np.full((1, 64), c))
        assert np.array_equal(m.rmsnorm(x, g, 0.0), oracle.bf16_bits_to_f64(g)[None] * np.sign(c))
    assert np.array_equal(m.rmsnorm(_bits(np.ones((1, 64))), g, 1e-5), oracle.bf16_bits_to_f64(g)[None])


def pin_rmsnorm_scale_invariance(m=OB):
    """With eps = 0, scaling a row by a power of two leaves the output unchanged."""
    x = _rand_bits((8, 256), 3)
    g = _rand_bits((256,), 4)
    y = m.rmsnorm(x, g, 0.0)
    for k in (-3, 1, 5):
        assert np.array_equal(m.rmsnorm(_bits(oracle.bf16_bits_to_f64(x) * 2.0 ** k), g, 0.0), y)


def pin_rmsnorm_unit_rms(m=OB):
    """gamma = 1, eps = 0, no rounding: every output row has mean square 1."""
    x = _rand_bits((8, 300), 5, 7.0)
    y = m.rmsnorm(x, _bits(np.ones(300)), 0.0, mirror=False)
    np.testing.assert_allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-13)


# ----------------------------------------------------------------------------
# block: out = x + mixer(rmsnorm(x))
# ----------------------------------------------------------------------------

def _tiny_block_inputs(seed=0, T=12, H=64, L=32, E=8, I=64, Is=64):
    rng = np.random.default_rng(seed)
    w = dict(w_router=rng.normal(0, 1 / np.sqrt(H), (E, H)).astype(np.float32),
             corr_bias=rng.uniform(-0.05, 0.05, E).astype(np.float32),
             w_fc1=_bits(rng.normal(0, 1 / np.sqrt(H), (L, H))), w_fc2=_bits(rng.normal(0, 1 / np.sqrt(L), (H, L))),
             w_sh_up=_bits(rng.normal(0, 1 / np.sqrt(H), (Is, H))),
             w_sh_down=_bits(rng.normal(0, 1 / np.sqrt(Is), (H, Is))))
    ups = [_bits(rng.normal(0, 1 / np.sqrt(L), (I, L))) for _ in range(E)]
    downs = [_bits(rng.normal(0, 1 / np.sqrt(I), (L, I))) for _ in range(E)]
    x = _bits(rng.normal(0, 2.0, (T, H)))
    return x, w, (lambda e: (ups[e], downs[e]))


def _block(m, x, gamma, eps, w, expert, K=3, keep=False):
    return m.block_forward(x, gamma, eps, w["w_router"], w["corr_bias"], w["w_fc1"], w["w_fc2"], w["w_sh_up"],
                           w["w_sh_down"], expert, K, 5.0, keep=keep)


def pin_block_zero_gamma_is_identity(m=OB):
    """gamma = 0 zeroes the normed rows; the layer maps zero rows to zero (no
    biases, relu^2(0) = 0), so the block returns x bit for bit."""
    x, w, expert = _tiny_block_inputs()
    r = _block(m, x, _bits(np.zeros(x.shape[1])), 1e-5, w, expert)
    assert np.array_equal(r["out"], oracle.bf16_bits_to_f64(x))
    assert not np.any(r["mixer"])


def pin_block_norm_makes_mixer_scale_free(m=OB):
    """With eps = 0 the mixer sees the same normed rows for x and 2^k x, so its
    output is identical; the block output is then bf16(2^k x + that output)."""
    x, w, expert = _tiny_block_inputs(1)
    g = _rand_bits((x.shape[1],), 9)
    a = _block(m, x, g, 0.0, w, expert)
    x4 = _bits(oracle.bf16_bits_to_f64(x) * 4.0)
    b = _block(m, x4, g, 0.0, w, expert)
    assert np.array_equal(a["mixer"], b["mixer"]) and np.any(a["mixer"])
    assert np.array_equal(b["out"], oracle.round_bf16(oracle.bf16_bits_to_f64(x4) + a["mixer"]))


def pin_block_output_is_residual_plus_mixer_on_the_bf16_grid(m=OB):
    """out - x is the mixer output up to one bf16 rounding of the sum, and the
    mixer output equals the layer's forward on the normed rows."""
    x, w, expert = _tiny_block_inputs(2)
    g = _rand_bits((x.shape[1],), 10)
    r = _block(m, x, g, 1e-5, w, expert)
    xs = oracle.bf16_bits_to_f64(x)
    assert np.array_equal(oracle.round_bf16(r["out"]), r["out"])
    # one rounding of (x + mixer): within half a bf16 step of the exact sum
    s = xs + r["mixer"]
    step = np.ldexp(1.0, np.frexp(np.abs(s))[1] - 8)
    assert np.all(np.abs(r["out"] - s) <= 0.5 * step + 1e-300)
    f = oracle.forward(oracle.f64_to_bf16_bits(r["xn"]), w["w_router"], w["corr_bias"], w["w_fc1"], w["w_fc2"],
                       w["w_sh_up"], w["w_sh_down"], expert, 3, 5.0)
    assert np.array_equal(f["out"], r["mixer"])


# ----------------------------------------------------------------------------
# bias update
# ----------------------------------------------------------------------------

def pin_bias_update_hand_case(m=OB):
    """E = 4, T*K = 4 (mean load 1), counts [3, 1, 0, 0], eta = 0.5, b = 0:
    b - 0.5 * ([3, 1, 0, 0] - 1) = [-1, 0, 0.5, 0.5]."""
    got = m.bias_update(np.zeros(4, np.float32), [3, 1, 0, 0], 0.5, 4)
    assert got.dtype == np.float32 and got.tolist() == [-1.0, 0.0, 0.5, 0.5]


def pin_bias_update_balanced_load_is_a_fixed_point(m=OB):
    b = np.random.default_rng(0).uniform(-0.1, 0.1, 64).astype(np.float32)
    assert np.array_equal(m.bias_update(b, np.full(64, 22), 1e-3, 64 * 22), b)


def pin_bias_update_moves_against_the_load(m=OB):
    """Overloaded experts go down, underloaded up, by eta times their excess;
    the excesses sum to zero."""
    rng = np.random.default_rng(1)
    E, T, K = 128, 500, 8
    counts = np.bincount(rng.choice(E, size=T * K, p=rng.dirichlet(np.ones(E))), minlength=E)
    b = rng.uniform(-0.05, 0.05, E).astype(np.float32)
    eta = np.float32(1e-3)
    new = m.bias_update(b, counts, eta, T * K)
    d = new.astype(np.float64) - b
    avg = T * K / E
    assert np.all(np.sign(d[counts > avg]) < 0) and np.all(np.sign(d[counts < avg]) > 0)
    np.testing.assert_allclose(d, -float(eta) * (counts - avg), atol=2e-8)
    assert abs(d.sum()) < 1e-6


PINS = [pin_rmsnorm_matches_torch_unrounded, pin_rmsnorm_two_roundings_closed_form, pin_rmsnorm_constant_row,
        pin_rmsnorm_scale_invariance, pin_rmsnorm_unit_rms, pin_block_zero_gamma_is_identity,
        pin_block_norm_makes_mixer_scale_free, pin_block_output_is_residual_plus_mixer_on_the_bf16_grid,
        pin_bias_update_hand_case, pin_bias_update_balanced_load_is_a_fixed_point,
        pin_bias_update_moves_against_the_load]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


MUTANTS = {
    "eps_outside_sqrt": ("1.0 / np.sqrt(var + eps)", "1.0 / (np.sqrt(var) + eps)"),
    "sum_not_mean": ("np.mean(x * x, axis=-1, keepdims=True)", "np.sum(x * x, axis=-1, keepdims=True)"),
    "gamma_dropped": ("y = g * t", "y = t"),
    "one_rounding": ("    if mirror:\n        t = round_bf16(t)\n", ""),
    "no_final_rounding": ("return round_bf16(y) if mirror else y", "return y"),
    "norm_skipped": ("xn = rmsnorm(x_bits, gamma_bits, eps)", "xn = bf16_bits_to_f64(x_bits) + 0 * rmsnorm(x_bits, gamma_bits, eps)"),
    "residual_dropped": ('res["out"] = round_bf16(bf16_bits_to_f64(x_bits) + mixer)', 'res["out"] = mixer'),
    "residual_unrounded": ('res["out"] = round_bf16(bf16_bits_to_f64(x_bits) + mixer)',
                           'res["out"] = bf16_bits_to_f64(x_bits) + mixer'),
    "bias_sign_flipped": ("(b - float(eta) * (load - avg))", "(b + float(eta) * (load - avg))"),
    "mean_over_tokens_not_slots": ("avg = float(n_slots) / float(E)", "avg = float(n_slots) / float(E) / 2"),
    "mean_over_loaded_experts": ("avg = float(n_slots) / float(E)",
                                 "avg = float(n_slots) / float(max(1, np.count_nonzero(load)))"),
    "bias_unscaled": ("(b - float(eta) * (load - avg))", "(b - (load - avg))"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_every_block_mutant_fails_a_pin(name):
    old, new = MUTANTS[name]
    src = open(SRC, encoding="utf-8").read()
    assert src.count(old) == 1, f"mutant {name}: snippet not found once in the oracle source"
    src = src.replace(old, new).replace("from .moe_oracle import", "from oracle.moe_oracle import")
    mod = types.ModuleType(f"block_mutant_{name}")
    exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)
    failed = 0
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mod)
        except Exception:
            failed += 1
    assert failed > 0, f"mutant {name} passes every pin"
