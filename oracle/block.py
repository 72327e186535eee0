"""The layer's neighbours on either side, for the oracle (numpy, float64):
the pre-norm RMSNorm, the block's residual add, and the bias update of the
auxiliary-loss-free load balancing.

TEST INFRASTRUCTURE ONLY, like the rest of this package.

Sources:
  [QA] "Nemotron 3 Ultra 架构 QA" (cctoctofx.netlify.app):
       CH2 Q2.8 -- the RMSNorm: the input is upcast to fp32, the mean of squares
       is taken over the hidden dimension, the row is multiplied by
       rsqrt(mean + eps) with eps = 1e-5, the result is cast back to the input
       dtype (bf16) and then multiplied by the learned weight gamma (bf16, so
       the product is rounded to bf16 once more);
       CH2 Q2.1 point 3 -- every mixer sits inside Pre-Norm + Residual;
       CH5 Q5.3 -- the correction bias (fp32, kept out of the gradient) is
       moved against the load: b_i <- b_i - eta * (load_i - mean load).
  [P1] the hybrid Mamba/MoE walkthrough (2kiu.com/news/4188757), its block
       sketch: residual = x; x = norm(x); x = residual + MoE(x).

Readings (listed in the design notes):
  * the norm's arithmetic is "at least fp32" on the page; here the mean of
    squares, the scale and x * scale are float64, so the two bf16 roundings
    (after the scale, after gamma) act on a unique value. The kernel does the
    same; torch's fp32 execution of the page's code can differ on rare elements
    by one bf16 step;
  * the residual add is bf16 + bf16 rounded once to bf16 (the mixer output is
    the layer's bf16 output);
  * the load of expert i is the number of (token, slot) pairs routed to it in
    the batch, the mean load is T*K/E, and the update is evaluated in float64
    (b - eta * (load - T*K/E)) and rounded once to the fp32 bias.
"""
from __future__ import annotations

from typing import Callable, Dict, Optional, Tuple

import numpy as np

from .moe_oracle import bf16_bits_to_f64, forward, round_bf16

__all__ = ["RMS_EPS", "rmsnorm", "f64_to_bf16_bits", "block_forward", "bias_update"]

RMS_EPS = 1e-5


def f64_to_bf16_bits(v) -> np.ndarray:
    """bf16 bit patterns of float64 values that are bf16 values (exact)."""
    v = np.asarray(v, dtype=np.float64)
    assert np.array_equal(round_bf16(v), v, equal_nan=True), "not bf16 values"
    return (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def rmsnorm(x_bits, gamma_bits, eps: float = RMS_EPS, mirror: bool = True) -> np.ndarray:
    """QA Q2.8: y = gamma * bf16( x * rsqrt(mean(x^2) + eps) ), one row per token.

    x_bits [T, H] and gamma_bits [H] are bf16 bit patterns. Returns float64
    values (bf16 values when mirror; with mirror=False nothing is rounded)."""
    x = bf16_bits_to_f64(x_bits)
    g = bf16_bits_to_f64(gamma_bits)
    var = np.mean(x * x, axis=-1, keepdims=True)
    t = x * (1.0 / np.sqrt(var + eps))
    if mirror:
        t = round_bf16(t)
    y = g * t
    return round_bf16(y) if mirror else y


def block_forward(x_bits, gamma_bits, eps, w_router, corr_bias, w_fc1_bits, w_fc2_bits, w_sh_up_bits,
                  w_sh_down_bits, expert: Callable[[int], Tuple[np.ndarray, np.ndarray]], K: int,
                  routed_scaling: float, idx_override: Optional[np.ndarray] = None, keep: bool = False,
                  n_group: int = 1, topk_group: int = 1) -> Dict[str, np.ndarray]:
    """The MoE block: out = x + LatentMoE(RMSNorm(x)) (QA Q2.1, Q2.8; P1's block).

    Returns the forward's results for the normed input plus ``xn`` (the normed
    rows), ``mixer`` (the layer output on them) and ``out`` (after the residual
    add), all bf16 values."""
    xn = rmsnorm(x_bits, gamma_bits, eps)
    res = forward(f64_to_bf16_bits(xn), w_router, corr_bias, w_fc1_bits, w_fc2_bits, w_sh_up_bits,
                  w_sh_down_bits, expert, K, routed_scaling, mirror=True, idx_override=idx_override, keep=keep,
                  n_group=n_group, topk_group=topk_group)
    mixer = res["out"]
    res["xn"] = xn
    res["mixer"] = mixer
    res["out"] = round_bf16(bf16_bits_to_f64(x_bits) + mixer)
    return res


def bias_update(bias, counts, eta: float, n_slots: int) -> np.ndarray:
    """QA Q5.3: b_i <- b_i - eta * (load_i - mean load), load_i = counts[i]
    (slots routed to expert i), mean load = n_slots / E with n_slots = T*K.
    Returns the new fp32 bias."""
    b = np.asarray(bias, dtype=np.float32).astype(np.float64)
    load = np.asarray(counts).astype(np.float64)
    E = b.shape[0]
    avg = float(n_slots) / float(E)
    return (b - float(eta) * (load - avg)).astype(np.float32)
