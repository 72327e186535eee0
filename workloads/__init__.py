"""Seeded synthetic inputs for the LatentMoE layer forward.

This module only makes inputs. It holds none of the layer's arithmetic, and both
the CPU oracle side (tests, bench's CPU baseline) and the GPU side take their
inputs from here.

Every tensor is drawn from a counter-based generator written with integer torch
ops, so the same (seed, tag, element index) gives the same bits on the CPU and
on the GPU, and any slice (one expert's weights, one token's row) can be
regenerated on its own:

* a 32-bit key per (seed, tensor tag, high half of the element index);
* two rounds of the "lowbias32" integer hash published by C. Wellons
  (hash-prospector): ``x ^= x>>16; x *= 0x7feb352d; x ^= x>>15;
  x *= 0x846ca68b; x ^= x>>16`` (all mod 2**32);
* "normal" values are the centred sum of four 16-bit uniforms (Irwin-Hall
  with n=4, unit variance after scaling, support +-3.46 sigma), formed exactly
  as an integer, converted exactly to float32 and scaled by one float32
  multiply, which IEEE rounds identically on every device;
* bf16 values come from that float32 by round-to-nearest-even on the bit
  pattern, in integer ops.

Shapes and value distributions follow the workloads the layer is stated on:
x ~ N(0,1) in bf16, weights ~ N(0, 1/fan_in) in bf16, the router weight in
fp32, and the correction bias uniform (the sizes are those of the Nemotron-3
family as given on the "Nemotron 3 Ultra 架构 QA" page, Q1.1 and CH5, and the
2kiu.com architecture walkthrough, section "LatentMoE 层").
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Dict, Optional

import numpy as np
import torch

__all__ = [
    "MoEConfig", "CONFIGS", "get_config", "gen_normal_bf16", "gen_normal_f32",
    "gen_uniform_f32", "make_inputs", "make_x", "make_weights", "expert_weights", "zipf_offsets",
    "f32_to_bf16_bits", "bf16_tensor_to_u16_numpy",
]

_M32 = 0xFFFFFFFF


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int
    H: int
    L: int
    E: int
    I: int
    K: int
    Is: int
    routed_scaling: float = 5.0
    bias_halfwidth: float = 0.0       # correction bias ~ U(-w, w); 0 -> all zeros
    skew: Optional[str] = None        # None or "zipf1.1"
    seed: int = 0
    weight_key: str = ""              # configs sharing weights share this key
    x_tag: int = 0                    # distinguishes x streams that share weights

    @property
    def TK(self) -> int:
        return self.T * self.K

    def dims(self):
        return dict(T=self.T, H=self.H, L=self.L, E=self.E, I=self.I, K=self.K,
                    Is=self.Is, routed_scaling=self.routed_scaling)


CONFIGS: Dict[str, MoEConfig] = {
    # Tiny LatentMoE, small enough for the oracle in seconds and for brute force.
    "tiny": MoEConfig("tiny", T=64, H=256, L=64, E=16, I=128, K=4, Is=256,
                      bias_halfwidth=0.1, seed=0, weight_key="tiny"),
    # Nano-width: 128 experts, top-8, uniform routing (zero bias).
    "nano": MoEConfig("nano", T=4096, H=4096, L=2048, E=128, I=5120, K=8, Is=8192,
                      bias_halfwidth=0.0, seed=1, weight_key="nano"),
    # Super-width: 128 experts, top-8, router logits offset by a Zipf(1.1) law.
    "super": MoEConfig("super", T=8192, H=6144, L=2048, E=128, I=5120, K=8, Is=10240,
                       bias_halfwidth=0.0, skew="zipf1.1", seed=2, weight_key="super"),
    # Ultra shape, 16K-token prefill.
    "ultra_prefill": MoEConfig("ultra_prefill", T=16384, H=8192, L=2048, E=512, I=5120,
                               K=22, Is=10240, bias_halfwidth=0.05, seed=3,
                               weight_key="ultra", x_tag=0),
    # Ultra shape decode: the same layer weights, another x stream.
    "ultra_decode64": MoEConfig("ultra_decode64", T=64, H=8192, L=2048, E=512, I=5120,
                                K=22, Is=10240, bias_halfwidth=0.05, seed=3,
                                weight_key="ultra", x_tag=1),
    "ultra_decode1": MoEConfig("ultra_decode1", T=1, H=8192, L=2048, E=512, I=5120,
                               K=22, Is=10240, bias_halfwidth=0.05, seed=3,
                               weight_key="ultra", x_tag=2),
}


def get_config(name: str, **overrides) -> MoEConfig:
    cfg = CONFIGS[name]
    return replace(cfg, **overrides) if overrides else cfg


# ----------------------------------------------------------------------------
# counter-based generator (integer torch ops, identical on every device)
# ----------------------------------------------------------------------------

def _mul32(x: torch.Tensor, c: int) -> torch.Tensor:
    """(x * c) mod 2**32 for int64 x in [0, 2**32), without int64 overflow."""
    lo = x & 0xFFFF
    hi = x >> 16
    return (lo * c + (((hi * c) & 0xFFFF) << 16)) & _M32


def _lowbias32(x: torch.Tensor) -> torch.Tensor:
    x = x ^ (x >> 16)
    x = _mul32(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


def _lowbias32_int(x: int) -> int:
    x &= _M32
    x ^= x >> 16
    x = (x * 0x7FEB352D) & _M32
    x ^= x >> 15
    x = (x * 0x846CA68B) & _M32
    x ^= x >> 16
    return x


def _stream_key(seed: int, tag: int) -> int:
    return _lowbias32_int(_lowbias32_int(seed * 0x9E3779B9 + 0x632BE5AB) ^ (tag * 0x85EBCA6B))


_CHUNK = 1 << 25


def _hash_pair(key: int, start: int, n: int, device) -> tuple:
    """Two independent 32-bit words for element indices [start, start+n)."""
    i = torch.arange(start, start + n, dtype=torch.int64, device=device)
    lo = i & _M32
    hi = i >> 32
    hk = _lowbias32((hi * 0x27D4EB2F + key) & _M32)
    a = _lowbias32(lo ^ hk)
    b = _lowbias32((a + 0x9E3779B9) & _M32 ^ hk)
    return a, b


def _normal_f32_chunk(key: int, start: int, n: int, std: float, device) -> torch.Tensor:
    a, b = _hash_pair(key, start, n, device)
    s = (a & 0xFFFF) + (a >> 16) + (b & 0xFFFF) + (b >> 16)       # in [0, 4*65535]
    c = 2 * s - 4 * 65535                                          # symmetric, |c| < 2**19
    # Irwin-Hall(4): var(s) = 4 * (65536**2 - 1) / 12 ; scale c to unit variance * std
    sd_c = 2.0 * math.sqrt(4.0 * (65536.0 ** 2 - 1.0) / 12.0)
    scale = torch.tensor(np.float32(std / sd_c), dtype=torch.float32, device=device)
    return c.to(torch.float32) * scale


def f32_to_bf16_bits(v: torch.Tensor) -> torch.Tensor:
    """float32 -> bf16 bit pattern (int64 in [0, 65536)), round to nearest even."""
    bits = v.contiguous().view(torch.int32).to(torch.int64) & _M32
    lsb = (bits >> 16) & 1
    return ((bits + 0x7FFF + lsb) >> 16) & 0xFFFF


def _bits_to_bf16(bits: torch.Tensor) -> torch.Tensor:
    signed = torch.where(bits >= 0x8000, bits - 0x10000, bits).to(torch.int16)
    return signed.view(torch.bfloat16)


def _fill(shape, fn, device, out_dtype) -> torch.Tensor:
    n = int(np.prod(shape)) if len(shape) else 1
    out = torch.empty(n, dtype=out_dtype, device=device)
    for s in range(0, n, _CHUNK):
        m = min(_CHUNK, n - s)
        out[s:s + m] = fn(s, m)
    return out.view(*shape)


def gen_normal_f32(seed: int, tag: int, shape, std: float, device="cpu", offset: int = 0):
    key = _stream_key(seed, tag)
    return _fill(shape, lambda s, m: _normal_f32_chunk(key, offset + s, m, std, device),
                 device, torch.float32)


def gen_normal_bf16(seed: int, tag: int, shape, std: float, device="cpu", offset: int = 0):
    key = _stream_key(seed, tag)
    return _fill(shape, lambda s, m: _bits_to_bf16(
        f32_to_bf16_bits(_normal_f32_chunk(key, offset + s, m, std, device))),
        device, torch.bfloat16)


def gen_uniform_f32(seed: int, tag: int, shape, halfwidth: float, device="cpu"):
    """U(-w, w) on the odd multiples of w / 2**24, exact in float32 up to the scale."""
    key = _stream_key(seed, tag)

    def fn(s, m):
        a, _ = _hash_pair(key, s, m, device)
        c = 2 * (a >> 8) - (2 ** 24 - 1)
        scale = torch.tensor(np.float32(halfwidth / 2 ** 24), dtype=torch.float32, device=device)
        return c.to(torch.float32) * scale
    return _fill(shape, fn, device, torch.float32)


# tensor tags (fixed, so each tensor has its own stream)
TAG_X, TAG_WR, TAG_BIAS, TAG_FC1, TAG_UP, TAG_DOWN, TAG_FC2, TAG_SU, TAG_SD, TAG_PERM = range(10)


def zipf_offsets(E: int, seed: int, s: float = 1.1) -> np.ndarray:
    """Per-expert logit offsets delta_e = ln(E * p_e), p_e proportional to rank_e**-s.

    The ranks are a seeded permutation of 1..E. Returned as float32.
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, TAG_PERM])))
    ranks = rng.permutation(E) + 1
    p = ranks.astype(np.float64) ** (-s)
    p /= p.sum()
    return np.log(E * p).astype(np.float32)


def _wseed(cfg: MoEConfig) -> int:
    # configs that share weights share the weight seed
    return {"tiny": 100, "nano": 101, "super": 102, "ultra": 103}.get(cfg.weight_key, 1000 + cfg.seed)


def expert_weights(cfg: MoEConfig, e0: int, e1: int, device="cpu"):
    """W_up[e0:e1] ([n,I,L]) and W_down[e0:e1] ([n,L,I]) as bf16, regenerable per expert."""
    ws = _wseed(cfg)
    n = e1 - e0
    up = gen_normal_bf16(ws, TAG_UP, (n, cfg.I, cfg.L), 1.0 / math.sqrt(cfg.L), device,
                         offset=e0 * cfg.I * cfg.L)
    down = gen_normal_bf16(ws, TAG_DOWN, (n, cfg.L, cfg.I), 1.0 / math.sqrt(cfg.I), device,
                           offset=e0 * cfg.L * cfg.I)
    return up, down


def make_x(cfg: MoEConfig, device="cpu") -> torch.Tensor:
    """The input rows x [T,H] bf16. Row t does not depend on T (a longer batch
    extends a shorter one)."""
    x = gen_normal_bf16(_wseed(cfg) * 7919 + cfg.x_tag, TAG_X, (cfg.T, cfg.H), 1.0, device)
    if cfg.skew == "zipf1.1":
        x[:, 0] = 1.0      # carries the per-expert logit offsets, see make_weights
    return x


def make_weights(cfg: MoEConfig, device="cpu", with_experts: bool = True) -> Dict[str, torch.Tensor]:
    """Router weight, bias and the weight tensors of the layer."""
    ws = _wseed(cfg)
    H, L, E, I, Is = cfg.H, cfg.L, cfg.E, cfg.I, cfg.Is
    d: Dict[str, torch.Tensor] = {}
    wr = gen_normal_f32(ws, TAG_WR, (E, H), 1.0 / math.sqrt(H), device)
    if cfg.skew == "zipf1.1":
        # the offsets enter through the router product itself: x[:,0] = 1 and
        # w_router[:,0] = delta_e gives logit_e = delta_e + (the rest)
        wr[:, 0] = torch.from_numpy(zipf_offsets(E, ws)).to(device)
    if cfg.bias_halfwidth > 0:
        bias = gen_uniform_f32(ws, TAG_BIAS, (E,), cfg.bias_halfwidth, device)
    else:
        bias = torch.zeros(E, dtype=torch.float32, device=device)
    d["w_router"] = wr
    d["corr_bias"] = bias
    d["w_fc1"] = gen_normal_bf16(ws, TAG_FC1, (L, H), 1.0 / math.sqrt(H), device)
    d["w_fc2"] = gen_normal_bf16(ws, TAG_FC2, (H, L), 1.0 / math.sqrt(L), device)
    d["w_sh_up"] = gen_normal_bf16(ws, TAG_SU, (Is, H), 1.0 / math.sqrt(H), device)
    d["w_sh_down"] = gen_normal_bf16(ws, TAG_SD, (H, Is), 1.0 / math.sqrt(Is), device)
    if with_experts:
        up, down = expert_weights(cfg, 0, E, device)
        d["w_up"] = up
        d["w_down"] = down
    return d


def make_inputs(cfg: MoEConfig, device="cpu", with_experts: bool = True) -> Dict[str, torch.Tensor]:
    """All inputs of one forward: x, router weight, bias and the seven weight tensors.

    bf16 tensors are torch.bfloat16, fp32 ones torch.float32, all on ``device``.
    """
    d = make_weights(cfg, device, with_experts)
    d["x"] = make_x(cfg, device)
    return d


def bf16_tensor_to_u16_numpy(t: torch.Tensor) -> np.ndarray:
    """bf16 torch tensor (any device) -> numpy uint16 bit patterns on the host."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
