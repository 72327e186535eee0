"""Algorithmic work of one LatentMoE forward: FLOPs and compulsory HBM bytes.

The FLOP split follows the per-token breakdown of the "Nemotron 3 Ultra 架构 QA"
page, Q3.1 (router, latent projections, the K active experts, the shared
expert); a multiply-add counts two FLOPs. Bytes count each weight that the
forward must read once (the router weight, fc1, fc2, the shared expert and every
expert that received at least one token), x read once and out written once.
"""
from __future__ import annotations

from typing import Dict, Optional

__all__ = ["flops", "total_flops", "weight_bytes", "compulsory_bytes", "param_counts"]


def flops(T: int, H: int, L: int, E: int, I: int, K: int, Is: int) -> Dict[str, int]:
    return dict(
        router=2 * T * H * E,            # x . W_r^T
        latent=4 * T * H * L,            # fc1 (H->L) and fc2 (L->H)
        experts=4 * T * K * L * I,       # K x (up L->I, down I->L)
        shared=4 * T * H * Is,           # shared up H->Is and down Is->H
    )


def total_flops(T, H, L, E, I, K, Is) -> int:
    return sum(flops(T, H, L, E, I, K, Is).values())


def param_counts(H: int, L: int, E: int, I: int, Is: int) -> Dict[str, int]:
    return dict(router=E * H, latent=2 * H * L, experts=2 * E * I * L, shared=2 * H * Is)


def weight_bytes(H, L, E, I, Is, n_touched: Optional[int] = None) -> Dict[str, int]:
    """Bytes of weights read once: fp32 router weight and bias, bf16 everything else."""
    n = E if n_touched is None else n_touched
    return dict(router=4 * E * H + 4 * E, latent=2 * 2 * H * L, experts=n * 2 * 2 * I * L,
                shared=2 * 2 * H * Is)


def compulsory_bytes(T, H, L, E, I, K, Is, n_touched: Optional[int] = None) -> int:
    """Weights touched (read once) plus x in and out written, all bf16 except the router."""
    return sum(weight_bytes(H, L, E, I, Is, n_touched).values()) + 2 * T * H * 2
