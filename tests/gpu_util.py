"""Helpers of the GPU parity tests: inputs on the device, the oracle on the host.

The inputs come from the seeded generators of ``workloads`` (generated on the
GPU; the generator gives the same bits on every device). The oracle receives
host copies of those inputs -- never anything the HIP library computed, except
that on near-tie tokens it may be told to follow the library's choice of
experts (several choices are correct there).
"""
from __future__ import annotations

import sys
import time
from typing import Dict

import numpy as np
import torch

import oracle
import workloads as W

# bar of the layer output: max |gpu - ref| / max |ref|
OUT_TOL = 2e-2
# gates: the fp32 logit of a dot product over H terms differs from the exact one
# by at most ~H * 2^-24 * sum|x w| in the worst case and ~sqrt(H) * 2^-24 * that
# typically; through the sigmoid (slope <= 1/4) and the renormalisation this
# bounds the relative gate error far below 1e-5 for the workloads here.
GATE_RTOL = 1e-5

_wcache: Dict[tuple, Dict[str, torch.Tensor]] = {}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def device_inputs(name: str, **over) -> Dict[str, torch.Tensor]:
    """All inputs of a workload on cuda:0; weights are cached per weight set (one
    large set at a time), x is generated per call."""
    cfg = W.get_config(name, **over)
    wk = (cfg.weight_key, cfg.H, cfg.L, cfg.E, cfg.I, cfg.Is, cfg.skew, cfg.bias_halfwidth)
    t0 = time.time()
    if wk not in _wcache:
        if cfg.E * cfg.I * cfg.L > 1e9:
            for k in [k for k in _wcache if k[3] * k[4] * k[2] > 1e9]:
                del _wcache[k]
            torch.cuda.empty_cache()
        _wcache[wk] = W.make_weights(cfg, device="cuda")
    d = dict(_wcache[wk])
    d["x"] = W.make_x(cfg, device="cuda")
    d["cfg"] = cfg
    torch.cuda.synchronize()
    log(f"[inputs] {name} T={cfg.T} ready in {time.time() - t0:.1f}s")
    return d


def u16(t: torch.Tensor) -> np.ndarray:
    return W.bf16_tensor_to_u16_numpy(t)


def host_f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def weights_of(d):
    return {k: d[k] for k in ("w_router", "corr_bias", "w_fc1", "w_up", "w_down", "w_fc2", "w_sh_up", "w_sh_down")}


def oracle_route(d, tokens=None, n_group=1, topk_group=1):
    cfg = d["cfg"]
    x = d["x"] if tokens is None else d["x"][tokens]
    return oracle.route(oracle.bf16_bits_to_f64(u16(x)), host_f32(d["w_router"]), host_f32(d["corr_bias"]),
                        cfg.K, cfg.routed_scaling, n_group=n_group, topk_group=topk_group)


def oracle_forward_tokens(d, tokens, idx_override=None, mirror=True, keep=False, n_group=1, topk_group=1,
                          expert=None):
    """The oracle on a subset of tokens (tokens are independent), experts copied on
    demand (or given by ``expert(e) -> (w_up bits, w_down bits)``)."""
    cfg = d["cfg"]
    cache = {}

    def host_expert(e):
        if e not in cache:
            cache[e] = (u16(d["w_up"][e]), u16(d["w_down"][e]))
        return cache[e]

    if expert is None:
        expert = host_expert

    return oracle.forward(u16(d["x"][tokens]), host_f32(d["w_router"]), host_f32(d["corr_bias"]),
                          u16(d["w_fc1"]), u16(d["w_fc2"]), u16(d["w_sh_up"]), u16(d["w_sh_down"]),
                          expert, cfg.K, cfg.routed_scaling, mirror=mirror, idx_override=idx_override, keep=keep,
                          n_group=n_group, topk_group=topk_group)


def check_routing(idx_gpu, gate_gpu, gap_gpu, ref, label=""):
    """Routing bar: idx bit-exact on tokens whose oracle gap >= the tie band; on the
    others the GPU's set must be a correct top-K within the band. Returns the flagged count."""
    idx_gpu = np.asarray(idx_gpu)
    flagged = ref.gap < oracle.GAP_FLAG
    ok = ~flagged
    mism = np.nonzero(np.any(idx_gpu[ok] != ref.idx[ok], axis=1))[0]
    assert mism.size == 0, f"{label}: {mism.size} unflagged tokens route differently (first {np.nonzero(ok)[0][mism[:5]]})"
    # flagged tokens: every chosen expert's exact choice score is within the band of the K-th best
    for t in np.nonzero(flagged)[0]:
        c = ref.choice[t]
        kth = np.sort(c)[::-1][idx_gpu.shape[1] - 1]
        assert np.all(c[idx_gpu[t]] >= kth - oracle.GAP_FLAG), f"{label}: token {t} choice outside the tie band"
        assert len(np.unique(idx_gpu[t])) == idx_gpu.shape[1]
    same = np.all(idx_gpu == ref.idx, axis=1)
    g = np.asarray(gate_gpu)[same].astype(np.float64)
    gr = ref.gate[same].astype(np.float64)
    if g.size:
        rel = np.max(np.abs(g - gr) / np.abs(gr))
        assert rel <= GATE_RTOL, f"{label}: gate relative error {rel:.3g}"
    if gap_gpu is not None:
        gg = np.asarray(gap_gpu, dtype=np.float64)
        fin = np.isfinite(ref.gap)
        assert np.all(np.isinf(gg[~fin]))
        err = np.max(np.abs(gg[fin] - ref.gap[fin])) if fin.any() else 0.0
        assert err < 1e-5, f"{label}: gap error {err:.3g}"
    return int(flagged.sum())


def check_group_routing(idx_gpu, gate_gpu, gap_gpu, ref, n_group, topk_group, label=""):
    """check_routing for group-limited selection. Flagged tokens (group or expert
    margin inside the tie band) must use at most topk_group groups and be a top-K,
    within the band, of the experts of the groups they use."""
    idx_gpu = np.asarray(idx_gpu)
    T, K = idx_gpu.shape
    E = ref.choice.shape[1]
    G = E // n_group
    flagged = ref.gap < oracle.GAP_FLAG
    ok = ~flagged
    mism = np.nonzero(np.any(idx_gpu[ok] != ref.idx[ok], axis=1))[0]
    assert mism.size == 0, f"{label}: {mism.size} unflagged tokens route differently (first {np.nonzero(ok)[0][mism[:5]]})"
    for t in np.nonzero(flagged)[0]:
        groups = np.unique(idx_gpu[t] // G)
        assert len(groups) <= topk_group and len(np.unique(idx_gpu[t])) == K, f"{label}: token {t}"
        pool = np.concatenate([np.arange(g * G, (g + 1) * G) for g in groups])
        c = ref.choice[t]
        kth = np.sort(c[pool])[::-1][K - 1]
        assert np.all(c[idx_gpu[t]] >= kth - oracle.GAP_FLAG), f"{label}: token {t} outside the tie band"
    same = np.all(idx_gpu == ref.idx, axis=1)
    g = np.asarray(gate_gpu)[same].astype(np.float64)
    gr = ref.gate[same].astype(np.float64)
    if g.size:
        rel = np.max(np.abs(g - gr) / np.abs(gr))
        assert rel <= GATE_RTOL, f"{label}: gate relative error {rel:.3g}"
    gg = np.asarray(gap_gpu, dtype=np.float64)
    fin = np.isfinite(ref.gap)
    assert np.all(np.isinf(gg[~fin]))
    err = np.max(np.abs(gg[fin] - ref.gap[fin])) if fin.any() else 0.0
    assert err < 1e-5, f"{label}: gap error {err:.3g}"
    return int(flagged.sum())


def relerr(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


def bf16_dev_to_f64(t: torch.Tensor) -> np.ndarray:
    return oracle.bf16_bits_to_f64(u16(t))


def grouped_tile_kinds(offsets: np.ndarray, BM: int = 256, ntl_list=(20, 8)):
    """Per permuted row: the height class of the grouped products' M tile that
    holds it (1..4 quarters of BM: an expert's tail tile of at most BM/4, BM/2,
    3BM/4 rows runs a shorter tile) and, for each product with ntl column tiles,
    whether any of that M tile's tiles lies in the last eighth of an XCD's range
    (the tiles handed out through the per-XCD counters).

    The order is the one the grouped launch uses: an expert's tiles are
    contiguous, its first M tile f, tile t = f * ntl + nt * ne + i for local M
    tile i of ne and column tile nt; the valid tiles are split over 8 XCDs in
    equal contiguous ranges, and each range's last size // 8 tiles are claimed."""
    offsets = np.asarray(offsets, dtype=np.int64)
    counts = np.diff(offsets)
    ne = (counts + BM - 1) // BM
    first = np.concatenate([[0], np.cumsum(ne)[:-1]])
    n_mtiles = int(ne.sum())
    rows = int(offsets[-1])
    hclass = np.zeros(rows, dtype=np.int8)
    claimed = {ntl: np.zeros(rows, dtype=bool) for ntl in ntl_list}
    ranges = {}
    for ntl in ntl_list:
        valid = n_mtiles * ntl
        q, r = divmod(valid, 8)
        rr = []
        for x in range(8):
            start = x * q + min(x, r)
            size = q + (1 if x < r else 0)
            rr.append((start + size - size // 8, start + size))
        ranges[ntl] = rr
    for e in np.nonzero(counts)[0]:
        for i in range(int(ne[e])):
            a = int(offsets[e]) + i * BM
            b = min(a + BM, int(offsets[e + 1]))
            hclass[a:b] = (b - a + BM // 4 - 1) // (BM // 4)
            for ntl in ntl_list:
                ts = int(first[e]) * ntl + np.arange(ntl) * int(ne[e]) + i
                claimed[ntl][a:b] = any(((ts >= lo) & (ts < hi)).any() for lo, hi in ranges[ntl])
    return hclass, claimed
