"""Parity at the benchmarked sizes, on the rows that exercise every kind of tile.

At the Ultra prefill shape (16384 tokens, 512 experts, K = 22) the grouped
expert products run full 256-row tiles, shorter tiles for each expert's tail
(at most 64, 128 or 192 rows) and, in the last eighth of each XCD's range,
tiles handed out through counters. Tokens are chosen so that their slots land
in every one of those kinds, and for each chosen token the layer output, z,
hs, y_lat and every one of its K expert rows of h and y are compared with the
oracle. Two forwards of the same input must also be bit-identical at the full
prefill and at the one-token decode.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_layer_correction_amd as M
from gpu_util import (OUT_TOL, bf16_dev_to_f64, check_routing, device_inputs, grouped_tile_kinds, log,
                      oracle_forward_tokens, oracle_route, relerr, weights_of)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    M.load_library()
    yield
    torch.cuda.synchronize()


def _view(ws, lay, name, dtype, shape):
    n = int(np.prod(shape))
    es = torch.tensor([], dtype=dtype).element_size()
    return ws[lay[name]:lay[name] + n * es].view(dtype).view(*shape)


def _forward(d):
    cfg = d["cfg"]
    dims = M.dims_from(d["x"], weights_of(d), cfg.K, cfg.routed_scaling)
    ws = torch.empty(M.workspace_bytes(dims), dtype=torch.uint8, device="cuda")
    log(f"[forward] {cfg.name} T={cfg.T} E={cfg.E} K={cfg.K}")
    out = M.forward(d["x"], weights_of(d), cfg.K, cfg.routed_scaling, ws=ws)
    torch.cuda.synchronize()
    return out, ws, M.workspace_layout(dims)


def _pick_tokens(slot_row, hclass, claimed, n_per_kind, n_total, seed):
    """Tokens with slots in every tile kind (n_per_kind each), topped up at random."""
    rng = np.random.default_rng(seed)
    T = slot_row.shape[0]
    kinds = {f"height {q}/4": hclass == q for q in (1, 2, 3, 4)}
    kinds.update({f"claimed (ntl={ntl})": c for ntl, c in claimed.items()})
    chosen = {0, T - 1}
    for name, row_mask in kinds.items():
        tok_has = row_mask[slot_row].any(axis=1)
        cand = np.nonzero(tok_has)[0]
        assert cand.size > 0, f"no token has a slot in a tile of kind {name}"
        chosen.update(rng.choice(cand, size=min(n_per_kind, cand.size), replace=False).tolist())
        log(f"[tiles] {name}: {int(row_mask.sum())} rows, {cand.size} tokens")
    rest = np.setdiff1d(np.arange(T), np.fromiter(chosen, dtype=np.int64))
    if len(chosen) < n_total:
        chosen.update(rng.choice(rest, size=n_total - len(chosen), replace=False).tolist())
    return np.array(sorted(chosen))


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_ultra_prefill_every_tile_kind():
    d = device_inputs("ultra_prefill")
    cfg = d["cfg"]
    out, ws, lay = _forward(d)
    TK = cfg.T * cfg.K
    idx = _view(ws, lay, "idx", torch.int32, (cfg.T, cfg.K)).cpu().numpy()
    gate = _view(ws, lay, "gate", torch.float32, (cfg.T, cfg.K)).cpu().numpy()
    gap = _view(ws, lay, "gap", torch.float32, (cfg.T,)).cpu().numpy()
    check_routing(idx, gate, gap, oracle_route(d), label="ultra_prefill")
    offsets = _view(ws, lay, "offsets", torch.int32, (cfg.E + 1,)).cpu().numpy()
    slot_row = _view(ws, lay, "slot_row", torch.int32, (cfg.T, cfg.K)).cpu().numpy()
    p = oracle.permute(idx, cfg.E)
    assert np.array_equal(offsets, p.offsets) and np.array_equal(slot_row, p.slot_row)
    ntl_up = (cfg.I + 255) // 256
    ntl_down = (cfg.L + 255) // 256
    hclass, claimed = grouped_tile_kinds(offsets, 256, (ntl_up, ntl_down))
    tokens = _pick_tokens(slot_row, hclass, claimed, 12, 64, seed=3)
    log(f"[oracle] ultra_prefill: {len(tokens)} tokens")
    assert len(tokens) >= 64

    ref_r = oracle_route(d, tokens)
    flagged = ref_r.gap < oracle.GAP_FLAG
    override = ref_r.idx.copy()
    override[flagged] = idx[tokens][flagged]
    ref = oracle_forward_tokens(d, tokens, idx_override=override, keep=True)
    tt = torch.as_tensor(tokens, device="cuda")
    errs = {
        "out": relerr(bf16_dev_to_f64(out[tt]), ref["out"]),
        "z": relerr(bf16_dev_to_f64(_view(ws, lay, "z", torch.bfloat16, (cfg.T, cfg.L))[tt]), ref["z"]),
        "hs": relerr(bf16_dev_to_f64(_view(ws, lay, "hs", torch.bfloat16, (cfg.T, cfg.Is))[tt]), ref["hs"]),
        "y_lat": relerr(bf16_dev_to_f64(_view(ws, lay, "y_lat", torch.bfloat16, (cfg.T, cfg.L))[tt]),
                        ref["y_lat"]),
    }
    # every slot of the chosen tokens: the GPU's row slot_row[t, j] against the
    # oracle's row of the same (token, expert) (both list a token's experts ascending)
    rows_gpu = slot_row[tokens].reshape(-1)
    rows_ref = ref["slot_row"].reshape(-1)
    rg = torch.as_tensor(rows_gpu.astype(np.int64), device="cuda")
    h = bf16_dev_to_f64(_view(ws, lay, "h", torch.bfloat16, (TK, cfg.I))[rg])
    y = bf16_dev_to_f64(_view(ws, lay, "y", torch.bfloat16, (TK, cfg.L))[rg])
    errs["h"] = relerr(h, ref["h"][rows_ref])
    errs["y"] = relerr(y, ref["y"][rows_ref])
    kinds = {f"height {q}/4": int(np.sum(hclass[rows_gpu] == q)) for q in (1, 2, 3, 4)}
    kinds.update({f"claimed ntl={k}": int(v[rows_gpu].sum()) for k, v in claimed.items()})
    log(f"[parity] ultra_prefill {len(tokens)} tokens, {rows_gpu.size} expert rows {kinds}: "
        + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    assert all(v > 0 for v in kinds.values())
    for k, v in errs.items():
        assert v < OUT_TOL, f"{k}: max|err|/max|ref| = {v:.3g}"


@pytest.mark.slow
@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", ["ultra_prefill", "ultra_decode1", "ultra_decode64"])
def test_forward_bit_identical_twice(name):
    d = device_inputs(name)
    cfg = d["cfg"]
    a, ws, lay = _forward(d)
    a = a.clone()
    ylat_a = _view(ws, lay, "y_lat", torch.bfloat16, (cfg.T, cfg.L)).clone()
    h_a = _view(ws, lay, "h", torch.bfloat16, (cfg.T * cfg.K, cfg.I)).clone()
    ws.fill_(0x5A)                       # the second forward must not depend on what the first left
    out = torch.full_like(a, 7.0)
    M.forward(d["x"], weights_of(d), cfg.K, cfg.routed_scaling, out=out, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, a), f"{name}: two forwards differ"
    assert torch.equal(_view(ws, lay, "y_lat", torch.bfloat16, (cfg.T, cfg.L)), ylat_a)
    assert torch.equal(_view(ws, lay, "h", torch.bfloat16, (cfg.T * cfg.K, cfg.I)), h_a)
    log(f"[determinism] {name}: out, y_lat and h bit-identical over two forwards")
