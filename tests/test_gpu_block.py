"""The layer's neighbours on an MI355X, through the C ABI: the pre-norm RMSNorm
(bit-exact against the oracle), the block out = x + LatentMoE(RMSNorm(x)) with
the residual add fused into the last product's epilogue, and the load-balancing
bias update (bit-exact).

Bars: normed rows bit-exact; routing as for the layer; the block output within
2e-2 of max|mixer output| of the oracle plus one bf16 step of the sum; the
block output also equal bit for bit to bf16(x + the library's own forward on
the normed rows), which pins the fused residual epilogue exactly.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_moe_layer_correction_amd as M
from gpu_util import (OUT_TOL, bf16_dev_to_f64, check_routing, device_inputs, host_f32, log, u16, weights_of)

pytestmark = pytest.mark.gpu

EPS = float(np.float32(1e-5))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    M.load_library()
    yield
    torch.cuda.synchronize()


def _gamma(H, seed=7, device="cuda"):
    g = torch.Generator().manual_seed(seed)
    v = 1.0 + 0.25 * torch.randn(H, generator=g)
    return v.to(torch.bfloat16).to(device)


def _dev(bits: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


# ----------------------------------------------------------------------------
# RMSNorm
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("T,H,scale,eps", [(64, 256, 1.0, EPS), (37, 8192, 3.0, EPS), (1, 8192, 1.0, EPS),
                                           (300, 2048, 1e-3, EPS), (5, 64, 40.0, 0.0), (16, 8, 1.0, 0.5),
                                           # 2, 6 and more than 8 16-byte chunks per thread
                                           (3, 4096, 1.0, EPS), (4, 12288, 2.0, EPS), (3, 20480, 1.0, EPS)])
def test_rmsnorm_bit_exact(T, H, scale, eps):
    g = torch.Generator().manual_seed(T * 1000 + H)
    x = (scale * torch.randn(T, H, generator=g)).to(torch.bfloat16)
    if T > 2 and eps > 0:
        x[1] = 0.0                                       # a zero row: the scale is 1/sqrt(eps)
        x[2, ::3] *= 1e4                                 # a row with a wide dynamic range
    x = x.cuda()
    gamma = _gamma(H)
    log(f"[rmsnorm] T={T} H={H} scale={scale} eps={eps}")
    y = M.rmsnorm(x, gamma, eps)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm(u16(x), u16(gamma), eps)
    got = bf16_dev_to_f64(y)
    bad = np.nonzero(got != ref)
    assert bad[0].size == 0, f"{bad[0].size} elements differ, first {bad[0][0]},{bad[1][0]}: {got[bad][0]} vs {ref[bad][0]}"
    # in place gives the same bits
    x2 = x.clone()
    M.rmsnorm(x2, gamma, eps, out=x2)
    torch.cuda.synchronize()
    assert torch.equal(x2, y)


def test_rmsnorm_ultra_prefill_rows_sampled():
    d = device_inputs("ultra_prefill")
    x = d["x"]
    gamma = _gamma(x.shape[1])
    y = M.rmsnorm(x, gamma, EPS)
    torch.cuda.synchronize()
    rows = np.r_[0:64, np.random.default_rng(3).choice(x.shape[0], 192, replace=False), x.shape[0] - 1]
    sel = torch.as_tensor(rows, device="cuda")
    ref = oracle.rmsnorm(u16(x[sel]), u16(gamma), EPS)
    assert np.array_equal(bf16_dev_to_f64(y[sel]), ref)


# ----------------------------------------------------------------------------
# block
# ----------------------------------------------------------------------------

def _run_block(d, gamma, out=None):
    cfg = d["cfg"]
    dims = M.dims_from(d["x"], weights_of(d), cfg.K, cfg.routed_scaling)
    ws = torch.empty(M.block_workspace_bytes(dims), dtype=torch.uint8, device="cuda")
    log(f"[block] {cfg.name} T={cfg.T} H={cfg.H} E={cfg.E} K={cfg.K}")
    out = M.block_forward(d["x"], weights_of(d), gamma, cfg.K, cfg.routed_scaling, EPS, ws=ws, out=out)
    torch.cuda.synchronize()
    lay = M.workspace_layout(dims)
    xn = ws[lay["total"]:lay["total"] + cfg.T * cfg.H * 2].view(torch.bfloat16).view(cfg.T, cfg.H)
    idx = ws[lay["idx"]:lay["idx"] + 4 * cfg.T * cfg.K].view(torch.int32).view(cfg.T, cfg.K).cpu().numpy()
    gate = ws[lay["gate"]:lay["gate"] + 4 * cfg.T * cfg.K].view(torch.float32).view(cfg.T, cfg.K).cpu().numpy()
    gap = ws[lay["gap"]:lay["gap"] + 4 * cfg.T].view(torch.float32).cpu().numpy()
    offsets = ws[lay["offsets"]:lay["offsets"] + 4 * (cfg.E + 1)].view(torch.int32).clone()
    return out, xn.clone(), idx, gate, gap, offsets


def _oracle_block(d, gamma, tokens, idx_gpu):
    cfg = d["cfg"]
    xs = u16(d["x"][torch.as_tensor(tokens, device="cuda")])
    xn = oracle.rmsnorm(xs, u16(gamma), EPS)
    r = oracle.route(xn, host_f32(d["w_router"]), host_f32(d["corr_bias"]), cfg.K, cfg.routed_scaling)
    override = r.idx.copy()
    flagged = r.gap < oracle.GAP_FLAG
    override[flagged] = idx_gpu[tokens][flagged]
    cache = {}

    def expert(e):
        if e not in cache:
            cache[e] = (u16(d["w_up"][e]), u16(d["w_down"][e]))
        return cache[e]

    return oracle.block_forward(xs, u16(gamma), EPS, host_f32(d["w_router"]), host_f32(d["corr_bias"]),
                                u16(d["w_fc1"]), u16(d["w_fc2"]), u16(d["w_sh_up"]), u16(d["w_sh_down"]), expert,
                                cfg.K, cfg.routed_scaling, idx_override=override), r, int(flagged.sum())


def _check_block(d, gamma, out, xn, idx, tokens, label):
    cfg = d["cfg"]
    sel = torch.as_tensor(tokens, device="cuda")
    ref, r, nflag = _oracle_block(d, gamma, tokens, idx)
    assert np.array_equal(bf16_dev_to_f64(xn[sel]), ref["xn"]), f"{label}: normed rows differ"
    got = bf16_dev_to_f64(out[sel])
    step = np.ldexp(1.0, np.frexp(np.abs(ref["out"]))[1] - 8)
    lim = OUT_TOL * np.max(np.abs(ref["mixer"])) + step
    err = np.max(np.abs(got - ref["out"]) - lim)
    rel = np.max(np.abs(got - ref["out"])) / np.max(np.abs(ref["mixer"]))
    log(f"[parity] {label}: block out max|err|/max|mixer| = {rel:.2e} ({nflag} tokens in the tie band)")
    assert err <= 0, f"{label}: block output off by {rel:.3g} of max|mixer|"
    return r


def _check_epilogue_exact(d, out, xn):
    """The fused residual add equals bf16(x + the library's forward on the same normed rows)."""
    cfg = d["cfg"]
    mix = M.forward(xn, weights_of(d), cfg.K, cfg.routed_scaling)
    torch.cuda.synchronize()
    s = (d["x"].float() + mix.float()).to(torch.bfloat16)       # bf16 + bf16 is exact in fp32; one rounding
    assert torch.equal(s, out)


@pytest.mark.parametrize("name,over", [("tiny", {}), ("tiny", dict(T=37)), ("tiny", dict(T=1)),
                                       ("tiny", dict(T=300)), ("tiny", dict(T=777, K=1)),
                                       ("tiny", dict(T=333, H=320, L=192, E=24, I=448, Is=576, K=5)),
                                       ("tiny", dict(T=29, H=320, L=192, E=24, I=448, Is=576, K=5))])
def test_block_tiny_full(name, over):
    d = device_inputs(name, **over)
    cfg = d["cfg"]
    gamma = _gamma(cfg.H)
    out, xn, idx, gate, gap, _ = _run_block(d, gamma)
    r = _check_block(d, gamma, out, xn, idx, np.arange(cfg.T), f"{name}{over}")
    check_routing(idx, gate, gap, r, label=f"{name}{over} block")
    _check_epilogue_exact(d, out, xn)


@pytest.mark.parametrize("name,n", [("ultra_decode1", 1), ("ultra_decode64", 3), ("ultra_prefill", 3)])
def test_block_ultra_sampled(name, n):
    d = device_inputs(name)
    cfg = d["cfg"]
    gamma = _gamma(cfg.H)
    out, xn, idx, gate, gap, _ = _run_block(d, gamma)
    rng = np.random.default_rng(17)
    tokens = np.unique(np.r_[rng.choice(cfg.T, size=min(n, cfg.T), replace=False), cfg.T - 1])
    _check_block(d, gamma, out, xn, idx, tokens, name)
    _check_epilogue_exact(d, out, xn)


def test_block_in_place():
    d = device_inputs("tiny", T=48)
    cfg = d["cfg"]
    gamma = _gamma(cfg.H)
    out, _, _, _, _, _ = _run_block(d, gamma)
    x = d["x"].clone()
    dims = M.dims_from(x, weights_of(d), cfg.K, cfg.routed_scaling)
    ws = torch.empty(M.block_workspace_bytes(dims), dtype=torch.uint8, device="cuda")
    M.block_forward(x, weights_of(d), gamma, cfg.K, cfg.routed_scaling, EPS, ws=ws, out=x)
    torch.cuda.synchronize()
    assert torch.equal(x, out)


def test_block_with_mxfp8_experts():
    """The block on MXFP8 experts equals the block on their dequantised bf16 values."""
    d = device_inputs("tiny", T=29)
    cfg = d["cfg"]
    gamma = _gamma(cfg.H)
    mx = M.quantize_experts_mxfp8(weights_of(d))
    deq = dict(weights_of(d))
    for n in ("w_up", "w_down"):
        c, s = mx[n].cpu().numpy(), mx[n + "_scale"].cpu().numpy()
        deq[n] = _dev(oracle.f64_to_bf16_bits(oracle.dequantize_mxfp8(c, s)))
    a = M.block_forward(d["x"], {k: v for k, v in weights_of(d).items() if k not in ("w_up", "w_down")}, gamma,
                        cfg.K, cfg.routed_scaling, EPS, mx=mx)
    b = M.block_forward(d["x"], deq, gamma, cfg.K, cfg.routed_scaling, EPS)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ----------------------------------------------------------------------------
# bias update
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("E,T,K,eta,seed", [(512, 16384, 22, 1e-3, 0), (16, 64, 4, 0.5, 1), (128, 1, 8, 1e-4, 2),
                                            (1000, 333, 7, 3e-3, 3)])
def test_bias_update_bit_exact(E, T, K, eta, seed):
    rng = np.random.default_rng(seed)
    counts = np.bincount(rng.choice(E, size=T * K, p=rng.dirichlet(np.full(E, 0.3))), minlength=E)
    offsets = np.zeros(E + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    bias = rng.uniform(-0.2, 0.2, E).astype(np.float32)
    eta32 = float(np.float32(eta))
    b = torch.from_numpy(bias.copy()).cuda()
    M.bias_update(torch.from_numpy(offsets).cuda(), b, eta32)
    torch.cuda.synchronize()
    ref = oracle.bias_update(bias, counts, eta32, T * K)
    assert np.array_equal(b.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_bias_update_after_a_forward():
    """The forward's own expert offsets feed the update; on a batch with no
    near-tie token they are the oracle's histogram, so the result is bit-exact."""
    d = device_inputs("tiny", T=256)
    cfg = d["cfg"]
    gamma = _gamma(cfg.H)
    _, xn, idx, _, _, offsets = _run_block(d, gamma)
    r = oracle.route(oracle.rmsnorm(u16(d["x"]), u16(gamma), EPS), host_f32(d["w_router"]),
                     host_f32(d["corr_bias"]), cfg.K, cfg.routed_scaling)
    assert np.all(r.gap >= oracle.GAP_FLAG)
    counts = oracle.permute(r.idx, cfg.E).counts
    b = d["corr_bias"].clone()
    M.bias_update(offsets, b, float(np.float32(1e-3)))
    torch.cuda.synchronize()
    ref = oracle.bias_update(host_f32(d["corr_bias"]), counts, float(np.float32(1e-3)), cfg.T * cfg.K)
    assert np.array_equal(b.cpu().numpy().view(np.uint32), ref.view(np.uint32))
