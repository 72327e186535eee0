"""MX expert weights (MXFP8 and MXFP4) on an MI355X: the quantisers against the
oracle's, bit for bit, and the few-token forward on MX experts against the
oracle run on the oracle's own dequantised experts.

Bars: codes and scales bit-exact; routing as in the bf16 forward; the layer
output within max|err| / max|ref| <= 2e-2 of the oracle; and, since the kernels
decode every weight to its exact bf16 value, the output equal bit for bit to
the bf16 forward given those dequantised weights.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import sparse_moe_layer_correction_amd as M
from gpu_util import (OUT_TOL, bf16_dev_to_f64, check_routing, device_inputs, log, oracle_forward_tokens,
                      oracle_route, relerr, u16, weights_of)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    M.load_library()
    yield
    torch.cuda.synchronize()


def _exact_bf16_bits(v: np.ndarray) -> np.ndarray:
    """float64 values that are bf16 values -> their bit patterns."""
    assert np.array_equal(oracle.round_bf16(v), v), "dequantised weight not a bf16 value"
    return (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


_ORACLE_Q = {"mxfp8": (oracle.quantize_mxfp8, oracle.dequantize_mxfp8),
             "mxfp4": (oracle.quantize_mxfp4, oracle.dequantize_mxfp4)}
FORMATS = ["mxfp8", "mxfp4"]


def _oracle_mx(bits: np.ndarray, fmt="mxfp8"):
    """The oracle's MX codes, scales and dequantised bf16 bits of bf16 ``bits``."""
    q, dq = _ORACLE_Q[fmt]
    codes, scales = q(oracle.bf16_bits_to_f64(bits))
    return codes, scales, _exact_bf16_bits(dq(codes, scales))


def _gpu_quant(bits: np.ndarray, fmt="mxfp8"):
    src = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    log(f"[quantize] {fmt} {tuple(bits.shape)}")
    c, s = (M.quantize_mxfp8 if fmt == "mxfp8" else M.quantize_mxfp4)(src)
    torch.cuda.synchronize()
    return c.cpu().numpy(), s.cpu().numpy()


def _finite_bf16_patterns() -> np.ndarray:
    p = np.arange(1 << 16, dtype=np.uint32)
    return p[((p >> 7) & 0xFF) != 0xFF].astype(np.uint16)        # 65024 patterns, no inf / NaN


@pytest.mark.parametrize("fmt", FORMATS)
def test_quantizer_every_finite_bf16_value(fmt):
    pats = _finite_bf16_patterns()
    rng = np.random.default_rng(5)
    mags = oracle.bf16_bits_to_f64(pats)
    blocks = [
        rng.permutation(pats),                          # mixed magnitudes: most elements far below the block max
        pats[np.argsort(np.abs(mags), kind="stable")],  # neighbours in magnitude: every scale, every code
    ]
    bits = np.concatenate(blocks).reshape(-1, 64)
    c, s = _gpu_quant(bits, fmt)
    rc, rs, _ = _oracle_mx(bits, fmt)
    assert np.array_equal(s, rs), f"scales differ in {np.count_nonzero(s != rs)} blocks"
    bad = np.nonzero(c != rc)
    assert bad[0].size == 0, f"{bad[0].size} codes differ, first at {bad[0][0]},{bad[1][0]}"


@pytest.mark.parametrize("fmt", FORMATS)
def test_quantizer_special_blocks(fmt):
    f = np.zeros((7, 32))
    f[1] = -0.0                                               # negative zeros keep their sign bit
    f[2, 0] = 448.0 * 2 ** 3; f[2, 1:] = np.arange(1, 32) * 2 ** -7     # one large element, the rest tiny
    f[3] = np.linspace(-1, 1, 32)
    # ties of the E4M3 grid at scale 2^0 (block max 256..511): 1 + k/16 for odd k
    f[4, 0] = 256.0; f[4, 1:] = 1.0 + (2 * np.arange(31) % 16 + 1) / 16.0
    f[5, 0] = 2.0 ** -120; f[5, 1] = -(2.0 ** -121)          # tiny block: the scale exponent clamps at -127
    # ties of the E2M1 grid at scale 2^0 (block max 6): halfway points of every step
    f[6, 0] = 6.0; f[6, 1:15] = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0] * 2) * np.repeat([1, -1], 7)
    bits = _exact_bf16_bits(oracle.round_bf16(f))
    c, s = _gpu_quant(bits, fmt)
    rc, rs, _ = _oracle_mx(bits, fmt)
    assert np.array_equal(s, rs) and np.array_equal(c, rc)
    assert c[1].tolist() == ([0x80] * 32 if fmt == "mxfp8" else [0x88] * 16)   # negative zeros keep their sign


def _quantize_experts(d, label, fmt="mxfp8"):
    """The GPU's MX experts, quantised from the workload's bf16 weights."""
    mx = M.quantize_experts_mx(weights_of(d), fmt)
    torch.cuda.synchronize()
    log(f"[quantize] {label} experts on the GPU ({fmt})")
    return mx


class _OracleExperts:
    """expert(e) for the oracle: the oracle's dequantised MXFP8 weights of expert e,
    after checking that the GPU's codes and scales of that expert equal the oracle's."""

    def __init__(self, d, mx, fmt="mxfp8"):
        self.d, self.mx, self.fmt, self.cache = d, mx, fmt, {}

    def _one(self, e):
        out = []
        for n in ("w_up", "w_down"):
            c, s, deq = _oracle_mx(u16(self.d[n][e]), self.fmt)
            assert np.array_equal(self.mx[n + "_scale"][e].cpu().numpy(), s), f"{n}[{e}] scales"
            assert np.array_equal(self.mx[n][e].cpu().numpy(), c), f"{n}[{e}] codes"
            out.append(deq)
        return tuple(out)

    def prefetch(self, experts):
        todo = [int(e) for e in experts if int(e) not in self.cache]
        with ThreadPoolExecutor(16) as pool:
            for e, r in zip(todo, pool.map(self._one, todo)):
                self.cache[e] = r
        log(f"[oracle] quantised {len(todo)} experts")

    def __call__(self, e):
        if e not in self.cache:
            self.cache[e] = self._one(e)
        return self.cache[e]


def _run_mx(d, mx):
    cfg = d["cfg"]
    dims = M.dims_from(d["x"], weights_of(d), cfg.K, cfg.routed_scaling)
    ws = torch.empty(M.workspace_bytes(dims), dtype=torch.uint8, device="cuda")
    log(f"[forward_mx] {cfg.name} T={cfg.T} H={cfg.H} E={cfg.E} K={cfg.K}")
    w = {k: v for k, v in weights_of(d).items() if k not in ("w_up", "w_down")}
    out = M.forward_mx(d["x"], w, mx, cfg.K, cfg.routed_scaling, ws=ws)
    torch.cuda.synchronize()
    lay = M.workspace_layout(dims)
    view = lambda n, dt, shp: ws[lay[n]:lay[n] + int(np.prod(shp)) * torch.tensor([], dtype=dt).element_size()] \
        .view(dt).view(*shp).cpu().numpy()
    return out, view("idx", torch.int32, (cfg.T, cfg.K)), view("gate", torch.float32, (cfg.T, cfg.K)), \
        view("gap", torch.float32, (cfg.T,))


def _compare(d, out, idx, tokens, experts, label):
    ref_r = oracle_route(d, tokens)
    override = ref_r.idx.copy()
    flagged = ref_r.gap < oracle.GAP_FLAG
    override[flagged] = idx[tokens][flagged]
    experts.prefetch(np.unique(override))
    ref = oracle_forward_tokens(d, tokens, idx_override=override, expert=experts)
    e = relerr(bf16_dev_to_f64(out[torch.as_tensor(tokens, device="cuda")]), ref["out"])
    log(f"[parity] {label}: out {e:.2e} on {len(tokens)} tokens")
    assert e < OUT_TOL, f"{label}: max|err|/max|ref| = {e:.3g}"


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("over", [{}, dict(T=37), dict(T=1), dict(K=16), dict(K=1)])
def test_forward_mx_tiny(over, fmt):
    d = device_inputs("tiny", **over)
    cfg = d["cfg"]
    mx = _quantize_experts(d, f"tiny{over}", fmt)
    experts = _OracleExperts(d, mx, fmt)
    experts.prefetch(range(cfg.E))                 # every expert's codes checked against the oracle's
    out, idx, gate, gap = _run_mx(d, mx)
    check_routing(idx, gate, gap, oracle_route(d), label="tiny mx")
    _compare(d, out, idx, np.arange(cfg.T), experts, f"tiny{over}")
    # the bf16 forward on the oracle's dequantised weights gives the same bits
    deq = dict(weights_of(d))
    for j, n in enumerate(("w_up", "w_down")):
        deq[n] = torch.from_numpy(np.stack([experts(e)[j] for e in range(cfg.E)]).view(np.int16)).cuda() \
            .view(torch.bfloat16)
    ref_out = M.forward(d["x"], deq, cfg.K, cfg.routed_scaling)
    torch.cuda.synchronize()
    assert torch.equal(ref_out, out)


@pytest.mark.slow
@pytest.mark.timeout(600)
@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("name", ["ultra_decode1", "ultra_decode64"])
def test_forward_mx_ultra(name, fmt):
    """Every token of the batch; the codes and scales of every expert they use
    are checked bit for bit against the oracle's quantiser (about 480 experts at
    64 tokens)."""
    d = device_inputs(name)
    cfg = d["cfg"]
    mx = _quantize_experts(d, name, fmt)
    out, idx, gate, gap = _run_mx(d, mx)
    check_routing(idx, gate, gap, oracle_route(d), label=f"{name} mx")
    _compare(d, out, idx, np.arange(cfg.T), _OracleExperts(d, mx, fmt), f"{name} {fmt}")


def test_forward_mx_rejects_many_tokens():
    d = device_inputs("tiny", T=65)
    cfg = d["cfg"]
    mx = _quantize_experts(d, "tiny T=65")
    with pytest.raises(RuntimeError):
        _run_mx(d, mx)
