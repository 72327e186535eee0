"""The allocation-free forward (moe_forward_noalloc, its workspace the library's
static device scratch) against moe_forward with a caller workspace: bit-identical
outputs on two calls in a row, the second with fewer tokens, and inside a
captured HIP graph replayed between eager calls."""
import numpy as np
import pytest
import torch

import sparse_moe_layer_correction_amd as M
import workloads as W
from gpu_util import device_inputs, log, weights_of

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests need an MI355X")
    M.load_library()
    yield
    torch.cuda.synchronize()


def _reference(d):
    cfg = d["cfg"]
    out = M.forward(d["x"], weights_of(d), cfg.K, cfg.routed_scaling)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("first,second", [
    (("tiny", {}), ("tiny", dict(T=37))),
    (("ultra_decode64", {}), ("ultra_decode1", {})),
    # the tiled path: grouped products whose XCD tails are claimed through the
    # counters in the scratch (zeroed by the permutation on every call), then a
    # smaller tiled batch on the same scratch
    (("tiny", dict(T=2048, H=512, L=256, E=32, I=1024, Is=512, K=4)), ("tiny", dict(T=300))),
])
def test_noalloc_equals_forward_twice(first, second):
    for name, over in (first, second):
        d = device_inputs(name, **over)
        cfg = d["cfg"]
        ref = _reference(d)
        out = torch.full_like(ref, 3.0)
        log(f"[noalloc] {name}{over} T={cfg.T}")
        M.forward_noalloc(d["x"], weights_of(d), cfg.K, cfg.routed_scaling, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"{name}{over}: allocation-free forward differs from moe_forward"
    log("[noalloc] two calls in a row, the second smaller, equal moe_forward bit for bit")


def test_noalloc_rejects_a_batch_beyond_its_scratch():
    d = device_inputs("tiny")
    cfg = W.get_config("tiny")
    x = torch.zeros(M.NOALLOC_SCRATCH_BYTES // (cfg.H * 2) + 1, cfg.H, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(M.MoEError, match="static scratch"):
        M.forward_noalloc(x, weights_of(d), cfg.K, cfg.routed_scaling)


def test_noalloc_in_a_captured_graph():
    d = device_inputs("ultra_decode1")
    cfg = d["cfg"]
    w = weights_of(d)
    ref = _reference(d)
    x_other = W.make_x(W.get_config("ultra_decode1", seed=cfg.seed + 5), device="cuda")
    ref_other = M.forward(x_other, w, cfg.K, cfg.routed_scaling).clone()
    out = torch.empty_like(ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        M.forward_noalloc(d["x"], w, cfg.K, cfg.routed_scaling, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        M.forward_noalloc(d["x"], w, cfg.K, cfg.routed_scaling, out=out)
    log("[noalloc] captured")
    for rep in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"replay {rep}"
        # an eager allocation-free call on other inputs in between (same scratch)
        o2 = M.forward_noalloc(x_other, w, cfg.K, cfg.routed_scaling)
        torch.cuda.synchronize()
        assert torch.equal(o2, ref_other)
    log("[noalloc] 3 graph replays equal moe_forward")
