"""The forward captured into a HIP graph (through torch.cuda.CUDAGraph) gives, on
every replay, exactly the output of the eager call: the library makes no
allocation, copy, memset or synchronisation inside a forward, so it can be
captured. Replays alternate with eager forwards on other inputs."""
import numpy as np
import pytest
import torch

import sparse_moe_layer_correction_amd as M
import workloads as W
from gpu_util import device_inputs, log, weights_of

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,over", [("tiny", {}), ("tiny", dict(T=300)), ("ultra_decode1", {})])
def test_graph_replays_match_eager(name, over):
    d = device_inputs(name, **over)
    cfg = d["cfg"]
    w = weights_of(d)
    dims = M.dims_from(d["x"], w, cfg.K, cfg.routed_scaling)
    ws = torch.empty(M.workspace_bytes(dims), dtype=torch.uint8, device="cuda")
    out = torch.empty(cfg.T, cfg.H, dtype=torch.bfloat16, device="cuda")
    eager = M.forward(d["x"], w, cfg.K, cfg.routed_scaling).clone()
    x_other = W.make_x(W.get_config(name, **dict(over, seed=cfg.seed + 17)), device="cuda")
    other = M.forward(x_other, w, cfg.K, cfg.routed_scaling).clone()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        M.forward(d["x"], w, cfg.K, cfg.routed_scaling, out=out, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        M.forward(d["x"], w, cfg.K, cfg.routed_scaling, out=out, ws=ws)
    log(f"[graph] {name}{over}: captured")
    for rep in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from the eager forward"
        # eager work in between, on other inputs, through the same workspace
        o2 = M.forward(x_other, w, cfg.K, cfg.routed_scaling, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(o2, other)
    log(f"[graph] {name}{over}: 3 replays equal the eager output")
