"""The library keeps no state between calls and creates no stream or event:
forwards issued at the same time from two host threads, each on its own stream
and workspace, must each give exactly their single-threaded output."""
import threading

import pytest
import torch

import sparse_moe_layer_correction_amd as M
import workloads as W
from gpu_util import device_inputs, log, weights_of

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,over", [("tiny", {}), ("ultra_decode1", {})])
def test_concurrent_host_threads(name, over):
    d = device_inputs(name, **over)
    cfg = d["cfg"]
    w = weights_of(d)
    xs = [d["x"], W.make_x(W.get_config(name, **dict(over, seed=cfg.seed + 29)), device="cuda")]
    refs = [M.forward(x, w, cfg.K, cfg.routed_scaling).clone() for x in xs]
    torch.cuda.synchronize()
    dims = M.dims_from(xs[0], w, cfg.K, cfg.routed_scaling)
    outs = [torch.empty(cfg.T, cfg.H, dtype=torch.bfloat16, device="cuda") for _ in xs]
    wss = [torch.empty(M.workspace_bytes(dims), dtype=torch.uint8, device="cuda") for _ in xs]
    streams = [torch.cuda.Stream() for _ in xs]
    errors = []
    rounds = 20

    def worker(i):
        try:
            torch.cuda.set_device(0)
            with torch.cuda.stream(streams[i]):
                for r in range(rounds):
                    outs[i].zero_()
                    M.forward(xs[i], w, cfg.K, cfg.routed_scaling, out=outs[i], ws=wss[i])
                    streams[i].synchronize()
                    if not torch.equal(outs[i], refs[i]):
                        errors.append(f"thread {i} round {r}: output differs from the single-threaded one")
                        return
        except Exception as e:          # reported by the main thread
            errors.append(f"thread {i}: {e!r}")

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(xs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=100)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    log(f"[streams] {name}{over}: {rounds} rounds on 2 host threads equal the single-threaded outputs")
