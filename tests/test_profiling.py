"""Host logic of the rocprofv3 summaries (no GPU): synthetic counter files with
known values go in, the figures the summaries must derive from them come out."""
import csv
import json

import pytest

from sparse_moe_layer_correction_amd import profiling as P

COLS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]

DENSE = "void moe::gemm_bf16_kernel<256, 256, 2, 2, -1, 1, 3>(moe::GemmLaunch)"
UP = "void moe::gemm_bf16_kernel<256, 256, 2, 4, 1, 2, 3>(moe::GemmLaunch)"
DOWN = "void moe::gemm_bf16_kernel<256, 256, 2, 2, 0, 1, 3>(moe::GemmLaunch)"
ORDER = [DENSE, DENSE, UP, DOWN, DENSE]          # router, fc1 + shared up, expert up, expert down, fc2 + shared down


def _write(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COLS)
        w.writeheader()
        for r in rows:
            w.writerow(r)


def _mfma_rows(order, forwards, util, mops, grbm, dur_ns):
    rows, d = [], 0
    for _ in range(forwards):
        for i, name in enumerate(order):
            d += 1
            # an unrelated kernel between the products must be ignored
            rows.append(dict(Dispatch_Id=1000 + d, Kernel_Name="void moe::topk_kernel<8>(...)",
                             Counter_Name="MfmaUtil", Counter_Value=0.0, Start_Timestamp=0, End_Timestamp=1))
            for c, v in (("MfmaUtil", util[i]), ("SQ_INSTS_VALU_MFMA_MOPS_BF16", mops[i]),
                         ("GRBM_GUI_ACTIVE", grbm[i])):
                rows.append(dict(Dispatch_Id=d, Kernel_Name=name, Counter_Name=c, Counter_Value=v,
                                 Start_Timestamp=10_000 * d, End_Timestamp=10_000 * d + dur_ns[i]))
    return rows


def _table(md):
    out = {}
    for line in open(md):
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if cells and cells[0] in P.GEMM_PHASES:
            out[cells[0]] = cells
    return out


def test_mfma_summary_derives_busy_ratio_and_clock(tmp_path):
    dims = (512, 256, 128, 16, 192, 4, 320)
    fl = P.gemm_phase_flops(*dims)
    # issued MFMA work: exactly the algorithm's for dense products, 1.25x for the grouped ones, 3x for the router
    ratio = [3.0, 1.0, 1.25, 1.25, 1.0]
    mops = [fl[p] * r / 512 for p, r in zip(P.GEMM_PHASES, ratio)]
    util = [10.0, 60.0, 50.0, 55.0, 65.0]
    dur = [1000, 2000, 4000, 3000, 2500]
    ghz = [1.5, 1.8, 1.75, 2.0, 2.1]
    n_xcc = 8
    grbm = [g * t * n_xcc for g, t in zip(ghz, dur)]     # summed over the XCDs
    _write(tmp_path / "ctr_counter_collection.csv", _mfma_rows(ORDER, 2, util, mops, grbm, dur))
    with open(tmp_path / "ctr_agent_info.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Agent_Type", "Num_Xcc"])
        w.writeheader()
        w.writerow({"Agent_Type": "CPU", "Num_Xcc": 0})
        w.writerow({"Agent_Type": "GPU", "Num_Xcc": n_xcc})
    out = tmp_path / "mfma.md"
    P.summarize_mfma("t", str(tmp_path / "ctr_counter_collection.csv"), str(out), "cmd", ",".join(map(str, dims)))
    tab = _table(out)
    assert list(tab) == list(P.GEMM_PHASES)
    for i, ph in enumerate(P.GEMM_PHASES):
        _, _, ms, tflops, busy, issued, clk, peak = tab[ph]
        assert float(ms) == pytest.approx(dur[i] / 1e6, abs=1e-3)
        assert float(tflops) == pytest.approx(fl[ph] / dur[i] / 1e3, rel=1e-2, abs=1)
        assert busy == f"{util[i]:.1f} %"
        assert float(issued) == pytest.approx(ratio[i], abs=1e-3)
        assert float(clk) == pytest.approx(ghz[i], abs=0.006)
        assert float(peak) == pytest.approx(2500 * ghz[i] / 2.4, abs=1)


def test_mfma_phase_flops_are_the_layer_products():
    T, H, L, E, I, K, Is = 3, 5, 7, 11, 13, 2, 17
    f = P.gemm_phase_flops(T, H, L, E, I, K, Is)
    assert f == {"router": 2 * T * H * E, "fc1_shared_up": 2 * T * H * L + 2 * T * H * Is,
                 "expert_up": 2 * T * K * L * I, "expert_down": 2 * T * K * I * L,
                 "fc2_shared_down": 2 * T * L * H + 2 * T * Is * H}


def test_mfma_summary_rejects_a_launch_out_of_order(tmp_path):
    bad = [DENSE, DENSE, DOWN, UP, DENSE]            # expert down where expert up belongs
    one = [1.0] * 5
    _write(tmp_path / "c.csv", _mfma_rows(bad, 1, one, one, one, [10] * 5))
    with pytest.raises(SystemExit, match="not the expert_up launch"):
        P.summarize_mfma("t", str(tmp_path / "c.csv"), str(tmp_path / "o.md"), "cmd", "1,1,1,1,1,1,1")


def test_mfma_summary_rejects_partial_forwards(tmp_path):
    one = [1.0] * 4
    _write(tmp_path / "c.csv", _mfma_rows(ORDER[:4], 1, one, one, one, [10] * 4))
    with pytest.raises(SystemExit, match="not whole forwards"):
        P.summarize_mfma("t", str(tmp_path / "c.csv"), str(tmp_path / "o.md"), "cmd", "1,1,1,1,1,1,1")


def test_traffic_scales_by_the_calibration_copy(tmp_path):
    # the counters read half the copied bytes on fetch and all of them on write
    cal_kib = P.CALIBRATION_BYTES / 1024
    fetch_rows, write_rows = [], []
    for d, (name, fk, wk) in enumerate([("copyBuffer", cal_kib / 2, cal_kib), (UP, 1000.0, 300.0),
                                        (UP, 1200.0, 300.0), (DOWN, 800.0, 100.0)]):
        fetch_rows.append(dict(Dispatch_Id=d, Kernel_Name=name, Counter_Name="FETCH_SIZE", Counter_Value=fk,
                               Start_Timestamp=0, End_Timestamp=1))
        write_rows.append(dict(Dispatch_Id=d, Kernel_Name=name, Counter_Name="WRITE_SIZE", Counter_Value=wk,
                               Start_Timestamp=0, End_Timestamp=1))
    _write(tmp_path / "f.csv", fetch_rows)
    _write(tmp_path / "w.csv", write_rows)
    out = tmp_path / "t.json"
    data = P.summarize_traffic("w", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), str(out), "cmds")
    rec = data["w"]
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    up = rec["phases"]["expert_up"]
    assert up["launches"] == 2
    assert up["fetch_bytes_per_launch"] == round(1100.0 * 1024 * 2)
    assert up["write_bytes_per_launch"] == round(300.0 * 1024)
    assert up["kernel_hash"] == P.kernel_source_hash("gemm")
    down = rec["phases"]["expert_down"]
    assert down["bytes_per_launch"] == round(800.0 * 1024 * 2) + round(100.0 * 1024)
    assert json.load(open(out)) == data


def test_source_hash_ignores_comments():
    assert P._code_only("int a; // note\n/* block\ncomment */ int b;\n\n") == "int a;\n int b;"
