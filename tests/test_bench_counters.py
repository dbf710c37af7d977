"""bench.py --counters-from: the committed traffic and clock files are derived
from rocprofv3 counter CSVs exactly as documented (products in the run's own
launch order, every dispatch averaged, units calibrated by the run's 1 GiB
copy).  CPU only, on a small synthetic run directory."""
import csv
import json
import os

import pytest

import bench

LABELS = ["mlp_fwd.xw1_gelu", "mlp_fwd.hw2", "mlp_bwd.htdy", "mlp_bwd.dyw2t_dgelu", "mlp_bwd.daw1t",
          "mlp_bwd.xtda"]


def _write_run(root, name, counters, per_kernel, copy_values, steps=2, src_hash="abc123"):
    """One counter run: `steps` steps of the six products (launch order LABELS),
    then the calibration copy.  per_kernel(label, step) -> {counter: value}."""
    d = os.path.join(root, name)
    os.makedirs(d)
    rows, disp = [], 0
    for st in range(steps):
        for lab in LABELS:
            disp += 1
            vals = per_kernel(lab, st)
            for c in counters:
                rows.append({"Dispatch_Id": disp, "Kernel_Name": f"void tpk::gemm_bf16_kernel<{lab}>",
                             "Counter_Name": c, "Counter_Value": vals[c],
                             "Start_Timestamp": 1000, "End_Timestamp": 1000 + vals.get("dur", 500000)})
    disp += 1
    for c in counters:
        rows.append({"Dispatch_Id": disp, "Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": c,
                     "Counter_Value": copy_values.get(c, 0), "Start_Timestamp": 0, "End_Timestamp": 1})
    with open(os.path.join(d, "c5_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)
    with open(os.path.join(root, name + ".log"), "w") as fh:
        fh.write("rocprofv3 chatter\n")
        fh.write(json.dumps({"profile": True, "kernel_source_hash": src_hash,
                             "kernels_ms": {lab: 0.5 for lab in LABELS}}) + "\n")


def test_counter_files(tmp_path, monkeypatch):
    root = str(tmp_path)
    idx = {lab: i for i, lab in enumerate(LABELS)}
    # FETCH_SIZE reads half the bytes (KiB) of the copy, WRITE_SIZE all of them
    _write_run(root, "pmc_fetch", ["FETCH_SIZE"], lambda lab, st: {"FETCH_SIZE": 1000.0 * (idx[lab] + 1) + st},
               {"FETCH_SIZE": 524288.0})
    _write_run(root, "pmc_write", ["WRITE_SIZE"], lambda lab, st: {"WRITE_SIZE": 100.0 * (idx[lab] + 1)},
               {"WRITE_SIZE": 1048576.0})
    _write_run(root, "c5pmc1", ["GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES"],
               lambda lab, st: {"GRBM_GUI_ACTIVE": 8 * 900000.0, "SQ_VALU_MFMA_BUSY_CYCLES": 900000.0 * 512,
                                "dur": 500000}, {})
    monkeypatch.setattr(bench, "TRAFFIC_FILE", os.path.join(root, "traffic.json"))
    monkeypatch.setattr(bench, "CLOCK_FILE", os.path.join(root, "clock.json"))
    bench.write_counter_files(root)
    t = json.load(open(os.path.join(root, "traffic.json")))
    c = json.load(open(os.path.join(root, "clock.json")))
    assert t["kernel_source_hash"] == c["kernel_source_hash"] == "abc123"
    assert t["fetch_size_scale"] == 2.0 and t["write_size_scale"] == 1.0
    for lab in LABELS:
        k = t["kernels"][lab]
        fetch_kib = 1000.0 * (idx[lab] + 1) + 0.5          # mean over the two steps
        assert k["fetch_bytes_per_launch"] == int(fetch_kib * 1024 * 2)
        assert k["write_bytes_per_launch"] == int(100.0 * (idx[lab] + 1) * 1024)
        assert k["hbm_bytes_per_launch"] == k["fetch_bytes_per_launch"] + k["write_bytes_per_launch"]
        assert c["kernels"][lab]["clock_ghz"] == 1.8       # 900000 cycles per XCD in 500 us
        assert c["kernels"][lab]["mfma_busy"] == 0.5
    assert c["mean_clock_ghz"] == 1.8


def test_counter_runs_from_different_sources(tmp_path):
    root = str(tmp_path)
    one = lambda lab, st: {"FETCH_SIZE": 1.0, "WRITE_SIZE": 1.0, "GRBM_GUI_ACTIVE": 8.0,
                           "SQ_VALU_MFMA_BUSY_CYCLES": 1.0}
    _write_run(root, "pmc_fetch", ["FETCH_SIZE"], one, {"FETCH_SIZE": 524288.0}, src_hash="a")
    _write_run(root, "pmc_write", ["WRITE_SIZE"], one, {"WRITE_SIZE": 1048576.0}, src_hash="b")
    _write_run(root, "c5pmc1", ["GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES"], one, {}, src_hash="a")
    with pytest.raises(SystemExit):
        bench.write_counter_files(root)
