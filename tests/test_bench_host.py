"""Host-side logic of bench.py (no GPU): the one-GPU guard, the HBM traffic
records built from rocprofv3 counter files, and their source-hash check."""
import csv
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, counter, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


DW = "void ckl::gemm_kernel<__bf16, 256, 256, 2, 4, false, false, 2>  _ZN3ckl11gemm_kernelIDF16bLi256ELb0ELb0ELi2E"
COPY = "__amd_rocclr_copyBuffer"


@pytest.fixture
def records_in(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "traffic_path", lambda kind: str(tmp_path / f"{kind}.json"))
    return tmp_path


def test_traffic_records_scale_by_the_copy_calibration(records_in):
    t = records_in
    # a 1 GiB copy that reads FETCH_SIZE = 2^19 KiB (counter in 2x units) and WRITE_SIZE = 2^20 KiB
    _counter_csv(t / "cal_f.csv", [(COPY, "FETCH_SIZE", 524288.0)] * 3)
    _counter_csv(t / "cal_w.csv", [(COPY, "WRITE_SIZE", 1048576.0)] * 3)
    # two dW launches with different counts, and an unrelated kernel that must not be counted
    _counter_csv(t / "f.csv", [(DW, "FETCH_SIZE", 1000.0), (DW, "FETCH_SIZE", 3000.0), ("dense_kernel", "FETCH_SIZE", 7.0)])
    _counter_csv(t / "w.csv", [(DW, "WRITE_SIZE", 500.0), (DW, "WRITE_SIZE", 500.0)])
    bench.traffic_summary(str(t / "f.csv"), str(t / "w.csv"), str(t / "cal_f.csv"), str(t / "cal_w.csv"), "cmds")
    assert not (t / "logits.json").exists()  # no logits rows in these files
    rec = json.load(open(t / "dw.json"))
    assert rec["launches"] == [2, 2]
    assert rec["copy_calibration"]["fetch_scale"] == 2.0 and rec["copy_calibration"]["write_scale"] == 1.0
    assert rec["fetch_bytes_per_launch"] == 2000.0 * 2.0 * 1024
    assert rec["write_bytes_per_launch"] == 500.0 * 1024
    assert rec["bytes_per_launch"] == (4000.0 + 500.0) * 1024
    assert rec["source_sha"] == bench.source_hash(bench.GEMM_SOURCES)
    assert rec["commands"] == "cmds"


def test_traffic_is_reported_only_for_the_sources_it_was_taken_on(records_in):
    t = records_in
    assert bench.traffic_from_profile("dw") is None  # no record
    rec = {"source_sha": bench.source_hash(bench.GEMM_SOURCES), "bytes_per_launch": 123.0}
    (t / "dw.json").write_text(json.dumps(rec))
    assert bench.traffic_from_profile("dw") == 123.0
    rec["source_sha"] = "0" * 16  # taken on other kernels
    (t / "dw.json").write_text(json.dumps(rec))
    assert bench.traffic_from_profile("dw") is None
    (t / "dw.json").write_text("{not json")
    assert bench.traffic_from_profile("dw") is None


def test_traffic_kinds_pick_the_three_gemms_apart():
    names = {
        "logits": "_ZN3ckl11gemm_kernelIDF16bLi256ELi256ELi2ELi4ELb1ELb1ELi0ELi128ELi2ELi16EEEvNS_10GemmParamsE",
        "dh": "_ZN3ckl11gemm_kernelIDF16bLi256ELi256ELi2ELi4ELb1ELb0ELi1ELi128ELi2ELi32EEEvNS_10GemmParamsE",
        "dw": "_ZN3ckl11gemm_kernelIDF16bLi256ELi256ELi2ELi4ELb0ELb0ELi2ELi128ELi2ELi32EEEvNS_10GemmParamsE",
    }
    for kind, name in names.items():
        hits = [k for k, (tags, _) in bench.TRAFFIC_KINDS.items() if all(tg in name for tg in tags)]
        assert hits == [kind]


def test_dtype_override_keeps_the_workload_and_renames_it():
    import bench
    from chunked_kl_loss_seq_amd import workloads as WL

    wl = bench.resolve_workload(2, "f32")
    base = WL.WORKLOADS[2]
    assert (wl.N, wl.d, wl.V, wl.K, wl.chunk, wl.ids, wl.mask) == (base.N, base.d, base.V, base.K, base.chunk,
                                                                      base.ids, base.mask)
    assert wl.dtype == "f32" and wl.name == "bf16-32k-vocab-f32" and base.dtype == "bf16"
    assert bench.resolve_workload(4) is WL.WORKLOADS[4] and bench.resolve_workload(1, "f32") is WL.WORKLOADS[1]
    # the same seeded draws of H and W, only without the bf16 rounding (the
    # cached ids, half of them the student's own top-100, follow the inputs)
    a = WL.make_custom(wl, 2, rows=8)
    b = WL.make(2, rows=8)
    assert np.array_equal(WL.round_bf16(a["H"]), b["H"]) and np.array_equal(WL.round_bf16(a["W"]), b["W"])
    assert a["ids"].shape == b["ids"].shape and not np.array_equal(a["H"], b["H"])
