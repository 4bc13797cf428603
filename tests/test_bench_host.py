"""Host-side logic of bench.py (no GPU): algorithmic byte counts, the
traffic record built from rocprofv3 counter files, its source-hash check,
and the one-GPU guard."""

import csv
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_of_the_large_verify_product():
    # 32768 rows x 28 super-blocks x 84 bytes of weights, q8_1 rows of 1.25 k
    # bytes per token, f32 outputs.
    w = 32768 * 28 * 84
    assert w == 77_070_336
    assert bench.mmvq_bytes(1) == w + 8960 + 4 * 32768 == 77_210_368
    assert bench.mmvq_bytes(8) == w + 8 * 8960 + 4 * 8 * 32768 == 78_190_592
    # q8_1 launch: bf16 in, q8_1 out
    assert bench.q8_bytes(1) == 2 * 7168 + 8960


def _write_counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for name, value in rows:
            wr.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})
            # a row of another counter in the same file is ignored
            wr.writerow({"Kernel_Name": name, "Counter_Name": "GRBM_COUNT", "Counter_Value": 1})


def test_traffic_record_scales_counters_by_the_copy(tmp_path):
    kib = 1024.0
    copy_kib = bench.COPY_BYTES / kib
    # FETCH_SIZE reads half of the copied bytes (factor 2), WRITE_SIZE all of them.
    fetch = [("elementwise_copy_kernel", copy_kib / 2)] * 4 + [("small copy", 3.0)]
    fetch += [("q2k::mmvq_m1_kernel<6, 4, 32, 0>", 38_000.0), ("q2k::mmvq_m1_kernel<6, 4, 32, 0>", 40_000.0)]
    fetch += [("q2k::mmvq_mfma_kernel<28, 2>", 42_000.0)]
    write = [("elementwise_copy_kernel", copy_kib)] * 4
    write += [("q2k::mmvq_m1_kernel<6, 4, 32, 0>", 128.0), ("q2k::mmvq_mfma_kernel<28, 2>", 1024.0)]
    fpath, wpath, out = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "traffic.json"
    _write_counter_csv(fpath, "FETCH_SIZE", fetch)
    _write_counter_csv(wpath, "WRITE_SIZE", write)
    bench.traffic_from(str(fpath), str(wpath), str(out))
    rec = json.loads(out.read_text())
    assert rec["FETCH_SIZE_factor"] == 2.0 and rec["WRITE_SIZE_factor"] == 1.0
    m1, m8 = rec["m1"], rec["m8"]
    assert m1["fetch_bytes"] == round(2 * 39_000.0 * kib)        # mean over dispatches, x factor
    assert m1["write_bytes"] == round(128.0 * kib)
    assert m1["bytes_per_launch"] == m1["fetch_bytes"] + m1["write_bytes"]
    assert m8["bytes_per_launch"] == round(2 * 42_000.0 * kib + 1024.0 * kib)
    assert m1["algorithmic_bytes"] == bench.mmvq_bytes(1)
    assert m1["ratio_to_algorithmic"] == round(m1["bytes_per_launch"] / bench.mmvq_bytes(1), 4)
    assert m1["kernel_hash"] == bench.kernel_hash(1) and m8["kernel_hash"] == bench.kernel_hash(8)


def test_traffic_record_needs_the_calibration_copies(tmp_path):
    fpath, wpath = tmp_path / "f.csv", tmp_path / "w.csv"
    _write_counter_csv(fpath, "FETCH_SIZE", [("q2k::mmvq_m1_kernel<6, 4, 32, 0>", 1.0)])
    _write_counter_csv(wpath, "WRITE_SIZE", [("q2k::mmvq_m1_kernel<6, 4, 32, 0>", 1.0)])
    with pytest.raises(SystemExit):
        bench.traffic_from(str(fpath), str(wpath), str(tmp_path / "out.json"))


def test_traffic_is_null_once_the_kernel_source_changes(tmp_path, monkeypatch):
    rec = {"m1": {"kernel_hash": bench.kernel_hash(1), "bytes_per_launch": 77_800_000},
           "m8": {"kernel_hash": "0" * 16, "bytes_per_launch": 88_000_000}}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.measured_traffic(1) == 77_800_000.0
    assert bench.measured_traffic(8) is None            # recorded on another source
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "absent.json"))
    assert bench.measured_traffic(1) is None


def test_committed_traffic_record_is_consistent():
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    for m in (1, 8):
        r = rec[f"m{m}"]
        assert r["algorithmic_bytes"] == bench.mmvq_bytes(m)
        assert r["bytes_per_launch"] == r["fetch_bytes"] + r["write_bytes"]
        # reading fewer bytes than the weight stream itself would mean a bad calibration
        assert r["bytes_per_launch"] >= 32768 * 28 * 84


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout.strip() == ""


def test_rocprof_record_from_kernel_trace(tmp_path, monkeypatch):
    """--rocprof-from averages the last 640 dispatches of each product
    instantiation in a kernel trace (the ones the roofline's events bracket);
    bench.py reports the average only while the kernel source hash matches."""
    timed = bench.ROOF_GRAPH * bench.ROOF_REPS
    header = '"Kind","Kernel_Name","Start_Timestamp","End_Timestamp"'
    lines = [header]
    t = 1000
    for m, warm_us, timed_us in ((1, 18.0, 13.5), (8, 30.0, 20.0)):
        name = f"void q2k::{bench.KERNEL_INSTANCES[m]}(unsigned char const*, float*)"
        warm = bench.ROOF_GRAPH * 21            # the untimed settle replays
        for i in range(warm + timed):
            dur = warm_us if i < warm else timed_us
            lines.append(f'"KERNEL_DISPATCH","{name}",{t},{t + int(dur * 1000)}')
            t += int(dur * 1000) + 100
    lines.append(f'"KERNEL_DISPATCH","void q2k::mmvq_m1_kernel<6, 4, 32, 1>(x)",{t},{t + 5000}')
    csv_path = tmp_path / "prof_kernel_trace.csv"
    csv_path.write_text("\n".join(lines) + "\n")
    out = tmp_path / "rec.json"
    bench.rocprof_from(str(csv_path), str(out))
    rec = json.loads(out.read_text())
    assert rec["m1"]["avg_us"] == 13.5 and rec["m8"]["avg_us"] == 20.0
    assert rec["m1"]["dispatches"] == timed
    assert rec["m1"]["frac"] == round(bench.mmvq_bytes(1) / 13.5 / 1e3 / 8000.0, 4)
    monkeypatch.setattr(bench, "ROCPROF_FILE", str(out))
    assert bench.measured_rocprof(1) == 13.5
    rec["m1"]["kernel_hash"] = "0" * 16
    out.write_text(json.dumps(rec))
    assert bench.measured_rocprof(1) is None


def test_kernel_sweep_table_from_trace(tmp_path, capsys, monkeypatch):
    """--kernel-sweep-from splits the trace per configuration by the untimed
    passes the run recorded (eager, sizing and settle passes differ from one
    configuration to the next) and averages the timed replays only."""
    monkeypatch.setattr(bench, "KERNEL_SWEEP_SHAPES", [(8192, 2048)])
    n, k = 8192, 2048
    per = n * (k // 256) * 84
    launches = min(max(2, min(1024, -(-(1 << 30) // per))), 128)
    reps = max(2, 1024 // launches)
    rec = {}
    lines = ['"Kind","Kernel_Name","Start_Timestamp","End_Timestamp"']
    t = 1000
    for m in range(2, 9):
        r = {"auto": "mfma", "mfma_us": 1.0, "dots_us": 2.0}
        for name, kern, untimed in (("mfma", "mmvq_mfma_kernel<8, 2, false>", 3 + m),
                                    ("dots", "mmvq_m1_kernel<5, 4, 16, 0>", 4 + m)):
            r[name + "_untimed_passes"] = untimed
            for i in range(launches * (untimed + reps)):
                dur = 50.0 if i < launches * untimed else (10.0 if name == "mfma" else 20.0) + m
                lines.append(f'"KERNEL_DISPATCH","void q2k::{kern}(x)",{t},{t + int(dur * 1000)}')
                t += int(dur * 1000) + 100
        rec[f"{n}x{k}_m{m}"] = r
    csv_path = tmp_path / "k.csv"
    csv_path.write_text("\n".join(lines) + "\n")
    js = tmp_path / "k.json"
    js.write_text(json.dumps({"product_kernels": rec}) + "\n")
    bench.kernel_sweep_from(str(csv_path), str(js))
    out = capsys.readouterr().out.strip().split("\n")
    assert len(out) == 2 + 7
    row4 = out[2 + 2]
    assert "| 4 |" in row4 and "14.000" in row4 and "24.000" in row4 and "mmvq_mfma_kernel<8, 2, false>" in row4
