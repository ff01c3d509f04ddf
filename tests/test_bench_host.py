"""Host-side logic of bench.py, on the CPU: the one-GPU refusal, the
algorithmic byte counts its roofline divides by, and the two profile
summarisers run on small synthetic rocprofv3 outputs (the counter scaling
by the copy kernel, and the windows that tell the step's dispatches from the
backward's and the rest)."""

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

STATE = "void based::mfma::linattn_state_kernel<4, 0, 1>(based::mfma::Params)"
MAIN = "void based::mfma::linattn_mfma_kernel<4, 1, 0, 0>(based::mfma::Params)"
QPASS = "based::bwdm::query_pass_kernel(based::bwdm::Params)"
SWAB = "void based::swab::swa_bwd_mfma_kernel<4>(based::swab::Params)"
DECODE = "void based::(anonymous namespace)::decode_step_kernel<unsigned short, 64, 273>(int)"
DECODE_C = "void based::(anonymous namespace)::decode_step_kernel<unsigned short, 64, 153>(int)"
COPY = "__amd_rocclr_copyBuffer"


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_bytes():
    # per (position, head), d_v 64, bf16 in / fp32 out
    assert bench.lin_bytes(64) == 448      # q, k, v read; y written
    assert bench.layer_bytes(64) == 704    # q, k, v read; y_lin and y_swa written
    assert bench.bwd_bytes(64) == 1088     # q, k, v, y, dy read; dq, dk, dv written
    # per head-step of decode: S and z read and written, the ring, q/k/v, outputs
    assert bench.decode_bytes(64, 64) == 152904
    assert bench.decode_bytes(64, 64, rows=153) == 152904 - 2 * 120 * (64 + 1) * 4


def _write_counters(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        w.writerows(rows)


def _dispatches():
    """The bench's dispatch order with calls = 2: the copy, the backward's
    input set-up (one layer call), the step (two layer calls), the backward
    (two calls of each op), then decode.  (id, kernel, fetch KiB, write KiB)."""
    copy_kib = bench.COPY_BYTES / 1024
    return [(1, COPY, 2 * copy_kib, copy_kib),                     # fetch reads twice the bytes, write once
            (2, STATE, 1000.0, 100.0), (3, MAIN, 3000.0, 900.0),     # set-up call
            (4, STATE, 1000.0, 100.0), (5, MAIN, 3000.0, 900.0),     # step 1
            (6, STATE, 1200.0, 100.0), (7, MAIN, 3400.0, 900.0),     # step 2
            (8, QPASS, 500.0, 50.0), (9, QPASS, 500.0, 50.0),
            (10, SWAB, 700.0, 70.0), (11, SWAB, 700.0, 70.0),
            (12, DECODE, 40.0, 40.0), (13, DECODE_C, 22.0, 22.0)]


def test_summarize_pmc_scales_and_windows(tmp_path):
    fetch, write = [], []
    for i, name, f, wr in _dispatches():
        # two instances of each counter per dispatch: the summariser adds them
        fetch += [{"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": "FETCH_SIZE", "Counter_Value": f / 2}] * 2
        write += [{"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": "WRITE_SIZE", "Counter_Value": wr / 2}] * 2
    _write_counters(str(tmp_path / "f"), fetch)
    _write_counters(str(tmp_path / "w"), write)
    out = tmp_path / "out"
    bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), 2, "cmd", out_dir=str(out))
    layer = json.loads((out / "traffic_layer.json").read_text())
    # fetch scaled by 1/2, write by 1; medians over the set-up and step calls
    assert layer["copy_fetch_factor"] == pytest.approx(0.5)
    assert layer["copy_write_factor"] == pytest.approx(1.0)
    k = layer["kernels"]
    assert k["based::mfma::linattn_state_kernel<4, 0, 1>"]["dispatches"] == 3
    assert k["based::mfma::linattn_state_kernel<4, 0, 1>"]["fetch_bytes"] == pytest.approx(1000.0 * 1024 * 0.5)
    assert k["based::mfma::linattn_mfma_kernel<4, 1, 0, 0>"]["write_bytes"] == pytest.approx(900.0 * 1024)
    assert layer["bytes_per_call"] == pytest.approx(((1000 + 3000) * 0.5 + 100 + 900) * 1024)
    assert layer["source_hash"] == bench.source_hash("layer")
    bwd = json.loads((out / "traffic_bwd.json").read_text())
    assert set(bwd["kernels"]) == {"based::bwdm::query_pass_kernel", "based::swab::swa_bwd_mfma_kernel<4>"}
    assert bwd["bytes_per_call"] == pytest.approx(((500 + 700) * 0.5 + 50 + 70) * 1024)
    dec = json.loads((out / "traffic_decode.json").read_text())
    assert dec["bytes_per_call"] == pytest.approx((40 * 0.5 + 40) * 1024)
    # the two state layouts' decode steps are told apart by the row count
    dc = json.loads((out / "traffic_decode_compact.json").read_text())
    assert dc["bytes_per_call"] == pytest.approx((22 * 0.5 + 22) * 1024)


def test_summarize_pmc_needs_the_copy(tmp_path):
    rows = [{"Dispatch_Id": i, "Kernel_Name": n, "Counter_Name": "FETCH_SIZE", "Counter_Value": f}
            for i, n, f, _ in _dispatches() if n != COPY]
    _write_counters(str(tmp_path / "f"), rows)
    _write_counters(str(tmp_path / "w"), [])
    with pytest.raises(SystemExit):
        bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), 2, "cmd", out_dir=str(tmp_path / "o"))


def test_summarize_stats_marks_step_and_backward(tmp_path):
    d = tmp_path / "stats"
    d.mkdir()
    rows, t = [], 1000
    for i, name, _, _ in _dispatches():
        dur = {STATE: 17_000, MAIN: 58_000, QPASS: 83_000, SWAB: 71_000}.get(name, 5_000)
        rows.append({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + dur, "Grid_Size_X": 131072,
                     "Workgroup_Size_X": 256})
        t += dur + 1000
    with open(d / "run_kernel_trace.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)
    bench.summarize_stats(str(d), "cmd", 2, out_dir=str(tmp_path / "out"))
    text = (tmp_path / "out" / "kernel_stats.md").read_text()
    lines = {ln.split("|")[1].strip().strip("`"): ln for ln in text.splitlines() if ln.startswith("| `")}
    # the set-up and step calls of the layer are marked step; the backward's
    # calls bwd; decode (after the backward) neither
    assert "| step | 3 | 17.0 |" in lines["based::mfma::linattn_state_kernel<4, 0, 1>"]
    assert "| step | 3 | 58.0 |" in lines["based::mfma::linattn_mfma_kernel<4, 1, 0, 0>"]
    assert "| bwd | 2 | 83.0 |" in lines["based::bwdm::query_pass_kernel"]
    assert "| bwd | 2 | 71.0 |" in lines["based::swab::swa_bwd_mfma_kernel<4>"]
    assert "|  | 1 | 5.0 |" in lines["based::decode_step_kernel<unsigned short, 64, 273>"]


def test_traffic_is_null_once_the_sources_change(tmp_path, monkeypatch):
    rec = {"bytes_per_call": 123.0, "source_hash": "not-the-current-sources"}
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "traffic_layer.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_hash", lambda op: "current")
    assert bench.load_traffic("layer") is None
    rec["source_hash"] = "current"
    (tmp_path / "profiles" / "traffic_layer.json").write_text(json.dumps(rec))
    assert bench.load_traffic("layer") == 123.0
