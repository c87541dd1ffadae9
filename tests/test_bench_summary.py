"""bench.py's rocprofv3 summarizer on small synthetic CSV files (no GPU): the copy calibration
scales FETCH_SIZE / WRITE_SIZE, kernel averages use the timed dispatches only (the warm-up
ones are dropped), the per-call traffic adds the call's kernels, and the record ties itself to
the kernel sources by SHA-256 so that bench.py drops it once a source changes."""
import csv
import hashlib
import json
import os

import pytest

import bench

WARM = int(bench.PROFILE_STEPS.split("--warmup ")[1].split()[0])
STEPS = int(bench.PROFILE_STEPS.split("--steps ")[1].split()[0])
KNAME = "void bsr::attn_decode_bf16_kernel<128, false, false, true>(bsr::RunArgs)"
PNAME = "(anonymous namespace)::read_pages_kernel(unsigned int const*, int)"
COPY = "__amd_rocclr_copyBuffer"


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def _fake_run(raw, name):
    d = os.path.join(raw, name)
    for tag in ("trace", "fetch", "write"):
        os.makedirs(d + "_" + tag)
    # trace: warm-up dispatches at 300 us, timed ones at 200 us (attention) and 150 us (probe)
    disp, did = [], 0
    for call in range(WARM + STEPS):
        for kname, us in ((KNAME, 300.0 if call < WARM else 200.0), (PNAME, 150.0)):
            did += 1
            disp.append(["KERNEL_DISPATCH", did, kname, 1000 * did * 10, 1000 * did * 10 + int(us * 1000)])
    _write(os.path.join(d + "_trace", "run_kernel_trace.csv"),
           ["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"], disp)
    n = WARM + STEPS
    avg = (WARM * 300.0 + STEPS * 200.0) / n
    _write(os.path.join(d + "_trace", "run_kernel_stats.csv"), ["Name", "Calls", "AverageNs", "MinNs", "MaxNs"],
           [[KNAME, n, avg * 1000, 200000, 300000], [PNAME, n, 150000, 150000, 150000]])
    # counters: three 512 MiB copies first (FETCH_SIZE reads half the bytes), then the kernels,
    # each dispatch's value split over two rows (per-XCD instances are summed)
    for tag, counter, copy_kib, k_kib, p_kib in (("fetch", "FETCH_SIZE", 262144.0, 500000.0, 400000.0),
                                                 ("write", "WRITE_SIZE", 524288.0, 1000.0, 0.0)):
        rows, did = [], 0
        for _ in range(3):
            did += 1
            rows += [[did, COPY, counter, copy_kib / 2], [did, COPY, counter, copy_kib / 2]]
        for _ in range(n):
            for kname, v in ((KNAME, k_kib), (PNAME, p_kib)):
                did += 1
                rows += [[did, kname, counter, v / 2], [did, kname, counter, v / 2]]
        _write(os.path.join(d + "_" + tag, "run_counter_collection.csv"),
               ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], rows)
    json.dump({"event_timed_us_per_call": 201.5}, open(d + "_event.json", "w"))


def test_summary_of_a_decode_profile(tmp_path, monkeypatch):
    raw, out = str(tmp_path / "raw"), str(tmp_path / "out")
    os.makedirs(out)
    _fake_run(raw, "decode_batch64")
    monkeypatch.setattr(bench, "profile_case_batch", lambda name: None)
    monkeypatch.setattr(bench, "profile_algorithmic", lambda name, b: 1_000_000_000)
    rec = bench.summarize_profile("decode_batch64", raw_dir=raw, out_dir=out)
    assert rec["kernel_avg_us"]["attn_decode_bf16_kernel"] == 200.0  # warm-up dispatches dropped
    assert rec["kernel_avg_us_all_dispatches"]["attn_decode_bf16_kernel"] == round((WARM * 300 + STEPS * 200)
                                                                                   / (WARM + STEPS), 2)
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["traffic_bytes_per_call"] == (500000 * 2 + 1000) * 1024  # the call is the attention kernel
    assert rec["traffic_over_algorithmic"] == round((500000 * 2 + 1000) * 1024 / 1e9, 4)
    assert rec["read_probe_gbs"] == round(400000 * 2 * 1024 / 150e-6 / 1e9, 1)
    assert rec["event_timed_us_per_call"] == 201.5
    for src, sha in rec["sources"].items():
        assert sha == hashlib.sha256(open(os.path.join(bench.ROOT, src), "rb").read()).hexdigest()
    assert rec["commands"] == bench.profile_commands("decode_batch64")
    md = open(os.path.join(out, "decode_batch64.md")).read()
    assert all(c in md for c in rec["commands"])


def test_missing_copy_calibration_is_an_error(tmp_path, monkeypatch):
    raw, out = str(tmp_path / "raw"), str(tmp_path / "out")
    os.makedirs(out)
    _fake_run(raw, "decode_batch64")
    path = os.path.join(raw, "decode_batch64_fetch", "run_counter_collection.csv")
    rows = [r for r in csv.reader(open(path))]
    _write(path, rows[0], [r for r in rows[1:] if r[1] != COPY])
    monkeypatch.setattr(bench, "profile_case_batch", lambda name: None)
    monkeypatch.setattr(bench, "profile_algorithmic", lambda name, b: 1)
    with pytest.raises(AssertionError, match="calibration"):
        bench.summarize_profile("decode_batch64", raw_dir=raw, out_dir=out)


def test_profile_commands_run_committed_files_only():
    for name in bench.PROFILE_CASES:
        for c in bench.profile_commands(name):
            assert c.startswith("timeout -s KILL ") and " rocprofv3 " in c
            prog = c.split(" -- ", 1)[1]
            assert prog.startswith("python3 bench.py --profile-case " + name)
            assert "_work" not in c
