"""Host-side arithmetic of bench.py (CPU): HBM bytes per launch from rocprofv3 counter CSVs,
scaled by a copy kernel of known size; the source-digest guard that drops counters taken on
other kernel sources; MFMA/VALU utilisation medians; the one-GPU refusal."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

COUNTER_FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
COPY_KERNEL = "void at::native::elementwise_kernel<MulFunctor<unsigned char>>(int)"
DRAFT_KERNEL = "void mtp::mtp_draft_head_kernel<3, false, 4>(mtp::LmheadLaunch)"
VERIFY_KERNEL = "void mtp::mtp_verify_logits_kernel<3, false>(mtp::LmheadLaunch)"


def _write_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COUNTER_FIELDS)
        w.writeheader()
        for i, (kernel, kib) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": kib})


@pytest.fixture
def tmp_profiles(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    monkeypatch.setattr(bench, "UTIL_FILE", str(tmp_path / "util.json"))
    return tmp_path


def test_counter_bytes_are_scaled_by_the_copy_kernel(tmp_profiles):
    copy_kib = bench.COPY_BYTES / 1024
    # a counter that reads half the bytes (FETCH_SIZE on this part) and one that is exact
    _write_csv(tmp_profiles / "fetch.csv", "FETCH_SIZE",
               [(COPY_KERNEL, copy_kib / 2), (DRAFT_KERNEL, 1000.0), (DRAFT_KERNEL, 1002.0), (DRAFT_KERNEL, 1004.0),
                (VERIFY_KERNEL, 4000.0)])
    _write_csv(tmp_profiles / "write.csv", "WRITE_SIZE",
               [(COPY_KERNEL, copy_kib), (DRAFT_KERNEL, 10.0), (DRAFT_KERNEL, 10.0), (DRAFT_KERNEL, 10.0),
                (VERIFY_KERNEL, 20.0)])
    bench.summarize_counters([("wl", str(tmp_profiles / "fetch.csv"), str(tmp_profiles / "write.csv"))])
    t = json.load(open(bench.TRAFFIC_FILE))
    w = t["workloads"]["wl"]
    assert w["fetch_scale"] == pytest.approx(2.0) and w["write_scale"] == pytest.approx(1.0)
    d = w["kernels"]["mtp_draft_head_kernel"]
    # median of the launches, KiB -> bytes, times the scale
    assert d["fetch_bytes"] == int(1002.0 * 1024 * 2.0) and d["write_bytes"] == int(10.0 * 1024)
    assert d["bytes_per_launch"] == d["fetch_bytes"] + d["write_bytes"] and d["launches"] == 3
    assert w["kernels"]["mtp_verify_logits_kernel"]["fetch_bytes"] == int(4000.0 * 1024 * 2.0)
    # served while the digest matches the kernel sources, dropped once they change
    assert bench.load_traffic("wl", "mtp_draft_head_kernel") == d["bytes_per_launch"]
    assert bench.load_traffic("other", "mtp_draft_head_kernel") is None
    t["source_digest"] = "0" * 16
    json.dump(t, open(bench.TRAFFIC_FILE, "w"))
    assert bench.load_traffic("wl", "mtp_draft_head_kernel") is None


def test_counter_summary_needs_the_copy_kernel(tmp_profiles):
    _write_csv(tmp_profiles / "fetch.csv", "FETCH_SIZE", [(DRAFT_KERNEL, 1000.0)])
    _write_csv(tmp_profiles / "write.csv", "WRITE_SIZE", [(DRAFT_KERNEL, 10.0)])
    with pytest.raises(SystemExit):
        bench.summarize_counters([("wl", str(tmp_profiles / "fetch.csv"), str(tmp_profiles / "write.csv"))])


def test_utilisation_medians_and_digest_guard(tmp_profiles):
    path = tmp_profiles / "util.csv"
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COUNTER_FIELDS)
        w.writeheader()
        for i, (mfma, valu) in enumerate([(20.0, 10.0), (24.0, 30.0), (30.0, 20.0)]):
            for name, v in (("MfmaUtil", mfma), ("VALUBusy", valu), ("MfmaFlopsBF16", 1e9 * (i + 1))):
                w.writerow({"Dispatch_Id": i, "Kernel_Name": VERIFY_KERNEL, "Counter_Name": name, "Counter_Value": v})
    bench.summarize_utilisation([("wl", str(path))])
    u = bench.load_utilisation("wl", "mtp_verify_logits_kernel")
    assert u == {"mfma_busy_pct": 24.0, "valu_busy_pct": 20.0, "mfma_bf16_flops": 2000000000, "launches": 3}
    t = json.load(open(bench.UTIL_FILE))
    t["source_digest"] = "0" * 16
    json.dump(t, open(bench.UTIL_FILE, "w"))
    assert bench.load_utilisation("wl", "mtp_verify_logits_kernel") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert json.loads(r.stdout.strip().splitlines()[-1])["n_gpus"] == 2
