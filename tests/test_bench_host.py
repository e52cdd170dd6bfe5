"""Host logic of the benchmark, on the CPU: the one-GPU rule, the scaling of
the HBM byte counters by the probe copy kernel's own reading, and the gate
that reports stored counter traffic only while the dominant kernel's sources
are unchanged."""
import csv
import os
import subprocess
import sys

import bench


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _csv(path, fields, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(r)


COPY = "ckks::(anonymous namespace)::copy_kernel(HIP_vector_type<unsigned long long, 2u> const*)"
KERN = "void ckks::(anonymous namespace)::some_kernel(ckks::Args)"


def test_summarize_counters_scales_by_the_copy_kernel(tmp_path):
    _csv(str(tmp_path / "trace" / "t_kernel_stats.csv"), ["Name", "Calls", "AverageNs"],
         [{"Name": COPY, "Calls": 16, "AverageNs": 350000.0}, {"Name": KERN, "Calls": 2, "AverageNs": 10000.0}])
    rows = []
    # the copy of 1 GiB: FETCH_SIZE counts half its bytes, WRITE_SIZE all of them (KiB)
    for d in (1, 2):
        rows.append({"Kernel_Name": COPY, "Counter_Name": "FETCH_SIZE", "Dispatch_Id": d, "Counter_Value": 524288.0})
    # the kernel: two dispatches of 1000 and 3000 KiB (two XCD rows each), averaged per dispatch
    for d, v in ((3, 1000.0), (4, 3000.0)):
        rows.append({"Kernel_Name": KERN, "Counter_Name": "FETCH_SIZE", "Dispatch_Id": d, "Counter_Value": v / 2})
        rows.append({"Kernel_Name": KERN, "Counter_Name": "FETCH_SIZE", "Dispatch_Id": d, "Counter_Value": v / 2})
    _csv(str(tmp_path / "fetch" / "x_counter_collection.csv"),
         ["Kernel_Name", "Counter_Name", "Dispatch_Id", "Counter_Value"], rows)
    rows = [{"Kernel_Name": COPY, "Counter_Name": "WRITE_SIZE", "Dispatch_Id": 1, "Counter_Value": 1048576.0},
            {"Kernel_Name": KERN, "Counter_Name": "WRITE_SIZE", "Dispatch_Id": 3, "Counter_Value": 500.0}]
    _csv(str(tmp_path / "write" / "x_counter_collection.csv"),
         ["Kernel_Name", "Counter_Name", "Dispatch_Id", "Counter_Value"], rows)
    out = bench.summarize_counters(str(tmp_path))
    assert "FETCH_SIZE scale 2.0000, WRITE_SIZE scale 1.0000" in out
    row = next(line for line in out.splitlines() if "some_kernel" in line)
    cells = [c.strip() for c in row.strip("|").split("|")]
    # read: 2000 KiB average x 2 x 1024 B = 4.096 MB; written: 500 KiB = 0.512 MB
    assert cells[-2] == "4.1" and cells[-1] == "0.5"
    assert cells[1] == "2" and cells[2] == "10.0"


def test_stored_traffic_is_gated_by_the_source_hash(tmp_path, monkeypatch):
    path = tmp_path / "traffic.txt"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.measured_traffic() is None  # no file
    body = "# comment: 1\nfetch_bytes_per_launch: 1000\nwrite_bytes_per_launch: 24\n"
    path.write_text("sources_sha256: %s\n" % bench.kernel_sources_sha256() + body)
    assert bench.measured_traffic() == 1024
    path.write_text("sources_sha256: %s\n" % ("0" * 64) + body)
    assert bench.measured_traffic() is None  # the kernel changed since the counters were taken
