"""bench.py's command line on a CPU-only host: more than one GPU is refused
with a message and exit status 2 before anything touches a device, and the
counter summary turns rocprofv3 --pmc output into the committed file format
(checked on a synthetic CSV, written to a temporary copy)."""
import csv
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2, r.stdout + r.stderr
    assert "one GPU" in r.stdout


def test_counter_summary_scales_by_the_copy_probe(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench

    def write(path, counter, decode_kib, copy_kib):
        with open(path, "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
            w.writeheader()
            w.writerow({"Kernel_Name": "at::native::elementwise copy", "Counter_Name": counter,
                        "Counter_Value": copy_kib})
            for v in decode_kib:
                w.writerow({"Kernel_Name": "decode_bsr_kernel<2, 128, 4>", "Counter_Name": counter,
                            "Counter_Value": v})

    fetch, wr = tmp_path / "f.csv", tmp_path / "w.csv"
    mib = bench.COPY_PROBE_MIB
    # FETCH reads half the copied bytes (scale 2), WRITE all of them (scale 1)
    write(fetch, "FETCH_SIZE", [1000.0, 1002.0], mib * 1024 / 2)
    write(wr, "WRITE_SIZE", [10.0], mib * 1024)
    monkeypatch.setattr(bench, "counters_file", lambda name: str(tmp_path / f"{name}.txt"))
    bench.summarize_counters(str(fetch), str(wr), "unit")
    vals = {}
    for line in open(tmp_path / "unit.txt"):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    assert abs(float(vals["fetch_scale"]) - 2.0) < 1e-9
    # the file keeps six significant digits
    assert abs(float(vals["scaled_fetch_bytes_per_launch"]) / (1001.0 * 1024 * 2) - 1) < 1e-5
    assert abs(float(vals["scaled_write_bytes_per_launch"]) / (10.0 * 1024) - 1) < 1e-5
    assert vals["decode_source_sha256_16"] == bench.source_digest()
