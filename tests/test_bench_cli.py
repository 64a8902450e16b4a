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


def _write_csv(path, counter, kernels, copy_kib):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        w.writerow({"Kernel_Name": "at::native::vectorized_elementwise_kernel<FillFunctor>",
                    "Counter_Name": counter, "Counter_Value": 3 * copy_kib})
        w.writerow({"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": counter,
                    "Counter_Value": copy_kib})
        for name, vals in kernels.items():
            for v in vals:
                w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})


def _read(path):
    vals = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    return vals


def test_counter_summary_scales_by_the_copy_probe(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench

    fetch, wr = tmp_path / "f.csv", tmp_path / "w.csv"
    mib = bench.COPY_PROBE_MIB
    dec = "decode_bsr_kernel<2, 128, 4>(DecodeParams)"
    # FETCH reads half the copied bytes (scale 2), WRITE all of them (scale 1);
    # a bigger fill kernel in the same run is not taken for the copy
    _write_csv(fetch, "FETCH_SIZE", {dec: [1000.0, 1002.0]}, mib * 1024 / 2)
    _write_csv(wr, "WRITE_SIZE", {dec: [10.0]}, mib * 1024)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    bench.summarize_counters(str(fetch), str(wr), "unit")
    path = tmp_path / "profiles" / "decode_bsr_counters_unit.txt"
    vals = _read(path)
    assert abs(float(vals["fetch_scale"]) - 2.0) < 1e-9
    # the file keeps six significant digits
    assert abs(float(vals["scaled_fetch_bytes_per_step"]) / (1001.0 * 1024 * 2) - 1) < 1e-5
    assert abs(float(vals["scaled_write_bytes_per_step"]) / (10.0 * 1024) - 1) < 1e-5
    assert vals["source_sha256_16"] == bench.source_digest(["decode_bsr_kernel"])
    # read back as the traffic of a step while the source is unchanged
    t = bench.read_traffic("unit", ["decode_bsr_kernel"])
    assert abs(t / (1001.0 * 1024 * 2 + 10.0 * 1024) - 1) < 1e-5


def test_counter_summary_sums_the_kernels_of_a_step(tmp_path, monkeypatch):
    """A shared-prefix step launches the tile kernel and the decode kernel:
    the traffic of the step is the sum of both kernels' per-launch means."""
    sys.path.insert(0, ROOT)
    import bench

    fetch, wr = tmp_path / "f.csv", tmp_path / "w.csv"
    mib = bench.COPY_PROBE_MIB
    ks = {"tile_attend_kernel<128, false>(TileParams)": [300.0, 310.0],
          "decode_bsr_kernel<2, 128, 4>(DecodeParams)": [100.0, 100.0]}
    _write_csv(fetch, "FETCH_SIZE", ks, mib * 1024)
    _write_csv(wr, "WRITE_SIZE", {k: [1.0, 3.0] for k in ks}, mib * 1024)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    bench.summarize_counters(str(fetch), str(wr), "unit")
    kernels = ["tile_attend_kernel", "decode_bsr_kernel"]
    vals = _read(tmp_path / "profiles" / "tile_attend_decode_bsr_counters_unit.txt")
    assert abs(float(vals["tile_attend_scaled_fetch_bytes_per_launch"]) / (305.0 * 1024) - 1) < 1e-5
    assert abs(float(vals["scaled_fetch_bytes_per_step"]) / (405.0 * 1024) - 1) < 1e-5
    assert abs(float(vals["scaled_write_bytes_per_step"]) / (4.0 * 1024) - 1) < 1e-5
    assert vals["source_sha256_16"] == bench.source_digest(kernels)
    assert bench.read_traffic("unit", kernels) is not None
    assert bench.read_traffic("unit", ["decode_bsr_kernel"]) is None  # no such summary


def test_source_digest_follows_code_not_comments():
    """The profiles record a digest of the kernel sources they were measured
    with: comments and layout do not enter it, code does, and the repository
    headers a source includes are part of it."""
    sys.path.insert(0, ROOT)
    import bench
    code = 'int f(int x) {\n  return x + 1;  // add one\n}\n/* end */ const char* s = "a // b";\n'
    assert bench._code_only(code) == bench._code_only(code.replace("add one", "plus 1")
                                                      .replace("\n", "\n\n  "))
    assert bench._code_only(code) != bench._code_only(code.replace("x + 1", "x + 2"))
    assert bench._code_only(code) != bench._code_only(code.replace('"a // b"', '"a // c"'))
    files = [os.path.basename(f) for f in bench._with_headers("attn_tile.hip")]
    assert files[0] == "attn_tile.hip" and "coherent.h" in files and "fi_bsr.h" in files
