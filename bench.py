"""Benchmark: skewed-batch paged GQA decode on one MI355X.

One step = one pass of the decode hot path over one batch: fi_decode_run, a
single kernel launch that attends over the planner's work items and folds the
partial states of cut requests up their merge trees, with the plan built once
per batch and uploaded before timing (a serving engine reuses one plan for every layer of a
decode step; the host planner's own time is reported beside it). Inputs are
resident in HBM. Before every timed step L2 and the 256 MB Infinity Cache
are flushed (a 1 GiB write, then a 1 GiB read of another buffer, so no dirty
line is left for the step to write back), outside the timed events.

Prints one JSON line: achieved HBM GB/s over the algorithmic bytes (active K
and V once per KV head + q read + output written) and microseconds per batch,
both from the median step (HIP events on the launch stream around each call),
the decode kernel's roofline fraction against 8 TB/s, and the float64 CPU
oracle timed on the host on the same workload.

    python bench.py [--steps K] [--warmup W] [--config 3]
    python bench.py --config 7|8|12     # prefill / append: TFLOP/s on matrix cores
    python bench.py --config 15         # latent attention (MLA) decode: HBM GB/s
    python bench.py --summarize-counters FETCH.csv WRITE.csv   # rocprofv3 --pmc output
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "achieved HBM GB/s (% of MI355X peak) + µs/batch, skewed-batch paged GQA decode"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0  # dense bf16 matrix-core peak
CSRC = os.path.join(ROOT, "block_sparse_kv_bsr_amd", "csrc")
COPY_PROBE_MIB = 1024
# the library kernels a step can launch, the source each is built from, and
# the short name counter summaries use
KERNELS = {"tile_attend_kernel": ("attn_tile.hip", "tile_attend"),
           "decode_bsr_kernel": ("decode_bsr.hip", "decode_bsr"),
           "decode_mma_kernel": ("decode_mma.hip", "decode_mma"),
           "mla_attend_kernel": ("mla_attend.hip", "mla_attend")}


def _with_headers(src: str) -> list:
    """src and every header of this repository it includes, directly or not
    (paths under csrc/ or include/), in a fixed order."""
    seen, todo = [], [os.path.join(CSRC, src)]
    while todo:
        path = todo.pop(0)
        if path in seen:
            continue
        seen.append(path)
        with open(path) as f:
            for ln in f:
                m = re.match(r'\s*#\s*include\s+"([^"]+)"', ln)
                if not m:
                    continue
                for d in (CSRC, os.path.join(ROOT, "include")):
                    cand = os.path.join(d, m.group(1))
                    if os.path.exists(cand):
                        todo.append(cand)
                        break
    return seen


def _code_only(text: str) -> str:
    """C/C++ source without its comments and with runs of white space
    collapsed: edits to comments and layout leave the digest unchanged."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c == '"' or c == "'":  # a literal, kept whole
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            i = text.find("\n", i)
            i = n if i < 0 else i
        elif text.startswith("/*", i):
            i = text.find("*/", i + 2)
            i = n if i < 0 else i + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_digest(kernels=("decode_bsr_kernel",)) -> str:
    """sha256 (16 hex digits) of the code (comments and layout aside) of the
    sources the given kernels are built from, with the repository headers
    they include."""
    h = hashlib.sha256()
    files = []
    for src in sorted({KERNELS[k][0] for k in kernels}):
        files += [f for f in _with_headers(src) if f not in files]
    for path in files:
        with open(path, encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def counters_file(workload_name: str, kernels=("decode_bsr_kernel",)) -> str:
    tag = "_".join(KERNELS[k][1] for k in kernels)
    return os.path.join(ROOT, "profiles", f"{tag}_counters_{workload_name}.txt")


def read_traffic(workload_name: str, kernels=("decode_bsr_kernel",)):
    """HBM bytes per step (FETCH + WRITE of every kernel of the step) from the
    committed counter summary, or None when there is none or a kernel's
    source changed since."""
    path = counters_file(workload_name, kernels)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256_16") != source_digest(kernels):
        return None
    try:
        return float(vals["scaled_fetch_bytes_per_step"]) + float(vals["scaled_write_bytes_per_step"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------- counters
def _pmc_rows(path, counter):
    import csv
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") == counter:
                rows.append((r.get("Kernel_Name", ""), float(r["Counter_Value"])))
    return rows


def summarize_counters(fetch_csv, write_csv, workload_name):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per
    dispatch) into bytes per launch of each library kernel found, scaled by
    what the same counter reads for a plain copy of COPY_PROBE_MIB MiB in the
    same program, and their sum per step (a step launches each once)."""
    out, kernels = {}, None
    for name, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        rows = _pmc_rows(path, counter)
        found = [k for k in KERNELS if any(k in kn for kn, _ in rows)]
        kernels = found if kernels is None else kernels
        if not found or found != kernels:
            raise SystemExit(f"{path}: library kernels {found} (expected {kernels})")
        cpy = [v for kn, v in rows if "copy" in kn.lower()]
        if not cpy:
            raise SystemExit(f"{path}: no copy dispatch with {counter}")
        probe = max(cpy)
        scale = COPY_PROBE_MIB * 1024.0 / probe
        out[f"{name}_copy_probe_kib"] = probe
        out[f"{name}_scale"] = scale
        total = 0.0
        for k in kernels:
            vals = [v for kn, v in rows if k in kn]
            short = KERNELS[k][1]
            out[f"{short}_{name}_kib_raw_mean"] = statistics.mean(vals)
            out[f"{short}_{name}_dispatches"] = len(vals)
            per = statistics.mean(vals) * 1024.0 * scale
            out[f"{short}_scaled_{name}_bytes_per_launch"] = per
            total += per
        out[f"scaled_{name}_bytes_per_step"] = total
    path = counters_file(workload_name, kernels)
    with open(path, "w") as f:
        f.write(f"# HBM traffic of {' + '.join(kernels)}, workload {workload_name}\n")
        f.write(f"# from: cd /tmp && TMPDIR=/tmp rocprofv3 --pmc FETCH_SIZE --output-format csv "
                f"-d <dir> -o pmc -- python $REPO/bench.py --config <id> --counters-run "
                f"--no-cpu-baseline\n")
        f.write(f"#  and: the same with --pmc WRITE_SIZE; then python bench.py --config <id> "
                f"--summarize-counters <fetch csv> <write csv>\n")
        f.write(f"# each counter scaled by (known bytes / counter) of a {COPY_PROBE_MIB} MiB copy\n")
        f.write(f"source_sha256_16 = {source_digest(kernels)}\n")
        for k, v in out.items():
            f.write(f"{k} = {v:.6g}\n")
    print(open(path).read())


# $REPO is the repository root, $OUT any directory for the profiler's output
TRACE_COMMAND = ("cd /tmp && TMPDIR=/tmp rocprofv3 --kernel-trace --stats --output-format csv "
                 "-d $OUT/trace_{cfg} -o trace -- python $REPO/bench.py --config {cfg} "
                 "--steps 20 --warmup 5 --no-cpu-baseline")


def summarize_trace(stats_csv, bench_log, w, config_id):
    """Write profiles/<kernels>_<workload>.md from a rocprofv3 --stats
    kernel summary and the bench line printed by the same traced run."""
    import csv
    line = [ln for ln in open(bench_log).read().splitlines() if ln.startswith("{")][-1]
    res = json.loads(line)
    kernels = res["roofline"]["kernel"].split(" + ")
    rows = []
    with open(stats_csv) as f:
        for r in csv.DictReader(f):
            rows.append((r["Name"], int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                         float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3,
                         float(r["Percentage"])))
    rows.sort(key=lambda x: -x[5])
    lib = {k: next((r for r in rows if k in r[0]), None) for k in kernels}
    missing = [k for k, r in lib.items() if r is None]
    if missing:
        raise SystemExit(f"{stats_csv}: no dispatch of {missing}")
    tag = "_".join(KERNELS[k][1] for k in kernels)
    path = os.path.join(ROOT, "profiles", f"{tag}_{w.name}.md")
    mla = hasattr(w, "num_heads")
    prefill = hasattr(w, "qo_indptr") and not mla
    kern_us = sum(r[2] for r in lib.values())
    ev_us = res["us_per_batch"]
    o = []
    o.append(f"# {' + '.join(kernels)} — {w.name}\n")
    tok = (w.total_kv_lens() if hasattr(w, "prefix_of") else w.kv_lens()).sum()
    if mla:
        desc = (f"batch {w.batch}, {int(tok):,} cached tokens (latent 512 + rotary key 64, "
                f"bf16), {w.num_heads} query heads, {w.num_qo_tokens} query token(s), page "
                f"size {w.page_size}; algorithmic work {w.flops():,} flop")
    else:
        desc = (f"batch {w.batch}, {int(tok):,} KV tokens, {w.num_qo_heads} query / "
                f"{w.num_kv_heads} KV heads, head_dim {w.head_dim}, page size {w.page_size}, "
                f"K/V {w.dtype}")
    if prefill:
        desc += f", {w.num_qo_tokens:,} query tokens ({'causal' if w.causal else 'unmasked'})"
    if getattr(w, "rope_theta", 0):
        desc += f", rotary embedding (theta {w.rope_theta:g}) applied to K in the kernel"
    if hasattr(w, "prefix_of"):
        desc += (f", the shared prefix held once in a second cache of {w.prefix_page_size}-token "
                 f"blocks")
    o.append(f"Workload (config {config_id}): {desc}.")
    if prefill:
        o.append(f"Algorithmic work per batch: {w.flops():,} flop "
                 f"(4 x head_dim x query heads per attended (query, token) pair).\n")
    elif mla:
        o.append(f"Algorithmic bytes per batch: {w.algorithmic_bytes():,} (every cached latent "
                 f"and rotary key once + q + output).\n")
    else:
        o.append(f"Algorithmic bytes per batch: {w.algorithmic_bytes():,} (K+V of every active "
                 f"token once per KV head + q + output).\n")
    o.append("Command (one MI355X; $REPO is the repository root, $OUT any output directory):\n")
    o.append("    " + TRACE_COMMAND.format(cfg=config_id) + "\n")
    o.append("`--stats` kernel summary, durations in microseconds:\n")
    o.append("| kernel | calls | avg | min | max | % of GPU time |")
    o.append("|---|---|---|---|---|---|")
    for n, c, a, mn, mx, pc in rows[:8]:
        o.append(f"| {n[:90]} | {c} | {a:.2f} | {mn:.2f} | {mx:.2f} | {pc:.2f} |")
    o.append("")
    o.append("The 1 GiB fill and the 1 GiB sum reduction are bench.py's L2/MALL flush "
             "before each step (outside the timed events); the streaming-read kernel measures "
             "the practical ceiling; the remaining torch kernels generate inputs.\n")
    parts = " + ".join(f"{k} {lib[k][2]:.2f}" for k in kernels)
    o.append(f"Library kernels per step (rocprofv3 averages): {parts} = {kern_us:.2f} us; "
             f"bench.py in the same run, HIP events around each step: median {ev_us} us "
             f"(p10-p90 {res['us_per_batch_p10_p90']}).")
    if prefill:
        tf_k = w.flops() / (kern_us * 1e-6) / 1e12
        o.append(f"Achieved: {tf_k:.1f} TFLOP/s ({100 * tf_k / PEAK_BF16_TFLOPS:.1f}% of the "
                 f"2.5 PFLOP/s bf16 dense peak) by the kernels' own durations; "
                 f"{res['value']} TFLOP/s ({100 * res['roofline']['frac']:.1f}%) by the events.")
    else:
        gb_k = w.algorithmic_bytes() / (kern_us * 1e-6) / 1e9
        o.append(f"Achieved: {gb_k / 1e3:.2f} TB/s ({100 * gb_k / PEAK_HBM_GBS:.1f}% of 8 TB/s) by "
                 f"the kernels' own durations; {res['value'] / 1e3:.2f} TB/s "
                 f"({100 * res['roofline']['frac']:.1f}%) by the events.")
        if mla:
            tf_k = w.flops() / (kern_us * 1e-6) / 1e12
            o.append(f"Matrix-core rate: {tf_k:.1f} TFLOP/s algorithmic "
                     f"({100 * tf_k / PEAK_BF16_TFLOPS:.1f}% of 2.5 PFLOP/s) by the kernels' "
                     f"durations.")
        if "practical_ceiling" in res:
            pc = res["practical_ceiling"]
            o.append(f"Streaming-read ceiling measured in the same run: {pc['gbs'] / 1e3:.2f} TB/s "
                     f"(the events figure is {100 * pc['frac']:.1f}% of it).")
    cf = counters_file(w.name, kernels)
    if os.path.exists(cf):
        vals = {}
        for ln in open(cf):
            if "=" in ln and not ln.startswith("#"):
                k, v = ln.split("=", 1)
                vals[k.strip()] = v.strip()
        if vals.get("source_sha256_16") == source_digest(kernels):
            fb_ = float(vals["scaled_fetch_bytes_per_step"])
            wb_ = float(vals["scaled_write_bytes_per_step"])
            alg = w.algorithmic_bytes()
            o.append(f"\nHBM traffic per step ({os.path.basename(cf)}, sources "
                     f"{vals['source_sha256_16']}): FETCH {fb_:.4g} B, WRITE {wb_:.4g} B; "
                     f"together {(fb_ + wb_) / alg:.3f}x the algorithmic bytes ("
                     + ("reads of the latents, rotary keys and q plus writes of the output"
                        if mla else "reads of K, V and q plus writes of the output") + ").")
    o.append(f"\nKernel sources sha256[:16]: {source_digest(kernels)}.")
    with open(path, "w") as f:
        f.write("\n".join(o) + "\n")
    print(open(path).read())


# ------------------------------------------------------- streaming ceiling
def stream_ceiling(dev, flush, nbytes=2 << 30, reps=5):
    """The box's practical HBM read rate: libfi_bench.so's streaming-read
    kernel (16-byte nontemporal loads) over 2 GiB, L2/MALL flushed before
    each pass, HIP events on the stream it runs on; median of `reps`."""
    import ctypes
    import torch
    L = ctypes.CDLL(os.path.join(ROOT, "block_sparse_kv_bsr_amd", "libfi_bench.so"))
    L.fi_bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                       ctypes.c_void_p]
    L.fi_bench_stream_read.restype = ctypes.c_int
    buf = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    ms = []
    for i in range(reps + 1):
        flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        rc = L.fi_bench_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), stream.cuda_stream)
        e1.record()
        if rc != 0:
            raise RuntimeError(f"fi_bench_stream_read failed: hipError {rc}")
        torch.cuda.synchronize()
        if i:  # the first pass warms the code object
            ms.append(e0.elapsed_time(e1))
    del buf
    return nbytes / (statistics.median(ms) * 1e-3) / 1e9


# ------------------------------------------------------------------ oracle
def _one_thread():
    """A context holding numpy's BLAS to one thread, and the thread count
    the oracle then uses. The oracle's products (one request and KV head at a
    time) are too small for BLAS threads to pay off: on a 16-thread host the
    default of 16 BLAS threads ran slower than one thread."""
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=1), 1
    except Exception:  # threadpoolctl missing: numpy's default threads
        import contextlib
        return contextlib.nullcontext(), os.cpu_count() or 1


def cpu_baseline(w, q, k, v, min_seconds=10.0, max_passes=3, kp_vp=None):
    """Time the float64 oracle on the host over whole batches of the same
    workload (inputs copied to host memory first, not timed), on one thread."""
    import torch
    sys.path.insert(0, ROOT)
    import oracle.attention as oa
    qh = q.float().cpu().numpy()
    if w.dtype == "fp8":  # the oracle attends over the dequantised cache
        kh = oa.dequantize_e4m3(k.view(torch.uint8).cpu().numpy(), w.k_scale)
        vh = oa.dequantize_e4m3(v.view(torch.uint8).cpu().numpy(), w.v_scale)
    else:
        kh, vh = k.float().cpu().numpy(), v.float().cpu().numpy()

    composed = hasattr(w, "prefix_of")
    if composed:
        kph, vph = kp_vp[0].float().cpu().numpy(), kp_vp[1].float().cpu().numpy()

    def run():
        if composed:
            oa.decode_attention_composed(qh, kh, vh, w.kv_indptr, w.kv_indices, w.last_page_len,
                                         kph, vph, w.prefix_indptr, w.prefix_indices,
                                         w.prefix_last_page_len, w.prefix_of, w.sm_scale)
        elif w.rope_theta:
            oa.decode_attention_rope(qh, kh, vh, w.kv_indptr, w.kv_indices, w.last_page_len,
                                     w.sm_scale, w.rope_theta, w.rope_scale)
        else:
            oa.decode_attention(qh, kh, vh, w.kv_indptr, w.kv_indices, w.last_page_len, w.sm_scale)

    ctx, threads = _one_thread()
    times = []
    with ctx:
        while len(times) < max_passes and sum(times) < min_seconds:
            t0 = time.perf_counter()
            run()
            times.append(time.perf_counter() - t0)
    per = statistics.median(times)
    tot_tokens = (w.total_kv_lens() if composed else w.kv_lens()).sum()
    return {"value": w.algorithmic_bytes() / per / 1e9, "unit": "GB/s", "cores": threads,
            "kind": "oracle", "seconds_per_batch": per,
            "sample": f"whole {w.name} batch ({int(tot_tokens)} KV tokens), "
                      f"{len(times)} pass(es), median; numpy float64, BLAS held to "
                      f"{threads} host thread(s)"}


def cpu_baseline_prefill(w, q, k, v, min_seconds=10.0):
    """Time the float64 prefill oracle on the host over whole requests of the
    workload, one after another, until min_seconds have passed; report its
    rate in the benchmark's unit (algorithmic TFLOP/s)."""
    import numpy as np
    sys.path.insert(0, ROOT)
    import oracle.attention as oa
    ctx, threads = _one_thread()
    if w.dtype == "fp8":  # the oracle attends over the dequantised cache
        import torch
        kh = oa.dequantize_e4m3(k.view(torch.uint8).cpu().numpy(), w.k_scale)
        vh = oa.dequantize_e4m3(v.view(torch.uint8).cpu().numpy(), w.v_scale)
    else:
        kh, vh = k.float().cpu().numpy(), v.float().cpu().numpy()
    qo = w.qo_indptr
    L = w.kv_lens()
    flops = 0
    spent = 0.0
    done = 0
    with ctx:
        for b in range(w.batch):
            n = int(qo[b + 1] - qo[b])
            if n == 0:
                continue
            qh = q[int(qo[b]):int(qo[b + 1])].float().cpu().numpy()
            ip = np.array([0, w.kv_indptr[b + 1] - w.kv_indptr[b]], dtype=np.int64)
            ix = w.kv_indices[w.kv_indptr[b]:w.kv_indptr[b + 1]]
            t0 = time.perf_counter()
            if w.rope_theta:
                oa.prefill_attention_rope(qh, kh, vh, np.array([0, n]), ip, ix,
                                          w.last_page_len[b:b + 1], w.causal, w.sm_scale,
                                          w.rope_theta, w.rope_scale)
            else:
                oa.prefill_attention(qh, kh, vh, np.array([0, n]), ip, ix,
                                     w.last_page_len[b:b + 1], w.causal, w.sm_scale)
            spent += time.perf_counter() - t0
            Lb = int(L[b])
            pairs = sum(max(0, Lb - n + i + 1) for i in range(n)) if w.causal else Lb * n
            flops += 4 * w.head_dim * w.num_qo_heads * pairs
            done += 1
            if spent >= min_seconds:
                break
    return {"value": flops / spent / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "seconds": round(spent, 2),
            "sample": f"the first {done} request(s) of {w.name} (whole requests, all heads), "
                      f"numpy float64, BLAS held to {threads} host thread(s)"}


# ------------------------------------------------------------ timing helpers
class CacheFlush:
    """Evicts L2 and the 256 MB Infinity Cache before a timed step, outside
    its events: a 1 GiB write, then a 1 GiB read of another buffer. The
    write alone would leave the Infinity Cache full of dirty lines that the
    timed kernel's own reads then evict, paying their write-back to HBM
    inside the timed region (2-5 us on the skewed batch, measured); after the
    read the caches hold clean lines of a buffer the step never touches."""

    def __init__(self, dev):
        import torch
        self.wbuf = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        self.rbuf = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        self.sink = torch.zeros(1, dtype=torch.float32, device=dev)

    def __call__(self):
        import torch
        self.wbuf.zero_()
        torch.sum(self.rbuf, dim=0, keepdim=True, out=self.sink)


def timed_steps(step, flush, steps, warmup):
    """Run `warmup` untimed steps, then `steps` steps each bracketed by HIP
    events on the current stream (the stream the library launches on), the
    cache flush before each outside the events. Returns (ms per step, wall
    seconds of the timed loop)."""
    import torch
    for _ in range(warmup):
        if flush:
            flush()
        step(None)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if flush:
            flush()
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return [e[0].elapsed_time(e[1]) for e in events], wall


def step_stats(step_ms):
    """Median (what `value` is computed from), mean, p10 and p90 in us."""
    s = sorted(step_ms)
    return {"us_per_batch": round(1e3 * statistics.median(s), 2),
            "us_per_batch_mean": round(1e3 * statistics.mean(s), 2),
            "us_per_batch_p10_p90": [round(1e3 * s[int(0.1 * (len(s) - 1))], 2),
                                     round(1e3 * s[int(0.9 * (len(s) - 1))], 2)]}


def copy_probe(dev):
    """For rocprofv3 --pmc runs: one plain copy of COPY_PROBE_MIB MiB, whose
    counter readings scale the library kernels' readings to bytes."""
    import torch
    src = torch.empty(COPY_PROBE_MIB << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()


def bench_prefill(args, w):
    """Prefill / append: one step = fi_prefill_run over the batch (one launch
    of the tile kernel; cut tiles merge inside it). Reported as
    algorithmic TFLOP/s (4 d H_q flops per attended (query, token) pair)
    against the bf16 dense matrix-core peak."""
    import torch
    import block_sparse_kv_bsr_amd as fb
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    fb.lib()
    dev = torch.device("cuda:0")
    q, k, v = w.make_values(dev)
    plan_t = []
    for _ in range(5):
        t0 = time.perf_counter()
        p = fb.prefill_plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.last_page_len,
                            w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size,
                            w.num_pool_pages, causal=w.causal, dtype=w.dtype,
                            rope=bool(w.rope_theta),
                            fixed_chunk_tokens=args.fixed_chunk_tokens,
                            items_per_cu=args.items_per_cu)
        plan_t.append(time.perf_counter() - t0)
    ws = torch.empty(max(256, p.info["workspace_bytes"]), dtype=torch.uint8, device=dev)
    p.upload(ws)
    out = torch.empty_like(q)
    lse = torch.empty((w.num_qo_tokens, w.num_qo_heads), dtype=torch.float32, device=dev)
    flush = None if args.no_flush else CacheFlush(dev)
    if args.counters_run:
        copy_probe(dev)
        args.steps, args.warmup = min(args.steps, 5), 1

    def step(ev):
        if ev:
            ev[0].record()
        fb.prefill(q, k, v, p, out=out, lse=lse, workspace=ws, k_scale=w.k_scale,
                   v_scale=w.v_scale, rope_theta=w.rope_theta or None, rope_scale=w.rope_scale)
        if ev:
            ev[1].record()

    step_ms, wall = timed_steps(step, flush, args.steps, args.warmup)
    st = step_stats(step_ms)
    med_ms = st["us_per_batch"] * 1e-3
    flops = w.flops()
    tflops = flops / (med_ms * 1e-3) / 1e12
    nbytes = w.algorithmic_bytes()
    kernels = ["tile_attend_kernel"]
    traffic = read_traffic(w.name, kernels)
    result = {
        "metric": "algorithmic TFLOP/s (% of MI355X bf16 dense peak) + µs/batch, "
                  "paged causal prefill / append attention",
        "value": round(tflops, 1),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(med_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the products are bf16 either way (fp8 K/V are widened on the way
        # in); config.kv_dtype names the cache's storage type
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "num_qo_heads": w.num_qo_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "page_size": w.page_size, "qo_tokens": w.num_qo_tokens,
                   "kv_dtype": w.dtype,
                   **({"rope_theta": w.rope_theta} if w.rope_theta else {}),
                   "kv_tokens": int(w.kv_lens().sum()), "causal": bool(w.causal),
                   "algorithmic_flops": flops, "algorithmic_bytes": nbytes,
                   "parallelism": "single-gpu", "plan_items": p.info["num_items"],
                   "plan_merges": p.info["num_merges"], "chunk_tokens": p.info["chunk_tokens"],
                   "l2_mall_flush_between_steps": not args.no_flush},
        **st,
        "timing": "median step; HIP events on the launch stream around each fi_prefill_run "
                  "(" + " + ".join(kernels) + ")",
        "hbm_gbs_algorithmic": round(nbytes / (med_ms * 1e-3) / 1e9, 1),
        "plan_host_us": round(1e6 * statistics.median(plan_t), 1),
        "wall_s_timed_loop": round(wall, 4),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": None if traffic is None else int(traffic),
                     "kernel": " + ".join(kernels)},
    }
    if not args.no_cpu_baseline and not args.counters_run:
        result["cpu_baseline"] = cpu_baseline_prefill(w, q, k, v)
    print(json.dumps(result), flush=True)
    return 0


def cpu_baseline_mla(w, qn, qp, ckv, kpe, min_seconds=10.0):
    """Time the float64 latent-attention oracle on the host over whole
    requests, one after another, until min_seconds have passed; report its
    rate in the benchmark's unit (algorithmic GB/s)."""
    import numpy as np
    sys.path.insert(0, ROOT)
    import oracle.attention as oa
    ctx, threads = _one_thread()
    ch, kh = ckv.float().cpu().numpy(), kpe.float().cpu().numpy()
    qo, L = w.qo_indptr, w.kv_lens()
    nbytes, spent, done = 0, 0.0, 0
    with ctx:
        for b in range(w.batch):
            q0, q1 = int(qo[b]), int(qo[b + 1])
            if q1 == q0:
                continue
            qa, qb = qn[q0:q1].float().cpu().numpy(), qp[q0:q1].float().cpu().numpy()
            ip = np.array([0, w.kv_indptr[b + 1] - w.kv_indptr[b]], dtype=np.int64)
            ix = w.kv_indices[w.kv_indptr[b]:w.kv_indptr[b + 1]]
            t0 = time.perf_counter()
            oa.mla_attention(qa, qb, ch, kh, np.array([0, q1 - q0]), ip, ix,
                             w.last_page_len[b:b + 1], w.sm_scale, w.causal)
            spent += time.perf_counter() - t0
            nbytes += int(L[b]) * (512 + 64) * 2 + (q1 - q0) * w.num_heads * (2 * 512 + 64) * 2
            done += 1
            if spent >= min_seconds:
                break
    return {"value": nbytes / spent / 1e9, "unit": "GB/s", "cores": int(threads),
            "kind": "oracle", "seconds": round(spent, 2),
            "sample": f"the first {done} request(s) of {w.name} (whole requests, all heads), "
                      f"numpy float64, BLAS held to {threads} host thread(s)"}


def bench_mla(args, w):
    """Multi-head latent attention decode: one step = fi_mla_run over the
    batch (one launch of the tile kernel; cut tiles merge inside it). Reported as
    achieved HBM GB/s of the algorithmic bytes (every cached latent and
    rotary key once, q, out) against the 8 TB/s peak: at 96 heads the work
    is 173 flop per byte, below the matrix cores' 312 flop per byte ridge."""
    import torch
    import block_sparse_kv_bsr_amd as fb
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    fb.lib()
    dev = torch.device("cuda:0")
    qn, qp, ckv, kpe = w.make_values(dev)
    plan_t = []
    for _ in range(5):
        t0 = time.perf_counter()
        p = fb.mla_plan(w.qo_indptr, w.kv_indptr, w.kv_indices, w.last_page_len, w.num_heads,
                        w.page_size, w.num_pool_pages, causal=w.causal,
                        fixed_chunk_tokens=args.fixed_chunk_tokens, items_per_cu=args.items_per_cu)
        plan_t.append(time.perf_counter() - t0)
    ws = torch.empty(max(256, p.info["workspace_bytes"]), dtype=torch.uint8, device=dev)
    p.upload(ws)
    out = torch.empty((w.num_qo_tokens, w.num_heads, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.num_qo_tokens, w.num_heads), dtype=torch.float32, device=dev)
    flush = None if args.no_flush else CacheFlush(dev)
    if args.counters_run:
        copy_probe(dev)
        args.steps, args.warmup = min(args.steps, 5), 1

    def step(ev):
        if ev:
            ev[0].record()
        fb.mla(qn, qp, ckv, kpe, p, w.sm_scale, out=out, lse=lse, workspace=ws)
        if ev:
            ev[1].record()

    step_ms, wall = timed_steps(step, flush, args.steps, args.warmup)
    st = step_stats(step_ms)
    med_ms = st["us_per_batch"] * 1e-3
    nbytes, flops = w.algorithmic_bytes(), w.flops()
    gbs = nbytes / (med_ms * 1e-3) / 1e9
    tflops = flops / (med_ms * 1e-3) / 1e12
    kernels = ["mla_attend_kernel"]
    traffic = read_traffic(w.name, kernels)
    result = {
        "metric": "achieved HBM GB/s (% of MI355X peak) + µs/batch, paged latent-attention "
                  "(MLA) decode",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(med_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "num_heads": w.num_heads,
                   "latent_dim": 512, "rope_dim": 64, "page_size": w.page_size,
                   "qo_tokens": w.num_qo_tokens, "kv_tokens": int(w.kv_lens().sum()),
                   "causal": bool(w.causal), "sm_scale": w.sm_scale,
                   "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
                   "parallelism": "single-gpu", "plan_items": p.info["num_items"],
                   "plan_merges": p.info["num_merges"], "chunk_tokens": p.info["chunk_tokens"],
                   "l2_mall_flush_between_steps": not args.no_flush},
        **st,
        "timing": "median step; HIP events on the launch stream around each fi_mla_run "
                  "(" + " + ".join(kernels) + ")",
        "tflops_algorithmic": round(tflops, 1),
        "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "plan_host_us": round(1e6 * statistics.median(plan_t), 1),
        "wall_s_timed_loop": round(wall, 4),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": None if traffic is None else int(traffic),
                     "kernel": " + ".join(kernels)},
    }
    if not args.no_cpu_baseline and not args.counters_run:
        result["cpu_baseline"] = cpu_baseline_mla(w, qn, qp, ckv, kpe)
    print(json.dumps(result), flush=True)
    return 0


# ------------------------------------------------------------------- bench
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--items-per-cu", type=int, default=0)
    ap.add_argument("--min-chunk-tokens", type=int, default=0)
    ap.add_argument("--fixed-chunk-tokens", type=int, default=0)
    ap.add_argument("--decode-kernel", type=int, default=0, choices=[0, 1, 2],
                    help="0 the library's choice, 1 vector-ALU kernel, 2 matrix-core kernel")
    ap.add_argument("--counters-run", action="store_true",
                    help="short run for rocprofv3 --pmc: a copy probe, then a few steps")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--summarize-trace", nargs=2, metavar=("STATS_CSV", "BENCH_LOG"),
                    help="write the profiles/ summary of a traced run (no GPU)")
    args = ap.parse_args()

    sys.path.insert(0, ROOT)
    from block_sparse_kv_bsr_amd.workloads import workload
    w = workload(args.config)

    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, w.name)
        return 0
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace, w, args.config)
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "this decode path runs on a single MI355X and has no multi-GPU mode.", flush=True)
        return 2
    if hasattr(w, "num_heads"):
        return bench_mla(args, w)
    if hasattr(w, "qo_indptr"):
        return bench_prefill(args, w)

    import torch
    import block_sparse_kv_bsr_amd as fb
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    fb.lib()
    dev = torch.device("cuda:0")
    composed = hasattr(w, "prefix_of")  # a prefix cache of its own block size
    vals = w.make_values(dev)
    q, k, v = vals[:3]
    kp_vp = vals[3:] if composed else None
    opts = dict(items_per_cu=args.items_per_cu, min_chunk_tokens=args.min_chunk_tokens,
                fixed_chunk_tokens=args.fixed_chunk_tokens, decode_kernel=args.decode_kernel)
    if not composed:
        opts["rope"] = bool(w.rope_theta)

    # host planner time (median of 20) and upload time
    plan_t = []
    for _ in range(20):
        t0 = time.perf_counter()
        if composed:
            p = fb.plan_composed(w.kv_indptr, w.kv_indices, w.last_page_len, w.prefix_indptr,
                                 w.prefix_indices, w.prefix_last_page_len, w.prefix_of,
                                 w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size,
                                 w.num_pool_pages, w.prefix_page_size, w.num_prefix_pool_pages,
                                 **opts)
        else:
            p = fb.plan(w.kv_indptr, w.kv_indices, w.last_page_len, w.num_qo_heads,
                        w.num_kv_heads, w.head_dim, w.page_size, w.num_pool_pages, w.dtype,
                        **opts)
        plan_t.append(time.perf_counter() - t0)
    ws = torch.empty(max(256, p.info["workspace_bytes"]), dtype=torch.uint8, device=dev)
    # upload time, host call to copy done: the first upload pins a staging
    # block; later ones (a new plan every step) reuse it (median of 20)
    up_t = []
    for _ in range(21):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        p.upload(ws)
        torch.cuda.synchronize()
        up_t.append(time.perf_counter() - t0)
    upload_first_s, upload_s = up_t[0], statistics.median(up_t[1:])

    out = torch.empty((w.batch, w.num_qo_heads, w.head_dim), dtype=q.dtype, device=dev)
    lse = torch.empty((w.batch, w.num_qo_heads), dtype=torch.float32, device=dev)
    flush = None if args.no_flush else CacheFlush(dev)
    if args.counters_run:
        copy_probe(dev)
        args.steps, args.warmup = min(args.steps, 5), 1

    def step(ev):
        if ev:
            ev[0].record()
        if composed:
            fb.decode_composed(q, k, v, kp_vp[0], kp_vp[1], p, out=out, lse=lse, workspace=ws)
        else:
            fb.decode(q, k, v, p, out=out, lse=lse, workspace=ws, k_scale=w.k_scale,
                      v_scale=w.v_scale, rope_theta=w.rope_theta or None,
                      rope_scale=w.rope_scale)
        if ev:
            ev[1].record()

    step_ms, wall = timed_steps(step, flush, args.steps, args.warmup)
    st = step_stats(step_ms)
    med_ms = st["us_per_batch"] * 1e-3
    nbytes = w.algorithmic_bytes()
    gbs = nbytes / (med_ms * 1e-3) / 1e9
    # a step is one fi_decode_run: the decode kernel, preceded by the tile
    # kernel when the plan has shared-prefix items
    decode_kernel = ("decode_mma_kernel" if p.info["decode_kernel"] == fb.binding.DECODE_KERNEL_MATRIX
                     else "decode_bsr_kernel")
    kernels = (["tile_attend_kernel"] if p.info["num_prefix_items"] else []) + [decode_kernel]
    traffic = read_traffic(w.name, kernels)
    result = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(med_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bf16": "bf16", "f32": "f32", "fp8": "fp8_e4m3 K/V, bf16 q/out"}[w.dtype]
                 + (", rotary embedding applied to K in the kernel" if w.rope_theta else ""),
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "num_qo_heads": w.num_qo_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "page_size": w.page_size,
                   "kv_tokens": int((w.total_kv_lens() if composed else w.kv_lens()).sum()),
                   **({"prefix_page_size": w.prefix_page_size} if composed else {}),
                   "algorithmic_bytes": nbytes, "parallelism": "single-gpu",
                   "plan_items": p.info["num_items"], "chunk_pages": p.info["chunk_pages"],
                   "prefix_items": p.info["num_prefix_items"],
                   "l2_mall_flush_between_steps": not args.no_flush},
        **st,
        "timing": "median step; HIP events on the launch stream around each fi_decode_run "
                  "(" + " + ".join(kernels) + ")",
        "pct_of_peak_hbm": round(100 * gbs / PEAK_HBM_GBS, 2),
        "plan_host_us": round(1e6 * statistics.median(plan_t), 1),
        "upload_us": round(1e6 * upload_s, 1),
        "upload_first_us": round(1e6 * upload_first_s, 1),
        "wall_s_timed_loop": round(wall, 4),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": None if traffic is None else int(traffic),
                     "kernel": " + ".join(kernels)},
    }
    if not args.counters_run:
        ceiling = stream_ceiling(dev, flush or CacheFlush(dev))
        result["practical_ceiling"] = {
            "gbs": round(ceiling, 1), "frac": round(gbs / ceiling, 4),
            "kernel": "streaming read of 2 GiB with 16-byte nontemporal loads "
                      "(libfi_bench.so), L2/MALL flushed, median of 5"}
    if not args.no_cpu_baseline and not args.counters_run:
        result["cpu_baseline"] = cpu_baseline(w, q, k, v, kp_vp=kp_vp)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
