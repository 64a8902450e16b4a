"""Build the C-ABI library ``libfi_bsr.so`` in-tree for gfx950, and the
benchmark's measurement helper ``libfi_bench.so`` (a streaming-read kernel,
not part of the library's interface).

Usage: ``python -m block_sparse_kv_bsr_amd.build``. Compiles every source each
time it runs (the sources are small); objects go to ``_build/`` at the repo
root and the libraries next to this file.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfi_bsr.so")
BENCH_LIB = os.path.join(PKG, "libfi_bench.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]
# Packed fp32 VALU ops are kept out of every device code object.
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
HIP_SOURCES = ["decode_bsr.hip", "decode_mma.hip", "attn_tile.hip", "merge_states.hip", "abi.hip",
               "staging.hip", "mla_attend.hip"]
CPP_SOURCES = ["plan.cpp", "prefill_plan.cpp"]
# Per-source device flags. The latent-attention kernel keeps its matrix
# accumulators in ordinary vector registers (everything fits in 256): with
# accumulation registers the compiler copied all 64 output accumulators out
# and back around the rarely taken rescale branch on every block.
EXTRA = {"mla_attend.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
BENCH_SOURCES = ["bench_stream.hip"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the device-only feature flag; drop that note
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "is not a recognized feature for this target" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([HIPCC, *COMMON, *DEVICE, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src),
                     "-o", obj])
        objs.append(obj)
    for src in CPP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append(["g++", *COMMON, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    bench_objs = []
    for src in BENCH_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        jobs.append([HIPCC, *COMMON, *DEVICE, "-c", os.path.join(CSRC, src), "-o", obj])
        bench_objs.append(obj)
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        outs = list(ex.map(_run, jobs))
    for lib, parts in ((LIB, objs), (BENCH_LIB, bench_objs)):
        tmp = lib + ".tmp"
        outs.append(_run([HIPCC, *DEVICE, "-shared", "-fPIC", *parts, "-o", tmp]))
        os.replace(tmp, lib)
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
