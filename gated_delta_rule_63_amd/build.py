"""Build libgdr.so in-tree with hipcc for gfx950.

    python -m gated_delta_rule_63_amd.build

Each ``csrc/*.hip`` file is compiled to an object under ``_build/`` (in parallel),
then linked into ``gated_delta_rule_63_amd/libgdr.so``.  Two measurement libraries are built beside
it: the benchmark's MFMA-rate probe (``csrc/probe/mfma_peak.hip``) into ``libgdr_probe.so``, and
``libgdr_stamps.so``, the same library with the flow kernel's clock counters compiled in
(``GDR_FLOW_STAMPS``; read by ``bench.py --flow-stamps``).  Packed-fp32 instruction selection is
switched off for every device compile.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgdr.so")
# measurement probe (a dense-MFMA rate kernel for the benchmark), a library of its own
PROBE_SRC = os.path.join(CSRC, "probe", "mfma_peak.hip")
PROBE_LIB = os.path.join(PKG, "libgdr_probe.so")
STAMPS_LIB = os.path.join(PKG, "libgdr_stamps.so")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str, defines=(), suffix: str = "") -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + suffix + ".o")
    cmd = [_hipcc(), *COMMON, *defines, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    workers = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    chunk = os.path.join(CSRC, "gdr_chunk.hip")
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        futs = [ex.submit(_compile, src) for src in srcs]
        fut_st = ex.submit(_compile, chunk, ("-DGDR_FLOW_STAMPS",), ".stamps")
        objs = [f.result() for f in futs]
        obj_st = fut_st.result()
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    tmp = PROBE_LIB + ".tmp"
    r = subprocess.run([_hipcc(), *COMMON, "-shared", PROBE_SRC, "-o", tmp], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {PROBE_SRC}:\n{r.stderr}")
    os.replace(tmp, PROBE_LIB)
    tmp = STAMPS_LIB + ".tmp"
    objs_st = [obj_st if os.path.basename(o) == "gdr_chunk.hip.o" else o for o in objs]
    r = subprocess.run([_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs_st, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, STAMPS_LIB)
    if verbose:
        print(f"built {LIB}, {PROBE_LIB} and {STAMPS_LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
