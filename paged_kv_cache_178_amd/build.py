"""Build the HIP library ``libnp_paged.so`` in-tree for gfx950, and its trace
build ``libnp_paged_trace.so`` (the decode kernels compiled with NP_TRACE:
per-workgroup schedule records and phase timestamps, for tests and
measurement only; see include/np_trace.h).

The host half (checks, planner) is compiled with g++ to keep it free of HIP;
the kernels and launchers with hipcc. All device code is built with packed
fp32 instructions disabled.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libnp_paged.so")
TRACE_LIB = os.path.join(PKG, "libnp_paged_trace.so")

HIP_SOURCES = ["np_decode.hip", "np_prefill.hip", "np_append.hip", "np_probe.hip"]
# Sources compiled a second time, with NP_TRACE, for the trace library.
TRACE_SOURCES = ["np_decode.hip"]
# Per-file flags. The prefill kernel masks by index with selects and never
# relies on NaN propagation, so it is built without NaN semantics (max and min
# lose their canonicalisation instructions).
EXTRA_FLAGS = {"np_prefill.hip": ["-fno-honor-nans"]}
HOST_SOURCES = ["np_host.cpp", "np_alloc.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in VGPRs (gfx950 has one register file), so the
    # softmax reads scores and rescales outputs without AGPR copies.
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library cannot be built")


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    return res


def build(verbose: bool = False, jobs: int = 8, trace: bool = True) -> str:
    """Compile every source and link ``libnp_paged.so`` (and, with `trace`,
    ``libnp_paged_trace.so``); returns the product library's path."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    incs = ["-I", INCLUDE, "-I", CSRC]
    steps = []
    objs = []
    trace_objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        steps.append(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", *incs, "-c",
                      os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
        trace_objs.append(obj)
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        steps.append([hipcc, *HIPCC_FLAGS, *EXTRA_FLAGS.get(src, []), *incs, "-c",
                      os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
        if trace and src in TRACE_SOURCES:
            tobj = os.path.join(BUILD, src + ".trace.o")
            steps.append([hipcc, *HIPCC_FLAGS, *EXTRA_FLAGS.get(src, []), "-DNP_TRACE", *incs,
                          "-c", os.path.join(CSRC, src), "-o", tobj])
            trace_objs.append(tobj)
        else:
            trace_objs.append(obj)
    # Longest compiles first.
    steps.sort(key=lambda c: "np_decode.hip" not in " ".join(c))
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(steps)))) as ex:
        for res in ex.map(_run, steps):
            if verbose and (res.stdout or res.stderr):
                sys.stderr.write(res.stdout + res.stderr)
    links = [(objs, LIB)] + ([(trace_objs, TRACE_LIB)] if trace else [])
    for obj_list, lib in links:
        tmp = lib + ".tmp"
        _run([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *obj_list, "-o", tmp])
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
