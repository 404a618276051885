"""Builds libtq.so (HIP kernels for gfx950 plus the host C++ of the C ABI) in this directory.

Usage: python kv_cache_vector_tq_amd/build_lib.py [--incremental] [-v]
(run by path: importing the package needs the built library).
Each source is compiled on its own (in parallel) and then linked with hipcc.  --incremental
recompiles only sources whose object is older than the source or than any header of csrc/ and
include/; the default recompiles everything.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtq.so")
# the quantize and attention kernels are instantiated per key code width (0..8 bits) in
# translation units of their own
SOURCES = (["tq_host.cpp", "tq_quantize.hip", "tq_attend.hip"] + [f"tq_quantize_k{kb}.hip" for kb in range(9)] +
           [f"tq_attend_k{kb}.hip" for kb in range(9)] + ["tq_bf16_attend.hip", "tq_probe.hip"])
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libtq")


def _flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
        # packed fp32 instructions stay off in all device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(HERE, "..", "include"),
    ]


def _newest_header() -> float:
    t = 0.0
    for d in (CSRC, os.path.join(HERE, "..", "include")):
        for f in os.listdir(d):
            if f.endswith(".h"):
                t = max(t, os.path.getmtime(os.path.join(d, f)))
    return t


def build(verbose: bool = False, incremental: bool = False) -> str:
    hipcc = _hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    headers = _newest_header()

    def compile_one(src):
        obj = os.path.join(objdir, src.rsplit(".", 1)[0] + ".o")
        if incremental and os.path.exists(obj) and os.path.getmtime(obj) > max(
                headers, os.path.getmtime(os.path.join(CSRC, src))):
            return obj
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc] + _flags() + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"compiling {src} failed:\n{msgs}")
        if verbose and msgs.strip():
            print(msgs)
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("linking libtq.so failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    path = build(verbose="-v" in sys.argv, incremental="--incremental" in sys.argv)
    print(path)
