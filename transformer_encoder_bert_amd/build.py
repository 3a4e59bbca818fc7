"""Build libftx.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Run as ``python -m transformer_encoder_bert_amd.build`` or through
``__graft_entry__.build()``.  Each source compiles in its own hipcc process (in
parallel), then one link step writes ``transformer_encoder_bert_amd/libftx.so``.
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
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libftx.so")
SOURCES = ("elementwise.hip", "gemm.hip", "attention.hip", "encoder.hip", "decoder.hip")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libftx.so)")


def compile_flags() -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Wno-unused-function",
            # packed-fp32 instructions are kept out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            f"-I{INCLUDE}", f"-I{CSRC}"]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the device feature flag; that warning is harmless
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    return p.returncode, out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    jobs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        jobs.append([cc] + compile_flags() + ["-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=min(len(jobs), os.cpu_count() or 1)) as ex:
        results = list(ex.map(_run, jobs))
    for cmd, (rc, out) in zip(jobs, results):
        if verbose or rc:
            print(" ".join(cmd))
            if out:
                print(out)
        if rc:
            raise RuntimeError(f"hipcc failed on {cmd[-3]}")
    tmp = LIB_PATH + ".tmp"
    link = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    rc, out = _run(link)
    if verbose or rc:
        print(" ".join(link))
        if out:
            print(out)
    if rc:
        raise RuntimeError("link of libftx.so failed")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
