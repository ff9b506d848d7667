"""Build libmlora.so (HIP, gfx950) in-tree with hipcc.

    python -m adapter_lora_segments_amd.build [--jobs N]

Every translation unit is compiled for gfx950 only, with packed-fp32 vector
instructions disabled; objects go to ``_build/`` at the repository root and
the shared library next to this file.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmlora.so")
PROBES_LIB = os.path.join(PKG, "libmlora_probes.so")

SOURCES = ["plan.cpp", "api.cpp", "kernels_bf16.hip", "kernels_gemm.hip", "kernels_gemm_mx.hip", "kernels_fp32.hip", "kernels_adamw.hip",
           "kernels_mx.hip", "scratch.hip"]
# measured-ceiling probes (include/mlora_probes.h), a library of their own
PROBE_SOURCES = ["probes.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = (r.stdout + r.stderr)
    # hipcc's host pass does not know the packed-fp32 feature; that line is noise.
    out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    # An inline-asm statement that clobbers a register the compiler reserves
    # (M0, EXEC, VCC) is undefined behaviour: refuse the build.
    if "Reserved registers on the clobber list" in out:
        raise RuntimeError(f"{src}: inline assembly clobbers a reserved register:\n{out}")
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def build(jobs: int = 4, verbose: bool = True) -> str:
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES + PROBE_SOURCES))
    for lib, parts in ((LIB, objs[:len(SOURCES)]), (PROBES_LIB, objs[len(SOURCES):])):
        tmp = lib + ".tmp"
        cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-o", tmp] + parts + \
            ["-Wl,-rpath,/opt/rocm/lib", "-Wl,--no-undefined"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
        shutil.move(tmp, lib)
        if verbose:
            print("built", lib)
    return LIB


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    a = ap.parse_args()
    build(a.jobs)


if __name__ == "__main__":
    main()
