"""Build libhkgemm.so in-tree with hipcc for gfx950.

    python -m fp8_gemm_02_amd._build            # build
    python -m fp8_gemm_02_amd._build --asm DIR  # also keep the device assembly in DIR
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libhkgemm.so")
SOURCES = [os.path.join(CSRC, "hk_gemm.hip"), os.path.join(CSRC, "hk_attn.hip"),
           os.path.join(CSRC, "hk_noalloc.hip")]
HEADERS = [os.path.join(CSRC, f) for f in ("hk_device.hpp", "hk_grid.hpp", "hk_kernels.hpp")] + [
    os.path.join(INCLUDE, "hk_gemm.h")]

ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; a ROCm install is required to build libhkgemm.so")


def compile_cmd(out: str, extra=()) -> list:
    return [hipcc(), "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
            # packed fp32 VALU forms are kept out of every kernel
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument",
            "-I", INCLUDE, "-I", CSRC, *extra, "-o", out, *SOURCES]


def build(asm_dir: str | None = None, extra=()) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    extra = list(extra)
    cwd = None
    if asm_dir:
        os.makedirs(asm_dir, exist_ok=True)
        extra += ["-save-temps"]
        cwd = asm_dir
    subprocess.run(compile_cmd(tmp, extra), check=True, cwd=cwd)
    os.replace(tmp, LIB)
    return LIB


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None, help="directory for -save-temps output")
    ap.add_argument("-D", action="append", default=[], help="extra preprocessor definitions")
    a = ap.parse_args()
    print(build(a.asm, ["-D" + d for d in a.D]))


if __name__ == "__main__":
    main()
