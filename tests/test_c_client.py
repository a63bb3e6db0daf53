"""The C ABI from a plain C99 program (tests/c/hk_c_client.c).

The client includes include/hk_gemm.h and include/hk_attn.h in a C99
translation unit built with -pedantic -Werror, links libhkgemm.so and HIP's
C runtime library, and calls the entry points directly.  Without a GPU it
checks argument validation (which happens before any HIP call); with one
it also runs hk_gemm_bf16, hk_gemm_fp8 and hk_attn_fwd_bf16 on small
integer-valued inputs whose exact results it computes itself (integer
products; the mean of V for all-zero queries).
"""
import os
import shutil
import subprocess

import pytest

import fp8_gemm_02_amd as hk

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c", "hk_c_client.c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _build(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    if not os.path.exists(hk.LIB_PATH):
        pytest.skip("libhkgemm.so is not built")
    out = str(tmp_path / "hk_c_client")
    libdir = os.path.dirname(hk.LIB_PATH)
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), "-isystem", os.path.join(ROCM, "include"),
           SRC, "-o", out, "-L", libdir, "-lhkgemm", "-L", os.path.join(ROCM, "lib"),
           "-lamdhip64", "-lm", "-Wl,-rpath," + libdir, "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    return out


def test_c_client_builds_and_validates(tmp_path):
    """The headers compile as strict C99; argument checks work from C."""
    exe = _build(tmp_path)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "hk_c_client OK" in r.stdout


@pytest.mark.gpu
def test_c_client_runs_the_kernels(tmp_path):
    exe = _build(tmp_path)
    r = subprocess.run([exe, "--gpu"], capture_output=True, text=True, timeout=120)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "hk_gemm_bf16 300x260x192 exact" in r.stdout
    assert "hk_gemm_fp8 300x260x192 exact" in r.stdout
    assert "hk_attn_fwd_bf16 all-zero queries" in r.stdout
    assert "hk_c_client OK" in r.stdout
