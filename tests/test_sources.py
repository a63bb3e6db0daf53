"""Static checks on the HIP sources (CPU only).

Direct HBM->LDS loads take their LDS address in M0.  The compiler must know
when M0 changes: an asm statement that writes M0 itself and lists it as
clobbered is undefined behaviour (the register is reserved), so every such
load takes M0 as an explicit "{m0}" input operand and no statement writes or
clobbers it.
"""
import glob
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = sorted(glob.glob(os.path.join(ROOT, "fp8_gemm_02_amd", "csrc", "*.h*")))


def _asm_statements(text):
    # every asm(...) / asm volatile(...) statement, up to its closing ");"
    return re.findall(r"\basm\s+(?:volatile\s*)?\((.*?)\);", text, re.S)


def test_sources_found():
    names = {os.path.basename(p) for p in SOURCES}
    assert {"hk_device.hpp", "hk_kernels.hpp", "hk_gemm.hip", "hk_attn.hpp"} <= names


def test_no_asm_statement_writes_or_clobbers_m0():
    for p in SOURCES:
        for st in _asm_statements(open(p).read()):
            assert not re.search(r'"m0"', st), (p, st)
            assert not re.search(r"s_mov_b32\s+m0", st), (p, st)


def test_direct_lds_loads_take_m0_as_an_operand():
    found = 0
    for p in SOURCES:
        for st in _asm_statements(open(p).read()):
            if re.search(r"(buffer|global)_load_\w+[^\"]*\blds\b|global_load_lds_", st):
                found += 1
                assert '"{m0}"' in st, (p, st)
                # the one wait state a direct load needs after M0 is written
                assert re.search(r'"s_nop 0\\n', st), (p, st)
    assert found >= 2
