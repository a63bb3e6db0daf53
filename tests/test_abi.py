"""The C ABI on the host: the library loads, exports what the header declares,
validates arguments before touching the GPU, and plans launches.

No test here computes anything on a GPU; calls that would launch use fake
pointers only where validation is expected to reject them first, or (without
a GPU) where the launch itself must fail cleanly with HK_ERROR_LAUNCH.
"""
import ctypes
import os
import re

import pytest

import fp8_gemm_02_amd as hk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hk_gemm.h")
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]

FAKE = 0x7F0000000000  # 16-byte aligned, never dereferenced in these tests


def _declared_functions():
    names = set()
    for path in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(hk_\w+)\s*\(", text, flags=re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def L():
    return hk.lib()


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("hk_gemm_bf16", "hk_gemm_fp8", "hk_gemm_mxfp8", "hk_gemm_ex", "hk_gemm_plan",
              "hk_grid_map", "hk_status_string", "hk_version", "hk_wall_clock_khz",
              "hk_attn_fwd_bf16"):
        assert n in names
    assert set(names) == set(hk.EXPORTED)


def test_library_exports_every_declared_symbol(L):
    for n in _declared_functions():
        assert hasattr(L, n), n


def test_status_strings(L):
    assert hk.status_string(0) == "HK_SUCCESS"
    assert hk.status_string(1) == "HK_ERROR_INVALID_VALUE"
    assert hk.status_string(2) == "HK_ERROR_NOT_SUPPORTED"
    assert hk.status_string(3) == "HK_ERROR_LAUNCH"
    assert hk.status_string(99) == "HK_UNKNOWN_STATUS"
    assert hk.hk_version() >= 200


BAD_BF16 = [
    dict(M=-1), dict(N=-1), dict(K=-1),
    dict(A=0), dict(B=0), dict(C=0),
    dict(lda=63), dict(ldb=63), dict(ldc=31),
    dict(C=FAKE + 1),          # C must be 2-byte aligned
    dict(A=FAKE + 1),          # bf16 operands must be 2-byte aligned
]


@pytest.mark.parametrize("bad", BAD_BF16, ids=[",".join(b) for b in BAD_BF16])
def test_invalid_arguments_rejected_before_any_hip_call(L, bad):
    a = dict(A=FAKE, B=FAKE, C=FAKE, M=32, N=32, K=64, lda=64, ldb=64, ldc=32)
    a.update(bad)
    st = L.hk_gemm_bf16(a["A"], a["B"], a["C"], a["M"], a["N"], a["K"], a["lda"], a["ldb"],
                        a["ldc"], None)
    assert st == hk.HK_ERROR_INVALID_VALUE


def test_fp8_rejects_non_finite_scales(L):
    for sa, sb in [(float("nan"), 1.0), (1.0, float("inf"))]:
        st = L.hk_gemm_fp8(FAKE, FAKE, FAKE, 32, 32, 64, 64, 64, 32, sa, sb, None)
        assert st == hk.HK_ERROR_INVALID_VALUE


def test_ex_rejects_bad_dtype_and_options(L):
    st = L.hk_gemm_ex(7, FAKE, FAKE, FAKE, 32, 32, 64, 64, 64, 32, 1.0, 1.0, None, None)
    assert st == hk.HK_ERROR_INVALID_VALUE
    for field, val in [("schedule", 9), ("grid_order", 5), ("group_m", -1), ("window", -2)]:
        o = hk.GemmOpts()
        setattr(o, field, val)
        st = L.hk_gemm_ex(0, FAKE, FAKE, FAKE, 32, 32, 64, 64, 64, 32, 1.0, 1.0,
                          ctypes.byref(o), None)
        assert st == hk.HK_ERROR_INVALID_VALUE, field
    for field, val in [("layout_a", 2), ("layout_b", -1)]:
        o = hk.GemmOpts()
        setattr(o, field, val)
        st = L.hk_gemm_ex(0, FAKE, FAKE, FAKE, 32, 32, 64, 64, 64, 32, 1.0, 1.0,
                          ctypes.byref(o), None)
        assert st == hk.HK_ERROR_INVALID_VALUE, field
    # the clock record takes 16-byte stores: a misaligned buffer is rejected
    for off in (8, 4, 1):
        o = hk.GemmOpts()
        o.clock_stamps = FAKE + off
        st = L.hk_gemm_ex(0, FAKE, FAKE, FAKE, 32, 32, 64, 64, 64, 32, 1.0, 1.0,
                          ctypes.byref(o), None)
        assert st == hk.HK_ERROR_INVALID_VALUE, off


def test_opts_struct_matches_the_header():
    text = open(HEADER).read()
    body = re.search(r"typedef struct hk_gemm_opts \{(.*?)\} hk_gemm_opts;", text, re.S).group(1)
    fields = re.findall(r"(int32_t|int64_t|uint64_t \*|const float \*|void \*)\s*(\w+);", body)
    ctype = {"int32_t": ctypes.c_int32, "int64_t": ctypes.c_int64, "uint64_t *": ctypes.c_void_p,
             "void *": ctypes.c_void_p, "const float *": ctypes.c_void_p}
    assert [(n, ctype[t]) for t, n in fields] == list(hk.GemmOpts._fields_)
    assert ctypes.sizeof(hk.GemmOpts) == 72
    assert hk.GemmOpts.clock_stamps.offset == 24 and hk.GemmOpts.workspace.offset == 32
    assert hk.GemmOpts.workspace_bytes.offset == 40 and hk.GemmOpts.repack.offset == 48
    assert hk.GemmOpts.scale_a_dev.offset == 56 and hk.GemmOpts.scale_b_dev.offset == 64


def test_chiplet_clocks_from_a_record():
    # chiplet 0: 1.9e6 shader cycles over 1e5 ticks of a 100 MHz counter = 1.9 GHz;
    # chiplet 1 recorded nothing
    st = [0] * 32
    st[0:4] = [10, 500, 10 + 1_900_000, 500 + 100_000]
    got = hk.chiplet_clocks_ghz(st, 100_000)
    assert abs(got[0] - 1.9) < 1e-12 and got[1] is None


# Operand layouts: K_STRIDED stores A as K x M (lda >= M) and B as K x N (ldb >= N).
def test_strided_layout_leading_dimension_checks(L):
    def ex(M, N, K, lda, ldb, la, lb):
        o = hk._opts(layout_a=la, layout_b=lb)
        return L.hk_gemm_ex(0, FAKE, FAKE, FAKE, M, N, K, lda, ldb, N, 1.0, 1.0, ctypes.byref(o),
                            None)
    # B stored K x N: ldb counts columns of B (N), not K
    assert ex(32, 48, 64, 64, 47, 0, 1) == hk.HK_ERROR_INVALID_VALUE
    # A stored K x M: lda counts M
    assert ex(40, 32, 64, 39, 64, 1, 0) == hk.HK_ERROR_INVALID_VALUE
    assert ex(40, 32, 64, 64, 63, 1, 0) == hk.HK_ERROR_INVALID_VALUE


def test_plan_strided_layouts():
    M, N, K = 8192, 8192, 8192
    names = {(0, 0): "hk_gemm_il4_bf16", (1, 0): "hk_gemm_il4_bf16_akm",
             (0, 1): "hk_gemm_il4_bf16_bkn", (1, 1): "hk_gemm_il4_bf16_akm_bkn"}
    for (la, lb), name in names.items():
        p = _plan(hk.HK_DTYPE_BF16, M, N, K, lda=M if la else K, ldb=N if lb else K,
                  layout_a=la, layout_b=lb)
        assert p["kernel_name"] == name and p["schedule"] == hk.HK_SCHEDULE_INTERLEAVE4
        assert p["workgroups"] == 256
    # ldb below K is fine for B stored K x N (it counts N)
    p = _plan(hk.HK_DTYPE_BF16, 512, 256, 1024, ldb=256, layout_b="k_strided")
    assert p["kernel_name"] == "hk_gemm_il4_bf16_bkn"
    # small outputs keep the 4-wave kernel (the small-tile kernel has no K-strided images)
    p = _plan(hk.HK_DTYPE_BF16, 256, 256, 256, layout_b="k_strided")
    assert p["kernel_name"] == "hk_gemm_il4_bf16_bkn"
    # both operands K-strided: K needs no chunk alignment
    p = _plan(hk.HK_DTYPE_BF16, 256, 256, 100, lda=256, ldb=256, layout_a=1, layout_b=1)
    assert p["kernel_name"] == "hk_gemm_il4_bf16_akm_bkn"


@pytest.mark.parametrize("case", [
    dict(N=260, ldb=260),           # N of a K-strided B not whole 16-byte chunks
    dict(ldb=264 + 4),              # stride not whole chunks
    dict(B=FAKE + 8),               # B not 16-byte aligned
    dict(K=100),                    # K-contiguous A with K not whole chunks
    dict(K=1 << 20, ldb=1 << 10),   # (K + 128) rows of B past the 31-bit offsets
], ids=lambda c: ",".join(c))
def test_plan_strided_layout_falls_back_to_basic(case):
    a = dict(M=512, N=256, K=1024, ldb=256, B=FAKE)
    a.update(case)
    p = _plan(hk.HK_DTYPE_BF16, a["M"], a["N"], a["K"], ldb=a["ldb"], B=a["B"], layout_b=1)
    assert p["kernel_name"] == "hk_gemm_basic_bf16"


def test_plan_strided_layout_other_schedules_unsupported():
    for sched in ("pingpong8", "smalltile", "interleave8", "producer_consumer"):
        with pytest.raises(hk.HKError):
            _plan(hk.HK_DTYPE_BF16, 1024, 1024, 1024, schedule=sched, layout_a=1, lda=1024)
    p = _plan(hk.HK_DTYPE_BF16, 1024, 1024, 1024, layout_b=1, ldb=1024, schedule="basic")
    assert p["kernel_name"] == "hk_gemm_basic_bf16"


def _mx(L, **kw):
    a = dict(A=FAKE, B=FAKE, C=FAKE, M=32, N=32, K=256, lda=256, ldb=256, ldc=32, SA=FAKE,
             SB=FAKE, ldsa=16, ldsb=16)
    a.update(kw)
    return L.hk_gemm_mxfp8(a["A"], a["B"], a["C"], a["M"], a["N"], a["K"], a["lda"], a["ldb"],
                           a["ldc"], a["SA"], a["SB"], a["ldsa"], a["ldsb"], None)


@pytest.mark.parametrize("bad", [dict(SA=0), dict(SB=0), dict(ldsa=7), dict(ldsb=0), dict(M=-1),
                                 dict(A=0), dict(lda=255), dict(ldc=31)],
                         ids=lambda b: ",".join(b))
def test_mxfp8_invalid_arguments(L, bad):
    assert _mx(L, **bad) == hk.HK_ERROR_INVALID_VALUE


@pytest.mark.parametrize("unsupported", [dict(K=48, lda=48, ldb=48, ldsa=16, ldsb=16),
                                         dict(SA=FAKE + 8), dict(SB=FAKE + 4), dict(ldsa=24),
                                         dict(ldsb=17), dict(A=FAKE + 16 + 8), dict(lda=264)],
                         ids=lambda b: ",".join(b))
def test_mxfp8_unsupported_layouts(L, unsupported):
    assert _mx(L, **unsupported) == hk.HK_ERROR_NOT_SUPPORTED


def test_mxfp8_needs_its_own_entry_point(L):
    st = L.hk_gemm_ex(hk.HK_DTYPE_MXFP8_E4M3, FAKE, FAKE, FAKE, 32, 32, 64, 64, 64, 32, 1.0, 1.0,
                      None, None)
    assert st == hk.HK_ERROR_INVALID_VALUE
    assert _mx(L, M=0) == hk.HK_SUCCESS and _mx(L, N=0, SA=0, SB=0) == hk.HK_SUCCESS


def test_plan_mxfp8():
    p = _plan(hk.HK_DTYPE_MXFP8_E4M3, 8192, 8192, 8192)
    assert p["kernel_name"] == "hk_gemm_il4_mxfp8" and p["tile_k"] == 128
    assert p["schedule"] == hk.HK_SCHEDULE_INTERLEAVE4 and p["workgroups"] == 256
    assert p["lds_bytes"] == 131072 + 16384  # two stages plus two groups of block scales
    # small outputs run the same kernel (the only one that carries block scales)
    p = _plan(hk.HK_DTYPE_MXFP8_E4M3, 256, 256, 256)
    assert p["kernel_name"] == "hk_gemm_il4_mxfp8" and p["workgroups"] == 1
    with pytest.raises(hk.HKError):
        _plan(hk.HK_DTYPE_MXFP8_E4M3, 256, 256, 256, schedule="pingpong8")


def test_empty_output_is_a_noop_success(L):
    # M == 0 or N == 0: nothing is read or written, null pointers allowed
    assert L.hk_gemm_bf16(0, 0, 0, 0, 16, 16, 16, 16, 16, None) == hk.HK_SUCCESS
    assert L.hk_gemm_bf16(0, 0, 0, 16, 0, 16, 16, 16, 16, None) == hk.HK_SUCCESS
    assert L.hk_gemm_fp8(0, 0, 0, 0, 0, 0, 0, 0, 0, 1.0, 1.0, None) == hk.HK_SUCCESS


def test_explicit_fast_schedule_needs_alignment(L):
    o = hk.GemmOpts()
    o.schedule = hk.HK_SCHEDULE_PINGPONG8
    # K not a multiple of 8 bf16 elements: the fast schedule cannot run it
    st = L.hk_gemm_ex(0, FAKE, FAKE, FAKE, 64, 64, 60, 60, 60, 64, 1.0, 1.0, ctypes.byref(o), None)
    assert st == hk.HK_ERROR_NOT_SUPPORTED
    # misaligned A pointer
    st = L.hk_gemm_ex(0, FAKE + 2, FAKE, FAKE, 64, 64, 64, 64, 64, 64, 1.0, 1.0,
                      ctypes.byref(o), None)
    assert st == hk.HK_ERROR_NOT_SUPPORTED


def _has_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.skipif(_has_gpu(), reason="checks the no-GPU launch path")
def test_valid_call_without_gpu_reports_launch_error(L):
    st = L.hk_gemm_bf16(FAKE, FAKE, FAKE, 256, 256, 256, 256, 256, 256, None)
    assert st == hk.HK_ERROR_LAUNCH
    st = L.hk_gemm_fp8(FAKE, FAKE, FAKE, 256, 256, 256, 256, 256, 256, 0.5, 2.0, None)
    assert st == hk.HK_ERROR_LAUNCH


# ------------------------------------------------------------------- planning

def _plan(dtype, M, N, K, lda=None, ldb=None, ldc=None, A=FAKE, B=FAKE, C=FAKE, **kw):
    return hk.hk_gemm_plan(dtype, A, B, C, M, N, K, lda or K, ldb or K, ldc or N, **kw)


@pytest.mark.parametrize("M,N,K,tiles", [(4096, 4096, 4096, (16, 16)),
                                         (8192, 8192, 8192, (32, 32)),
                                         (8192, 28672, 8192, (32, 112)),
                                         (8191, 28670, 8200, (32, 112))])
def test_plan_fast_path_for_every_workload(M, N, K, tiles):
    p = _plan(hk.HK_DTYPE_BF16, M, N, K)
    assert p["schedule"] == hk.HK_SCHEDULE_INTERLEAVE4
    assert p["kernel_name"] == "hk_gemm_il4_bf16"
    assert (p["tiles_m"], p["tiles_n"]) == tiles
    # persistent: one workgroup per compute unit (256 on MI355X; the same
    # count is assumed when no device is visible)
    assert p["workgroups"] == min(tiles[0] * tiles[1], 256)
    assert p["threads"] == 256 and p["lds_bytes"] == 131072
    assert p["tile_k"] == 64
    assert p["grid_order"] == hk.HK_GRID_XCD


@pytest.mark.parametrize("dtype,name", [(hk.HK_DTYPE_BF16, "hk_gemm_st4_bf16"),
                                        (hk.HK_DTYPE_FP8_E4M3, "hk_gemm_st4_fp8")])
@pytest.mark.parametrize("M,N,tiles", [(256, 256, (2, 2)), (2048, 2048, (16, 16)),
                                       (300, 4000, (3, 32))])
def test_plan_small_outputs_use_128_tiles(dtype, name, M, N, tiles):
    # at most one 256 x 256 tile per four compute units
    p = _plan(dtype, M, N, 256)
    assert p["schedule"] == hk.HK_SCHEDULE_SMALLTILE and p["kernel_name"] == name
    assert (p["tile_m"], p["tile_n"]) == (128, 128)
    assert (p["tiles_m"], p["tiles_n"]) == tiles
    assert p["workgroups"] == tiles[0] * tiles[1]  # one workgroup per tile
    assert p["threads"] == 256 and p["lds_bytes"] == 131072


def test_plan_small_tiles_on_request():
    p = _plan(hk.HK_DTYPE_BF16, 8192, 8192, 8192, schedule="smalltile")
    assert p["kernel_name"] == "hk_gemm_st4_bf16" and p["workgroups"] == 64 * 64


def test_plan_small_output_threshold():
    # 64 tiles of 256 x 256 on 256 compute units: small; 65: the 4-wave kernel
    assert _plan(hk.HK_DTYPE_BF16, 2048, 2048, 64)["schedule"] == hk.HK_SCHEDULE_SMALLTILE
    assert _plan(hk.HK_DTYPE_BF16, 2048, 2049, 64)["schedule"] == hk.HK_SCHEDULE_INTERLEAVE4


def test_plan_fp8():
    p = _plan(hk.HK_DTYPE_FP8_E4M3, 8192, 8192, 8192)
    assert p["schedule"] == hk.HK_SCHEDULE_INTERLEAVE4
    assert p["kernel_name"] == "hk_gemm_il4_fp8" and p["tile_k"] == 128
    assert p["workgroups"] == 256  # persistent: one workgroup per compute unit
    assert p["threads"] == 256 and p["lds_bytes"] == 131072
    # the ping-pong kernel on request: persistent as well
    p = _plan(hk.HK_DTYPE_FP8_E4M3, 8192, 8192, 8192, schedule="pingpong8")
    assert p["kernel_name"] == "hk_gemm_pp8_fp8" and p["workgroups"] == 256
    assert p["threads"] == 512
    p = _plan(hk.HK_DTYPE_FP8_E4M3, 512, 768, 1024, schedule="pingpong8")
    assert p["workgroups"] == 6  # fewer tiles than compute units: one workgroup each


@pytest.mark.parametrize("K,lda,Aoff", [(60, 60, 0), (64, 66, 0), (64, 64, 2)])
def test_plan_falls_back_to_basic(K, lda, Aoff):
    p = _plan(hk.HK_DTYPE_BF16, 100, 100, K, lda=lda, A=FAKE + Aoff)
    assert p["schedule"] == hk.HK_SCHEDULE_BASIC
    assert p["kernel_name"] == "hk_gemm_basic_bf16"
    assert (p["tiles_m"], p["tiles_n"]) == (2, 2)


def test_plan_fp8_fast_path_needs_16_byte_k():
    assert _plan(hk.HK_DTYPE_FP8_E4M3, 64, 64, 8, lda=16, ldb=16)["schedule"] == hk.HK_SCHEDULE_BASIC
    assert _plan(hk.HK_DTYPE_FP8_E4M3, 64, 64, 32)["schedule"] == hk.HK_SCHEDULE_SMALLTILE


def test_plan_zero_k_uses_the_fill_kernel():
    assert _plan(hk.HK_DTYPE_BF16, 8, 8, 0, lda=1, ldb=1)["kernel_name"] == "hk_zero_c"


def test_plan_options_are_honoured():
    p = _plan(hk.HK_DTYPE_BF16, 4096, 4096, 4096, grid_order="row_major", group_m=4, window=128)
    assert p["grid_order"] == hk.HK_GRID_ROW_MAJOR and p["group_m"] == 4 and p["window"] == 128


def test_plan_rejects_huge_strides():
    with pytest.raises(hk.HKError) as e:
        _plan(hk.HK_DTYPE_BF16, 8, 8, 8, lda=2 ** 30, ldb=8)
    assert e.value.status == hk.HK_ERROR_NOT_SUPPORTED


@pytest.mark.parametrize("schedule,dtype,name,threads", [
    ("interleave4", hk.HK_DTYPE_BF16, "hk_gemm_il4_bf16", 256),
    ("interleave4", hk.HK_DTYPE_FP8_E4M3, "hk_gemm_il4_fp8", 256),
    ("interleave8", hk.HK_DTYPE_BF16, "hk_gemm_i8_bf16", 512),
    ("pingpong8", hk.HK_DTYPE_FP8_E4M3, "hk_gemm_pp8_fp8", 512)])
def test_plan_explicit_schedules(schedule, dtype, name, threads):
    # a large output on request of a schedule (small tiles tested above)
    p = _plan(dtype, 8192, 8192, 8192, schedule=schedule)
    assert p["kernel_name"] == name and p["threads"] == threads
    assert (p["tile_m"], p["tile_n"]) == (256, 256) and p["lds_bytes"] == 131072


def test_plan_producer_consumer():
    p = _plan(hk.HK_DTYPE_BF16, 8192, 8192, 8192, schedule="producer_consumer")
    assert p["kernel_name"] == "hk_gemm_ws_bf16" and p["threads"] == 512
    assert (p["tile_m"], p["tile_n"]) == (256, 128) and (p["tiles_m"], p["tiles_n"]) == (32, 64)
    assert p["workgroups"] == 32 * 64 and p["lds_bytes"] == 2 * (256 + 128) * 128
    with pytest.raises(hk.HKError) as e:
        _plan(hk.HK_DTYPE_FP8_E4M3, 256, 256, 256, schedule="producer_consumer")
    assert e.value.status == hk.HK_ERROR_NOT_SUPPORTED


def test_interleave8_is_bf16_only():
    with pytest.raises(hk.HKError) as e:
        _plan(hk.HK_DTYPE_FP8_E4M3, 256, 256, 256, schedule="interleave8")
    assert e.value.status == hk.HK_ERROR_NOT_SUPPORTED


# ---------------------------------------------------------------- attention

def _attn(L, **kw):
    a = dict(Q=FAKE, K=FAKE, V=FAKE, O=FAKE, lse=None, B=1, Hq=4, Hkv=2, N=256, D=128,
             scale=0.088, causal=0, strides=None)
    a.update(kw)
    st = a["strides"]
    if st is not None:
        s = hk.AttnStrides()
        for name, tri in zip("qkvo", st):
            getattr(s, name)[:] = tri
        st = ctypes.byref(s)
    return L.hk_attn_fwd_bf16(a["Q"], a["K"], a["V"], a["O"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                              a["N"], a["D"], a["scale"], a["causal"], st, None)


@pytest.mark.parametrize("bad", [dict(B=-1), dict(Hq=-1), dict(N=-1), dict(Hkv=0), dict(Hq=3),
                                 dict(D=0), dict(scale=float("nan")), dict(scale=float("inf")),
                                 dict(scale=0.0), dict(scale=-0.5),
                                 dict(Q=0), dict(K=0), dict(V=0), dict(O=0),
                                 dict(strides=[(0, 0, 127), (0, 0, 128), (0, 0, 128), (0, 0, 128)]),
                                 dict(strides=[(-8, 0, 128), (0, 0, 128), (0, 0, 128), (0, 0, 128)])],
                         ids=lambda b: ",".join(b))
def test_attn_invalid_arguments(L, bad):
    assert _attn(L, **bad) == hk.HK_ERROR_INVALID_VALUE


@pytest.mark.parametrize("unsupported", [dict(D=96), dict(D=256), dict(Q=FAKE + 8),
                                         dict(O=FAKE + 2), dict(lse=FAKE + 2),
                                         dict(strides=[(0, 0, 132), (0, 0, 128), (0, 0, 128),
                                                       (0, 0, 128)]),
                                         dict(N=1 << 22, strides=[(0, 0, 128), (0, 0, 1024),
                                                                  (0, 0, 128), (0, 0, 128)])],
                         ids=lambda b: ",".join(b))
def test_attn_unsupported(L, unsupported):
    assert _attn(L, **unsupported) == hk.HK_ERROR_NOT_SUPPORTED


def test_attn_empty_is_a_noop_success(L):
    assert _attn(L, B=0, Q=0, K=0, V=0, O=0) == hk.HK_SUCCESS
    assert _attn(L, N=0, Q=0, K=0, V=0, O=0) == hk.HK_SUCCESS
    assert _attn(L, Hq=0, Q=0, K=0, V=0, O=0) == hk.HK_SUCCESS


def test_plan_fp8_strided_layouts():
    """FP8 (per-tensor scales) with K-strided operands runs on the 4-wave
    kernel; other fast schedules and block scales refuse such operands."""
    FP8 = hk.HK_DTYPE_FP8_E4M3
    for la, lb, name in ((0, 1, "hk_gemm_il4_fp8_bkn"), (1, 0, "hk_gemm_il4_fp8_akm"),
                         (1, 1, "hk_gemm_il4_fp8_akm_bkn")):
        kw = dict(layout_a=la, layout_b=lb, lda=1024 if la else 1024, ldb=1024)
        assert _plan(FP8, 1024, 1024, 1024, **kw)["kernel_name"] == name
        assert _plan(FP8, 1024, 1024, 1024, schedule="interleave4", **kw)["kernel_name"] == name
        for sched in ("pingpong8", "smalltile"):
            with pytest.raises(hk.HKError):
                _plan(FP8, 1024, 1024, 1024, schedule=sched, **kw)
    # a K-strided N that is not whole 16-byte chunks: the plain kernel
    assert _plan(FP8, 1024, 1000, 1024, layout_b=1, ldb=1000)["kernel_name"] == "hk_gemm_basic_fp8"
    # K-rows up to K + 255 are read (128 per stage): the 31-bit offset bound
    # is (K + 256) rows of B, tighter than BF16's K + 128
    K = (1 << 21) - 192
    assert (K + 128) * 1024 + 512 < 2 ** 31 <= (K + 256) * 1024 + 512
    assert _plan(FP8, 1024, 1024, K, layout_b=1, ldb=1024)["kernel_name"] == "hk_gemm_basic_fp8"
    assert _plan(FP8, 1024, 1024, K - 128, layout_b=1,
                 ldb=1024)["kernel_name"] == "hk_gemm_il4_fp8_bkn"
    with pytest.raises(hk.HKError):
        _plan(hk.HK_DTYPE_MXFP8_E4M3, 1024, 1024, 1024, layout_b=1, ldb=1024)


# Repacking straddling operands into a caller-provided workspace.
def test_repack_options_are_validated(L):
    def ex(**f):
        o = hk.GemmOpts()
        for k, v in f.items():
            setattr(o, k, v)
        return L.hk_gemm_ex(0, FAKE, FAKE, FAKE, 32, 32, 64, 64, 64, 32, 1.0, 1.0,
                            ctypes.byref(o), None)
    assert ex(repack=3) == hk.HK_ERROR_INVALID_VALUE
    assert ex(repack=-1) == hk.HK_ERROR_INVALID_VALUE
    assert ex(reserved=1) == hk.HK_ERROR_INVALID_VALUE
    assert ex(workspace=FAKE, workspace_bytes=-1) == hk.HK_ERROR_INVALID_VALUE
    assert ex(workspace_bytes=4096) == hk.HK_ERROR_INVALID_VALUE      # no buffer
    assert ex(workspace=FAKE + 64, workspace_bytes=4096) == hk.HK_ERROR_INVALID_VALUE
    # always repacking with no room for the copy (lda = 72 straddles lines)
    o = hk._opts(repack="always")
    st = L.hk_gemm_ex(0, FAKE, FAKE, FAKE, 32, 32, 64, 72, 64, 32, 1.0, 1.0, ctypes.byref(o), None)
    assert st == hk.HK_ERROR_INVALID_VALUE


def test_device_scale_pointers_are_validated(L):
    """Device-resident scales are for per-tensor FP8 only and must be dword
    aligned; both are checked before any HIP call."""
    def ex(dtype, **f):
        o = hk.GemmOpts()
        for k, v in f.items():
            setattr(o, k, v)
        return L.hk_gemm_ex(dtype, FAKE, FAKE, FAKE, 32, 32, 64, 64, 64, 32, 1.0, 1.0,
                            ctypes.byref(o), None)
    for field in ("scale_a_dev", "scale_b_dev"):
        assert ex(hk.HK_DTYPE_BF16, **{field: FAKE}) == hk.HK_ERROR_INVALID_VALUE, field
        assert ex(hk.HK_DTYPE_MXFP8_E4M3, **{field: FAKE}) == hk.HK_ERROR_INVALID_VALUE, field
        for off in (1, 2, 3):
            st = ex(hk.HK_DTYPE_FP8_E4M3, **{field: FAKE + off})
            assert st == hk.HK_ERROR_INVALID_VALUE, (field, off)
    # a non-finite by-value scale with no pointer to replace it is still rejected
    o = hk.GemmOpts()
    o.scale_a_dev = FAKE
    st = L.hk_gemm_ex(hk.HK_DTYPE_FP8_E4M3, FAKE, FAKE, FAKE, 32, 32, 64, 64, 64, 32, 1.0,
                      float("nan"), ctypes.byref(o), None)
    assert st == hk.HK_ERROR_INVALID_VALUE
    # the plan (validation only) accepts aligned FP8 pointers
    o = hk._opts(scale_a_dev=FAKE, scale_b_dev=FAKE + 4)
    info = hk.PlanInfo()
    assert L.hk_gemm_plan(hk.HK_DTYPE_FP8_E4M3, FAKE, FAKE, FAKE, 32, 32, 64, 64, 64, 32,
                          ctypes.byref(o), ctypes.byref(info)) == hk.HK_SUCCESS


def _ws(M, N, K, lda, ldb, dtype=0, **opts):
    return hk.hk_gemm_workspace_size(dtype, FAKE, FAKE, FAKE, M, N, K, lda, ldb, N, **opts)


def test_workspace_size_policy():
    def c256(x):
        return (x + 255) // 256 * 256
    # the ragged MLP shape: both operands straddle (16 400-byte rows); each is
    # copied to 17 KiB rows
    assert _ws(8191, 28670, 8200, 8200, 8200) == c256(8191 * 17408) + c256(28670 * 17408)
    # only the straddling operand is copied
    assert _ws(8191, 28670, 8200, 8256, 8200) == c256(28670 * 17408)
    # whole-line strides: nothing to do; K-strided operands are never copied
    assert _ws(8192, 8192, 8192, 8192, 8192) == 0
    assert _ws(8192, 8192, 8200, 8192, 8200, layout_a=1, layout_b=1) == 0
    # too small to pay for the copy unless asked; never means never
    assert _ws(1024, 1024, 1032, 1032, 1032) == 0
    assert _ws(1024, 1024, 1032, 1032, 1032, repack="always") == 2 * c256(1024 * 3072)
    assert _ws(8191, 28670, 8200, 8200, 8200, repack="never") == 0
    # 16 KiB rows after rounding would be a multiple of 8 KiB: one KiB more
    assert _ws(8000, 9000, 8184, 8184, 8184) == c256(8000 * 17408) + c256(9000 * 17408)
    # FP8: 8208-byte rows (K a whole number of 16-byte chunks) round to 9 KiB
    assert _ws(8191, 28670, 8208, 8208, 8208, dtype=1) == c256(8191 * 9216) + c256(28670 * 9216)
    # the plain fallback (misaligned pointer) takes operands as they are
    assert hk.hk_gemm_workspace_size(0, FAKE + 2, FAKE, FAKE, 8191, 28670, 8200, 8200, 8200,
                                     28670) == 0
