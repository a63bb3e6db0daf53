"""Python binding of libhkgemm.so (C ABI in include/hk_gemm.h).

Argument marshalling only: every step of the product runs in the library's
HIP kernels.  Functions take device pointers as ints or torch tensors (their
``data_ptr()``), and a stream as a HIP stream handle, a ``torch.cuda.Stream``
or None (torch's current stream on the current device).

The library must have been built (``python -m fp8_gemm_02_amd._build`` or
``__graft_entry__.build()``); there is no fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhkgemm.so")

HK_SUCCESS = 0
HK_ERROR_INVALID_VALUE = 1
HK_ERROR_NOT_SUPPORTED = 2
HK_ERROR_LAUNCH = 3

HK_DTYPE_BF16 = 0
HK_DTYPE_FP8_E4M3 = 1
HK_DTYPE_MXFP8_E4M3 = 2

HK_SCHEDULE_AUTO = 0
HK_SCHEDULE_PINGPONG8 = 1
HK_SCHEDULE_INTERLEAVE4 = 2
HK_SCHEDULE_BASIC = 3
HK_SCHEDULE_INTERLEAVE8 = 4
HK_SCHEDULE_SMALLTILE = 5
HK_SCHEDULE_PRODUCER_CONSUMER = 6

HK_GRID_AUTO = 0
HK_GRID_ROW_MAJOR = 1
HK_GRID_XCD = 2

HK_REPACK_AUTO = 0
HK_REPACK_NEVER = 1
HK_REPACK_ALWAYS = 2

HK_LAYOUT_K_CONTIGUOUS = 0  # A stored M x K, B stored N x K
HK_LAYOUT_K_STRIDED = 1     # A stored K x M, B stored K x N

SCHEDULES = {"auto": 0, "pingpong8": 1, "interleave4": 2, "basic": 3, "interleave8": 4,
             "smalltile": 5, "producer_consumer": 6}
GRID_ORDERS = {"auto": 0, "row_major": 1, "xcd": 2}
LAYOUTS = {"k_contiguous": 0, "k_strided": 1}
REPACKS = {"auto": 0, "never": 1, "always": 2}

EXPORTED = ("hk_gemm_bf16", "hk_gemm_fp8", "hk_gemm_mxfp8", "hk_gemm_ex", "hk_gemm_plan",
            "hk_gemm_ex_noalloc", "hk_gemm_workspace_size", "hk_grid_map", "hk_status_string",
            "hk_version", "hk_wall_clock_khz", "hk_attn_fwd_bf16")


class HKError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s" % (where, status_string(status)))


class GemmOpts(ctypes.Structure):
    _fields_ = [("schedule", ctypes.c_int32), ("grid_order", ctypes.c_int32),
                ("group_m", ctypes.c_int32), ("window", ctypes.c_int32),
                ("layout_a", ctypes.c_int32), ("layout_b", ctypes.c_int32),
                ("clock_stamps", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_int64), ("repack", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("scale_a_dev", ctypes.c_void_p),
                ("scale_b_dev", ctypes.c_void_p)]


class AttnStrides(ctypes.Structure):
    """(batch, head, token) strides in elements of Q, K, V and O."""
    _fields_ = [("q", ctypes.c_int64 * 3), ("k", ctypes.c_int64 * 3),
                ("v", ctypes.c_int64 * 3), ("o", ctypes.c_int64 * 3)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("schedule", ctypes.c_int32), ("grid_order", ctypes.c_int32),
                ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32),
                ("tile_k", ctypes.c_int32), ("threads", ctypes.c_int32),
                ("tiles_m", ctypes.c_int64), ("tiles_n", ctypes.c_int64),
                ("workgroups", ctypes.c_int64), ("lds_bytes", ctypes.c_int32),
                ("group_m", ctypes.c_int32), ("window", ctypes.c_int32),
                ("kernel_name", ctypes.c_char * 96)]

    def as_dict(self):
        d = {name: getattr(self, name) for name, _ in self._fields_ if name != "kernel_name"}
        d["kernel_name"] = self.kernel_name.decode()
        return d


_lib = None


def lib():
    """Load libhkgemm.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError("libhkgemm.so is not built (%s); run python -m fp8_gemm_02_amd._build"
                          % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    i64, i32, vp, f32 = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_float
    L.hk_gemm_bf16.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, vp]
    L.hk_gemm_fp8.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, f32, f32, vp]
    L.hk_gemm_mxfp8.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i64, vp, vp, i64, i64, vp]
    L.hk_gemm_ex.argtypes = [i32, vp, vp, vp, i64, i64, i64, i64, i64, i64, f32, f32,
                             ctypes.POINTER(GemmOpts), vp]
    L.hk_gemm_ex_noalloc.argtypes = [i32, vp, vp, vp, i64, i64, i64, i64, i64, i64, f32, f32,
                                     ctypes.POINTER(GemmOpts), vp]
    L.hk_gemm_plan.argtypes = [i32, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                               ctypes.POINTER(GemmOpts), ctypes.POINTER(PlanInfo)]
    L.hk_gemm_workspace_size.argtypes = [i32, vp, vp, vp, i64, i64, i64, i64, i64, i64,
                                         ctypes.POINTER(GemmOpts), ctypes.POINTER(i64)]
    L.hk_grid_map.argtypes = [i32, i64, i64, i32, i32, i32, i64, vp, vp, vp]
    L.hk_status_string.argtypes = [i32]
    L.hk_status_string.restype = ctypes.c_char_p
    L.hk_version.argtypes = []
    L.hk_wall_clock_khz.argtypes = []
    L.hk_attn_fwd_bf16.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, f32, i32,
                                   ctypes.POINTER(AttnStrides), vp]
    for name in ("hk_gemm_bf16", "hk_gemm_fp8", "hk_gemm_mxfp8", "hk_gemm_ex", "hk_gemm_plan",
                 "hk_gemm_ex_noalloc", "hk_gemm_workspace_size", "hk_grid_map", "hk_version", "hk_wall_clock_khz",
                 "hk_attn_fwd_bf16"):
        getattr(L, name).restype = i32
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().hk_status_string(int(status)).decode()


def _ptr(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(s) -> int:
    if s is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if isinstance(s, int):
        return s
    return int(s.cuda_stream)


def _opts(schedule=0, grid_order=0, group_m=0, window=0, layout_a=0, layout_b=0,
          clock_stamps=None, workspace=None, workspace_bytes=None, repack=0,
          scale_a_dev=None, scale_b_dev=None):
    if isinstance(schedule, str):
        schedule = SCHEDULES[schedule]
    if isinstance(grid_order, str):
        grid_order = GRID_ORDERS[grid_order]
    layout_a = LAYOUTS[layout_a] if isinstance(layout_a, str) else layout_a
    layout_b = LAYOUTS[layout_b] if isinstance(layout_b, str) else layout_b
    o = GemmOpts()
    o.schedule, o.grid_order, o.group_m, o.window = schedule, grid_order, group_m, window
    o.layout_a, o.layout_b = layout_a, layout_b
    o.clock_stamps = _ptr(clock_stamps) or None
    o.workspace = _ptr(workspace) or None
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None or isinstance(workspace, int) else \
            workspace.numel() * workspace.element_size()
    o.workspace_bytes = int(workspace_bytes)
    o.repack = REPACKS[repack] if isinstance(repack, str) else int(repack)
    o.scale_a_dev = _ptr(scale_a_dev) or None
    o.scale_b_dev = _ptr(scale_b_dev) or None
    return o


def _check(status: int, where: str, raise_on_error: bool):
    if raise_on_error and status != HK_SUCCESS:
        raise HKError(status, where)
    return status


def hk_gemm_bf16(A, B, C, M, N, K, lda, ldb, ldc, stream=None, raise_on_error=True):
    st = lib().hk_gemm_bf16(_ptr(A), _ptr(B), _ptr(C), M, N, K, lda, ldb, ldc, _stream(stream))
    return _check(st, "hk_gemm_bf16", raise_on_error)


def hk_gemm_fp8(A, B, C, M, N, K, lda, ldb, ldc, scale_a, scale_b, stream=None,
                raise_on_error=True):
    st = lib().hk_gemm_fp8(_ptr(A), _ptr(B), _ptr(C), M, N, K, lda, ldb, ldc,
                           float(scale_a), float(scale_b), _stream(stream))
    return _check(st, "hk_gemm_fp8", raise_on_error)


def hk_gemm_mxfp8(A, B, C, M, N, K, lda, ldb, ldc, scales_a, scales_b, ld_scales_a,
                  ld_scales_b, stream=None, raise_on_error=True):
    """MXFP8: E4M3 A and B with E8M0 scale bytes, one per 32 K-elements of a row."""
    st = lib().hk_gemm_mxfp8(_ptr(A), _ptr(B), _ptr(C), M, N, K, lda, ldb, ldc, _ptr(scales_a),
                             _ptr(scales_b), ld_scales_a, ld_scales_b, _stream(stream))
    return _check(st, "hk_gemm_mxfp8", raise_on_error)


def hk_gemm_ex(dtype, A, B, C, M, N, K, lda, ldb, ldc, scale_a=1.0, scale_b=1.0,
               schedule=0, grid_order=0, group_m=0, window=0, layout_a=0, layout_b=0,
               stream=None, raise_on_error=True, clock_stamps=None, workspace=None,
               workspace_bytes=None, repack=0, scale_a_dev=None, scale_b_dev=None):
    """clock_stamps: None, or a 16-byte aligned device buffer of 32 uint64 (a
    torch tensor or a pointer) for the launch's clock record.  workspace: None,
    or a 256-byte aligned device buffer (tensor: its size is taken; pointer:
    give workspace_bytes) for repacked operands; repack: "auto", "never",
    "always" (or the HK_REPACK_* value).  scale_a_dev, scale_b_dev: None, or a
    device fp32 (tensor or pointer) read when the kernel runs in place of
    scale_a (scale_b); FP8 only."""
    o = _opts(schedule, grid_order, group_m, window, layout_a, layout_b, clock_stamps,
              workspace, workspace_bytes, repack, scale_a_dev, scale_b_dev)
    st = lib().hk_gemm_ex(int(dtype), _ptr(A), _ptr(B), _ptr(C), M, N, K, lda, ldb, ldc,
                          float(scale_a), float(scale_b), ctypes.byref(o), _stream(stream))
    return _check(st, "hk_gemm_ex", raise_on_error)


def hk_gemm_plan(dtype, A, B, C, M, N, K, lda, ldb, ldc, schedule=0, grid_order=0,
                 group_m=0, window=0, layout_a=0, layout_b=0):
    """Return the launch description as a dict; raises HKError on invalid input."""
    o = _opts(schedule, grid_order, group_m, window, layout_a, layout_b)
    info = PlanInfo()
    st = lib().hk_gemm_plan(int(dtype), _ptr(A), _ptr(B), _ptr(C), M, N, K, lda, ldb, ldc,
                            ctypes.byref(o), ctypes.byref(info))
    _check(st, "hk_gemm_plan", True)
    return info.as_dict()


HK_NOALLOC_SCRATCH_BYTES = 256 << 20


def hk_gemm_ex_noalloc(dtype, A, B, C, M, N, K, lda, ldb, ldc, scale_a=1.0, scale_b=1.0,
                       schedule=0, grid_order=0, group_m=0, window=0, layout_a=0, layout_b=0,
                       stream=None, raise_on_error=True, clock_stamps=None, repack=0,
                       scale_a_dev=None, scale_b_dev=None):
    """hk_gemm_ex with any repack workspace taken from the library's own device
    array (HK_NOALLOC_SCRATCH_BYTES per GPU): the call allocates nothing."""
    o = _opts(schedule, grid_order, group_m, window, layout_a, layout_b, clock_stamps,
              repack=repack, scale_a_dev=scale_a_dev, scale_b_dev=scale_b_dev)
    st = lib().hk_gemm_ex_noalloc(int(dtype), _ptr(A), _ptr(B), _ptr(C), M, N, K, lda, ldb, ldc,
                                  float(scale_a), float(scale_b), ctypes.byref(o),
                                  _stream(stream))
    return _check(st, "hk_gemm_ex_noalloc", raise_on_error)


def hk_gemm_workspace_size(dtype, A, B, C, M, N, K, lda, ldb, ldc, schedule=0, grid_order=0,
                           group_m=0, window=0, layout_a=0, layout_b=0, repack=0):
    """Workspace bytes hk_gemm_ex would use for repacked operands (0 = none)."""
    o = _opts(schedule, grid_order, group_m, window, layout_a, layout_b, repack=repack)
    out = ctypes.c_int64(0)
    st = lib().hk_gemm_workspace_size(int(dtype), _ptr(A), _ptr(B), _ptr(C), M, N, K, lda, ldb,
                                      ldc, ctypes.byref(o), ctypes.byref(out))
    _check(st, "hk_gemm_workspace_size", True)
    return int(out.value)


def hk_grid_map(grid_order, tiles_m, tiles_n, group_m, window, nxcd, wg):
    """Map workgroup ids (sequence of ints) to (tm, tn) lists with the device's map."""
    import numpy as np
    if isinstance(grid_order, str):
        grid_order = GRID_ORDERS[grid_order]
    wg = np.ascontiguousarray(wg, dtype=np.int64)
    tm = np.zeros_like(wg)
    tn = np.zeros_like(wg)
    st = lib().hk_grid_map(int(grid_order), tiles_m, tiles_n, group_m, window, nxcd, wg.size,
                           wg.ctypes.data, tm.ctypes.data, tn.ctypes.data)
    _check(st, "hk_grid_map", True)
    return tm, tn


def hk_version() -> int:
    return int(lib().hk_version())


def hk_wall_clock_khz() -> int:
    """Rate of the constant-rate counter in the clock record, kHz (0 = unknown)."""
    return int(lib().hk_wall_clock_khz())


def chiplet_clocks_ghz(stamps, wall_khz: int):
    """Mean shader clock of each chiplet over one launch, from its clock record.

    stamps: 32 integers as written by the 4-wave kernels (see hk_gemm_opts);
    chiplets whose workgroup did not record (zero spans) are None.
    """
    out = []
    for x in range(8):
        t0, r0, t1, r1 = (int(v) for v in stamps[4 * x:4 * x + 4])
        dr = r1 - r0
        out.append(None if dr <= 0 or t1 <= t0 or wall_khz <= 0
                   else (t1 - t0) / dr * wall_khz * 1e3 / 1e9)
    return out


def gemm_nt(A, B, scale_a=None, scale_b=None, out=None, stream=None, **opts):
    """C = A @ B.T for 2-D torch device tensors (bf16, or uint8/float8_e4m3fn with scales).

    A convenience over hk_gemm_ex: allocates C (bf16) with torch when `out` is
    None; strides are taken from the tensors (rows must be K-contiguous).
    """
    import torch
    M, K = A.shape
    N, K2 = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ: %d vs %d" % (K, K2))
    if A.stride(1) != 1 or B.stride(1) != 1:
        raise ValueError("A and B rows must be contiguous along K")
    fp8 = A.dtype in (torch.uint8, torch.float8_e4m3fn)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    if out.stride(1) != 1:
        raise ValueError("C rows must be contiguous")
    dtype = HK_DTYPE_FP8_E4M3 if fp8 else HK_DTYPE_BF16
    hk_gemm_ex(dtype, A, B, out, M, N, K, A.stride(0) if M > 1 else max(K, 1),
               B.stride(0) if N > 1 else max(K, 1), out.stride(0) if M > 1 else max(N, 1),
               1.0 if scale_a is None else scale_a, 1.0 if scale_b is None else scale_b,
               stream=stream, **opts)
    return out


def matmul(A, B, scale_a=None, scale_b=None, out=None, stream=None, **opts):
    """C = A @ B for 2-D torch device tensors A (M x K) and B (K x N), bf16, or
    uint8/float8_e4m3fn with scales, where each operand is contiguous along one
    of its two dimensions (a plain tensor or a transposed view of one).

    The storage decides the layout: A with unit stride along K is stored M x K
    (K_CONTIGUOUS), along M it is stored K x M (K_STRIDED); B with unit stride
    along K is an N x K array seen transposed (K_CONTIGUOUS), along N it is
    stored K x N (K_STRIDED).  Allocates C (bf16) with torch when `out` is None.
    """
    import torch
    M, K = A.shape
    K2, N = B.shape
    if K2 != K:
        raise ValueError("inner dimensions differ: %d vs %d" % (K, K2))

    def layout(kstride, rstride, rows):
        # (layout, leading dimension) from the strides along K and along rows
        if kstride == 1 and (rows <= 1 or rstride >= K):
            return HK_LAYOUT_K_CONTIGUOUS, rstride if rows > 1 else max(K, 1)
        if rstride == 1 and (K <= 1 or kstride >= rows):
            return HK_LAYOUT_K_STRIDED, kstride if K > 1 else max(rows, 1)
        raise ValueError("each operand must be contiguous along one dimension")

    la, lda = layout(A.stride(1), A.stride(0), M)
    lb, ldb = layout(B.stride(0), B.stride(1), N)
    fp8 = A.dtype in (torch.uint8, torch.float8_e4m3fn)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    if out.stride(1) != 1:
        raise ValueError("C rows must be contiguous")
    dtype = HK_DTYPE_FP8_E4M3 if fp8 else HK_DTYPE_BF16
    hk_gemm_ex(dtype, A, B, out, M, N, K, lda, ldb, out.stride(0) if M > 1 else max(N, 1),
               1.0 if scale_a is None else scale_a, 1.0 if scale_b is None else scale_b,
               layout_a=la, layout_b=lb, stream=stream, **opts)
    return out


def hk_attn_fwd_bf16(Q, K, V, O, lse, B, Hq, Hkv, N, D, scale, causal, strides=None,
                     stream=None, raise_on_error=True):
    """Attention forward (include/hk_attn.h).  strides: None (packed B x H x N x D)
    or four (batch, head, token) stride triples for Q, K, V, O in elements."""
    st = None
    if strides is not None:
        st = AttnStrides()
        for name, tri in zip("qkvo", strides):
            getattr(st, name)[:] = [int(x) for x in tri]
    rc = lib().hk_attn_fwd_bf16(_ptr(Q), _ptr(K), _ptr(V), _ptr(O),
                                _ptr(lse) if lse is not None else None, B, Hq, Hkv, N, D,
                                float(scale), int(bool(causal)),
                                ctypes.byref(st) if st is not None else None, _stream(stream))
    return _check(rc, "hk_attn_fwd_bf16", raise_on_error)


def attention(q, k, v, causal=False, scale=None, return_lse=False, out=None, stream=None):
    """softmax(scale * q k^T [+ causal mask]) v for torch bf16 device tensors of
    shape (B, Hq, N, D) and (B, Hkv, N, D) with D contiguous (any strides
    otherwise; a (B, N, H, D) tensor seen through .transpose(1, 2) works).
    Returns O (B, Hq, N, D), and the fp32 log-sum-exp (B, Hq, N) if asked."""
    import torch
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, N, D) or v.shape != k.shape:
        raise ValueError("k and v must be (B, Hkv, N, D) with q's B, N and D")
    for t in (q, k, v):
        if t.stride(3) != 1:
            raise ValueError("the head dimension must be contiguous")
    if out is None:
        out = torch.empty((B, Hq, N, D), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device) if return_lse else None
    scale = D ** -0.5 if scale is None else scale
    strides = [t.stride()[:3] for t in (q, k, v, out)]
    hk_attn_fwd_bf16(q, k, v, out, lse, B, Hq, Hkv, N, D, scale, causal, strides=strides,
                     stream=stream)
    return (out, lse) if return_lse else out
