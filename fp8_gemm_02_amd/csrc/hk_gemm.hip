// hk_gemm.hip -- kernels and C ABI of libhkgemm.so (declared in include/hk_gemm.h).
//
// The host side validates arguments before any HIP call, picks a schedule
// and a workgroup order, and enqueues exactly one kernel on the caller's
// stream.  It allocates nothing and never synchronises.
#include <hip/hip_runtime.h>

#include <math.h>
#include <mutex>
#include <stdint.h>
#include <string.h>

#include "hk_gemm.h"
#include "hk_kernels.hpp"

#define HK_VERSION 300  // 0.3.0: device-resident FP8 scales

// ------------------------------------------------------------------ kernels
//
// Unmangled names so that profiler output reads as the schedule and dtype.

extern "C" __global__ void __launch_bounds__(hk::kPP8Threads)
hk_gemm_pp8_bf16(hk::GemmArgs g) {
    __shared__ hk::i32x4 alo0[hk::kPP8HalfI4], ahi0[hk::kPP8HalfI4], b0[hk::kPP8StageI4];
    __shared__ hk::i32x4 alo1[hk::kPP8HalfI4], ahi1[hk::kPP8HalfI4], b1[hk::kPP8StageI4];
    const hk::PP8Buf buf0 = {(HK_LDS hk::i32x4*)alo0, (HK_LDS hk::i32x4*)ahi0, (HK_LDS hk::i32x4*)b0};
    const hk::PP8Buf buf1 = {(HK_LDS hk::i32x4*)alo1, (HK_LDS hk::i32x4*)ahi1, (HK_LDS hk::i32x4*)b1};
    hk::pp8_body<false, 1>(g, buf0, buf1);
}

extern "C" __global__ void __launch_bounds__(hk::kPP8Threads)
hk_gemm_pp8_fp8(hk::GemmArgs g) {
    __shared__ hk::i32x4 alo0[hk::kPP8HalfI4], ahi0[hk::kPP8HalfI4], b0[hk::kPP8StageI4];
    __shared__ hk::i32x4 alo1[hk::kPP8HalfI4], ahi1[hk::kPP8HalfI4], b1[hk::kPP8StageI4];
    const hk::PP8Buf buf0 = {(HK_LDS hk::i32x4*)alo0, (HK_LDS hk::i32x4*)ahi0, (HK_LDS hk::i32x4*)b0};
    const hk::PP8Buf buf1 = {(HK_LDS hk::i32x4*)alo1, (HK_LDS hk::i32x4*)ahi1, (HK_LDS hk::i32x4*)b1};
    hk::pp8_body<true, 1>(g, buf0, buf1);
}

// Two stage buffers of an A and a B image (32 KiB each): 128 KiB.
#define HK_IL4_LDS                                                                   \
    __shared__ hk::i32x4 a0[hk::kIL4StageI4], b0[hk::kIL4StageI4], a1[hk::kIL4StageI4], \
        b1[hk::kIL4StageI4];                                                           \
    const hk::IL4Buf buf0 = {(HK_LDS hk::i32x4*)a0, (HK_LDS hk::i32x4*)b0};            \
    const hk::IL4Buf buf1 = {(HK_LDS hk::i32x4*)a1, (HK_LDS hk::i32x4*)b1}

extern "C" __global__ void __launch_bounds__(hk::kIL4Threads)
hk_gemm_il4_bf16(hk::GemmArgs g) {
    HK_IL4_LDS;
    hk::il4_bf16_body<false, false>(g, buf0, buf1);
}

// operands stored K-strided: A as K x M ("akm"), B as K x N ("bkn")
extern "C" __global__ void __launch_bounds__(hk::kIL4Threads)
hk_gemm_il4_bf16_akm(hk::GemmArgs g) {
    HK_IL4_LDS;
    hk::il4_bf16_body<true, false>(g, buf0, buf1);
}

extern "C" __global__ void __launch_bounds__(hk::kIL4Threads)
hk_gemm_il4_bf16_bkn(hk::GemmArgs g) {
    HK_IL4_LDS;
    hk::il4_bf16_body<false, true>(g, buf0, buf1);
}

extern "C" __global__ void __launch_bounds__(hk::kIL4Threads)
hk_gemm_il4_bf16_akm_bkn(hk::GemmArgs g) {
    HK_IL4_LDS;
    hk::il4_bf16_body<true, true>(g, buf0, buf1);
}

extern "C" __global__ void __launch_bounds__(hk::kIL4Threads)
hk_gemm_il4_fp8(hk::GemmArgs g) {
    HK_IL4_LDS;
    hk::il4_fp8_body<false>(g, buf0, buf1, nullptr);
}

// FP8 operands stored K-strided: A as K x M ("akm"), B as K x N ("bkn")
extern "C" __global__ void __launch_bounds__(hk::kIL4Threads)
hk_gemm_il4_fp8_akm(hk::GemmArgs g) {
    HK_IL4_LDS;
    hk::il4_fp8_body<false, true, false>(g, buf0, buf1, nullptr);
}

extern "C" __global__ void __launch_bounds__(hk::kIL4Threads)
hk_gemm_il4_fp8_bkn(hk::GemmArgs g) {
    HK_IL4_LDS;
    hk::il4_fp8_body<false, false, true>(g, buf0, buf1, nullptr);
}

extern "C" __global__ void __launch_bounds__(hk::kIL4Threads)
hk_gemm_il4_fp8_akm_bkn(hk::GemmArgs g) {
    HK_IL4_LDS;
    hk::il4_fp8_body<false, true, true>(g, buf0, buf1, nullptr);
}

// MXFP8: the FP8 4-wave kernel plus two 8 KiB buffers of block scales (144 KiB).
extern "C" __global__ void __launch_bounds__(hk::kIL4Threads)
hk_gemm_il4_mxfp8(hk::GemmArgs g) {
    HK_IL4_LDS;
    __shared__ hk::i32x4 scl[2 * hk::kMxGroupBytes / 16];
    hk::il4_fp8_body<true>(g, buf0, buf1, (HK_LDS uint8_t*)scl);
}

extern "C" __global__ void __launch_bounds__(hk::kI8Threads)
hk_gemm_i8_bf16(hk::GemmArgs g) {
    HK_IL4_LDS;
    hk::i8_body(g, buf0, buf1);
}

extern "C" __global__ void __launch_bounds__(hk::kSTThreads)
hk_gemm_st4_bf16(hk::GemmArgs g) {
    __shared__ hk::i32x4 ring[hk::kSTStages * 2 * hk::kSTStageI4];
    hk::st4_body<false>(g, (HK_LDS hk::i32x4*)ring);
}

extern "C" __global__ void __launch_bounds__(hk::kSTThreads)
hk_gemm_st4_fp8(hk::GemmArgs g) {
    __shared__ hk::i32x4 ring[hk::kSTStages * 2 * hk::kSTStageI4];
    hk::st4_body<true>(g, (HK_LDS hk::i32x4*)ring);
}

// Producer/consumer ablation: 4 loading waves, 4 computing waves, 256 x 128 tiles.
extern "C" __global__ void __launch_bounds__(hk::kWSThreads)
hk_gemm_ws_bf16(hk::GemmArgs g) {
    __shared__ hk::i32x4 a0[hk::kWSStageAI4], b0[hk::kWSStageBI4], a1[hk::kWSStageAI4],
        b1[hk::kWSStageBI4];
    const hk::IL4Buf buf0 = {(HK_LDS hk::i32x4*)a0, (HK_LDS hk::i32x4*)b0};
    const hk::IL4Buf buf1 = {(HK_LDS hk::i32x4*)a1, (HK_LDS hk::i32x4*)b1};
    hk::ws_body(g, buf0, buf1);
}

extern "C" __global__ void __launch_bounds__(hk::kBasicThreads)
hk_gemm_basic_bf16(hk::GemmArgs g) {
    __shared__ hk::i32x4 sA[hk::kBasicStageI4], sB[hk::kBasicStageI4];
    hk::basic_body<false>(g, (HK_LDS hk::i32x4*)sA, (HK_LDS hk::i32x4*)sB);
}

extern "C" __global__ void __launch_bounds__(hk::kBasicThreads)
hk_gemm_basic_fp8(hk::GemmArgs g) {
    __shared__ hk::i32x4 sA[hk::kBasicStageI4], sB[hk::kBasicStageI4];
    hk::basic_body<true>(g, (HK_LDS hk::i32x4*)sA, (HK_LDS hk::i32x4*)sB);
}

// ------------------------------------------------------------- host side

namespace {

constexpr int kMaxDevices = 64;
constexpr int32_t kDefaultGroupM = 8;
constexpr int32_t kMI355XCUs = 256;
constexpr int64_t kMaxRowBytes = (int64_t)1 << 31;  // strides the 32-bit offsets can address

std::once_flag g_cu_once[kMaxDevices];
int32_t g_cu_count[kMaxDevices];

// Number of compute units of the current device (cached; read once per device).
// Without a usable device, assume MI355X's 256 so that planning still works.
int32_t current_cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return kMI355XCUs;
    }
    std::call_once(g_cu_once[dev], [dev]() {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0) {
            (void)hipGetLastError();
            cus = kMI355XCUs;
        }
        g_cu_count[dev] = cus;
    });
    return g_cu_count[dev];
}

struct Plan {
    int32_t dtype;
    int32_t schedule;
    int32_t grid_order;
    int32_t tile;    // tile rows (M)
    int32_t tile_n;  // tile columns (N); equal to tile unless set otherwise
    int32_t threads;
    int32_t lds_bytes;
    int64_t tiles_m, tiles_n;
    int64_t grid;  // workgroups launched (persistent kernels: at most one per CU)
    hk::GemmArgs args;
    const void* kernel;
    const char* name;
};

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

hk_status validate(int32_t dtype, const void* A, const void* B, const void* C, int64_t M,
                   int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                   const hk_gemm_opts* opts) {
    if (dtype != HK_DTYPE_BF16 && dtype != HK_DTYPE_FP8_E4M3 && dtype != HK_DTYPE_MXFP8_E4M3)
        return HK_ERROR_INVALID_VALUE;
    if (M < 0 || N < 0 || K < 0) return HK_ERROR_INVALID_VALUE;
    if (opts) {
        if (opts->schedule < HK_SCHEDULE_AUTO || opts->schedule > HK_SCHEDULE_PRODUCER_CONSUMER)
            return HK_ERROR_INVALID_VALUE;
        if (opts->grid_order < HK_GRID_AUTO || opts->grid_order > HK_GRID_XCD)
            return HK_ERROR_INVALID_VALUE;
        if (opts->group_m < 0 || opts->window < 0) return HK_ERROR_INVALID_VALUE;
        for (int32_t l : {opts->layout_a, opts->layout_b})
            if (l != HK_LAYOUT_K_CONTIGUOUS && l != HK_LAYOUT_K_STRIDED)
                return HK_ERROR_INVALID_VALUE;
        if (!aligned(opts->clock_stamps, 16)) return HK_ERROR_INVALID_VALUE;
        if (opts->repack < HK_REPACK_AUTO || opts->repack > HK_REPACK_ALWAYS ||
            opts->reserved != 0 || opts->workspace_bytes < 0 ||
            (opts->workspace == nullptr && opts->workspace_bytes != 0) ||
            !aligned(opts->workspace, 256))
            return HK_ERROR_INVALID_VALUE;
        // scales read from device memory: FP8 per-tensor scales only
        if ((opts->scale_a_dev != nullptr || opts->scale_b_dev != nullptr) &&
            dtype != HK_DTYPE_FP8_E4M3)
            return HK_ERROR_INVALID_VALUE;
        if (!aligned(opts->scale_a_dev, 4) || !aligned(opts->scale_b_dev, 4))
            return HK_ERROR_INVALID_VALUE;
    }
    if (M == 0 || N == 0) return HK_SUCCESS;
    if (C == nullptr || ldc < N || !aligned(C, 2)) return HK_ERROR_INVALID_VALUE;
    if (K > 0) {
        const bool at = opts && opts->layout_a == HK_LAYOUT_K_STRIDED;
        const bool bt = opts && opts->layout_b == HK_LAYOUT_K_STRIDED;
        if (A == nullptr || B == nullptr || lda < (at ? M : K) || ldb < (bt ? N : K))
            return HK_ERROR_INVALID_VALUE;
        if (dtype == HK_DTYPE_BF16 && (!aligned(A, 2) || !aligned(B, 2)))
            return HK_ERROR_INVALID_VALUE;
    }
    return HK_SUCCESS;
}

// Fills *p; assumes validate() passed and M, N > 0.
hk_status make_plan(int32_t dtype, const void* A, const void* B, const void* C, int64_t M,
                    int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc, float scale_a,
                    float scale_b, const hk_gemm_opts* opts, Plan* p) {
    memset(p, 0, sizeof(*p));
    const int64_t esz = dtype == HK_DTYPE_BF16 ? 2 : 1;
    if (M > INT32_MAX - 512 || N > INT32_MAX - 512 || K > INT32_MAX / 2)
        return HK_ERROR_NOT_SUPPORTED;
    const int64_t lda_b = (K > 0 ? lda : 0) * esz, ldb_b = (K > 0 ? ldb : 0) * esz;
    if (lda_b >= kMaxRowBytes || ldb_b >= kMaxRowBytes) return HK_ERROR_NOT_SUPPORTED;

    int32_t sched = opts ? opts->schedule : HK_SCHEDULE_AUTO;
    int32_t order = opts ? opts->grid_order : HK_GRID_AUTO;
    if (order == HK_GRID_AUTO) order = HK_GRID_XCD;

    // Fast path: 16-byte direct loads need 16-byte aligned rows and whole
    // 16-byte chunks; 256 rows of stride must fit the 31-bit offsets.  An
    // operand stored K-strided is read in rows of K: its M (or N) must be
    // whole chunks, and K + 128 rows (the stages past K included) must fit.
    const bool at = opts && opts->layout_a == HK_LAYOUT_K_STRIDED;
    const bool bt = opts && opts->layout_b == HK_LAYOUT_K_STRIDED;
    const int64_t chunk = 16 / esz;
    auto operand_ok = [&](const void* X, bool trans, int64_t rows, int64_t ld, int64_t ld_b) {
        if (!aligned(X, 16) || ld % chunk != 0) return false;
        // K-rows read reach K + 127 (BF16, 64 per stage) or K + 255 (FP8, 128)
        if (trans) return rows % chunk == 0 && (K + 256 / esz) * ld_b + 512 < kMaxRowBytes;
        return K % chunk == 0 && ld_b * hk::kPP8Tile < kMaxRowBytes;
    };
    const bool fast_ok = operand_ok(A, at, M, lda, lda_b) && operand_ok(B, bt, N, ldb, ldb_b);
    const bool trans = at || bt;
    if (trans) {
        // the 4-wave BF16 and per-tensor FP8 kernels read K-strided images;
        // BASIC reads anything
        const bool il4_ok = dtype == HK_DTYPE_BF16 || dtype == HK_DTYPE_FP8_E4M3;
        if (sched == HK_SCHEDULE_AUTO)
            sched = fast_ok && il4_ok ? HK_SCHEDULE_INTERLEAVE4 : HK_SCHEDULE_BASIC;
        if (sched != HK_SCHEDULE_BASIC && (sched != HK_SCHEDULE_INTERLEAVE4 || !il4_ok))
            return HK_ERROR_NOT_SUPPORTED;
    }
    if (dtype == HK_DTYPE_MXFP8_E4M3) {
        // block scales: only the 4-wave kernel carries them, on the fast path
        if (sched != HK_SCHEDULE_AUTO && sched != HK_SCHEDULE_INTERLEAVE4)
            return HK_ERROR_NOT_SUPPORTED;
        if (!fast_ok || K % 32 != 0) return HK_ERROR_NOT_SUPPORTED;
        sched = HK_SCHEDULE_INTERLEAVE4;
    }
    // Measured on MI355X: the 4-wave interleave is the faster kernel for both
    // dtypes at 8192^3; outputs with few 256 x 256 tiles (at most one per
    // four compute units) run faster on 128 x 128 tiles with more stages in
    // flight.
    const int32_t cus = current_cu_count();
    if (sched == HK_SCHEDULE_AUTO) {
        const int64_t tiles256 = ((M + 255) / 256) * ((N + 255) / 256);
        sched = !fast_ok ? HK_SCHEDULE_BASIC
                         : (tiles256 * 4 <= cus ? HK_SCHEDULE_SMALLTILE : HK_SCHEDULE_INTERLEAVE4);
    }
    if (sched != HK_SCHEDULE_BASIC && !fast_ok) return HK_ERROR_NOT_SUPPORTED;
    if ((sched == HK_SCHEDULE_INTERLEAVE8 || sched == HK_SCHEDULE_PRODUCER_CONSUMER) &&
        dtype != HK_DTYPE_BF16)
        return HK_ERROR_NOT_SUPPORTED;

    const bool fp8 = dtype != HK_DTYPE_BF16;
    const bool mx = dtype == HK_DTYPE_MXFP8_E4M3;
    if (sched == HK_SCHEDULE_PINGPONG8) {
        p->tile = hk::kPP8Tile;
        p->threads = hk::kPP8Threads;
        p->lds_bytes = 4 * hk::kPP8StageI4 * 16;
        p->kernel = fp8 ? (const void*)hk_gemm_pp8_fp8 : (const void*)hk_gemm_pp8_bf16;
        p->name = fp8 ? "hk_gemm_pp8_fp8" : "hk_gemm_pp8_bf16";
    } else if (sched == HK_SCHEDULE_INTERLEAVE8) {
        p->tile = hk::kIL4Tile;
        p->threads = hk::kI8Threads;
        p->lds_bytes = 4 * hk::kIL4StageI4 * 16;
        p->kernel = (const void*)hk_gemm_i8_bf16;
        p->name = "hk_gemm_i8_bf16";
    } else if (sched == HK_SCHEDULE_PRODUCER_CONSUMER) {
        p->tile = hk::kWSTileM;
        p->tile_n = hk::kWSTileN;
        p->threads = hk::kWSThreads;
        p->lds_bytes = 2 * (hk::kWSStageAI4 + hk::kWSStageBI4) * 16;
        p->kernel = (const void*)hk_gemm_ws_bf16;
        p->name = "hk_gemm_ws_bf16";
    } else if (sched == HK_SCHEDULE_SMALLTILE) {
        p->tile = hk::kSTTile;
        p->threads = hk::kSTThreads;
        p->lds_bytes = hk::kSTStages * 2 * hk::kSTStageI4 * 16;
        p->kernel = fp8 ? (const void*)hk_gemm_st4_fp8 : (const void*)hk_gemm_st4_bf16;
        p->name = fp8 ? "hk_gemm_st4_fp8" : "hk_gemm_st4_bf16";
    } else if (sched == HK_SCHEDULE_INTERLEAVE4) {
        p->tile = hk::kIL4Tile;
        p->threads = hk::kIL4Threads;
        p->lds_bytes = 4 * hk::kIL4StageI4 * 16;
        if (mx) {
            p->kernel = (const void*)hk_gemm_il4_mxfp8;
            p->name = "hk_gemm_il4_mxfp8";
        } else if (fp8 && at && bt) {
            p->kernel = (const void*)hk_gemm_il4_fp8_akm_bkn;
            p->name = "hk_gemm_il4_fp8_akm_bkn";
        } else if (fp8 && at) {
            p->kernel = (const void*)hk_gemm_il4_fp8_akm;
            p->name = "hk_gemm_il4_fp8_akm";
        } else if (fp8 && bt) {
            p->kernel = (const void*)hk_gemm_il4_fp8_bkn;
            p->name = "hk_gemm_il4_fp8_bkn";
        } else if (fp8) {
            p->kernel = (const void*)hk_gemm_il4_fp8;
            p->name = "hk_gemm_il4_fp8";
        } else if (at && bt) {
            p->kernel = (const void*)hk_gemm_il4_bf16_akm_bkn;
            p->name = "hk_gemm_il4_bf16_akm_bkn";
        } else if (at) {
            p->kernel = (const void*)hk_gemm_il4_bf16_akm;
            p->name = "hk_gemm_il4_bf16_akm";
        } else if (bt) {
            p->kernel = (const void*)hk_gemm_il4_bf16_bkn;
            p->name = "hk_gemm_il4_bf16_bkn";
        } else {
            p->kernel = (const void*)hk_gemm_il4_bf16;
            p->name = "hk_gemm_il4_bf16";
        }
        if (mx) p->lds_bytes += 2 * (int64_t)hk::kMxGroupBytes;
    } else {
        p->tile = hk::kBasicTile;
        p->threads = hk::kBasicThreads;
        p->lds_bytes = 2 * hk::kBasicStageI4 * 16;
        p->kernel = fp8 ? (const void*)hk_gemm_basic_fp8 : (const void*)hk_gemm_basic_bf16;
        p->name = fp8 ? "hk_gemm_basic_fp8" : "hk_gemm_basic_bf16";
    }
    p->dtype = dtype;
    p->schedule = sched;
    p->grid_order = order;
    if (p->tile_n == 0) p->tile_n = p->tile;
    p->tiles_m = (M + p->tile - 1) / p->tile;
    p->tiles_n = (N + p->tile_n - 1) / p->tile_n;
    if (p->tiles_m * p->tiles_n > INT32_MAX) return HK_ERROR_NOT_SUPPORTED;

    p->grid = p->tiles_m * p->tiles_n;
    // the 4-wave and ping-pong kernels are persistent: one workgroup per compute unit
    if ((sched == HK_SCHEDULE_INTERLEAVE4 || sched == HK_SCHEDULE_PINGPONG8) && p->grid > cus)
        p->grid = cus;
    hk::GemmArgs& g = p->args;
    g.A = (const uint8_t*)A;
    g.B = (const uint8_t*)B;
    g.C = (uint16_t*)C;
    g.M = (int32_t)M;
    g.N = (int32_t)N;
    g.K = (int32_t)K;
    g.lda_b = (uint32_t)lda_b;
    g.ldb_b = (uint32_t)ldb_b;
    g.ldc = ldc;
    g.scale_pa = opts ? opts->scale_a_dev : nullptr;
    g.scale_pb = opts ? opts->scale_b_dev : nullptr;
    // with one factor read on the device, g.scale carries the other
    g.scale = !(fp8 && !mx)        ? 1.0f
              : g.scale_pa && g.scale_pb ? 1.0f
              : g.scale_pa       ? scale_b
              : g.scale_pb       ? scale_a
                                 : scale_a * scale_b;
    g.SA = nullptr;
    g.SB = nullptr;
    g.ldsa = g.ldsb = 0;
    g.a_t = at;
    g.b_t = bt;
    g.stamps = opts ? opts->clock_stamps : nullptr;
    g.c_align = (aligned(C, 16) && ldc % 8 == 0) ? 16
                : (aligned(C, 8) && ldc % 4 == 0)  ? 8
                : (aligned(C, 4) && ldc % 2 == 0)  ? 4
                                                   : 2;
    g.grid.order = order == HK_GRID_ROW_MAJOR ? hk::kGridRowMajor : hk::kGridXcd;
    g.grid.tiles_m = (int32_t)p->tiles_m;
    g.grid.tiles_n = (int32_t)p->tiles_n;
    g.grid.group_m = (opts && opts->group_m > 0) ? opts->group_m : kDefaultGroupM;
    g.grid.window = (opts && opts->window > 0) ? opts->window : cus;
    g.grid.nxcd = (cus % 8 == 0) ? 8 : 1;
    return HK_SUCCESS;
}

// ------------------------------------------------------------- repacking
//
// Rows of a K-contiguous operand whose stride is not a whole number of
// 128-byte cache lines make every 128-byte stage segment but one in eight
// span two lines; the call can first copy such an operand to a padded stride
// in a caller-provided workspace (include/hk_gemm.h, hk_repack).

struct Repack {
    int64_t a_ld_b = 0, b_ld_b = 0;  // padded strides in bytes; 0 = operand not repacked
    int64_t a_off = 0, b_off = 0;    // byte offsets of the copies in the workspace
    int64_t bytes = 0;               // workspace used
};

// The padded stride: the row rounded up to 1024 bytes, plus 1024 when that
// is a multiple of 8192 (measured on the 8191 x 28670 x 8200 product: 17 KiB
// rows ran 2615 us, 16 KiB + 128 B 2707 us, 16 KiB + 256 B 2629 us).
int64_t padded_stride(int64_t row_bytes) {
    int64_t s = (row_bytes + 1023) / 1024 * 1024;
    if (s % 8192 == 0) s += 1024;
    return s;
}

// Which operands a call with plan p repacks, given avail workspace bytes.
// Returns HK_ERROR_INVALID_VALUE for REPACK_ALWAYS without room.
hk_status plan_repack(const Plan& p, int64_t M, int64_t N, int64_t K, const hk_gemm_opts* opts,
                      int64_t avail, Repack* r) {
    *r = Repack();
    const int32_t mode = opts ? opts->repack : HK_REPACK_AUTO;
    if (mode == HK_REPACK_NEVER || K == 0 || p.schedule == HK_SCHEDULE_BASIC) return HK_SUCCESS;
    const int64_t esz = p.dtype == HK_DTYPE_BF16 ? 2 : 1;
    const int64_t row_bytes = K * esz;
    const bool at = opts && opts->layout_a == HK_LAYOUT_K_STRIDED;
    const bool bt = opts && opts->layout_b == HK_LAYOUT_K_STRIDED;
    const bool rep_a = !at && p.args.lda_b % hk::kRowBytes != 0;
    const bool rep_b = !bt && p.args.ldb_b % hk::kRowBytes != 0;
    if (!rep_a && !rep_b) return HK_SUCCESS;
    // the copy reads and writes (M + N) K elements; the straddling costs a
    // share of the 2 M N K product: it pays when M N / (M + N) is large
    if (mode == HK_REPACK_AUTO && M * N < 4096 * (M + N)) return HK_SUCCESS;
    Repack q;
    const int64_t stride = padded_stride(row_bytes);
    if (rep_a) {
        q.a_ld_b = stride;
        q.a_off = 0;
        q.bytes = (M * stride + 255) / 256 * 256;
    }
    if (rep_b) {
        q.b_ld_b = stride;
        q.b_off = q.bytes;
        q.bytes += (N * stride + 255) / 256 * 256;
    }
    if (q.bytes > avail) return mode == HK_REPACK_ALWAYS ? HK_ERROR_INVALID_VALUE : HK_SUCCESS;
    *r = q;
    return HK_SUCCESS;
}

// Copy the rows of up to two operands (A's rows, then B's), each row cpr
// 16-byte chunks, from src (row stride sld chunks) to dst (stride dld
// chunks), in one launch: one row per workgroup at a time, four chunks per
// thread in flight.  The stores are nontemporal: on the ragged MLP shape
// they took the two copies from 42.6 + 182.3 to 39.4 + 166.1 us, and the
// product on the copies did not slow down.
typedef uint32_t repack_u32x4 __attribute__((ext_vector_type(4)));
struct RepackJob {
    const repack_u32x4* src;
    int64_t sld;
    repack_u32x4* dst;
    int64_t dld;
    int64_t rows;
};
__global__ void __launch_bounds__(256) hk_repack_rows(RepackJob ja, RepackJob jb, int32_t cpr) {
    const int64_t rows = ja.rows + jb.rows;
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const bool in_a = r < ja.rows;
        const RepackJob& j = in_a ? ja : jb;
        const int64_t rr = in_a ? r : r - ja.rows;
        const repack_u32x4* s = j.src + rr * j.sld;
        repack_u32x4* d = j.dst + rr * j.dld;
        int32_t c = (int32_t)threadIdx.x;
        for (; c + 768 < cpr; c += 1024) {
            const repack_u32x4 v0 = s[c], v1 = s[c + 256], v2 = s[c + 512], v3 = s[c + 768];
            __builtin_nontemporal_store(v0, d + c);
            __builtin_nontemporal_store(v1, d + c + 256);
            __builtin_nontemporal_store(v2, d + c + 512);
            __builtin_nontemporal_store(v3, d + c + 768);
        }
        for (; c < cpr; c += 256) __builtin_nontemporal_store(s[c], d + c);
    }
}

// One launch copying A's and/or B's rows (rows = 0 skips an operand); strides
// in bytes, all multiples of 16.
hk_status repack_rows(const void* a_src, int64_t a_src_ld_b, void* a_dst, int64_t a_dst_ld_b,
                      int64_t a_rows, const void* b_src, int64_t b_src_ld_b, void* b_dst,
                      int64_t b_dst_ld_b, int64_t b_rows, int64_t row_bytes, hipStream_t stream) {
    const RepackJob ja{(const repack_u32x4*)a_src, a_src_ld_b / 16, (repack_u32x4*)a_dst,
                       a_dst_ld_b / 16, a_rows};
    const RepackJob jb{(const repack_u32x4*)b_src, b_src_ld_b / 16, (repack_u32x4*)b_dst,
                       b_dst_ld_b / 16, b_rows};
    const int64_t rows = a_rows + b_rows;
    const int64_t blocks = rows < 8192 ? rows : 8192;
    hipLaunchKernelGGL(hk_repack_rows, dim3((uint32_t)blocks), dim3(256), 0, stream, ja, jb,
                       (int32_t)(row_bytes / 16));
    if (hipGetLastError() != hipSuccess) return HK_ERROR_LAUNCH;
    return HK_SUCCESS;
}

// C = 0 for K == 0 (the empty sum), any dtype.
__global__ void hk_zero_c(uint16_t* C, int64_t M, int64_t N, int64_t ldc) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < M * N) C[(i / N) * ldc + i % N] = 0;
}

hk_status launch(const Plan& p, hipStream_t stream) {
    const int64_t grid = p.grid;
    hk::GemmArgs args = p.args;
    void* kargs[] = {&args};
    hipError_t e = hipLaunchKernel(p.kernel, dim3((uint32_t)grid), dim3((uint32_t)p.threads),
                                   kargs, 0, stream);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return HK_ERROR_LAUNCH;
    }
    return HK_SUCCESS;
}

hk_status zero_c(void* C, int64_t M, int64_t N, int64_t ldc, hipStream_t stream) {
    const int64_t total = M * N;
    const int64_t blocks = (total + 255) / 256;
    if (blocks > INT32_MAX) return HK_ERROR_NOT_SUPPORTED;
    hipLaunchKernelGGL(hk_zero_c, dim3((uint32_t)blocks), dim3(256), 0, stream, (uint16_t*)C, M,
                       N, ldc);
    if (hipGetLastError() != hipSuccess) return HK_ERROR_LAUNCH;
    return HK_SUCCESS;
}

hk_status gemm_common(int32_t dtype, const void* A, const void* B, void* C, int64_t M, int64_t N,
                      int64_t K, int64_t lda, int64_t ldb, int64_t ldc, float scale_a,
                      float scale_b, const hk_gemm_opts* opts, hipStream_t stream) {
    // block-scaled FP8 needs its scale arrays: hk_gemm_mxfp8
    if (dtype == HK_DTYPE_MXFP8_E4M3) return HK_ERROR_INVALID_VALUE;
    hk_status s = validate(dtype, A, B, C, M, N, K, lda, ldb, ldc, opts);
    if (s != HK_SUCCESS) return s;
    // a by-value scale counts unless a device pointer replaces it
    if (dtype == HK_DTYPE_FP8_E4M3 &&
        ((!isfinite(scale_a) && !(opts && opts->scale_a_dev)) ||
         (!isfinite(scale_b) && !(opts && opts->scale_b_dev))))
        return HK_ERROR_INVALID_VALUE;
    if (M == 0 || N == 0) return HK_SUCCESS;
    Plan p;
    s = make_plan(dtype, A, B, C, M, N, K, lda, ldb, ldc, scale_a, scale_b, opts, &p);
    if (s != HK_SUCCESS) return s;
    if (K == 0) return zero_c(C, M, N, ldc, stream);
    Repack rp;
    s = plan_repack(p, M, N, K, opts, opts ? opts->workspace_bytes : 0, &rp);
    if (s != HK_SUCCESS) return s;
    if (rp.bytes == 0) return launch(p, stream);
    // copy the straddling operands to padded strides, then run on the copies
    const int64_t esz = dtype == HK_DTYPE_BF16 ? 2 : 1;
    uint8_t* ws = (uint8_t*)opts->workspace;
    const void* A2 = A;
    const void* B2 = B;
    int64_t lda2 = lda, ldb2 = ldb;
    s = repack_rows(A, lda * esz, ws + rp.a_off, rp.a_ld_b, rp.a_ld_b ? M : 0, B, ldb * esz,
                    ws + rp.b_off, rp.b_ld_b, rp.b_ld_b ? N : 0, K * esz, stream);
    if (s != HK_SUCCESS) return s;
    if (rp.a_ld_b) {
        A2 = ws + rp.a_off;
        lda2 = rp.a_ld_b / esz;
    }
    if (rp.b_ld_b) {
        B2 = ws + rp.b_off;
        ldb2 = rp.b_ld_b / esz;
    }
    Plan p2;
    s = make_plan(dtype, A2, B2, C, M, N, K, lda2, ldb2, ldc, scale_a, scale_b, opts, &p2);
    if (s != HK_SUCCESS) return s;
    p2.args.stamps = p.args.stamps;
    return launch(p2, stream);
}

hk_status gemm_mx(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                  int64_t lda, int64_t ldb, int64_t ldc, const void* SA, const void* SB,
                  int64_t ldsa, int64_t ldsb, hipStream_t stream) {
    hk_status s = validate(HK_DTYPE_MXFP8_E4M3, A, B, C, M, N, K, lda, ldb, ldc, nullptr);
    if (s != HK_SUCCESS) return s;
    if (M == 0 || N == 0) return HK_SUCCESS;
    if (K > 0) {
        const int64_t nb = (K + 31) / 32;
        if (SA == nullptr || SB == nullptr || ldsa < nb || ldsb < nb) return HK_ERROR_INVALID_VALUE;
        // scales travel as 16-byte direct loads of whole rows
        if (!aligned(SA, 16) || !aligned(SB, 16) || ldsa % 16 != 0 || ldsb % 16 != 0 ||
            ldsa * hk::kIL4Tile >= kMaxRowBytes || ldsb * hk::kIL4Tile >= kMaxRowBytes)
            return HK_ERROR_NOT_SUPPORTED;
    }
    Plan p;
    s = make_plan(HK_DTYPE_MXFP8_E4M3, A, B, C, M, N, K, lda, ldb, ldc, 1.0f, 1.0f, nullptr,
                  &p);
    if (s != HK_SUCCESS) return s;
    if (K == 0) return zero_c(C, M, N, ldc, stream);
    p.args.SA = (const uint8_t*)SA;
    p.args.SB = (const uint8_t*)SB;
    p.args.ldsa = (uint32_t)ldsa;
    p.args.ldsb = (uint32_t)ldsb;
    return launch(p, stream);
}

}  // namespace

// ------------------------------------------------------------------ C ABI

extern "C" {

hk_status hk_gemm_bf16(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                       int64_t lda, int64_t ldb, int64_t ldc, hk_stream_t stream) {
    return gemm_common(HK_DTYPE_BF16, A, B, C, M, N, K, lda, ldb, ldc, 1.0f, 1.0f, nullptr,
                       (hipStream_t)stream);
}

hk_status hk_gemm_fp8(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                      int64_t lda, int64_t ldb, int64_t ldc, float scale_a, float scale_b,
                      hk_stream_t stream) {
    return gemm_common(HK_DTYPE_FP8_E4M3, A, B, C, M, N, K, lda, ldb, ldc, scale_a, scale_b,
                       nullptr, (hipStream_t)stream);
}

hk_status hk_gemm_mxfp8(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                        int64_t lda, int64_t ldb, int64_t ldc, const void* scales_a,
                        const void* scales_b, int64_t ld_scales_a, int64_t ld_scales_b,
                        hk_stream_t stream) {
    return gemm_mx(A, B, C, M, N, K, lda, ldb, ldc, scales_a, scales_b, ld_scales_a, ld_scales_b,
                   (hipStream_t)stream);
}

hk_status hk_gemm_ex(int32_t dtype, const void* A, const void* B, void* C, int64_t M, int64_t N,
                     int64_t K, int64_t lda, int64_t ldb, int64_t ldc, float scale_a,
                     float scale_b, const hk_gemm_opts* opts, hk_stream_t stream) {
    return gemm_common(dtype, A, B, C, M, N, K, lda, ldb, ldc, scale_a, scale_b, opts,
                       (hipStream_t)stream);
}

hk_status hk_gemm_plan(int32_t dtype, const void* A, const void* B, const void* C, int64_t M,
                       int64_t N, int64_t K, int64_t lda, int64_t ldb, int64_t ldc,
                       const hk_gemm_opts* opts, hk_gemm_plan_info* out) {
    if (out == nullptr) return HK_ERROR_INVALID_VALUE;
    hk_status s = validate(dtype, A, B, C, M, N, K, lda, ldb, ldc, opts);
    if (s != HK_SUCCESS) return s;
    memset(out, 0, sizeof(*out));
    if (M == 0 || N == 0) return HK_SUCCESS;
    Plan p;
    s = make_plan(dtype, A, B, C, M, N, K, lda, ldb, ldc, 1.0f, 1.0f, opts, &p);
    if (s != HK_SUCCESS) return s;
    out->schedule = p.schedule;
    out->grid_order = p.grid_order;
    out->tile_m = p.tile;
    out->tile_n = p.tile_n;
    out->tile_k = hk::kRowBytes / (dtype == HK_DTYPE_BF16 ? 2 : 1);
    out->threads = p.threads;
    out->tiles_m = p.tiles_m;
    out->tiles_n = p.tiles_n;
    out->workgroups = p.grid;
    out->lds_bytes = p.lds_bytes;
    out->group_m = p.args.grid.group_m;
    out->window = p.args.grid.window;
    strncpy(out->kernel_name, K == 0 ? "hk_zero_c" : p.name, sizeof(out->kernel_name) - 1);
    return HK_SUCCESS;
}

hk_status hk_gemm_workspace_size(int32_t dtype, const void* A, const void* B, const void* C,
                                 int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                                 int64_t ldc, const hk_gemm_opts* opts, int64_t* bytes) {
    if (bytes == nullptr) return HK_ERROR_INVALID_VALUE;
    *bytes = 0;
    if (dtype == HK_DTYPE_MXFP8_E4M3) return HK_SUCCESS;  // hk_gemm_mxfp8 never repacks
    hk_status s = validate(dtype, A, B, C, M, N, K, lda, ldb, ldc, opts);
    if (s != HK_SUCCESS) return s;
    if (M == 0 || N == 0 || K == 0) return HK_SUCCESS;
    Plan p;
    s = make_plan(dtype, A, B, C, M, N, K, lda, ldb, ldc, 1.0f, 1.0f, opts, &p);
    if (s != HK_SUCCESS) return s;
    Repack rp;
    s = plan_repack(p, M, N, K, opts, INT64_MAX, &rp);
    if (s != HK_SUCCESS) return s;
    *bytes = rp.bytes;
    return HK_SUCCESS;
}

hk_status hk_grid_map(int32_t grid_order, int64_t tiles_m, int64_t tiles_n, int32_t group_m,
                      int32_t window, int32_t nxcd, int64_t count, const int64_t* wg,
                      int64_t* tm, int64_t* tn) {
    if (grid_order != HK_GRID_ROW_MAJOR && grid_order != HK_GRID_XCD)
        return HK_ERROR_INVALID_VALUE;
    if (tiles_m <= 0 || tiles_n <= 0 || tiles_m * tiles_n > INT32_MAX || group_m <= 0 ||
        window <= 0 || nxcd <= 0 || count < 0)
        return HK_ERROR_INVALID_VALUE;
    if (count > 0 && (wg == nullptr || tm == nullptr || tn == nullptr))
        return HK_ERROR_INVALID_VALUE;
    const int64_t total = tiles_m * tiles_n;
    for (int64_t i = 0; i < count; ++i)
        if (wg[i] < 0 || wg[i] >= total) return HK_ERROR_INVALID_VALUE;
    hk::GridParams gp;
    gp.order = grid_order == HK_GRID_ROW_MAJOR ? hk::kGridRowMajor : hk::kGridXcd;
    gp.tiles_m = (int32_t)tiles_m;
    gp.tiles_n = (int32_t)tiles_n;
    gp.group_m = group_m;
    gp.window = window;
    gp.nxcd = nxcd;
    for (int64_t i = 0; i < count; ++i) {
        uint32_t a, b;
        hk::tile_of((uint32_t)wg[i], gp, &a, &b);
        tm[i] = a;
        tn[i] = b;
    }
    return HK_SUCCESS;
}

const char* hk_status_string(hk_status status) {
    switch (status) {
        case HK_SUCCESS: return "HK_SUCCESS";
        case HK_ERROR_INVALID_VALUE: return "HK_ERROR_INVALID_VALUE";
        case HK_ERROR_NOT_SUPPORTED: return "HK_ERROR_NOT_SUPPORTED";
        case HK_ERROR_LAUNCH: return "HK_ERROR_LAUNCH";
    }
    return "HK_UNKNOWN_STATUS";
}

int32_t hk_version(void) { return HK_VERSION; }

int32_t hk_wall_clock_khz(void) {
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return khz;
}

}  // extern "C"
