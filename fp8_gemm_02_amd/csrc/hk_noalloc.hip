// hk_noalloc.hip -- hk_gemm_ex_noalloc (declared in include/hk_gemm.h): the
// product of hk_gemm_ex with the repack workspace taken from a device array
// the library owns, for callers that cannot allocate device memory.
//
// The array is a file-scope static __device__ object.  In host code its name
// stands for a host-side shadow, not for device memory, so it is never passed
// to a kernel or a copy: the device address comes from hipGetSymbolAddress,
// once per device (with that device current, at the entry point's first call
// on it), and is kept per device.  Every call on one GPU uses that GPU's
// copy; nothing in it needs to start at zero (a repack writes every byte the
// product then reads), and calls that overlap on one GPU race on it.
#include <hip/hip_runtime.h>

#include <mutex>
#include <stdint.h>

#include "hk_gemm.h"

namespace {

constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[HK_NOALLOC_SCRATCH_BYTES];

std::once_flag g_once[kMaxDevices];
void* g_scratch[kMaxDevices];
hipError_t g_err[kMaxDevices];

// The current device's address of `scratch`, looked up once per device.
hk_status scratch_of_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return HK_ERROR_LAUNCH;
    }
    std::call_once(g_once[dev], [dev]() {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) (void)hipGetLastError();
        g_err[dev] = e;
        g_scratch[dev] = e == hipSuccess ? p : nullptr;
    });
    if (g_err[dev] != hipSuccess || g_scratch[dev] == nullptr) return HK_ERROR_LAUNCH;
    *out = g_scratch[dev];
    return HK_SUCCESS;
}

}  // namespace

extern "C" hk_status hk_gemm_ex_noalloc(int32_t dtype, const void* A, const void* B, void* C,
                                        int64_t M, int64_t N, int64_t K, int64_t lda,
                                        int64_t ldb, int64_t ldc, float scale_a, float scale_b,
                                        const hk_gemm_opts* opts, hk_stream_t stream) {
    hk_gemm_opts o = {};
    if (opts) {
        if (opts->workspace != nullptr || opts->workspace_bytes != 0)
            return HK_ERROR_INVALID_VALUE;
        o = *opts;
    }
    // the scratch this call would use, by the same rule as hk_gemm_ex (this
    // also validates every argument before any HIP call)
    int64_t need = 0;
    hk_status s = hk_gemm_workspace_size(dtype, A, B, C, M, N, K, lda, ldb, ldc, &o, &need);
    if (s != HK_SUCCESS) return s;
    if (need > (int64_t)HK_NOALLOC_SCRATCH_BYTES) return HK_ERROR_NOT_SUPPORTED;
    if (need > 0) {
        void* ws = nullptr;
        s = scratch_of_current_device(&ws);
        if (s != HK_SUCCESS) return s;
        o.workspace = ws;
        o.workspace_bytes = (int64_t)HK_NOALLOC_SCRATCH_BYTES;
    }
    return hk_gemm_ex(dtype, A, B, C, M, N, K, lda, ldb, ldc, scale_a, scale_b, &o, stream);
}
