// hk_attn.hip -- attention-forward kernels and their C ABI (include/hk_attn.h).
//
// Validates arguments before any HIP call, then enqueues one kernel on the
// caller's stream; allocates nothing and never synchronises.
#include <hip/hip_runtime.h>

#include <math.h>
#include <mutex>
#include <stdint.h>
#include <string.h>

#include "hk_attn.h"
#include "hk_attn.hpp"

// Two buffers of a K and a V block image: 4 x 64 x D bf16.  Without a mask
// one workgroup per 128-query block (the hardware's dispatch keeps the
// compute units fed); with a causal mask a persistent grid over pairs of
// query blocks, the longest with the shortest, so that every workgroup does
// the same work (measured at B=4, H=16, N=4096, D=128: 988 against 889
// TFLOP/s; without the mask the persistent form lost, 1067 against 1106).
#define HK_ATTN_KERNEL(NAME, D, CAUSAL)                                           \
    extern "C" __global__ void __launch_bounds__(                                 \
        hk::kAttnThreads, (CAUSAL) ? hk::attn_slots<(D)>() : 2) NAME(hk::AttnArgs g) { \
        __shared__ hk::i32x4 lds[4 * hk::kAttnKV * (D) * 2 / 16];                 \
        if constexpr (CAUSAL)                                                     \
            hk::attn_fwd_persist<(D), true>(g, (HK_LDS uint8_t*)lds);             \
        else                                                                      \
            hk::attn_fwd_body<(D), false>(g, (HK_LDS uint8_t*)lds);               \
    }

HK_ATTN_KERNEL(hk_attn_fwd_d64, 64, false)
HK_ATTN_KERNEL(hk_attn_fwd_d64_causal, 64, true)
HK_ATTN_KERNEL(hk_attn_fwd_d128, 128, false)
HK_ATTN_KERNEL(hk_attn_fwd_d128_causal, 128, true)

namespace {

constexpr int64_t kMaxBytes = (int64_t)1 << 31;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

constexpr int kMaxDevices = 64;
std::once_flag g_cu_once[kMaxDevices];
int32_t g_cu_count[kMaxDevices];

// Compute units of the current device (read once per device); 256 (MI355X)
// when the runtime cannot say.
int32_t cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return 256;
    }
    std::call_once(g_cu_once[dev], [dev]() {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0) {
            (void)hipGetLastError();
            cus = 256;
        }
        g_cu_count[dev] = cus;
    });
    return g_cu_count[dev];
}

}  // namespace

extern "C" hk_status hk_attn_fwd_bf16(const void* Q, const void* K, const void* V, void* O,
                                      float* lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t N,
                                      int64_t D, float scale, int32_t causal,
                                      const hk_attn_strides* strides, hk_stream_t stream) {
    if (B < 0 || Hq < 0 || N < 0 || Hkv < 1 || D < 1 || Hq % Hkv != 0 || !(isfinite(scale) && scale > 0.0f))
        return HK_ERROR_INVALID_VALUE;
    hk_attn_strides st;
    if (strides) {
        st = *strides;
    } else {
        const int64_t q[3] = {Hq * N * D, N * D, D}, kv[3] = {Hkv * N * D, N * D, D};
        memcpy(st.q, q, sizeof q);
        memcpy(st.k, kv, sizeof kv);
        memcpy(st.v, kv, sizeof kv);
        memcpy(st.o, q, sizeof q);
    }
    const int64_t* all[4] = {st.q, st.k, st.v, st.o};
    for (const int64_t* s : all)
        if (s[0] < 0 || s[1] < 0 || s[2] < D) return HK_ERROR_INVALID_VALUE;
    if (B * Hq * N == 0) return HK_SUCCESS;
    if (!Q || !K || !V || !O) return HK_ERROR_INVALID_VALUE;

    if (D != 64 && D != 128) return HK_ERROR_NOT_SUPPORTED;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) ||
        ((uintptr_t)lse & 3u) != 0)
        return HK_ERROR_NOT_SUPPORTED;
    for (const int64_t* s : all)
        for (int i = 0; i < 3; ++i)
            if (s[i] % 8 != 0) return HK_ERROR_NOT_SUPPORTED;
    // 32-bit buffer offsets over a head's rows, the blocks past N included
    if ((N + 128) * st.k[2] * 2 >= kMaxBytes || (N + 128) * st.v[2] * 2 >= kMaxBytes)
        return HK_ERROR_NOT_SUPPORTED;
    if (B > INT32_MAX || Hq > INT32_MAX || N > INT32_MAX - 256) return HK_ERROR_NOT_SUPPORTED;

    hk::AttnArgs g;
    memset(&g, 0, sizeof g);
    g.Q = (const uint16_t*)Q;
    g.K = (const uint16_t*)K;
    g.V = (const uint16_t*)V;
    g.O = (uint16_t*)O;
    g.lse = lse;
    g.B = (int32_t)B;
    g.Hq = (int32_t)Hq;
    g.Hkv = (int32_t)Hkv;
    g.N = (int32_t)N;
    g.nqb = (int32_t)((N + hk::kAttnQ - 1) / hk::kAttnQ);
    g.group = (int32_t)(Hq / Hkv);
    g.c = scale * 1.4426950408889634f;
    memcpy(g.sq, st.q, sizeof g.sq);
    memcpy(g.sk, st.k, sizeof g.sk);
    memcpy(g.sv, st.v, sizeof g.sv);
    memcpy(g.so, st.o, sizeof g.so);
    // work units: query blocks, or under a causal mask pairs of them (the
    // longest with the shortest)
    g.upH = causal ? (g.nqb + 1) / 2 : g.nqb;
    if (B * Hq * g.nqb > INT32_MAX) return HK_ERROR_NOT_SUPPORTED;
    g.nunits = (int32_t)(B * Hq * g.upH);
    // causal: persistent, as many workgroups per compute unit as its
    // registers take; otherwise one workgroup per query block
    const int64_t slots = (D == 64 ? hk::attn_slots<64>() : hk::attn_slots<128>()) *
                          (int64_t)cu_count();
    const int64_t grid = !causal ? B * Hq * g.nqb : g.nunits < slots ? g.nunits : slots;

    const void* kern = D == 64 ? (causal ? (const void*)hk_attn_fwd_d64_causal
                                         : (const void*)hk_attn_fwd_d64)
                               : (causal ? (const void*)hk_attn_fwd_d128_causal
                                         : (const void*)hk_attn_fwd_d128);
    void* kargs[] = {&g};
    if (hipLaunchKernel(kern, dim3((uint32_t)grid), dim3(hk::kAttnThreads), kargs, 0,
                        (hipStream_t)stream) != hipSuccess) {
        (void)hipGetLastError();
        return HK_ERROR_LAUNCH;
    }
    return HK_SUCCESS;
}
