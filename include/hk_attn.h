/*
 * hk_attn.h -- C ABI of libhkgemm.so's attention forward on one MI355X (gfx950).
 *
 * The operation.  "How to make AMD GPUs go brrr" (GeekNews summary, section
 * "Real kernel example") names attention forward as the second hot loop built
 * on the GEMM's wave schedules, and "HipKittens: fast and furious AMD kernels"
 * (section "Performance results") reports it over several head dimensions D
 * and sequence lengths N, causal and non-causal.  Neither page writes it out
 * or gives an interface, so this one is ours: scaled dot-product attention
 *
 *     s_ij   = scale * sum_{d<D} Q[b,h,i,d] * K[b,g(h),j,d]
 *     O[b,h,i,:] = bf16_rne( sum_j softmax_j(s_i.) * V[b,g(h),j,:] )
 *     lse[b,h,i] = log sum_j exp(s_ij)
 *
 * over keys j < N (j <= i with causal != 0), for 0 <= b < B, 0 <= h < Hq,
 * 0 <= i < N, with g(h) = h / (Hq / Hkv): each key/value head serves Hq/Hkv
 * consecutive query heads (grouped-query attention; Hkv = Hq is plain
 * multi-head attention).  Q, K and V are BF16 bit patterns, the softmax and
 * both products run in FP32, O is BF16 (round to nearest even) and lse is
 * FP32.
 *
 * Layout.  Element (b, h, t, d) of Q, K, V or O sits at
 * b*s[0] + h*s[1] + t*s[2] + d (elements; d contiguous), with the strides in
 * hk_attn_strides; strides == NULL means packed B x H x N x D for all four.
 * lse, when not NULL, is packed B x Hq x N fp32.
 *
 * Ownership, ordering, errors: as for the GEMM entry points (hk_gemm.h).
 * Device pointers owned by the caller; one kernel enqueued on `stream`; no
 * allocation, no synchronisation.  HK_ERROR_INVALID_VALUE, before any HIP
 * call: negative B, Hq, Hkv or N; Hkv < 1 or Hq not a multiple of Hkv;
 * D < 1; a scale that is not finite and positive; a NULL Q, K, V or O when
 * there is work; a negative stride or a token stride below D.
 * HK_ERROR_NOT_SUPPORTED: D other than 64 or 128; Q, K, V or O not 16-byte aligned; a stride not a multiple
 * of 8; (N + 128) token strides of K or V spanning 2^31 bytes or more.
 * B * Hq * N == 0 is a no-op success.
 */
#ifndef HK_ATTN_H
#define HK_ATTN_H

#include <stdint.h>

#include "hk_gemm.h"

#ifdef __cplusplus
extern "C" {
#endif

/* (batch, head, token) strides in elements of Q, K, V and O. */
typedef struct hk_attn_strides {
    int64_t q[3];
    int64_t k[3];
    int64_t v[3];
    int64_t o[3];
} hk_attn_strides;

hk_status hk_attn_fwd_bf16(const void *Q, const void *K, const void *V, void *O, float *lse,
                           int64_t B, int64_t Hq, int64_t Hkv, int64_t N, int64_t D,
                           float scale, int32_t causal, const hk_attn_strides *strides,
                           hk_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* HK_ATTN_H */
