// hk_attn.hpp -- attention forward on gfx950: O = softmax(scale * Q K^T
// [+ causal mask]) V over BF16 Q, K, V, FP32 softmax and accumulation, BF16 O.
//
// The pages' second workload ("How to make AMD GPUs go brrr", section "Real
// kernel example": the attention-forward hot loop runs on the same wave
// schedules as the BF16 GEMM and uses exp2 and column sums; "HipKittens: fast
// and furious AMD kernels", section "Performance results": causal and
// non-causal, several head dimensions and sequence lengths).
//
// One workgroup of 4 waves takes 128 query rows of one (batch, head); each
// wave owns 32 of them (two 16-row blocks) and keeps their Q fragments in
// registers.  Keys and values stream through LDS in blocks of 64 (direct
// HBM->LDS loads, two buffers), and each block updates the running softmax
// (online: running max m and sum l per query, in log2 units, the output
// rescaled by exp2(m_old - m_new)).
//
// Everything is computed transposed, which keeps every per-query quantity in
// one lane and the probabilities in the registers that produced them:
//
//   S^T (keys x queries) = K Q^T    16x16x32 MFMA, "A" = K rows, "B" = Q rows:
//                                   lane l holds query l%16, keys 4(l/16)..+3
//   O^T (d x queries)   += V^T P^T  "A" = V^T (transposing LDS reads of V),
//                                   "B" = P^T: lane l's 8 K-slots are its own
//                                   probabilities of two 16-key blocks
//
// so the result lane l holds query l%16, d = 4(l/16)..+3: four consecutive
// outputs of one row, stored as one 8-byte write.  The row max needs two
// cross-lane exchanges per block (the four lanes that share a query); the row
// sum stays per lane until the end.
//
// Two workgroups share a compute unit (2 waves per SIMD), so one wave's
// softmax arithmetic runs while the other's matrix instructions do.
//
// The softmax reference point moves lazily: only when a query's block max
// exceeds it by more than kLazy (log2 units) is the output rescaled, so most
// blocks skip the rescale; the weights then stay below 2^kLazy.
#pragma once

#include "hk_device.hpp"

namespace hk {

struct AttnArgs {
    const uint16_t* Q;
    const uint16_t* K;
    const uint16_t* V;
    uint16_t* O;
    float* lse;          // optional: B x Hq x N, natural log
    int32_t B, Hq, Hkv, N;
    int32_t nqb;         // query blocks of 128 per (batch, head)
    int32_t group;       // Hq / Hkv
    int32_t upH;         // work units per (batch, head): query blocks, or causal pairs of them
    int32_t nunits;      // B * Hq * upH
    float c;             // scale * log2(e)
    int64_t sq[3], sk[3], sv[3], so[3];  // (batch, head, token) strides, elements
};

constexpr int kAttnThreads = 256;
// Persistent (causal) workgroups per compute unit: as many as the registers
// allow (D = 128 kernels take up to 256 registers per lane, D = 64 ones up
// to 168).
template <int D>
constexpr int attn_slots() { return D == 64 ? 3 : 2; }

constexpr int kAttnQ = 128;   // query rows per workgroup
constexpr int kAttnKV = 64;   // keys per block
constexpr float kLazy = 8.0f; // log2 headroom before the softmax reference moves

// LDS image of one block of K or V: 64 rows (keys) x D bf16, 16-byte chunk c
// of row r at physical chunk c ^ key(r).
//  K (read by rows: 16 lanes, 16 rows, one chunk): the key spreads 16 rows
//  over all 64 banks.
//  V (transposing reads: a half-wave touches 8 consecutive rows, 32 bytes
//  each, at one chunk pair): the key, even, permutes chunk pairs so that
//  those 8 rows land on distinct banks.
template <int D>
__device__ __forceinline__ uint32_t attn_kswz(uint32_t r) {
    return D == 128 ? (r & 15u) : ((r >> 1) & 7u);
}
template <int D>
__device__ __forceinline__ uint32_t attn_vswz(uint32_t r) {
    return D == 128 ? 2u * (r & 7u) : 2u * ((r >> 1) & 3u);
}

// max of x over the four lanes l, l^16, l^32, l^48 (the lanes that share a
// query): lane l^16 through ds_swizzle (bit mode: and 0x1F, xor 0x10, within
// 32 lanes), lane l^32 through ds_bpermute (byte address x32 = 4 (l ^ 32)).
//
// In the block loop the max goes through v_permlane16_swap / v_permlane32_swap
// instead, which stay off the LDS pipe: swapping a register with a copy of
// itself leaves in the pair, per lane, its own value and its partner's (rows
// of 16 lanes swapped pairwise, or the two halves), and max is symmetric in
// the pair.  Issued as assembly (the compiler folded away one half of the
// pair of the builtin), with the two wait states a VALU write needs before a
// permlane reads it.
__device__ __forceinline__ float max_across_groups(float x) {
    float a = x, b = x;
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
    float c = fmaxf(a, b), d = c;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(c), "+v"(d));
    return fmaxf(c, d);
}
__device__ __forceinline__ float sum_across_groups(float x, int32_t x32) {
    const int u = __builtin_bit_cast(int, x);
    const float y = x + __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(u, 0x401F));
    const int v = __builtin_bit_cast(int, y);
    return y + __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(x32, v));
}

// workgroup -> (batch * Hq + head, query block).  Workgroups are dealt to
// the 8 chiplets round-robin; when the count allows, each chiplet gets a
// contiguous range of heads, so that a head's K and V stay in one L2.
// Within a head the query blocks run from the last (the most keys under a
// causal mask) to the first.
__device__ __forceinline__ void attn_tile_of(uint32_t w, uint32_t total, uint32_t nqb,
                                             uint32_t* bh, uint32_t* qblk) {
    uint32_t idx = w;
    if (total % 8u == 0) idx = (w % 8u) * (total / 8u) + w / 8u;
    *bh = idx / nqb;
    *qblk = nqb - 1u - idx % nqb;
}

// Persistent form: workgroup b takes work units b, b + G, b + 2G, ... (G =
// grid size, a multiple of 8 when there are at least that many units, so a
// workgroup's units stay on its chiplet).  Without a causal mask a unit is one
// query block.  With one, unit u of a (batch, head) is the pair of query
// blocks nqb-1-u and u (the middle block alone when nqb is odd): the longest
// and the shortest, 2 (nqb + 1) key blocks together, so that every
// workgroup gets the same work.  As above, each chiplet gets a contiguous
// range of (batch, head)s when the count allows.
__device__ __forceinline__ void attn_unit_of(uint32_t U, uint32_t total, uint32_t upH,
                                             uint32_t* bh, uint32_t* u) {
    uint32_t idx = U;
    if (total % 8u == 0) idx = (U % 8u) * (total / 8u) + U / 8u;
    *bh = idx / upH;
    *u = idx % upH;
}
// query block of member mem (0, 1) of unit u; members() of a unit: 1 or 2
template <bool kCausal>
__device__ __forceinline__ uint32_t attn_unit_qblk(uint32_t u, uint32_t mem, uint32_t nqb) {
    if (!kCausal) return nqb - 1u - u;
    return mem == 0 ? nqb - 1u - u : u;
}
template <bool kCausal>
__device__ __forceinline__ uint32_t attn_unit_members(uint32_t u, uint32_t nqb) {
    return (kCausal && nqb - 1u - u != u) ? 2u : 1u;
}

template <int D, bool kCausal>
__device__ __forceinline__ void attn_fwd_body(const AttnArgs& g, HK_LDS uint8_t* lds) {
    constexpr int kDC = D / 32;                    // 32-wide d chunks (S MFMAs)
    constexpr int kDB = D / 16;                    // 16-wide d blocks (O MFMAs)
    constexpr int kVPre = kDB / 2;                 // V d blocks read before the softmax
    constexpr uint32_t kRowB = D * 2;              // bytes per K/V row
    constexpr uint32_t kImgB = kAttnKV * kRowB;    // bytes per K or V block image
    constexpr uint32_t kRowsPerLoad = 1024u / kRowB;
    constexpr uint32_t kChunksPerRow = kRowB / 16u;
    constexpr int kLoads = (int)(kAttnKV / (kRowsPerLoad * 4u));  // per thread per matrix

    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t g4 = lane >> 4, r16 = lane & 15u;

    uint32_t bh, qblk;
    attn_tile_of(blockIdx.x, (uint32_t)(g.B * g.Hq) * (uint32_t)g.nqb, (uint32_t)g.nqb, &bh,
                 &qblk);
    const int32_t b = (int32_t)bh / g.Hq, h = (int32_t)bh % g.Hq;
    const int32_t kvh = h / g.group;
    const int32_t q0 = (int32_t)qblk * kAttnQ;
    const int32_t q0w = q0 + 32 * (int32_t)wave;
    const int32_t N = g.N;

    // blocks of keys this workgroup needs
    const int32_t kend = kCausal ? min(N, q0 + kAttnQ) : N;
    const int32_t nblk = (kend + kAttnKV - 1) / kAttnKV;

    // ---- Q fragments ("B" operand of S^T): lane l holds query q0w + 16qb +
    // l%16, d = 32dc + 8(l/16) .. +7.  Rows past N read as zero.
    i32x4 qf[2][kDC];
    {
        const uint16_t* Qh = g.Q + (int64_t)b * g.sq[0] + (int64_t)h * g.sq[1];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int32_t q = q0w + 16 * qb + (int32_t)r16;
#pragma unroll
            for (int dc = 0; dc < kDC; ++dc) {
                qf[qb][dc] = i32x4{0, 0, 0, 0};
                if (q < N)
                    qf[qb][dc] = *reinterpret_cast<const i32x4*>(
                        Qh + (int64_t)q * g.sq[2] + 32 * dc + 8 * (int32_t)g4);
            }
        }
    }

    // ---- K and V blocks: direct loads into LDS.  Buffer resources over the
    // (batch, kv head) rows 0..N-1: rows past N read as zero.
    const uint32_t ktok_b = (uint32_t)g.sk[2] * 2u, vtok_b = (uint32_t)g.sv[2] * 2u;
    const i32x4 rk = make_rsrc_words(g.K + (int64_t)b * g.sk[0] + (int64_t)kvh * g.sk[1],
                                     (uint32_t)((N - 1) * ktok_b + kRowB));
    const i32x4 rv = make_rsrc_words(g.V + (int64_t)b * g.sv[0] + (int64_t)kvh * g.sv[1],
                                     (uint32_t)((N - 1) * vtok_b + kRowB));
    // load i of a matrix: rows kRowsPerLoad * (wave + 4i) .. of the block;
    // lane l -> row + l / kChunksPerRow, physical chunk l % kChunksPerRow
    uint32_t voff_k[kLoads], voff_v[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const uint32_t row = kRowsPerLoad * (wave + 4u * i) + lane / kChunksPerRow;
        const uint32_t pc = lane % kChunksPerRow;
        voff_k[i] = row * ktok_b + ((pc ^ attn_kswz<D>(row)) * 16u);
        voff_v[i] = row * vtok_b + ((pc ^ attn_vswz<D>(row)) * 16u);
    }
    // block j into buffer p (= j % 2)
    auto issue = [&](int32_t j, uint32_t p) {
        HK_LDS uint8_t* kimg = lds + p * 2u * kImgB;
        HK_LDS uint8_t* vimg = kimg + kImgB;
        const uint32_t kb = (uint32_t)j * kAttnKV;
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const uint32_t blk = wave + 4u * i;
            // the block's row offset rides in the VGPR offset, which the
            // buffer range check covers (the SGPR offset is not checked)
            load_lds_b128(rk, (HK_LDS void*)(kimg + blk * 1024u), voff_k[i] + kb * ktok_b, 0u);
            load_lds_b128(rv, (HK_LDS void*)(vimg + blk * 1024u), voff_v[i] + kb * vtok_b, 0u);
        }
    };

    // ---- fragment reads
    // K ("A" operand of S^T): key row 16kb + l%16, chunk 4dc + l/16
    auto read_k = [&](const HK_LDS uint8_t* kimg, int kb, int dc) -> i32x4 {
        const uint32_t r = 16u * kb + r16;
        const uint32_t ch = (4u * dc + g4) ^ attn_kswz<D>(r);
        return *(const HK_LDS i32x4*)(kimg + r * kRowB + ch * 16u);
    };
    // V^T ("A" operand of O^T) for d block db and keys 32c .. 32c+31: two
    // transposing reads, of key rows 16(2c+hh) + 4(l/16) + r (r = (l/4)%4),
    // d = 16db + 4(l%4) .. +3; output lane l gets d = 16db + l%16 and those
    // four keys (measured lane map: within 16 lanes, output lane i's element
    // r comes from source lane i/4 + 4r, position i%4).
    const uint32_t va = lane & 3u, vr = (lane >> 2) & 3u;
    auto read_vt = [&](const HK_LDS uint8_t* vimg, int db, int c) -> i32x4 {
        typedef short s16x4 __attribute__((ext_vector_type(4)));
        s16x4 part[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const uint32_t r = 16u * (2u * c + hh) + 4u * g4 + vr;
            const uint32_t ch = (2u * db + (va >> 1)) ^ attn_vswz<D>(r);
            part[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (HK_LDS s16x4*)(vimg + r * kRowB + ch * 16u + (va & 1u) * 8u));
        }
        return __builtin_shufflevector(__builtin_bit_cast(i32x2, part[0]),
                                       __builtin_bit_cast(i32x2, part[1]), 0, 1, 2, 3);
    };

    f32x4 o[kDB][2];
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) o[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m[2] = {-INFINITY, -INFINITY};  // softmax reference per query (log2 units)
    float l[2] = {0.f, 0.f};              // this lane's share of the sum of weights
    const int32_t x32 = (int32_t)((lane ^ 32u) << 2);

    // One barrier per block: past it, block j has landed (every wave waited
    // for its own part) and every wave has finished block j - 1, whose
    // buffer then takes block j + 1.
    if (nblk > 0) issue(0, 0u);
    // The block loop runs unrolled by two, so that each block's buffer is a
    // constant and its LDS reads take the buffer offset as an immediate.
    auto block = [&](int32_t j, auto pc) {
        constexpr uint32_t p = decltype(pc)::value;
        wait_vmcnt0();
        wait_lgkmcnt0();
        fenced_barrier();
        if (j + 1 < nblk) issue(j + 1, p ^ 1u);
        const HK_LDS uint8_t* kimg = lds + p * 2u * kImgB;
        const HK_LDS uint8_t* vimg = kimg + kImgB;
        const int32_t k0 = j * kAttnKV;

        // a wave whose queries all lie before this block has nothing to add
        if (!kCausal || k0 <= q0w + 31) {
            // Phases, each fenced from the next so that the reads of a phase
            // are all in flight before its first consumer waits: K reads;
            // S MFMAs; the V reads of the first kVPre d blocks (landing
            // during the softmax); softmax; the other V reads; O MFMAs.
            // ---- S^T = K Q^T
            i32x4 kf[4][kDC];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int dc = 0; dc < kDC; ++dc) kf[kb][dc] = read_k(kimg, kb, dc);
            __builtin_amdgcn_sched_barrier(0);
            f32x4 s[4][2];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                s[kb][0] = s[kb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int dc = 0; dc < kDC; ++dc) {
                    s[kb][0] = mfma_bf16_16x16x32(kf[kb][dc], qf[0][dc], s[kb][0]);
                    s[kb][1] = mfma_bf16_16x16x32(kf[kb][dc], qf[1][dc], s[kb][1]);
                }
            }
            // ---- masked scores (causal, or keys past N) become -inf, on a
            // separate path that blocks away from the edges skip
            const bool masked = (kCausal && k0 + kAttnKV - 1 > q0w) || k0 + kAttnKV > N;
            if (masked) {
                // key = k0 + 16kb + 4(l/16) + v and q = q0w + 16qb + l%16:
                // compare the lane's constant part against a scalar threshold
                const int32_t dq = 4 * (int32_t)g4 - (int32_t)r16;
                const int32_t g4x4 = 4 * (int32_t)g4;
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const bool after_q = dq > q0w - k0 + 16 * (qb - kb) - v;  // key > q
                            const bool past_n = g4x4 >= N - k0 - 16 * kb - v;         // key >= N
                            if ((kCausal && after_q) || past_n) s[kb][qb][v] = -INFINITY;
                        }
            }
            __builtin_amdgcn_sched_barrier(0);
            i32x4 vf[kDB][2];
#pragma unroll
            for (int db = 0; db < kVPre; ++db)
#pragma unroll
                for (int c = 0; c < 2; ++c) vf[db][c] = read_vt(vimg, db, c);
            __builtin_amdgcn_sched_barrier(0);
            // ---- online softmax, per query (lane l%16) in log2 units.  With
            // c = scale * log2(e) > 0, max_j (c s_j) = c max_j s_j, and each
            // weight is exp2(c s_j - m): one fma and one exp2 per score.
            i32x4 pf[2][2];  // P^T fragments: [qb][c]
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                float mx = s[0][qb][0];
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int v = 0; v < 4; ++v) mx = fmaxf(mx, s[kb][qb][v]);
                mx = max_across_groups(mx);
                mx *= g.c;
                // The reference point m moves only when some query of the
                // wave gains more than kLazy over it: until then the weights
                // stay below 2^kLazy, and O and l carry the same stale
                // factor, which the final O / l cancels.
                if (__builtin_amdgcn_ballot_w64(mx > m[qb] + kLazy) != 0) {
                    const float mnew = fmaxf(m[qb], mx);
                    // (a query with no visible key yet keeps m = -inf)
                    const float alpha =
                        mnew == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[qb] - mnew);
                    m[qb] = mnew;
                    l[qb] *= alpha;
#pragma unroll
                    for (int db = 0; db < kDB; ++db) o[db][qb] *= alpha;
                }
                const float nm = -m[qb];
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    float p[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        p[e] = __builtin_amdgcn_exp2f(
                            __builtin_fmaf(s[2 * c + e / 4][qb][e % 4], g.c, nm));
                    // the sum takes the fp32 weights, so that LSE is exact to
                    // fp32 sums; O carries the bf16 ones
                    l[qb] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
                    pf[qb][c] = i32x4{(int)pack_bf16x2(p[0], p[1]), (int)pack_bf16x2(p[2], p[3]),
                                      (int)pack_bf16x2(p[4], p[5]), (int)pack_bf16x2(p[6], p[7])};
                }
            }
            // ---- O^T += V^T P^T
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int db = kVPre; db < kDB; ++db)
#pragma unroll
                for (int c = 0; c < 2; ++c) vf[db][c] = read_vt(vimg, db, c);
#pragma unroll
            for (int db = 0; db < kDB; ++db)
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    o[db][0] = mfma_bf16_16x16x32(vf[db][c], pf[0][c], o[db][0]);
                    o[db][1] = mfma_bf16_16x16x32(vf[db][c], pf[1][c], o[db][1]);
                }
        }
    };
    for (int32_t j = 0; j < nblk; j += 2) {
        block(j, std::integral_constant<uint32_t, 0>{});
        if (j + 1 < nblk) block(j + 1, std::integral_constant<uint32_t, 1>{});
    }


    // ---- epilogue: O = O^T / l, LSE = (m + log2 l) ln 2
    uint16_t* Oh = g.O + (int64_t)b * g.so[0] + (int64_t)h * g.so[1];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const float lt = sum_across_groups(l[qb], x32);
        const int32_t q = q0w + 16 * qb + (int32_t)r16;
        if (q < N) {
            const float inv = 1.0f / lt;
            uint16_t* orow = Oh + (int64_t)q * g.so[2] + 4 * (int32_t)g4;
#pragma unroll
            for (int db = 0; db < kDB; ++db) {
                const f32x4 v = o[db][qb] * inv;
                *reinterpret_cast<uint2*>(orow + 16 * db) =
                    make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
            }
            if (g.lse && g4 == 0)
                g.lse[((int64_t)b * g.Hq + h) * N + q] =
                    (m[qb] + __builtin_amdgcn_logf(lt)) * 0.69314718055994531f;
        }
    }
}


template <int D, bool kCausal>
__device__ __forceinline__ void attn_fwd_persist(const AttnArgs& g, HK_LDS uint8_t* lds) {
    constexpr int kDC = D / 32;                    // 32-wide d chunks (S MFMAs)
    constexpr int kDB = D / 16;                    // 16-wide d blocks (O MFMAs)
    constexpr int kVPre = kDB / 2;                 // V d blocks read before the softmax
    constexpr uint32_t kRowB = D * 2;              // bytes per K/V row
    constexpr uint32_t kImgB = kAttnKV * kRowB;    // bytes per K or V block image
    constexpr uint32_t kRowsPerLoad = 1024u / kRowB;
    constexpr uint32_t kChunksPerRow = kRowB / 16u;
    constexpr int kLoads = (int)(kAttnKV / (kRowsPerLoad * 4u));  // per thread per matrix

    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t g4 = lane >> 4, r16 = lane & 15u;

    const int32_t N = g.N;
    // The sequence of tiles this workgroup runs: member mem of unit U.
    struct Tile {
        int32_t b, h, kvh, q0, nblk;
        uint32_t U, mem;
        bool live;
    };
    auto make_tile = [&](uint32_t U, uint32_t mem) {
        Tile t;
        t.U = U;
        t.mem = mem;
        t.live = U < (uint32_t)g.nunits;
        uint32_t bh = 0, u = 0;
        if (t.live) attn_unit_of(U, (uint32_t)g.nunits, (uint32_t)g.upH, &bh, &u);
        t.b = (int32_t)bh / g.Hq;
        t.h = (int32_t)bh % g.Hq;
        t.kvh = t.h / g.group;
        t.q0 = (int32_t)attn_unit_qblk<kCausal>(u, mem, (uint32_t)g.nqb) * kAttnQ;
        // blocks of keys the tile needs
        const int32_t kend = kCausal ? min(N, t.q0 + kAttnQ) : N;
        t.nblk = (kend + kAttnKV - 1) / kAttnKV;
        return t;
    };
    auto next_of = [&](const Tile& t) {
        uint32_t bh = 0, u = 0;
        attn_unit_of(t.U, (uint32_t)g.nunits, (uint32_t)g.upH, &bh, &u);
        if (t.mem + 1u < attn_unit_members<kCausal>(u, (uint32_t)g.nqb)) return make_tile(t.U, 1u);
        return make_tile(t.U + gridDim.x, 0u);
    };

    // ---- Q fragments ("B" operand of S^T): lane l holds query q0w + 16qb +
    // l%16, d = 32dc + 8(l/16) .. +7.  Rows past N read as zero.
    i32x4 qf[2][kDC];
    auto load_q = [&](const Tile& t) {
        const uint16_t* Qh = g.Q + (int64_t)t.b * g.sq[0] + (int64_t)t.h * g.sq[1];
        const int32_t q0w = t.q0 + 32 * (int32_t)wave;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int32_t q = q0w + 16 * qb + (int32_t)r16;
#pragma unroll
            for (int dc = 0; dc < kDC; ++dc) {
                qf[qb][dc] = i32x4{0, 0, 0, 0};
                if (q < N)
                    qf[qb][dc] = *reinterpret_cast<const i32x4*>(
                        Qh + (int64_t)q * g.sq[2] + 32 * dc + 8 * (int32_t)g4);
            }
        }
    };

    // ---- K and V blocks: direct loads into LDS.  Buffer resources over the
    // (batch, kv head) rows 0..N-1: rows past N read as zero.
    const uint32_t ktok_b = (uint32_t)g.sk[2] * 2u, vtok_b = (uint32_t)g.sv[2] * 2u;
    auto rsrc_k = [&](const Tile& t) {
        return make_rsrc_words(g.K + (int64_t)t.b * g.sk[0] + (int64_t)t.kvh * g.sk[1],
                               (uint32_t)((N - 1) * ktok_b + kRowB));
    };
    auto rsrc_v = [&](const Tile& t) {
        return make_rsrc_words(g.V + (int64_t)t.b * g.sv[0] + (int64_t)t.kvh * g.sv[1],
                               (uint32_t)((N - 1) * vtok_b + kRowB));
    };
    // load i of a matrix: rows kRowsPerLoad * (wave + 4i) .. of the block;
    // lane l -> row + l / kChunksPerRow, physical chunk l % kChunksPerRow
    uint32_t voff_k[kLoads], voff_v[kLoads];
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
        const uint32_t row = kRowsPerLoad * (wave + 4u * i) + lane / kChunksPerRow;
        const uint32_t pc = lane % kChunksPerRow;
        voff_k[i] = row * ktok_b + ((pc ^ attn_kswz<D>(row)) * 16u);
        voff_v[i] = row * vtok_b + ((pc ^ attn_vswz<D>(row)) * 16u);
    }
    // block j of a tile into buffer buf
    auto issue = [&](const i32x4& rk, const i32x4& rv, int32_t j, uint32_t buf) {
        HK_LDS uint8_t* kimg = lds + buf * 2u * kImgB;
        HK_LDS uint8_t* vimg = kimg + kImgB;
        const uint32_t kb = (uint32_t)j * kAttnKV;
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const uint32_t blk = wave + 4u * i;
            // the block's row offset rides in the VGPR offset, which the
            // buffer range check covers (the SGPR offset is not checked)
            load_lds_b128(rk, (HK_LDS void*)(kimg + blk * 1024u), voff_k[i] + kb * ktok_b, 0u);
            load_lds_b128(rv, (HK_LDS void*)(vimg + blk * 1024u), voff_v[i] + kb * vtok_b, 0u);
        }
    };

    // ---- fragment reads
    // K ("A" operand of S^T): key row 16kb + l%16, chunk 4dc + l/16
    auto read_k = [&](const HK_LDS uint8_t* kimg, int kb, int dc) -> i32x4 {
        const uint32_t r = 16u * kb + r16;
        const uint32_t ch = (4u * dc + g4) ^ attn_kswz<D>(r);
        return *(const HK_LDS i32x4*)(kimg + r * kRowB + ch * 16u);
    };
    // V^T ("A" operand of O^T) for d block db and keys 32c .. 32c+31: two
    // transposing reads, of key rows 16(2c+hh) + 4(l/16) + r (r = (l/4)%4),
    // d = 16db + 4(l%4) .. +3; output lane l gets d = 16db + l%16 and those
    // four keys (measured lane map: within 16 lanes, output lane i's element
    // r comes from source lane i/4 + 4r, position i%4).
    const uint32_t va = lane & 3u, vr = (lane >> 2) & 3u;
    auto read_vt = [&](const HK_LDS uint8_t* vimg, int db, int c) -> i32x4 {
        typedef short s16x4 __attribute__((ext_vector_type(4)));
        s16x4 part[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const uint32_t r = 16u * (2u * c + hh) + 4u * g4 + vr;
            const uint32_t ch = (2u * db + (va >> 1)) ^ attn_vswz<D>(r);
            part[hh] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (HK_LDS s16x4*)(vimg + r * kRowB + ch * 16u + (va & 1u) * 8u));
        }
        return __builtin_shufflevector(__builtin_bit_cast(i32x2, part[0]),
                                       __builtin_bit_cast(i32x2, part[1]), 0, 1, 2, 3);
    };

    f32x4 o[kDB][2];
    float m[2], l[2];  // softmax reference per query (log2 units); this lane's share of the sum
    const int32_t x32 = (int32_t)((lane ^ 32u) << 2);

    // One barrier per block: past it, block j has landed (every wave waited
    // for its own part) and every wave has finished the previous block, whose
    // buffer then takes the next one: block j + 1 of this tile, or, from the
    // last block, the next tile's block 0.  The buffer parity runs on across
    // tiles.  The next tile's Q fragments load right after the last block's
    // S products (the last readers of qf), so they land during its softmax,
    // its O products and the store of O.
    Tile cur = make_tile(blockIdx.x, 0u);
    if (!cur.live) return;
    i32x4 rk = rsrc_k(cur), rv = rsrc_v(cur);
    load_q(cur);
    issue(rk, rv, 0, 0u);
    uint32_t buf = 0;
    for (;;) {
#pragma unroll
        for (int db = 0; db < kDB; ++db)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) o[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
        m[0] = m[1] = -INFINITY;
        l[0] = l[1] = 0.f;
        const int32_t b = cur.b, h = cur.h, q0 = cur.q0, nblk = cur.nblk;
        const int32_t q0w = q0 + 32 * (int32_t)wave;
        (void)q0;
    for (int32_t j = 0; j < nblk; ++j, buf ^= 1u) {
        wait_vmcnt0();
        wait_lgkmcnt0();
        fenced_barrier();
        const bool last = j + 1 == nblk;
        // the next tile is worked out in the last block only, so that none of
        // its state stays in registers across the block loop
        Tile nx;
        nx.live = false;
        if (!last) {
            issue(rk, rv, j + 1, buf ^ 1u);
        } else {
            nx = next_of(cur);
            if (nx.live) issue(rsrc_k(nx), rsrc_v(nx), 0, buf ^ 1u);
        }
        const HK_LDS uint8_t* kimg = lds + buf * 2u * kImgB;
        const HK_LDS uint8_t* vimg = kimg + kImgB;
        const int32_t k0 = j * kAttnKV;

        // a wave whose queries all lie before this block has nothing to add
        if (!kCausal || k0 <= q0w + 31) {
            // Phases, each fenced from the next so that the reads of a phase
            // are all in flight before its first consumer waits: K reads;
            // S MFMAs; the V reads of the first kVPre d blocks (landing
            // during the softmax); softmax; the other V reads; O MFMAs.
            // ---- S^T = K Q^T
            i32x4 kf[4][kDC];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int dc = 0; dc < kDC; ++dc) kf[kb][dc] = read_k(kimg, kb, dc);
            __builtin_amdgcn_sched_barrier(0);
            f32x4 s[4][2];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                s[kb][0] = s[kb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int dc = 0; dc < kDC; ++dc) {
                    s[kb][0] = mfma_bf16_16x16x32(kf[kb][dc], qf[0][dc], s[kb][0]);
                    s[kb][1] = mfma_bf16_16x16x32(kf[kb][dc], qf[1][dc], s[kb][1]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            // ---- masked scores (causal, or keys past N) become -inf, on a
            // separate path that blocks away from the edges skip
            const bool masked = (kCausal && k0 + kAttnKV - 1 > q0w) || k0 + kAttnKV > N;
            if (masked) {
                // key = k0 + 16kb + 4(l/16) + v and q = q0w + 16qb + l%16:
                // compare the lane's constant part against a scalar threshold
                const int32_t dq = 4 * (int32_t)g4 - (int32_t)r16;
                const int32_t g4x4 = 4 * (int32_t)g4;
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                        for (int v = 0; v < 4; ++v) {
                            const bool after_q = dq > q0w - k0 + 16 * (qb - kb) - v;  // key > q
                            const bool past_n = g4x4 >= N - k0 - 16 * kb - v;         // key >= N
                            if ((kCausal && after_q) || past_n) s[kb][qb][v] = -INFINITY;
                        }
            }
            __builtin_amdgcn_sched_barrier(0);
            i32x4 vf[kDB][2];
#pragma unroll
            for (int db = 0; db < kVPre; ++db)
#pragma unroll
                for (int c = 0; c < 2; ++c) vf[db][c] = read_vt(vimg, db, c);
            __builtin_amdgcn_sched_barrier(0);
            // ---- online softmax, per query (lane l%16) in log2 units.  With
            // c = scale * log2(e) > 0, max_j (c s_j) = c max_j s_j, and each
            // weight is exp2(c s_j - m): one fma and one exp2 per score.
            i32x4 pf[2][2];  // P^T fragments: [qb][c]
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                float mx = s[0][qb][0];
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int v = 0; v < 4; ++v) mx = fmaxf(mx, s[kb][qb][v]);
                mx = max_across_groups(mx);
                mx *= g.c;
                // The reference point m moves only when some query of the
                // wave gains more than kLazy over it: until then the weights
                // stay below 2^kLazy, and O and l carry the same stale
                // factor, which the final O / l cancels.
                if (__builtin_amdgcn_ballot_w64(mx > m[qb] + kLazy) != 0) {
                    const float mnew = fmaxf(m[qb], mx);
                    // (a query with no visible key yet keeps m = -inf)
                    const float alpha =
                        mnew == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[qb] - mnew);
                    m[qb] = mnew;
                    l[qb] *= alpha;
#pragma unroll
                    for (int db = 0; db < kDB; ++db) o[db][qb] *= alpha;
                }
                const float nm = -m[qb];
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    float p[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        p[e] = __builtin_amdgcn_exp2f(
                            __builtin_fmaf(s[2 * c + e / 4][qb][e % 4], g.c, nm));
                    // the sum takes the fp32 weights, so that LSE is exact to
                    // fp32 sums; O carries the bf16 ones
                    l[qb] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
                    pf[qb][c] = i32x4{(int)pack_bf16x2(p[0], p[1]), (int)pack_bf16x2(p[2], p[3]),
                                      (int)pack_bf16x2(p[4], p[5]), (int)pack_bf16x2(p[6], p[7])};
                }
            }
            // ---- O^T += V^T P^T
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int db = kVPre; db < kDB; ++db)
#pragma unroll
                for (int c = 0; c < 2; ++c) vf[db][c] = read_vt(vimg, db, c);
#pragma unroll
            for (int db = 0; db < kDB; ++db)
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    o[db][0] = mfma_bf16_16x16x32(vf[db][c], pf[0][c], o[db][0]);
                    o[db][1] = mfma_bf16_16x16x32(vf[db][c], pf[1][c], o[db][1]);
                }
        }
    }

    // ---- epilogue: O = O^T / l, LSE = (m + log2 l) ln 2
    uint16_t* Oh = g.O + (int64_t)b * g.so[0] + (int64_t)h * g.so[1];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const float lt = sum_across_groups(l[qb], x32);
        const int32_t q = q0w + 16 * qb + (int32_t)r16;
        if (q < N) {
            const float inv = 1.0f / lt;
            uint16_t* orow = Oh + (int64_t)q * g.so[2] + 4 * (int32_t)g4;
#pragma unroll
            for (int db = 0; db < kDB; ++db) {
                const f32x4 v = o[db][qb] * inv;
                *reinterpret_cast<uint2*>(orow + 16 * db) =
                    make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
            }
            if (g.lse && g4 == 0)
                g.lse[((int64_t)b * g.Hq + h) * N + q] =
                    (m[qb] + __builtin_amdgcn_logf(lt)) * 0.69314718055994531f;
        }
    }
        cur = next_of(cur);
        if (!cur.live) break;
        rk = rsrc_k(cur);
        rv = rsrc_v(cur);
        load_q(cur);
    }
    wait_all();  // no LDS write may outlive the workgroup
}

}  // namespace hk
