// hk_kernels.hpp -- kernel bodies for C = A * B^T on gfx950.
//
// Two bodies share one data layout:
//
//  * pp8_body: the fast path.  A 256 x 256 output tile per workgroup of 512
//    threads (8 waves).  K advances 128 bytes per stage (64 bf16 or 128 e4m3),
//    so both dtypes use the same LDS image: 256 rows x 8 chunks of 16 bytes per
//    operand per stage, two stages (128 KiB).  Operands go HBM -> LDS with
//    direct buffer loads (no register round trip), whose per-lane global
//    addresses are permuted so that the fixed lane -> LDS placement of those
//    loads produces an XOR-swizzled image that the fragment reads see without
//    bank conflicts ("How to make AMD GPUs go brrr", section "HipKittens
//    memory-access patterns": asynchronous HBM->shared loads, HBM address
//    swizzling, one swizzle per register layout).  The waves form two groups
//    of four (one wave per SIMD each) running the 8-wave ping-pong from the
//    section "Intra-processor scheduling: wave patterns": while one group
//    issues its cluster of matrix-core instructions, the other issues its
//    cluster of LDS reads and HBM->LDS loads; workgroup barriers swap them.
//
//  * basic_body: a plain fallback with no alignment requirements: 64 x 64
//    tile, 4 waves, element-wise bounds-checked loads into LDS, one stage.
//
// Both compute C^T blocks on the matrix cores (B rows as the MFMA "A" operand,
// A rows as its "B" operand) so that each lane ends up holding four
// consecutive columns of one C row, which it stores as one 8-byte write.
#pragma once

#include "hk_device.hpp"
#include "hk_grid.hpp"

namespace hk {

struct GemmArgs {
    const uint8_t* A;
    const uint8_t* B;
    uint16_t* C;
    int32_t M, N, K;        // K in elements
    uint32_t lda_b, ldb_b;  // row strides of A and B in bytes
    int64_t ldc;            // row stride of C in elements
    float scale;            // multiplies the fp32 accumulator (FP8 only)
    int32_t c_align;        // guaranteed alignment of 4-column groups of C: 8, 4 or 2
    GridParams grid;
};

constexpr int kRowBytes = 128;  // bytes of K per stage in every tile row
constexpr int kChunks = 8;      // 16-byte chunks per tile row per stage

// ---------------------------------------------------------------- swizzle
//
// Physical chunk of logical K-chunk kc in tile row r: kc ^ key(r).  A
// fragment read for the 16x16 matrix-core shapes has lanes 0..15 on 16
// consecutive rows at the same logical chunk; the key spreads them over the
// 8 chunk positions (= all LDS banks of a 128-byte row).  Variant 1 keys on
// r mod 8; variant 2 keys on (r / 2) mod 8, for bank groups spanning two rows.
template <int kSwz>
__device__ __forceinline__ uint32_t swz_key(uint32_t row) {
    if constexpr (kSwz == 0) return 0u;
    else if constexpr (kSwz == 1) return row & 7u;
    else return (row >> 1) & 7u;
}

// -------------------------------------------------------------- fast path

constexpr int kPP8Tile = 256;
constexpr int kPP8Threads = 512;
constexpr int kPP8StageI4 = kPP8Tile * kChunks;  // 16-byte chunks per operand per stage

template <bool kFp8, int kSwz>
__device__ __forceinline__ void pp8_body(const GemmArgs& g, HK_LDS i32x4* sA0, HK_LDS i32x4* sB0,
                                         HK_LDS i32x4* sA1, HK_LDS i32x4* sB1) {
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // Group 0 (waves 0-3) loads the A tile and owns output rows 0..127 of the
    // tile; group 1 (waves 4-7) loads the B tile and owns rows 128..255.
    // Within a group, wave wq owns the 64-column strip wq.
    const uint32_t grp = wave >> 2;
    const uint32_t wq = wave & 3u;

    uint32_t tm, tn;
    tile_of(blockIdx.x, g.grid, &tm, &tn);
    const int32_t m0 = (int32_t)tm * kPP8Tile;
    const int32_t n0 = (int32_t)tn * kPP8Tile;
    const uint32_t kbytes = (uint32_t)g.K * (kFp8 ? 1u : 2u);
    const uint32_t nk = (kbytes + kRowBytes - 1) / kRowBytes;

    // ---- HBM -> LDS loads: this wave moves 8 blocks of 8 rows of its
    // group's operand per stage; block b = 4i + wq holds tile rows 8b..8b+7
    // and lane l lands on row 8b + l/8, physical chunk l%8.
    const bool loads_a = (grp == 0);
    const uint32_t ld_b = loads_a ? g.lda_b : g.ldb_b;
    const int32_t rows_left = loads_a ? g.M - m0 : g.N - n0;
    const uint8_t* src = loads_a ? g.A + (int64_t)m0 * ld_b : g.B + (int64_t)n0 * ld_b;
    uint64_t span = (uint64_t)rows_left * ld_b;  // rows past the edge read as zero
    if (span > kOobOffset) span = kOobOffset;
    const auto rsrc = make_rsrc(src, (uint32_t)span);
    const uint32_t lrow = wq * 8u + (lane >> 3);             // tile row for i = 0
    const uint32_t lkc = (lane & 7u) ^ swz_key<kSwz>(lrow);  // logical chunk it must hold
    const uint32_t voff0 = lrow * ld_b + lkc * 16u;
    const uint32_t vstep = 32u * ld_b;                       // block b -> b + 4

    auto issue_loads = [&](HK_LDS i32x4* dA, HK_LDS i32x4* dB, uint32_t t) {
        HK_LDS i32x4* dst = loads_a ? dA : dB;
        // K chunks past the end of the row (the K tail) read as zero
        const bool kvalid = t * (uint32_t)kRowBytes + lkc * 16u < kbytes;
        const uint32_t vo = voff0 + t * (uint32_t)kRowBytes;
#pragma unroll
        for (uint32_t i = 0; i < 8; ++i)
            load_lds_b128(rsrc, dst + (i * 4u + wq) * 64u, kvalid ? vo + i * vstep : kOobOffset);
    };

    // ---- LDS -> register fragments.  Fragment rows start at multiples of 16,
    // so the swizzle key depends on the lane only.
    const uint32_t r16 = lane & 15u;
    const uint32_t g4 = lane >> 4;
    const uint32_t key = swz_key<kSwz>(r16);
    const uint32_t fa0 = (grp * 128u + r16) * kChunks + ((0u + g4) ^ key);
    const uint32_t fa1 = (grp * 128u + r16) * kChunks + ((4u + g4) ^ key);
    const uint32_t fb0 = (wq * 64u + r16) * kChunks + ((0u + g4) ^ key);
    const uint32_t fb1 = (wq * 64u + r16) * kChunks + ((4u + g4) ^ key);

    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    i32x4 af[4][2], bfr[4][2];

    // matrix-core cluster over output row blocks mbase..mbase+3
    auto mma = [&](const int mbase) {
        if constexpr (!kFp8) {
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb)
                        acc[mbase + mb][nb] =
                            mfma_bf16_16x16x32(bfr[nb][c], af[mb][c], acc[mbase + mb][nb]);
        } else {
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
                    acc[mbase + mb][nb] = mfma_fp8_16x16x128(bfr[nb][0], bfr[nb][1], af[mb][0],
                                                             af[mb][1], acc[mbase + mb][nb]);
        }
    };

    // One stage t, as four barrier-separated phases.  Group 0 runs
    // M C M C, group 1 runs the same one phase later, so in every phase one
    // group issues memory work while the other issues matrix-core work.
    auto stage = [&](const HK_LDS i32x4* rA, const HK_LDS i32x4* rB, HK_LDS i32x4* wA,
                     HK_LDS i32x4* wB, uint32_t t) {
        // memory: A-side fragments of row blocks 0-3, all B-side fragments,
        // and this group's half of stage t+1 into the other buffer (free:
        // every wave finished reading stage t-1 before this phase began)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            af[mb][0] = rA[fa0 + mb * 128];
            af[mb][1] = rA[fa1 + mb * 128];
        }
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
            bfr[nb][0] = rB[fb0 + nb * 128];
            bfr[nb][1] = rB[fb1 + nb * 128];
        }
        if (t + 1 < nk) issue_loads(wA, wB, t + 1);
        wait_lgkmcnt0();
        fenced_barrier();
        // compute
        __builtin_amdgcn_s_setprio(1);
        mma(0);
        __builtin_amdgcn_s_setprio(0);
        fenced_barrier();
        // memory: A-side fragments of row blocks 4-7
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            af[mb][0] = rA[fa0 + (mb + 4) * 128];
            af[mb][1] = rA[fa1 + (mb + 4) * 128];
        }
        if (grp == 1) wait_vmcnt0();  // group 1's loads of stage t+1 have landed
        wait_lgkmcnt0();
        fenced_barrier();
        // compute
        __builtin_amdgcn_s_setprio(1);
        mma(4);
        __builtin_amdgcn_s_setprio(0);
        if (grp == 0) wait_vmcnt0();  // group 0's loads of stage t+1 have landed
        fenced_barrier();
    };

    if (nk > 0) {
        issue_loads(sA0, sB0, 0);
        wait_vmcnt0();
    }
    fenced_barrier();
    if (grp == 1) fenced_barrier();  // start group 1 one phase behind
    for (uint32_t t = 0; t < nk; t += 2) {
        stage(sA0, sB0, sA1, sB1, t);
        if (t + 1 < nk) stage(sA1, sB1, sA0, sB0, t + 1);
    }
    if (grp == 0) fenced_barrier();  // match group 1's barrier count

    // ---- epilogue: lane holds C[m][n..n+3] for each (mb, nb)
    const int32_t mrow = m0 + (int32_t)(grp * 128u + r16);
    const int32_t ncol = n0 + (int32_t)(wq * 64u + g4 * 4u);
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
        const int32_t m = mrow + mb * 16;
        if (m < g.M) {
            uint16_t* crow = g.C + (int64_t)m * g.ldc;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const int32_t n = ncol + nb * 16;
                if (n < g.N) {
                    f32x4 v = acc[mb][nb];
                    if constexpr (kFp8) v *= g.scale;
                    store_bf16x4(crow + n, n, g.N, v, g.c_align);
                }
            }
        }
    }
}

// --------------------------------------------------------------- fallback

constexpr int kBasicTile = 64;
constexpr int kBasicThreads = 256;
constexpr int kBasicStageI4 = kBasicTile * kChunks;

template <bool kFp8>
__device__ __forceinline__ void basic_body(const GemmArgs& g, HK_LDS i32x4* sA, HK_LDS i32x4* sB) {
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wave = tid >> 6;
    const uint32_t wm = wave >> 1, wn = wave & 1u;  // 2 x 2 waves of 32 x 32

    uint32_t tm, tn;
    tile_of(blockIdx.x, g.grid, &tm, &tn);
    const int32_t m0 = (int32_t)tm * kBasicTile;
    const int32_t n0 = (int32_t)tn * kBasicTile;
    constexpr uint32_t kElems = kFp8 ? 128u : 64u;  // K elements per stage
    const uint32_t nk = ((uint32_t)g.K + kElems - 1) / kElems;

    // loader: thread -> tile row tid/4, bytes 32*(tid%4) .. +32 of that row
    const uint32_t lr = tid >> 2;
    const uint32_t lb = (tid & 3u) * 32u;
    const int32_t am = m0 + (int32_t)lr, bn = n0 + (int32_t)lr;
    HK_LDS uint8_t* sAb = (HK_LDS uint8_t*)sA;
    HK_LDS uint8_t* sBb = (HK_LDS uint8_t*)sB;

    const uint32_t r16 = lane & 15u, g4 = lane >> 4;
    f32x4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (uint32_t t = 0; t < nk; ++t) {
        const int64_t k0 = (int64_t)t * kElems;
        if constexpr (kFp8) {
#pragma unroll 4
            for (uint32_t e = 0; e < 32; ++e) {
                const int64_t k = k0 + lb + e;
                uint8_t va = 0, vb = 0;
                if (am < g.M && k < g.K) va = g.A[(int64_t)am * g.lda_b + k];
                if (bn < g.N && k < g.K) vb = g.B[(int64_t)bn * g.ldb_b + k];
                sAb[lr * kRowBytes + lb + e] = va;
                sBb[lr * kRowBytes + lb + e] = vb;
            }
        } else {
            const uint16_t* A16 = reinterpret_cast<const uint16_t*>(g.A);
            const uint16_t* B16 = reinterpret_cast<const uint16_t*>(g.B);
            const int64_t lda = g.lda_b / 2, ldb = g.ldb_b / 2;
#pragma unroll 4
            for (uint32_t e = 0; e < 16; ++e) {
                const int64_t k = k0 + lb / 2 + e;
                uint16_t va = 0, vb = 0;
                if (am < g.M && k < g.K) va = A16[(int64_t)am * lda + k];
                if (bn < g.N && k < g.K) vb = B16[(int64_t)bn * ldb + k];
                ((HK_LDS uint16_t*)sAb)[(lr * kRowBytes + lb) / 2 + e] = va;
                ((HK_LDS uint16_t*)sBb)[(lr * kRowBytes + lb) / 2 + e] = vb;
            }
        }
        __syncthreads();
        i32x4 af[2][2], bfr[2][2];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                af[b][c] = sA[(wm * 32u + b * 16u + r16) * kChunks + c * 4u + g4];
                bfr[b][c] = sB[(wn * 32u + b * 16u + r16) * kChunks + c * 4u + g4];
            }
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                if constexpr (kFp8) {
                    acc[mb][nb] = mfma_fp8_16x16x128(bfr[nb][0], bfr[nb][1], af[mb][0], af[mb][1],
                                                     acc[mb][nb]);
                } else {
                    acc[mb][nb] = mfma_bf16_16x16x32(bfr[nb][0], af[mb][0], acc[mb][nb]);
                    acc[mb][nb] = mfma_bf16_16x16x32(bfr[nb][1], af[mb][1], acc[mb][nb]);
                }
            }
        __syncthreads();
    }

    const int32_t mrow = m0 + (int32_t)(wm * 32u + r16);
    const int32_t ncol = n0 + (int32_t)(wn * 32u + g4 * 4u);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        const int32_t m = mrow + mb * 16;
        if (m < g.M) {
            uint16_t* crow = g.C + (int64_t)m * g.ldc;
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const int32_t n = ncol + nb * 16;
                if (n < g.N) {
                    f32x4 v = acc[mb][nb];
                    if constexpr (kFp8) v *= g.scale;
                    store_bf16x4(crow + n, n, g.N, v, g.c_align);
                }
            }
        }
    }
}

}  // namespace hk
