// hk_kernels.hpp -- kernel bodies for C = A * B^T on gfx950.
//
// The fast bodies share one data layout.  A workgroup computes a 256 x 256
// tile of C; K advances 128 bytes per stage (64 bf16 or 128 e4m3), so both
// dtypes use the same LDS image: 256 rows x 8 chunks of 16 bytes per operand
// per stage, two stages (128 KiB).  Operands go HBM -> LDS with direct buffer
// loads (no register round trip), whose per-lane global addresses are
// permuted so that the fixed lane -> LDS placement of those loads produces an
// XOR-swizzled image that the fragment reads see without bank conflicts
// ("How to make AMD GPUs go brrr", section "HipKittens memory-access
// patterns": asynchronous HBM->shared loads, HBM address swizzling, one
// swizzle per register layout).  Schedules ("Intra-processor scheduling:
// wave patterns"):
//
//  * il4_bf16_body, il4_fp8_body: 4 waves (one per SIMD), each interleaving
//    its own loads and LDS reads with its matrix-core instructions; one
//    workgroup per compute unit walks its share of the tiles.  The default.
//  * pp8_body: the 8-wave ping-pong; two groups of four waves swap between a
//    cluster of matrix-core instructions and a cluster of memory work at
//    workgroup barriers.
//  * i8_body: 8 waves (two per SIMD), each interleaving like the 4-wave
//    kernel (BF16 only).
//  * basic_body: a plain fallback with no alignment requirements: 64 x 64
//    tile, 4 waves, element-wise bounds-checked loads into LDS, one stage.
//
// All compute C^T blocks on the matrix cores (B rows as the MFMA "A" operand,
// A rows as its "B" operand) so that each lane ends up holding four
// consecutive columns of one C row, which it stores as one 8-byte write.
#pragma once

#include <type_traits>

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
    // FP8 only (1 otherwise): the accumulator scale scale_a * scale_b, or,
    // when exactly one factor comes from device memory, the other factor
    float scale;
    // FP8 only: NULL, or a device fp32 that replaces scale_a (scale_b), read
    // when the kernel runs
    const float* scale_pa;
    const float* scale_pb;
    int32_t c_align;        // guaranteed alignment of 8-column (16) or 4-column groups of C (8, 4, 2)
    GridParams grid;
    // MXFP8 only: E8M0 scale bytes, one per 32 K-elements of a row
    const uint8_t* SA;
    const uint8_t* SB;
    uint32_t ldsa, ldsb;    // row strides of the scale arrays in bytes
    // operand stored transposed: A[k * lda + m], B[k * ldb + n] (basic kernel;
    // the 4-wave BF16 kernel takes the layout as template arguments)
    int32_t a_t, b_t;
    // optional clock record (clock_stamp_begin); written by the persistent kernels only
    uint64_t* stamps;
};

// The FP8 accumulator scale: the host's fp32 product when both factors were
// passed by value, else the same fp32 product with the device-resident
// factors read now (equal values give the same bits either way).
__device__ __forceinline__ float fp8_scale(const GemmArgs& g) {
    if (g.scale_pa == nullptr && g.scale_pb == nullptr) return g.scale;
    const float a = g.scale_pa != nullptr ? *g.scale_pa : g.scale;
    const float b = g.scale_pb != nullptr ? *g.scale_pb : g.scale;
    return a * b;
}

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

// ----------------------------------------------------------- 8-wave ping-pong

constexpr int kPP8Tile = 256;
constexpr int kPP8Threads = 512;
constexpr int kPP8StageI4 = kPP8Tile * kChunks;  // 16-byte chunks per operand per stage
constexpr int kPP8HalfI4 = kPP8StageI4 / 2;       // one A region (128 rows)

// LDS of one stage buffer: each region is its own array, so the compiler's
// tracking of asynchronous LDS writes can tell a refill of one region from
// reads of another.
struct PP8Buf {
    HK_LDS i32x4* alo;  // A tile rows 0-63 and 128-191 (16 KiB)
    HK_LDS i32x4* ahi;  // A tile rows 64-127 and 192-255 (16 KiB)
    HK_LDS i32x4* b;    // B tile rows 0-255 (32 KiB)
};

// Chiplet-rotated K order of the persistent kernels.  All CUs walk
// the K stages of their tiles in lockstep, and the 8 chiplets share each
// A (or B) panel of a window: with one K order, all 8 L2s miss on the same
// lines at the same moment and queue at the last-level cache (fabric read
// latency about 1.5 times hipBLASLt's, measured with TCC_EA0_RDREQ_LEVEL).
// Chiplet x (workgroup w runs on chiplet w mod 8) starts its tiles' whole
// stages x/8 of the way into K and wraps around; the CUs of one chiplet keep
// one order, so their L2 sharing is untouched.  The partial last stage and
// the stages past K keep their places.  Only the order of the fp32 sums
// changes.
__device__ __forceinline__ uint32_t chiplet_k_rotation(uint32_t nk_whole) {
    return ((blockIdx.x & 7u) * nk_whole) >> 3;
}
__device__ __forceinline__ uint32_t rotated_stage(uint32_t s, uint32_t rot, uint32_t nk_whole) {
    if (s >= nk_whole) return s;
    const uint32_t r = s + rot;
    return r >= nk_whole ? r - nk_whole : r;
}

// Persistent like the 4-wave kernels: one workgroup per compute unit walks
// tiles w = b, b + G, ... (G = grid size), and the stage pipeline runs
// through tile boundaries (stages past a tile's last one are the next
// tile's first), with the chiplet-rotated K order, global direct loads for
// the whole stages of tiles inside C and 16-byte C stores.
template <bool kFp8, int kSwz>
__device__ __forceinline__ void pp8_body(const GemmArgs& g, const PP8Buf buf0, const PP8Buf buf1) {
    clock_stamp_begin(g.stamps);
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // Group 0 (waves 0-3) owns output rows 0..127 of the tile and issues all
    // HBM->LDS loads; group 1 (waves 4-7) owns rows 128..255.  Within a group,
    // wave wq owns the 64-column strip wq.
    const uint32_t grp = wave >> 2;
    const uint32_t wq = wave & 3u;
    const uint32_t total = (uint32_t)g.grid.tiles_m * (uint32_t)g.grid.tiles_n;
    const uint32_t kbytes = (uint32_t)g.K * (kFp8 ? 1u : 2u);
    const uint32_t nk = (kbytes + kRowBytes - 1) / kRowBytes;
    const uint32_t nk_pad = (nk + 1u) & ~1u;  // stages run in pairs
    const uint32_t nk_whole = kbytes / kRowBytes;
    const uint32_t krot = chiplet_k_rotation(nk_whole);

    // ---- HBM -> LDS.  A stage of an operand is 32 blocks of 8 rows; one
    // 16-byte load per lane moves a block (lane l -> row 8b + l/8, physical
    // chunk l%8, which holds logical chunk (l%8) ^ key(row)).  The regions of
    // a stage buffer free up at different times: B and A-lo after the first
    // memory phase of both groups, A-hi after the second.  Group 0 refills
    // each region as soon as it is free:
    //   batch HI(s): A-hi of stage s       (4 loads per wave), one stage ahead
    //   batch LO(s): B and A-lo of stage s (12 loads per wave), two stages ahead
    // so every batch has six phases to land.  Stages past a tile's K (the
    // pad stage and the ones past the last tile) read zeros, which keeps
    // every wait count constant.
    const uint32_t kc_lane = (lane & 7u) ^ swz_key<kSwz>(wq * 8u + (lane >> 3));
    const uint32_t vrow_a = (lane >> 3) * g.lda_b + kc_lane * 16u;
    const uint32_t vrow_b = (lane >> 3) * g.ldb_b + kc_lane * 16u;
    // This wave's blocks: region block r = wq + 4j.  In A-lo, region blocks
    // 0-7 are tile blocks 0-7 and 8-15 are tile blocks 16-23; in A-hi, region
    // blocks 0-7 are tile blocks 8-15 and 8-15 are tile blocks 24-31.
    uint32_t vhi[4], vlo_a[4], vlo_b[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t rb = wq + 4u * j;
        const uint32_t tile_lo = rb < 8 ? rb : rb + 8u;
        vlo_a[j] = vrow_a + tile_lo * 8u * g.lda_b;
        vhi[j] = vrow_a + (tile_lo + 8u) * 8u * g.lda_b;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) vlo_b[j] = vrow_b + (wq + 4u * j) * 8u * g.ldb_b;

    // Buffer resources of a tile's A and B row panels; rows past the matrix
    // edge read as zero, and a tile past the end gets empty resources.
    struct Tile {
        i32x4 ra, rb;
        int32_t m0, n0;
    };
    auto tile = [&](uint32_t w) {
        Tile t;
        uint32_t tm = 0, tn = 0;
        if (w < total) tile_of(w, g.grid, &tm, &tn);
        t.m0 = (int32_t)tm * kPP8Tile;
        t.n0 = (int32_t)tn * kPP8Tile;
        const uint64_t sa = w < total ? (uint64_t)(g.M - t.m0) * g.lda_b : 0;
        const uint64_t sb = w < total ? (uint64_t)(g.N - t.n0) * g.ldb_b : 0;
        t.ra = make_rsrc_words(g.A + (int64_t)t.m0 * g.lda_b,
                               (uint32_t)(sa > kOobOffset ? kOobOffset : sa));
        t.rb = make_rsrc_words(g.B + (int64_t)t.n0 * g.ldb_b,
                               (uint32_t)(sb > kOobOffset ? kOobOffset : sb));
        return t;
    };

    // One load of region block `block` of stage s0 of tile tt.  Masked: lanes
    // whose chunk is at or past K (every lane, for a stage past the end) read
    // zero.  glob: the tile lies inside C and the stage inside K, so the
    // unchecked global form reads only the operand.
    auto ld = [&](auto masked, auto glob, const Tile& tt, bool is_a, HK_LDS i32x4* dst,
                  uint32_t block, uint32_t voff, uint32_t s0) {
        const uint32_t s = rotated_stage(s0, krot, nk_whole);
        const uint32_t koff = s * (uint32_t)kRowBytes;
        if constexpr (decltype(glob)::value) {
            const uint8_t* base = is_a ? g.A + (int64_t)tt.m0 * g.lda_b + koff
                                       : g.B + (int64_t)tt.n0 * g.ldb_b + koff;
            load_lds_global_b128(base, (HK_LDS void*)(dst + block * 64u), voff);
            return;
        }
        // the stage offset rides in the (uniform) scalar offset; a masked lane's
        // vector offset alone already lies past the end of the buffer
        if constexpr (decltype(masked)::value)
            voff = koff + kc_lane * 16u < kbytes ? voff : kOobOffset;
        load_lds_b128(is_a ? tt.ra : tt.rb, (HK_LDS void*)(dst + block * 64u), voff, koff);
    };
    auto issue_hi = [&](auto masked, auto glob, const Tile& tt, const PP8Buf& d, uint32_t s) {
#pragma unroll
        for (int j = 0; j < 4; ++j) ld(masked, glob, tt, true, d.ahi, wq + 4u * j, vhi[j], s);
    };
    auto issue_lo = [&](auto masked, auto glob, const Tile& tt, const PP8Buf& d, uint32_t s) {
#pragma unroll
        for (int j = 0; j < 8; ++j) ld(masked, glob, tt, false, d.b, wq + 4u * j, vlo_b[j], s);
#pragma unroll
        for (int j = 0; j < 4; ++j) ld(masked, glob, tt, true, d.alo, wq + 4u * j, vlo_a[j], s);
    };

    // ---- LDS -> register fragments.  Fragment rows start at multiples of 16,
    // so the swizzle key depends on the lane only.  Group g's A rows are
    // region rows g*64 .. g*64+63 of both A-lo and A-hi.
    const uint32_t r16 = lane & 15u;
    const uint32_t g4 = lane >> 4;
    const uint32_t key = swz_key<kSwz>(r16);
    const uint32_t fa0 = (grp * 64u + r16) * kChunks + ((0u + g4) ^ key);
    const uint32_t fa1 = (grp * 64u + r16) * kChunks + ((4u + g4) ^ key);
    const uint32_t fb0 = (wq * 64u + r16) * kChunks + ((0u + g4) ^ key);
    const uint32_t fb1 = (wq * 64u + r16) * kChunks + ((4u + g4) ^ key);

    f32x4 acc[8][4];
    auto zero_acc = [&]() {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    };
    // A fragment is the lane's two 16-byte chunks of one row block: K chunks
    // g and g+4 of the stage.  BF16 feeds them to two 16x16x32 MFMAs (one
    // K slice each); FP8 feeds the pair to one 16x16x128 MFMA.
    auto frag = [](const HK_LDS i32x4* p, uint32_t o0, uint32_t o1) {
        return __builtin_shufflevector(p[o0], p[o1], 0, 1, 2, 3, 4, 5, 6, 7);
    };

    // matrix-core cluster over output row blocks mbase..mbase+3
    auto mma = [&](const int mbase, const i32x8 (&af)[4], const i32x8 (&bfr)[4]) {
        if constexpr (!kFp8) {
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb)
                        acc[mbase + mb][nb] = mfma_bf16_16x16x32(half_of(bfr[nb], c),
                                                                 half_of(af[mb], c),
                                                                 acc[mbase + mb][nb]);
        } else {
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
                    acc[mbase + mb][nb] =
                        mfma_fp8_16x16x128(bfr[nb], af[mb], acc[mbase + mb][nb]);
        }
    };

    // One stage t as four barrier-separated phases.  Group 0 runs
    // M1 C1 M2 C2, group 1 runs the same one phase later, so in every phase
    // one group issues memory work while the other issues matrix-core work.
    // cur holds stage t; oth holds stage t+1 (or is being filled with it).
    // The loader sends HI of stage sh of tile th and LO of stage sl of tile tl
    // (the next stage and the one after, possibly of the next tile).
    const bool loader = (grp == 0);
    auto stage = [&](auto masked, auto glob, const PP8Buf& cur, const PP8Buf& oth,
                     const Tile& th, uint32_t sh, const Tile& tl, uint32_t sl) {
        i32x8 af[4], bfr[4];
        // M1: A-lo fragments (row blocks 0-3) and all B fragments of stage t;
        // the loader sends HI(t+1) into the other buffer, whose A-hi was last
        // read in the previous stage's second memory phase
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) af[mb] = frag(cur.alo, fa0 + mb * 128, fa1 + mb * 128);
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) bfr[nb] = frag(cur.b, fb0 + nb * 128, fb1 + nb * 128);
        if (loader) issue_hi(masked, glob, th, oth, sh);
        wait_lgkmcnt0();
        fenced_barrier();
        // C1; then HI(t) must have landed (newer in flight: LO(t+1), HI(t+1))
        __builtin_amdgcn_s_setprio(1);
        mma(0, af, bfr);
        pin_all(acc);
        __builtin_amdgcn_s_setprio(0);
        if (loader) wait_vmcnt<16>();
        fenced_barrier();
        // M2: A-hi fragments (row blocks 4-7); every wave has finished with
        // this buffer's B and A-lo, so the loader sends LO(t+2) into them
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) af[mb] = frag(cur.ahi, fa0 + mb * 128, fa1 + mb * 128);
        if (loader) issue_lo(masked, glob, tl, cur, sl);
        wait_lgkmcnt0();
        fenced_barrier();
        // C2; then LO(t+1) must have landed (newer in flight: HI(t+1), LO(t+2))
        __builtin_amdgcn_s_setprio(1);
        mma(4, af, bfr);
        pin_all(acc);
        __builtin_amdgcn_s_setprio(0);
        if (loader) wait_vmcnt<16>();
        fenced_barrier();
    };

    // prologue: LO(0), HI(0), LO(1) of the first tile in flight; LO(0) must
    // have landed
    const std::true_type masked;
    const std::false_type unmasked;
    const std::false_type checked;
    const std::true_type unchecked;
    uint32_t w = blockIdx.x;
    Tile cur = tile(w);
    if (loader) {
        issue_lo(masked, checked, cur, buf0, 0);
        issue_hi(masked, checked, cur, buf0, 0);
        issue_lo(masked, checked, cur, buf1, 1);
        wait_vmcnt<16>();
    }
    fenced_barrier();
    if (grp == 1) fenced_barrier();  // start group 1 one phase behind
    zero_acc();

    for (;;) {
        const uint32_t w_next = w + gridDim.x;
        const Tile nxt = tile(w_next);
        // Stage pair (t, t+1) loads up to stage t+3, all whole stages of this
        // tile while t + 4 <= nk_whole.
        uint32_t t = 0;
        const bool inside = cur.m0 + kPP8Tile <= g.M && cur.n0 + kPP8Tile <= g.N;
        if (inside) {
            for (; t + 4 <= nk_whole; t += 2) {
                stage(unmasked, unchecked, buf0, buf1, cur, t + 1, cur, t + 2);
                stage(unmasked, unchecked, buf1, buf0, cur, t + 2, cur, t + 3);
            }
        } else {
            for (; t + 4 <= nk_whole; t += 2) {
                stage(unmasked, checked, buf0, buf1, cur, t + 1, cur, t + 2);
                stage(unmasked, checked, buf1, buf0, cur, t + 2, cur, t + 3);
            }
        }
        // the last pairs: stages at or past the end of this tile's K are the
        // next tile's first (stage s of this tile is stage s - nk_pad of the next)
        auto pick = [&](uint32_t s, uint32_t* s_out) -> const Tile& {
            const bool mine = s < nk_pad;
            *s_out = mine ? s : s - nk_pad;
            return mine ? cur : nxt;
        };
        for (; t < nk_pad; t += 2) {
            uint32_t h0, l0, h1, l1;
            const Tile& th0 = pick(t + 1, &h0);
            const Tile& tl0 = pick(t + 2, &l0);
            stage(masked, checked, buf0, buf1, th0, h0, tl0, l0);
            const Tile& th1 = pick(t + 2, &h1);
            const Tile& tl1 = pick(t + 3, &l1);
            stage(masked, checked, buf1, buf0, th1, h1, tl1, l1);
        }

        // ---- epilogue, at the start of this group's next memory phase: lane
        // holds C[m][n..n+3] for each (mb, nb)
        const uint32_t le = lane_id_here();
        const int32_t mrow = cur.m0 + (int32_t)(grp * 128u + (le & 15u));
        const float sc = kFp8 ? fp8_scale(g) : 1.0f;
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
            const int32_t m = mrow + mb * 16;
            store_c_rows(g.C + (int64_t)m * g.ldc, m < g.M, cur.n0 + (int32_t)(wq * 64u), le >> 4,
                         g.N, acc[mb], sc, g.c_align);
        }
        if (w_next >= total) break;
        w = w_next;
        cur = nxt;
        zero_acc();
    }
    if (grp == 0) fenced_barrier();  // match group 1's barrier count
    wait_all();                      // no LDS write may outlive the workgroup
    clock_stamp_end(wave);
}

// ------------------------------------------------------- 4-wave interleave
//
// "How to make AMD GPUs go brrr", section "Intra-processor scheduling: wave
// patterns": one wave per SIMD, each interleaving its own HBM->LDS loads and
// LDS reads with its matrix-core instructions.  A 256 x 256 tile of C per
// workgroup of 4 waves in a 2 x 2 arrangement; each wave owns a 128 x 128
// sub-tile as 8 x 8 blocks of 16 x 16 (256 fp32 accumulators per lane,
// pinned to the accumulation registers).
//
// LDS: two stage buffers, each an A and a B image of 256 rows x 128 bytes of
// K (64 BF16 or 128 E4M3) with the row layout of the ping-pong kernel (key
// row % 8, conflict-free for 16-row fragment reads).  A stage is split into
// two slices of matrix-core work, and each wave reads the fragments of the
// next slice while the matrix cores consume the current one's:
//
//   slice 0 of stage t:  MFMA  |  fragment reads
//   -- wait for this wave's reads and stage t+1's loads; workgroup barrier --
//   slice 1 of stage t:  MFMA  |  load stage t+2, read stage t+1's first fragments
//
// The barrier is the only one per stage: past it, every wave has finished
// reading stage t (so its buffer may be refilled with stage t+2) and every
// wave's share of stage t+1 has landed (so it may be read).
constexpr int kIL4Tile = 256;
constexpr int kIL4Threads = 256;
constexpr int kIL4StageI4 = kIL4Tile * kChunks;  // 16-byte chunks per operand per stage

struct IL4Buf {
    HK_LDS i32x4* a;
    HK_LDS i32x4* b;
};

// BF16 form: v_mfma_f32_16x16x32_bf16, which on gfx950 costs about 12% less
// energy per FLOP than the 32 x 32 shape when the matrix cores are kept busy
// (the sustained clock of this power-bound GEMM follows the energy per
// stage).  The two slices of a stage are its two K slices of 32 (chunks 0-3
// and 4-7):
//
//   slice 0 of stage t:  64 MFMA on F(t, 0)  |  read F(t, 1)
//   slice 1 of stage t:  64 MFMA on F(t, 1)  |  load stage t+2, read F(t+1, 0)
//
// Persistent: the grid has one workgroup per compute unit and workgroup b
// computes tiles w = b, b + G, b + 2G, ... (G = grid size), which keeps the
// workgroup-to-chiplet dealing and the co-resident windows of the tile map.
// The stage pipeline runs through tile boundaries: the two stages loaded
// past a tile's last one are the next tile's first two, so between tiles
// only the store of C remains.
//
// kAT, kBT: the operand is stored transposed (A as K x M, B as K x N: M or N
// contiguous, row stride lda or ldb), so that C = A^T B^T, A^T B or A B as
// well as A B^T.  A stage of such an operand is 64 K-rows x 512 bytes (the
// tile's 256 rows of the other index), loaded with the same direct loads (one
// load covers two K-rows; K-rows past K read zero through the buffer bounds)
// into an image whose 16-byte chunk c of K-row k sits at c ^ km_key(k).  A
// fragment (16 rows x 32 K) is built by two transposing reads
// (ds_read_b64_tr_b16).  Within each group of 16 lanes, output lane i's
// element r comes from source lane (i >> 2) + 4r, position i & 3 (measured
// on gfx950).  So source lane (a + 4r) of lane group g addresses K-row
// 8g + 4h + r, rows 4a .. 4a+3 of the block, and output lane i receives row
// i, K 8g + 4h .. +3: half of the MFMA operand, exactly what a K-contiguous
// image gives.  The key puts the 8 K-rows that one half-wave's read touches
// on distinct 32-byte bank groups.
__device__ __forceinline__ uint32_t km_key(uint32_t k) {
    return ((k & 3u) | (((k >> 3) & 3u) << 2)) << 1;
}
constexpr uint32_t kKMRowBytes = kIL4Tile * 2u;    // one K-row of a transposed stage image
constexpr uint32_t kKMStageRows = kRowBytes / 2u;  // 64 K-rows of bf16 per stage

template <bool kAT, bool kBT>
__device__ __forceinline__ void il4_bf16_body(const GemmArgs& g, const IL4Buf buf0,
                                              const IL4Buf buf1) {
    clock_stamp_begin(g.stamps);
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t wm = wave >> 1;  // A rows wm*128 .. +127
    const uint32_t wn = wave & 1u;  // B rows (C columns) wn*128 .. +127
    const uint32_t total = (uint32_t)g.grid.tiles_m * (uint32_t)g.grid.tiles_n;
    const uint32_t kbytes = (uint32_t)g.K * 2u;
    const uint32_t nk = (kbytes + kRowBytes - 1) / kRowBytes;
    const uint32_t nk_pad = (nk + 1u) & ~1u;  // stages run in pairs
    const uint32_t nk_whole = kbytes / kRowBytes;

    // ---- HBM -> LDS: block b = 8 rows, lane l -> row 8b + l/8, physical
    // chunk l%8 holding logical chunk (l%8) ^ (l/8).  Wave w sends blocks
    // w + 4j (j = 0..7) of A and of B: 16 loads per stage.
    const uint32_t kc_lane = (lane & 7u) ^ (lane >> 3);
    // Transposed operand: block wave + 4j = K-rows 2(wave + 4j), +1 of the
    // stage; lane l -> K-row 2 * block + l/32, physical chunk l%32.
    uint32_t voff_a[8], voff_b[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t row = (wave + 4u * j) * 8u + (lane >> 3);
        const uint32_t krow = 2u * (wave + 4u * j) + (lane >> 5);
        const uint32_t kmo = ((lane & 31u) ^ km_key(krow)) * 16u;
        voff_a[j] = kAT ? krow * g.lda_b + kmo : row * g.lda_b + kc_lane * 16u;
        voff_b[j] = kBT ? krow * g.ldb_b + kmo : row * g.ldb_b + kc_lane * 16u;
    }
    // Buffer resources of tile w's A and B row panels; rows past the matrix
    // edge read as zero.  A tile past the end (w >= total) gets empty
    // resources, so its loads read zeros and only keep the wait counts even.
    struct Tile {
        i32x4 ra, rb;
        int32_t m0, n0;
    };
    // rows r0 .. of an operand with `rows` rows: K-contiguous, the panel ends
    // with row rows - 1; transposed, it ends at K-row K - 1, row rows - 1
    auto panel = [&](bool trans, const uint8_t* X, uint32_t ld_b, int32_t rows, int32_t r0,
                     bool live) {
        const uint64_t sz = !live   ? 0
                            : trans ? (uint64_t)(g.K - 1) * ld_b + (uint64_t)(rows - r0) * 2u
                                    : (uint64_t)(rows - r0) * ld_b;
        const uint8_t* base = X + (trans ? (int64_t)r0 * 2 : (int64_t)r0 * ld_b);
        return make_rsrc_words(base, (uint32_t)(sz > kOobOffset ? kOobOffset : sz));
    };
    auto tile = [&](uint32_t w) {
        Tile t;
        uint32_t tm = 0, tn = 0;
        if (w < total) tile_of(w, g.grid, &tm, &tn);
        t.m0 = (int32_t)tm * kIL4Tile;
        t.n0 = (int32_t)tn * kIL4Tile;
        t.ra = panel(kAT, g.A, g.lda_b, g.M, t.m0, w < total);
        t.rb = panel(kBT, g.B, g.ldb_b, g.N, t.n0, w < total);
        return t;
    };
    // Load i (0-7: A block wave+4i, 8-15: B block wave+4(i-8)) of stage s of
    // tile tt into buffer d.  Masked: lanes whose chunk lies at or past K
    // (every lane, for a stage past the end) read zeros; the main loop, whose
    // stages all lie inside K, skips that select.
    const uint32_t krot = chiplet_k_rotation(nk_whole);
    // glob: the tile lies inside C and the stage inside K, so the unchecked
    // global form of the load reads only the operands
    auto send = [&](auto masked, const Tile& tt, const IL4Buf& d, uint32_t s0, int i,
                    auto glob) {
        const uint32_t s = rotated_stage(s0, krot, nk_whole);
        const uint32_t koff = s * (uint32_t)kRowBytes;
        const uint32_t blk = wave + 4u * (uint32_t)(i & 7);
        const bool km = i < 8 ? kAT : kBT;
        if constexpr (decltype(glob)::value) {
            const uint8_t* x = i < 8 ? g.A : g.B;
            const uint32_t ld_b = i < 8 ? g.lda_b : g.ldb_b;
            const int64_t r0 = i < 8 ? tt.m0 : tt.n0;
            // K-strided: the stage's first K-row, the tile's first column
            const uint8_t* base = km ? x + r0 * 2 + (int64_t)s * kKMStageRows * ld_b
                                     : x + r0 * ld_b + koff;
            load_lds_global_b128(base, (HK_LDS void*)((i < 8 ? d.a : d.b) + blk * 64u),
                                 i < 8 ? voff_a[i & 7] : voff_b[i & 7]);
            return;
        }
        const uint32_t ld_b = i < 8 ? g.lda_b : g.ldb_b;
        uint32_t vo = i < 8 ? voff_a[i & 7] : voff_b[i & 7];
        uint32_t so = koff;
        if (km) {
            // K-rows past K fall outside the buffer and read zeros.  The
            // stage's K-row offset goes into the VGPR offset: the buffer
            // range check does not count the SGPR offset.
            vo += s * kKMStageRows * ld_b;
            so = 0;
        } else if constexpr (decltype(masked)::value) {
            vo = koff + kc_lane * 16u < kbytes ? vo : kOobOffset;
        }
        load_lds_b128(i < 8 ? tt.ra : tt.rb, (HK_LDS void*)((i < 8 ? d.a : d.b) + blk * 64u), vo,
                      so);
    };

    // ---- LDS -> fragments.  Slice s of a 16-row block: lane l holds 8 bf16
    // of row (block base + l%16), logical chunk 4s + l/16.
    const uint32_t r16 = lane & 15u;
    const uint32_t g4 = lane >> 4;
    const uint32_t fo0 = r16 * kChunks + ((0u + g4) ^ (r16 & 7u));
    const uint32_t fo1 = r16 * kChunks + ((4u + g4) ^ (r16 & 7u));
    const uint32_t arow = wm * 128u;
    const uint32_t brow = wn * 128u;
    // transposed image: lane l (group g4, i = l%16, a = i%4, r = i/4) addresses
    // K-row 8 g4 + r (+ 32s + 4h), rows 4a .. 4a+3 of the block: chunk
    // 2 (block base / 16) + a/2 of that K-row, byte 8 (a%2).  km_key of those
    // K-rows is 2 (r | g4 << 2) for every s and h.
    const uint32_t km_a = lane & 3u;
    const uint32_t km_kk = ((lane >> 2) & 3u) | (g4 << 2);
    const uint32_t km_row =
        (8u * g4 + ((lane >> 2) & 3u)) * kKMRowBytes + (km_a & 1u) * 8u + (km_a >> 1) * 16u;
    auto read_km = [&](const HK_LDS i32x4* img, int s, uint32_t blk16) -> i32x4 {
        typedef short s16x4 __attribute__((ext_vector_type(4)));
        const HK_LDS uint8_t* p = (const HK_LDS uint8_t*)img + km_row + 32u * (blk16 ^ km_kk) +
                                  (uint32_t)(32 * s) * kKMRowBytes;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((HK_LDS s16x4*)p);
        const s16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((HK_LDS s16x4*)(p + 4u * kKMRowBytes));
        return __builtin_shufflevector(__builtin_bit_cast(i32x2, lo), __builtin_bit_cast(i32x2, hi),
                                       0, 1, 2, 3);
    };
    // fragment f of slice s: f = 0..7 A blocks, 8..15 B blocks
    auto read = [&](const IL4Buf& d, int s, int f) -> i32x4 {
        if (f < 8 ? kAT : kBT)
            return read_km(f < 8 ? d.a : d.b, s,
                           f < 8 ? arow / 16u + (uint32_t)f : brow / 16u + (uint32_t)(f - 8));
        const HK_LDS i32x4* base = f < 8 ? d.a + (arow + 16u * (uint32_t)f) * kChunks
                                         : d.b + (brow + 16u * (uint32_t)(f - 8)) * kChunks;
        return base[s == 0 ? fo0 : fo1];
    };

    f32x4 acc[8][8];
    auto zero_acc = [&]() {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc_settle();  // the zeroed accumulators before the first MFMA reads them
    };

    // MFMA q of a slice: A block mb = q / 8 as the "B" operand and B block nb
    // as the "A" operand (C^T, so a lane holds 4 consecutive columns of a C
    // row), nb running 0-7 on even rows and 7-0 on odd ones, so that every
    // MFMA shares a fragment with the one before it (about 0.6 % faster than
    // restarting each row at nb = 0: the chip is power-bound, and fewer
    // operand reads leave it more clock).  Fragments are read in the order the
    // list consumes them: A block 0, B blocks 0-7, A blocks 1-7.
    i32x4 fx[16], fy[16];
    auto mfma = [&](const i32x4 (&fr)[16], int q) {
        const int mb = q >> 3;
        const int nb = (mb & 1) ? 7 - (q & 7) : (q & 7);
        mfma_bf16_16x16x32_pinned(acc[mb][nb], fr[8 + nb], fr[mb]);
    };
    auto rd = [&](i32x4 (&fr)[16], const IL4Buf& d, int s, int r) {
        constexpr int kOrder[16] = {0, 8, 9, 10, 11, 12, 13, 14, 15, 1, 2, 3, 4, 5, 6, 7};
        fr[kOrder[r]] = read(d, s, kOrder[r]);
    };
    // 64 MFMAs per slice.  Slice 0 reads the 16 fragments of slice 1 within
    // its first 48 MFMAs, so that they have landed by the workgroup barrier
    // that ends it.
    auto slice0 = [&](const IL4Buf& cur) {
#pragma unroll
        for (int q = 0; q < 64; ++q) {
            mfma(fx, q);
            if (q % 3 == 2 && q / 3 < 16) rd(fy, cur, 1, q / 3);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // slice 1 of a stage: MFMAs on fy, the 16 loads of stage s of tile tt
    // into cur, and the reads of the next stage's slice 0 from nxt into fx
    auto slice1 = [&](auto masked, const Tile& tt, uint32_t s, const IL4Buf& cur,
                      const IL4Buf& nxt, auto glob) {
#pragma unroll
        for (int q = 0; q < 64; ++q) {
            mfma(fy, q);
            if ((q & 3) == 1) send(masked, tt, cur, s, q >> 2, glob);
            if ((q & 3) == 3) rd(fx, nxt, 0, q >> 2);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // stage t (in cur; the next stage in nxt) loading stage s of tile tt
    auto stage = [&](auto masked, const Tile& tt, uint32_t s, const IL4Buf& cur,
                     const IL4Buf& nxt, auto glob) {
        slice0(cur);
        wait_lgkmcnt0();  // F(t, 1) is in registers: this wave is done with stage t
        wait_vmcnt0();    // this wave's share of stage t+1 has landed
        fenced_barrier();
        slice1(masked, tt, s, cur, nxt, glob);
    };

    const std::true_type masked;
    const std::false_type unmasked;
    uint32_t w = blockIdx.x;
    Tile cur = tile(w);
    const std::false_type checked;
    const std::true_type unchecked;
#pragma unroll
    for (int i = 0; i < 16; ++i) send(masked, cur, buf0, 0, i, checked);
#pragma unroll
    for (int i = 0; i < 16; ++i) send(masked, cur, buf1, 1, i, checked);
    wait_vmcnt<16>();
    fenced_barrier();
#pragma unroll
    for (int r = 0; r < 16; ++r) rd(fx, buf0, 0, r);
    zero_acc();

    for (;;) {
        const uint32_t w_next = w + gridDim.x;
        const Tile nxt = tile(w_next);
        // Stage pair (t, t+1) loads stages t+2 and t+3, all inside K while
        // t + 4 <= the number of whole stages.
        uint32_t t = 0;
        // the whole-stage count taken afresh per tile: kept across the tile
        // loop, the compiler holds the loop-entry test in a register of its
        // own, which spills
        uint32_t nkw = nk_whole;
        asm volatile("" : "+s"(nkw));
        // a tile inside C: its whole stages take the global loads
        const bool inside = cur.m0 + kIL4Tile <= g.M && cur.n0 + kIL4Tile <= g.N;
        if (inside) {
            for (; t + 4 <= nkw; t += 2) {
                stage(unmasked, cur, t + 2, buf0, buf1, unchecked);
                stage(unmasked, cur, t + 3, buf1, buf0, unchecked);
            }
        } else {
            for (; t + 4 <= nkw; t += 2) {
                stage(unmasked, cur, t + 2, buf0, buf1, checked);
                stage(unmasked, cur, t + 3, buf1, buf0, checked);
            }
        }
        // the last pairs: stages at or past the end of this tile's K load
        // the next tile's first two stages (stage s of this tile is stage
        // s - nk_pad of the next)
        auto pick = [&](uint32_t s, uint32_t* s_out) {
            const bool mine = s < nk_pad;
            *s_out = mine ? s : s - nk_pad;
            Tile r;
            r.ra = mine ? cur.ra : nxt.ra;
            r.rb = mine ? cur.rb : nxt.rb;
            return r;
        };
        for (; t < nk_pad; t += 2) {
            uint32_t s0, s1;
            const Tile t0 = pick(t + 2, &s0);
            stage(masked, t0, s0, buf0, buf1, checked);
            const Tile t1 = pick(t + 3, &s1);
            stage(masked, t1, s1, buf1, buf0, checked);
        }
        acc_settle();  // the last MFMA results before the epilogue reads them

        // ---- epilogue: lane holds C[m][n..n+3] for each (mb, nb)
        const uint32_t le = lane_id_here();
        const int32_t mrow = cur.m0 + (int32_t)(arow + (le & 15u));
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
            const int32_t m = mrow + mb * 16;
            store_c_rows(g.C + (int64_t)m * g.ldc, m < g.M, cur.n0 + (int32_t)brow, le >> 4, g.N,
                         acc[mb], 1.0f, g.c_align);
        }
        if (w_next >= total) break;
        w = w_next;
        cur = nxt;
        zero_acc();
    }
    wait_all();  // no LDS write may outlive the workgroup
    clock_stamp_end(wave);
}

// FP8 form of the persistent 4-wave interleave: v_mfma_scale_f32_16x16x128_f8f6f4
// (E4M3 operands, unit block scales).  Same tile, LDS images, loads, tile
// walk and pipeline across tiles as the BF16 form; a stage row of 128 bytes
// is 128 E4M3 values, the whole K of one instruction, so a stage is one
// MFMA per 16 x 16 block (64 per wave).  A block's fragment is the lane's
// chunks g and g+4 (g = lane / 16) of row l%16, identically for A and B,
// which pairs the same K values on both sides.
//
// A full stage of fragments (16 blocks x 32 bytes per lane) is half the
// register file, so fragments are not double-buffered by stage.  Instead
// the stage is split by A blocks and each fragment is refilled as soon as
// its last reader has issued:
//
//   slice 0 of stage t:  MFMA A(t, 0-3) x B(t), A-block-major
//                        | read A(t, 2-7)
//   -- wait for this wave's reads and stage t+1's loads; workgroup barrier --
//   slice 1 of stage t:  MFMA A(t, 4-7) x B(t), B-block-major
//                        | after the last MFMA on B(t, n): read B(t+1, n);
//                        | read A(t+1, 0-1); load stage t+2
//
// The barrier is the only one per stage, with the same meaning as in the
// BF16 form.  A(t, 2) and A(t, 3) are read in slice 0 itself, 16 and 24
// MFMAs ahead of their first use.
//
// kMx: MXFP8, one E8M0 scale per 32 K-values of a row (OCP MX v1.0) in place
// of the per-tensor scales.  A stage's 128 K are 4 scale blocks, and the
// fragment layout above already gives lane group g block g's values of its
// row, so lane l's scale operand for a block is byte 4s + l/16 of the row's
// scales (stage s).  Scales travel HBM -> LDS in groups of four stages (16
// bytes per row: 4 KiB per operand per group, one direct load of 64 rows
// per wave and operand), issued with the loads of the group's first stage,
// into two group buffers used in turn across tiles.  Each fragment's scale
// is read (ds_read_u8) next to the fragment.  Blocks at or past K / 32 (the
// zero-filled stages at the end of K) get scale 127 (x1), whatever the
// bytes past a row's end hold.
constexpr int kMxGroupStages = 4;
constexpr uint32_t kMxGroupBytes = 2u * kIL4Tile * 16u;  // A and B scales of a group

// kAT, kBT (per-tensor FP8 only): the operand is stored K-strided (A as K x M,
// B as K x N, one byte per element, row stride lda or ldb).  A stage of such
// an operand is 128 K-rows x 256 bytes (the tile's 256 rows of M or N); one
// direct load covers four K-rows, and 16-byte chunk c of K-row k sits at
// c ^ km8_key(k).  A fragment (16 rows, the lane's 32 K values) is built by
// four transposing reads (ds_read_b64_tr_b8).  Within each group of 16 lanes,
// output lane i's byte r comes from source lane 2r + i/8, byte i%8 of its 8
// (measured on gfx950).  So source lane s of lane group g addresses K-row
// 16g + s/2 (+ 8, + 64, + 72 for the other reads), the half s%2 of the
// block's 16-byte chunk, and output lane i receives row i's 8 consecutive K
// values: the same operand a K-contiguous image gives.  The key puts the 8
// K-rows of one lane group on distinct chunks, and those of lane groups g
// and g+1 on disjoint sets of chunks.
__device__ __forceinline__ uint32_t km8_key(uint32_t k) {
    return (k & 7u) | (((k >> 4) & 1u) << 3);
}
constexpr uint32_t kKM8RowBytes = kIL4Tile;    // one K-row of an 8-bit transposed stage image
constexpr uint32_t kKM8StageRows = kRowBytes;  // 128 K-rows of E4M3 per stage

template <bool kMx, bool kAT = false, bool kBT = false>
__device__ __forceinline__ void il4_fp8_body(const GemmArgs& g, const IL4Buf buf0,
                                             const IL4Buf buf1, HK_LDS uint8_t* scl) {
    static_assert(!(kMx && (kAT || kBT)), "block scales take K-contiguous operands only");
    clock_stamp_begin(g.stamps);
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t wm = wave >> 1;  // A rows wm*128 .. +127
    const uint32_t wn = wave & 1u;  // B rows (C columns) wn*128 .. +127
    const uint32_t total = (uint32_t)g.grid.tiles_m * (uint32_t)g.grid.tiles_n;
    const uint32_t kbytes = (uint32_t)g.K;
    const uint32_t nk = (kbytes + kRowBytes - 1) / kRowBytes;
    const uint32_t nk_pad = (nk + 1u) & ~1u;  // stages run in pairs
    const uint32_t nk_whole = kbytes / kRowBytes;

    // ---- HBM -> LDS, as in the BF16 form: block b = 8 rows, lane l -> row
    // 8b + l/8, physical chunk l%8 holding logical chunk (l%8) ^ (l/8); wave
    // w sends blocks w + 4j (j = 0..7) of A and of B.
    const uint32_t kc_lane = (lane & 7u) ^ (lane >> 3);
    // K-strided operand: block b = K-rows 4b .. 4b+3 of the stage; lane l ->
    // K-row 4b + l/16, physical chunk l%16
    uint32_t voff_a[8], voff_b[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t row = (wave + 4u * j) * 8u + (lane >> 3);
        const uint32_t krow = 4u * (wave + 4u * j) + (lane >> 4);
        const uint32_t kmo = ((lane & 15u) ^ km8_key(krow)) * 16u;
        voff_a[j] = kAT ? krow * g.lda_b + kmo : row * g.lda_b + kc_lane * 16u;
        voff_b[j] = kBT ? krow * g.ldb_b + kmo : row * g.ldb_b + kc_lane * 16u;
    }
    struct Tile {
        i32x4 ra, rb;
        i32x4 rsa, rsb;  // MXFP8: the tile's scale rows
        int32_t m0, n0;
    };
    // rows r0 .. of an operand with `rows` rows: K-contiguous, the panel ends
    // with row rows - 1; K-strided, it ends at K-row K - 1, row rows - 1
    auto panel = [&](bool trans, const uint8_t* X, uint32_t ld_b, int32_t rows, int32_t r0,
                     bool live) {
        const uint64_t sz = !live   ? 0
                            : trans ? (uint64_t)(g.K - 1) * ld_b + (uint64_t)(rows - r0)
                                    : (uint64_t)(rows - r0) * ld_b;
        const uint8_t* base = X + (trans ? (int64_t)r0 : (int64_t)r0 * ld_b);
        return make_rsrc_words(base, (uint32_t)(sz > kOobOffset ? kOobOffset : sz));
    };
    auto tile = [&](uint32_t w) {
        Tile t;
        uint32_t tm = 0, tn = 0;
        if (w < total) tile_of(w, g.grid, &tm, &tn);
        t.m0 = (int32_t)tm * kIL4Tile;
        t.n0 = (int32_t)tn * kIL4Tile;
        t.ra = panel(kAT, g.A, g.lda_b, g.M, t.m0, w < total);
        t.rb = panel(kBT, g.B, g.ldb_b, g.N, t.n0, w < total);
        if constexpr (kMx) {
            const uint64_t xa = w < total ? (uint64_t)(g.M - t.m0) * g.ldsa : 0;
            const uint64_t xb = w < total ? (uint64_t)(g.N - t.n0) * g.ldsb : 0;
            t.rsa = make_rsrc_words(g.SA + (int64_t)t.m0 * g.ldsa,
                                    (uint32_t)(xa > kOobOffset ? kOobOffset : xa));
            t.rsb = make_rsrc_words(g.SB + (int64_t)t.n0 * g.ldsb,
                                    (uint32_t)(xb > kOobOffset ? kOobOffset : xb));
        }
        return t;
    };
    // ---- MXFP8 scales.  Group q of a tile (stages 4q .. 4q+3) lives in group
    // buffer (seq + q) & 1, where seq counts the groups of earlier tiles.
    // Buffer layout: A scales of the tile's 256 rows (16 bytes each: stage-in-
    // group major, block minor), then B's.  Wave w loads rows 64w .. 64w+63.
    const uint32_t nblocks = (uint32_t)g.K / 32u;
    const uint32_t ngroups = (nk_pad + kMxGroupStages - 1) / kMxGroupStages;
    auto send_scales = [&](const Tile& tt, uint32_t s, uint32_t seq) {
        if constexpr (kMx) {
            if (s % kMxGroupStages == 0) {
                HK_LDS uint8_t* d = scl + (seq & 1u) * kMxGroupBytes + wave * 64u * 16u;
                const uint32_t koff = (s / kMxGroupStages) * 16u;
                load_lds_b128(tt.rsa, (HK_LDS void*)d, (wave * 64u + lane) * g.ldsa, koff);
                load_lds_b128(tt.rsb, (HK_LDS void*)(d + kIL4Tile * 16u),
                              (wave * 64u + lane) * g.ldsb, koff);
            }
        }
    };
    // scale byte of lane (row r16 of a 16-row block at tile row `row0`, block
    // g4) for stage s of the tile whose group sequence starts at seq
    auto rd_scale = [&](auto masked, uint32_t operand, uint32_t row0, uint32_t s,
                        uint32_t seq) -> uint32_t {
        const HK_LDS uint8_t* p = scl + ((seq + s / kMxGroupStages) & 1u) * kMxGroupBytes +
                                  operand * (kIL4Tile * 16u) +
                                  (row0 + (lane & 15u)) * 16u + (s % kMxGroupStages) * 4u +
                                  (lane >> 4);
        uint32_t v = *p;
        if constexpr (decltype(masked)::value) v = 4u * s + (lane >> 4) < nblocks ? v : 127u;
        return v;
    };
    const uint32_t krot = kMx ? 0u : chiplet_k_rotation(nk_whole);
    // glob: the tile lies inside C and the stage inside K, so the unchecked
    // global form of the load reads only the operands.  MXFP8 and the kernels
    // with A K-strided keep the buffer form: measured, it was as fast for
    // MXFP8 and faster with A stored K x M.
    auto send = [&](auto masked, const Tile& tt, const IL4Buf& d, uint32_t s0, int i,
                    auto glob) {
        const uint32_t s = rotated_stage(s0, krot, nk_whole);
        const uint32_t koff = s * (uint32_t)kRowBytes;
        const uint32_t blk = wave + 4u * (uint32_t)(i & 7);
        if constexpr (decltype(glob)::value && !kMx && !kAT) {
            const bool km = i < 8 ? kAT : kBT;
            const uint8_t* x = i < 8 ? g.A : g.B;
            const uint32_t ld_b = i < 8 ? g.lda_b : g.ldb_b;
            const int64_t r0 = i < 8 ? tt.m0 : tt.n0;
            // K-strided: the stage's first K-row, the tile's first column
            const uint8_t* base = km ? x + r0 + (int64_t)s * kKM8StageRows * ld_b
                                     : x + r0 * ld_b + koff;
            load_lds_global_b128(base, (HK_LDS void*)((i < 8 ? d.a : d.b) + blk * 64u),
                                 i < 8 ? voff_a[i & 7] : voff_b[i & 7]);
            return;
        }
        uint32_t vo = i < 8 ? voff_a[i & 7] : voff_b[i & 7];
        uint32_t so = koff;
        if (i < 8 ? kAT : kBT) {
            // K-rows past K fall outside the buffer and read zeros; the
            // stage's K-row offset goes into the VGPR offset, which the
            // buffer range check covers
            vo += s * kKM8StageRows * (i < 8 ? g.lda_b : g.ldb_b);
            so = 0;
        } else if constexpr (decltype(masked)::value) {
            vo = koff + kc_lane * 16u < kbytes ? vo : kOobOffset;
        }
        if (i < 8)
            load_lds_b128(tt.ra, (HK_LDS void*)(d.a + blk * 64u), vo, so);
        else
            load_lds_b128(tt.rb, (HK_LDS void*)(d.b + blk * 64u), vo, so);
    };

    // ---- LDS -> fragments: lane l holds row (block base + l%16), logical
    // chunks g and g+4 (g = l/16) as one 32-byte operand.
    const uint32_t r16 = lane & 15u;
    const uint32_t g4 = lane >> 4;
    const uint32_t fo0 = r16 * kChunks + ((0u + g4) ^ (r16 & 7u));
    const uint32_t fo1 = r16 * kChunks + ((4u + g4) ^ (r16 & 7u));
    const uint32_t arow = wm * 128u;
    const uint32_t brow = wn * 128u;
    // K-strided image: lane l (group g4, s = l%16) reads K-row 16 g4 + s/2
    // (+ 8, + 64, + 72), half s%2 of the block's chunk; km8_key of those
    // K-rows is (s/2) | (g4 % 2) << 3 for all four reads.
    const uint32_t km8_kk = (r16 >> 1) | ((g4 & 1u) << 3);
    const uint32_t km8_row = (16u * g4 + (r16 >> 1)) * kKM8RowBytes + (r16 & 1u) * 8u;
    auto read_km8 = [&](const HK_LDS i32x4* img, uint32_t blk16) -> i32x8 {
        const HK_LDS uint8_t* p = (const HK_LDS uint8_t*)img + km8_row + 16u * (blk16 ^ km8_kk);
        i32x2 v[4];
#pragma unroll
        for (int c = 0; c < 4; ++c)
            v[c] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (HK_LDS i32x2*)(p + (uint32_t)(8 * (c & 1) + 64 * (c >> 1)) * kKM8RowBytes));
        const i32x4 lo = __builtin_shufflevector(v[0], v[1], 0, 1, 2, 3);
        const i32x4 hi = __builtin_shufflevector(v[2], v[3], 0, 1, 2, 3);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    auto rd_a = [&](const IL4Buf& d, int mb) -> i32x8 {
        if constexpr (kAT) return read_km8(d.a, arow / 16u + (uint32_t)mb);
        const HK_LDS i32x4* p = d.a + (arow + 16u * (uint32_t)mb) * kChunks;
        return __builtin_shufflevector(p[fo0], p[fo1], 0, 1, 2, 3, 4, 5, 6, 7);
    };
    auto rd_b = [&](const IL4Buf& d, int nb) -> i32x8 {
        if constexpr (kBT) return read_km8(d.b, brow / 16u + (uint32_t)nb);
        const HK_LDS i32x4* p = d.b + (brow + 16u * (uint32_t)nb) * kChunks;
        return __builtin_shufflevector(p[fo0], p[fo1], 0, 1, 2, 3, 4, 5, 6, 7);
    };

    f32x4 acc[8][8];
    uint32_t xa[8], xb[8];  // MXFP8: scale operands of the fragments in fa, fb
    uint32_t seq = 0;       // group sequence number of the current tile's group 0
    auto zero_acc = [&]() {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        acc_settle();  // the zeroed accumulators before the first MFMA reads them
    };
    // E8M0 exponent 127: block scale 1
    const uint32_t one = 127u;
    i32x8 fa[8], fb[8];
    // C^T block (mb, nb): B block nb as the "A" operand, A block mb as "B"
    auto mfma = [&](int mb, int nb) {
        if constexpr (kMx)
            mfma_mxfp8_16x16x128_pinned(acc[mb][nb], fb[nb], fa[mb], xb[nb], xa[mb]);
        else
            mfma_fp8_16x16x128_pinned(acc[mb][nb], fb[nb], fa[mb], one);
    };
    // fragment reads with their scales: stage s of the tile whose groups start
    // at sequence number sq
    auto get_a = [&](auto masked, const IL4Buf& d, int mb, uint32_t s, uint32_t sq) {
        fa[mb] = rd_a(d, mb);
        if constexpr (kMx) xa[mb] = rd_scale(masked, 0u, arow + 16u * (uint32_t)mb, s, sq);
    };
    auto get_b = [&](auto masked, const IL4Buf& d, int nb, uint32_t s, uint32_t sq) {
        fb[nb] = rd_b(d, nb);
        if constexpr (kMx) xb[nb] = rd_scale(masked, 1u, brow + 16u * (uint32_t)nb, s, sq);
    };

    // slice 0 of stage t (in cur)
    auto slice0 = [&](auto masked, const IL4Buf& cur, uint32_t t) {
#pragma unroll
        for (int q = 0; q < 32; ++q) {
            // rows of A blocks 0-3, B blocks reversed on odd rows (each MFMA
            // shares a fragment with the one before it)
            const int mb = q >> 3;
            mfma(mb, (mb & 1) ? 7 - (q & 7) : (q & 7));
            if (q % 3 == 0 && q / 3 < 6) get_a(masked, cur, 2 + q / 3, t, seq);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // slice 1 of stage t (in cur; stage t+1 in nxt, stage u1 of the tile whose
    // groups start at sequence sq1), loading stage s of tile tt (groups from ss)
    auto slice1 = [&](auto masked, const Tile& tt, uint32_t s, uint32_t ss, const IL4Buf& cur,
                      const IL4Buf& nxt, uint32_t u1, uint32_t sq1, auto glob) {
#pragma unroll
        for (int q = 0; q < 32; ++q) {
            // columns of B blocks 0-7 (ascending: each column's fragment is
            // refilled for the next stage once consumed), A blocks 4-7
            // reversed on odd columns
            const int nb = q >> 2;
            mfma(4 + ((nb & 1) ? 3 - (q & 3) : (q & 3)), nb);
            if (q & 1) send(masked, tt, cur, s, q >> 1, glob);
            else if ((q & 3) == 0 && q > 0) get_b(masked, nxt, (q >> 2) - 1, u1, sq1);
            else if (q == 2) get_a(masked, nxt, 0, u1, sq1);
            else if (q == 6) get_a(masked, nxt, 1, u1, sq1);
            else if (q == 10) send_scales(tt, s, ss + s / kMxGroupStages);
            __builtin_amdgcn_sched_barrier(0);
        }
        get_b(masked, nxt, 7, u1, sq1);
    };
    // stage t of the current tile; stage t+1 is stage u1 of the tile with group
    // sequence sq1 (this tile, or the next one past the end of K)
    auto stage = [&](auto masked, uint32_t t, const Tile& tt, uint32_t s, uint32_t ss,
                     const IL4Buf& cur, const IL4Buf& nxt, uint32_t u1, uint32_t sq1, auto glob) {
        slice0(masked, cur, t);
        wait_lgkmcnt0();  // A(t, 2-7) are in registers: this wave is done with stage t
        wait_vmcnt0();    // this wave's share of stage t+1 has landed
        fenced_barrier();
        slice1(masked, tt, s, ss, cur, nxt, u1, sq1, glob);
    };

    const std::true_type masked;
    const std::false_type unmasked;
    uint32_t w = blockIdx.x;
    Tile cur = tile(w);
    const std::false_type checked;
    const std::true_type unchecked;
    send_scales(cur, 0, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) send(masked, cur, buf0, 0, i, checked);
#pragma unroll
    for (int i = 0; i < 16; ++i) send(masked, cur, buf1, 1, i, checked);
    wait_vmcnt<16>();
    fenced_barrier();
    get_a(masked, buf0, 0, 0, 0);
    get_a(masked, buf0, 1, 0, 0);
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) get_b(masked, buf0, nb, 0, 0);
    zero_acc();

    for (;;) {
        const uint32_t w_next = w + gridDim.x;
        const Tile nxt = tile(w_next);
        uint32_t t = 0;
        // the whole-stage count taken afresh per tile (see il4_bf16_body)
        uint32_t nkw = nk_whole;
        asm volatile("" : "+s"(nkw));
        // a tile inside C: its whole stages take the global loads
        const bool inside = cur.m0 + kIL4Tile <= g.M && cur.n0 + kIL4Tile <= g.N;
        if (!kMx && !kAT && inside) {
            for (; t + 4 <= nkw; t += 2) {
                stage(unmasked, t, cur, t + 2, seq, buf0, buf1, t + 1, seq, unchecked);
                stage(unmasked, t + 1, cur, t + 3, seq, buf1, buf0, t + 2, seq, unchecked);
            }
        } else {
            for (; t + 4 <= nkw; t += 2) {
                stage(unmasked, t, cur, t + 2, seq, buf0, buf1, t + 1, seq, checked);
                stage(unmasked, t + 1, cur, t + 3, seq, buf1, buf0, t + 2, seq, checked);
            }
        }
        // stages at or past the end of this tile's K load the next tile's
        // first two (stage s of this tile is stage s - nk_pad of the next)
        auto pick = [&](uint32_t s, uint32_t* s_out) {
            const bool mine = s < nk_pad;
            *s_out = mine ? s : s - nk_pad;
            Tile r;
            r.ra = mine ? cur.ra : nxt.ra;
            r.rb = mine ? cur.rb : nxt.rb;
            if constexpr (kMx) {
                r.rsa = mine ? cur.rsa : nxt.rsa;
                r.rsb = mine ? cur.rsb : nxt.rsb;
            }
            return r;
        };
        const uint32_t seq_next = seq + ngroups;
        for (; t < nk_pad; t += 2) {
            uint32_t s0, s1;
            const Tile t0 = pick(t + 2, &s0);
            const uint32_t q0 = t + 2 < nk_pad ? seq : seq_next;
            stage(masked, t, t0, s0, q0, buf0, buf1, t + 1, seq, checked);
            const Tile t1 = pick(t + 3, &s1);
            const uint32_t q1 = t + 3 < nk_pad ? seq : seq_next;
            // stage t+2 is the next tile's stage 0 once t+2 reaches the end
            const uint32_t u2 = t + 2 < nk_pad ? t + 2 : 0u;
            const uint32_t qu = t + 2 < nk_pad ? seq : seq_next;
            stage(masked, t + 1, t1, s1, q1, buf1, buf0, u2, qu, checked);
        }
        acc_settle();  // the last MFMA results before the epilogue reads them

        // ---- epilogue: lane holds C[m][n..n+3] of block (mb, nb), times sA*sB
        const uint32_t le = lane_id_here();
        const int32_t mrow = cur.m0 + (int32_t)(arow + (le & 15u));
        const float sc = fp8_scale(g);
#pragma unroll
        for (int mb = 0; mb < 8; ++mb) {
            const int32_t m = mrow + mb * 16;
            store_c_rows(g.C + (int64_t)m * g.ldc, m < g.M, cur.n0 + (int32_t)brow, le >> 4, g.N,
                         acc[mb], sc, g.c_align);
        }
        if (w_next >= total) break;
        w = w_next;
        cur = nxt;
        seq = seq_next;
        zero_acc();
    }
    wait_all();  // no LDS write may outlive the workgroup
    clock_stamp_end(wave);
}

// ------------------------------------------------------- 8-wave interleave
//
// Eight waves (two per SIMD), each interleaving its own memory work with its
// own matrix-core instructions, so that both waves of a SIMD issue
// v_mfma_f32_16x16x32_bf16 at the same time.  On gfx950 one wave cannot
// issue that instruction back to back at the full rate, two waves can, and
// it costs less energy per FLOP than the 32 x 32 shape, which is what sets
// the sustained clock of a power-bound GEMM.  Wave w owns output rows
// (w / 4) * 128 .. +127 and columns (w % 4) * 64 .. +63 of the 256 x 256 tile
// as 8 x 4 blocks of 16 x 16 (128 accumulators per lane).
//
// LDS and pipeline as in the 4-wave kernel, with the two K slices of 32
// (chunks 0-3 and 4-7 of a 128-byte stage row) in place of its halves:
//
//   slice 0 of stage t:  MFMA on F(t, 0)  |  read F(t, 1)
//   -- wait for F(t, 1) and stage t+1's loads, workgroup barrier --
//   slice 1 of stage t:  MFMA on F(t, 1)  |  load stage t+2, read F(t+1, 0)
//
// The image rows use the ping-pong kernel's key (row % 8), conflict-free for
// 16-row fragment reads.  BF16 only.
constexpr int kI8Threads = 512;

__device__ __forceinline__ void i8_body(const GemmArgs& g, const IL4Buf buf0, const IL4Buf buf1) {
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t wm = wave >> 2;  // A rows wm*128 .. +127
    const uint32_t wn = wave & 3u;  // B rows (C columns) wn*64 .. +63

    uint32_t tm, tn;
    tile_of(blockIdx.x, g.grid, &tm, &tn);
    const int32_t m0 = (int32_t)tm * kIL4Tile;
    const int32_t n0 = (int32_t)tn * kIL4Tile;
    const uint32_t kbytes = (uint32_t)g.K * 2u;
    const uint32_t nk = (kbytes + kRowBytes - 1) / kRowBytes;

    // ---- HBM -> LDS: block b = 8 rows, lane l -> row 8b + l/8, physical
    // chunk l%8 holding logical chunk (l%8) ^ (l/8).  Wave w sends blocks
    // w + 8j (j = 0..3) of A and of B: 8 loads per stage.
    const uint32_t kc_lane = (lane & 7u) ^ (lane >> 3);
    uint32_t span_a, span_b;
    {
        const uint64_t sa = (uint64_t)(g.M - m0) * g.lda_b;
        const uint64_t sb = (uint64_t)(g.N - n0) * g.ldb_b;
        span_a = (uint32_t)(sa > kOobOffset ? kOobOffset : sa);
        span_b = (uint32_t)(sb > kOobOffset ? kOobOffset : sb);
    }
    const i32x4 rsrc_a = make_rsrc_words(g.A + (int64_t)m0 * g.lda_b, span_a);
    const i32x4 rsrc_b = make_rsrc_words(g.B + (int64_t)n0 * g.ldb_b, span_b);
    uint32_t voff_a[4], voff_b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t row = (wave + 8u * j) * 8u + (lane >> 3);
        voff_a[j] = row * g.lda_b + kc_lane * 16u;
        voff_b[j] = row * g.ldb_b + kc_lane * 16u;
    }
    // load i (0-3: A block wave+8i, 4-7: B block wave+8(i-4)) of stage s
    auto send = [&](auto masked, const IL4Buf& d, uint32_t s, int i) {
        const uint32_t koff = s * (uint32_t)kRowBytes;
        const uint32_t blk = wave + 8u * (uint32_t)(i & 3);
        uint32_t vo = i < 4 ? voff_a[i & 3] : voff_b[i & 3];
        if constexpr (decltype(masked)::value) vo = koff + kc_lane * 16u < kbytes ? vo : kOobOffset;
        if (i < 4)
            load_lds_b128(rsrc_a, (HK_LDS void*)(d.a + blk * 64u), vo, koff);
        else
            load_lds_b128(rsrc_b, (HK_LDS void*)(d.b + blk * 64u), vo, koff);
    };

    // ---- LDS -> fragments.  Slice s of a 16-row block: lane l holds 8 bf16
    // of row (block base + l%16), logical chunk 4s + l/16.
    const uint32_t r16 = lane & 15u;
    const uint32_t g4 = lane >> 4;
    const uint32_t fo0 = r16 * kChunks + ((0u + g4) ^ (r16 & 7u));
    const uint32_t fo1 = r16 * kChunks + ((4u + g4) ^ (r16 & 7u));
    const uint32_t arow = wm * 128u;
    const uint32_t brow = wn * 64u;
    // fragment f of slice s: f = 0..7 A blocks, 8..11 B blocks
    auto read = [&](const IL4Buf& d, int s, int f) -> i32x4 {
        const HK_LDS i32x4* base = f < 8 ? d.a + (arow + 16u * (uint32_t)f) * kChunks
                                         : d.b + (brow + 16u * (uint32_t)(f - 8)) * kChunks;
        return base[s == 0 ? fo0 : fo1];
    };

    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // MFMA q of a slice: B block nb = q % 4 as the "A" operand, A block
    // mb = q / 4 as the "B" operand (C^T, so a lane holds 4 consecutive
    // columns of one C row).  Fragments are read in the order the list
    // consumes them: A block 0, B blocks 0-3, A blocks 1-7.
    i32x4 fx[12], fy[12];
    auto mfma = [&](const i32x4 (&fr)[12], int q) {
        const int mb = q >> 2, nb = q & 3;
        acc[mb][nb] = mfma_bf16_16x16x32(fr[8 + nb], fr[mb], acc[mb][nb]);
    };
    auto rd = [&](i32x4 (&fr)[12], const IL4Buf& d, int s, int r) {
        constexpr int kOrder[12] = {0, 8, 9, 10, 11, 1, 2, 3, 4, 5, 6, 7};
        fr[kOrder[r]] = read(d, s, kOrder[r]);
    };
    auto slice0 = [&](const IL4Buf& cur) {
#pragma unroll
        for (int q = 0; q < 32; ++q) {
            mfma(fx, q);
            if ((q & 1) && q < 24) rd(fy, cur, 1, q >> 1);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto slice1 = [&](auto masked, const IL4Buf& cur, const IL4Buf& nxt, uint32_t t) {
#pragma unroll
        for (int q = 0; q < 32; ++q) {
            mfma(fy, q);
            if (q < 16) {
                if (q & 1) rd(fx, nxt, 0, q >> 1);
                else send(masked, cur, t + 2, q >> 1);
            } else if ((q & 1) && q < 24) {
                rd(fx, nxt, 0, 8 + ((q - 16) >> 1));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto stage = [&](auto masked, const IL4Buf& cur, const IL4Buf& nxt, uint32_t t) {
        slice0(cur);
        wait_lgkmcnt0();  // F(t, 1) is in registers: this wave is done with stage t
        wait_vmcnt0();    // this wave's share of stage t+1 has landed
        fenced_barrier();
        slice1(masked, cur, nxt, t);
    };

    const std::true_type masked;
    const std::false_type unmasked;
#pragma unroll
    for (int i = 0; i < 8; ++i) send(masked, buf0, 0, i);
#pragma unroll
    for (int i = 0; i < 8; ++i) send(masked, buf1, 1, i);
    wait_vmcnt<8>();
    fenced_barrier();
#pragma unroll
    for (int r = 0; r < 12; ++r) rd(fx, buf0, 0, r);
    const uint32_t nk_whole = kbytes / kRowBytes;
    uint32_t t = 0;
    for (; t + 4 <= nk_whole; t += 2) {
        stage(unmasked, buf0, buf1, t);
        stage(unmasked, buf1, buf0, t + 1);
    }
    for (; t < nk; t += 2) {
        stage(masked, buf0, buf1, t);
        stage(masked, buf1, buf0, t + 1);
    }
    wait_all();

    // ---- epilogue: lane holds C[m][n..n+3] for each (mb, nb)
    const int32_t mrow = m0 + (int32_t)(arow + r16);
    const int32_t ncol = n0 + (int32_t)(brow + g4 * 4u);
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
        const int32_t m = mrow + mb * 16;
        if (m < g.M) {
            uint16_t* crow = g.C + (int64_t)m * g.ldc;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const int32_t n = ncol + nb * 16;
                if (n < g.N) store_bf16x4(crow + n, n, g.N, acc[mb][nb], g.c_align);
            }
        }
    }
}

// ----------------------------------------------- producer / consumer waves
//
// Wave specialisation, the alternative the pages measure their 8-wave
// ping-pong against ("How to make AMD GPUs go brrr", section
// "Intra-processor scheduling: wave patterns"): four producer waves issue
// every HBM->LDS load, four consumer waves only read fragments and issue
// MFMAs.  A SIMD's register file is split evenly between its waves, so a
// consumer (sharing its SIMD with a producer) holds 128 accumulators: a
// 128 x 64 sub-tile, which makes the workgroup tile 256 x 128.  BF16 only;
// kept as the ablation of that design.
//
// LDS: two stage buffers of A (256 rows) and B (128 rows) x 128 bytes of K,
// rows keyed row % 8 as in the other kernels.  One barrier per stage:
//
//   consumers:  slice 0 of stage t (MFMA on F(t,0) | read F(t,1)); wait for
//               the reads; barrier; slice 1 (MFMA on F(t,1) | read F(t+1,0))
//   producers:  wait for their loads of stage t+1; barrier; load stage t+2
//               into the buffer the consumers just left
constexpr int kWSThreads = 512;
constexpr int kWSTileM = 256;
constexpr int kWSTileN = 128;
constexpr int kWSStageAI4 = kWSTileM * kChunks;
constexpr int kWSStageBI4 = kWSTileN * kChunks;

__device__ __forceinline__ void ws_body(const GemmArgs& g, const IL4Buf buf0, const IL4Buf buf1) {
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool producer = wave >= 4u;

    uint32_t tm, tn;
    tile_of(blockIdx.x, g.grid, &tm, &tn);
    const int32_t m0 = (int32_t)tm * kWSTileM;
    const int32_t n0 = (int32_t)tn * kWSTileN;
    const uint32_t kbytes = (uint32_t)g.K * 2u;
    const uint32_t nk = (kbytes + kRowBytes - 1) / kRowBytes;
    const uint32_t nk_pad = (nk + 1u) & ~1u;
    const uint32_t nk_whole = kbytes / kRowBytes;
    const std::true_type masked;
    const std::false_type unmasked;

    if (producer) {
        // producer p sends A blocks p + 4j (j = 0..7) and B blocks p + 4j
        // (j = 0..3): 12 loads per stage
        const uint32_t p = wave - 4u;
        const uint32_t kc_lane = (lane & 7u) ^ (lane >> 3);
        uint32_t span_a, span_b;
        {
            const uint64_t sa = (uint64_t)(g.M - m0) * g.lda_b;  // rows past the edge read zero
            const uint64_t sb = (uint64_t)(g.N - n0) * g.ldb_b;
            span_a = (uint32_t)(sa > kOobOffset ? kOobOffset : sa);
            span_b = (uint32_t)(sb > kOobOffset ? kOobOffset : sb);
        }
        const i32x4 rsrc_a = make_rsrc_words(g.A + (int64_t)m0 * g.lda_b, span_a);
        const i32x4 rsrc_b = make_rsrc_words(g.B + (int64_t)n0 * g.ldb_b, span_b);
        uint32_t voff_a[8], voff_b[4];
#pragma unroll
        for (int j = 0; j < 8; ++j)
            voff_a[j] = ((p + 4u * j) * 8u + (lane >> 3)) * g.lda_b + kc_lane * 16u;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            voff_b[j] = ((p + 4u * j) * 8u + (lane >> 3)) * g.ldb_b + kc_lane * 16u;
        auto issue = [&](auto msk, const IL4Buf& d, uint32_t s) {
            const uint32_t koff = s * (uint32_t)kRowBytes;
            const bool in_k = !decltype(msk)::value || koff + kc_lane * 16u < kbytes;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                load_lds_b128(rsrc_a, (HK_LDS void*)(d.a + (p + 4u * j) * 64u),
                              in_k ? voff_a[j] : kOobOffset, koff);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                load_lds_b128(rsrc_b, (HK_LDS void*)(d.b + (p + 4u * j) * 64u),
                              in_k ? voff_b[j] : kOobOffset, koff);
        };
        issue(masked, buf0, 0);
        issue(masked, buf1, 1);
        wait_vmcnt<12>();  // stage 0 landed
        fenced_barrier();
        for (uint32_t t = 0; t < nk_pad; t += 2) {
            wait_vmcnt0();  // stage t+1 landed
            fenced_barrier();
            if (t + 2 < nk_pad) {
                if (t + 2 < nk_whole) issue(unmasked, buf0, t + 2);
                else issue(masked, buf0, t + 2);
            }
            wait_vmcnt0();
            fenced_barrier();
            if (t + 3 < nk_pad) {
                if (t + 3 < nk_whole) issue(unmasked, buf1, t + 3);
                else issue(masked, buf1, t + 3);
            }
        }
        wait_all();  // no LDS write may outlive the workgroup
        return;
    }

    // ---- consumers: wave c owns A rows (c / 2) * 128 .. +127 and B rows
    // (c % 2) * 64 .. +63 as 8 x 4 blocks of 16 x 16
    const uint32_t wm = wave >> 1;
    const uint32_t wn = wave & 1u;
    const uint32_t r16 = lane & 15u;
    const uint32_t g4 = lane >> 4;
    const uint32_t fo0 = r16 * kChunks + ((0u + g4) ^ (r16 & 7u));
    const uint32_t fo1 = r16 * kChunks + ((4u + g4) ^ (r16 & 7u));
    const uint32_t arow = wm * 128u;
    const uint32_t brow = wn * 64u;
    auto read = [&](const IL4Buf& d, int s, int f) -> i32x4 {
        const HK_LDS i32x4* base = f < 8 ? d.a + (arow + 16u * (uint32_t)f) * kChunks
                                         : d.b + (brow + 16u * (uint32_t)(f - 8)) * kChunks;
        return base[s == 0 ? fo0 : fo1];
    };
    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    i32x4 fx[12], fy[12];
    auto mfma = [&](const i32x4 (&fr)[12], int q) {
        const int mb = q >> 2, nb = q & 3;
        acc[mb][nb] = mfma_bf16_16x16x32(fr[8 + nb], fr[mb], acc[mb][nb]);
    };
    // fragments in consumption order: A block 0, B blocks 0-3, A blocks 1-7
    auto rd = [&](i32x4 (&fr)[12], const IL4Buf& d, int s, int r) {
        constexpr int kOrder[12] = {0, 8, 9, 10, 11, 1, 2, 3, 4, 5, 6, 7};
        fr[kOrder[r]] = read(d, s, kOrder[r]);
    };
    auto stage = [&](const IL4Buf& cur, const IL4Buf& nxt) {
#pragma unroll
        for (int q = 0; q < 32; ++q) {
            mfma(fx, q);
            if ((q & 1) && q < 24) rd(fy, cur, 1, q >> 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        wait_lgkmcnt0();  // F(t, 1) is in registers: done with this stage's buffer
        fenced_barrier();
#pragma unroll
        for (int q = 0; q < 32; ++q) {
            mfma(fy, q);
            if ((q & 1) && q < 24) rd(fx, nxt, 0, q >> 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        pin_all(acc);
    };
    fenced_barrier();  // stage 0 landed
#pragma unroll
    for (int r = 0; r < 12; ++r) rd(fx, buf0, 0, r);
    for (uint32_t t = 0; t < nk_pad; t += 2) {
        stage(buf0, buf1);
        stage(buf1, buf0);
    }
    wait_all();

    const int32_t mrow = m0 + (int32_t)(arow + r16);
    const int32_t ncol = n0 + (int32_t)(brow + g4 * 4u);
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
        const int32_t m = mrow + mb * 16;
        if (m < g.M) {
            uint16_t* crow = g.C + (int64_t)m * g.ldc;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const int32_t n = ncol + nb * 16;
                if (n < g.N) store_bf16x4(crow + n, n, g.N, acc[mb][nb], g.c_align);
            }
        }
    }
}

// --------------------------------------------------------- small outputs
//
// For outputs with few 256 x 256 tiles, where the GEMM is bound by the
// latency of the first loads rather than by the matrix cores: 128 x 128
// tiles (four times as many workgroups), 4 waves in a 2 x 2 arrangement of
// 64 x 64 sub-tiles (4 x 4 blocks of 16 x 16), and a ring of four stage
// buffers (4 x 32 KiB) with three stages in flight ahead of the one being
// computed.  K up to three stages (192 BF16 or 384 E4M3) is fetched before
// the first matrix-core instruction; one barrier per stage:
//
//   stage t:  wait for this wave's share of stage t; workgroup barrier
//             (stage t is visible, buffer (t-1) % 4 is free);
//             load stage t+3 into buffer (t+3) % 4;
//             read and compute stage t
//
// Loads, LDS image rows and fragment layout are those of the 4-wave
// kernels (direct HBM -> LDS loads, key row % 8).
constexpr int kSTTile = 128;
constexpr int kSTThreads = 256;
constexpr int kSTStages = 4;
constexpr int kSTStageI4 = kSTTile * kChunks;  // 16-byte chunks per operand per stage

template <bool kFp8>
__device__ __forceinline__ void st4_body(const GemmArgs& g, HK_LDS i32x4* ring) {
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t wm = wave >> 1;  // A rows wm*64 .. +63
    const uint32_t wn = wave & 1u;  // B rows (C columns) wn*64 .. +63

    uint32_t tm, tn;
    tile_of(blockIdx.x, g.grid, &tm, &tn);
    const int32_t m0 = (int32_t)tm * kSTTile;
    const int32_t n0 = (int32_t)tn * kSTTile;
    const uint32_t kbytes = (uint32_t)g.K * (kFp8 ? 1u : 2u);
    const uint32_t nk = (kbytes + kRowBytes - 1) / kRowBytes;

    // ---- HBM -> LDS: an operand's stage is 16 blocks of 8 rows (lane l ->
    // row 8b + l/8, physical chunk l%8 holding logical chunk (l%8) ^ (l/8));
    // wave w sends blocks w + 4j (j = 0..3) of A and of B: 8 loads per stage.
    const uint32_t kc_lane = (lane & 7u) ^ (lane >> 3);
    uint32_t span_a, span_b;
    {
        const uint64_t sa = (uint64_t)(g.M - m0) * g.lda_b;  // rows past the edge read as zero
        const uint64_t sb = (uint64_t)(g.N - n0) * g.ldb_b;
        span_a = (uint32_t)(sa > kOobOffset ? kOobOffset : sa);
        span_b = (uint32_t)(sb > kOobOffset ? kOobOffset : sb);
    }
    const i32x4 rsrc_a = make_rsrc_words(g.A + (int64_t)m0 * g.lda_b, span_a);
    const i32x4 rsrc_b = make_rsrc_words(g.B + (int64_t)n0 * g.ldb_b, span_b);
    uint32_t voff_a[4], voff_b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t row = (wave + 4u * j) * 8u + (lane >> 3);
        voff_a[j] = row * g.lda_b + kc_lane * 16u;
        voff_b[j] = row * g.ldb_b + kc_lane * 16u;
    }
    auto buf_a = [&](uint32_t s) { return ring + (s % kSTStages) * 2u * kSTStageI4; };
    auto buf_b = [&](uint32_t s) { return ring + ((s % kSTStages) * 2u + 1u) * kSTStageI4; };
    // the 8 loads of stage s; lanes whose chunk lies at or past K (every
    // lane, for a stage past the end) read zeros, which keeps the wait
    // counts constant
    auto issue = [&](uint32_t s) {
        const uint32_t koff = s * (uint32_t)kRowBytes;
        const bool in_k = koff + kc_lane * 16u < kbytes;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t blk = wave + 4u * j;
            load_lds_b128(rsrc_a, (HK_LDS void*)(buf_a(s) + blk * 64u), in_k ? voff_a[j] : kOobOffset,
                          koff);
            load_lds_b128(rsrc_b, (HK_LDS void*)(buf_b(s) + blk * 64u), in_k ? voff_b[j] : kOobOffset,
                          koff);
        }
    };

    // ---- fragments: lane l holds row (block base + l%16), logical chunks
    // g and g+4 (g = l/16): the two K slices of 32 for BF16, the whole 128
    // E4M3 of one MFMA for FP8
    const uint32_t r16 = lane & 15u;
    const uint32_t g4 = lane >> 4;
    const uint32_t fo0 = r16 * kChunks + ((0u + g4) ^ (r16 & 7u));
    const uint32_t fo1 = r16 * kChunks + ((4u + g4) ^ (r16 & 7u));
    const uint32_t arow = wm * 64u;
    const uint32_t brow = wn * 64u;

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (uint32_t s = 0; s < kSTStages - 1; ++s) issue(s);
    for (uint32_t t = 0; t < nk; ++t) {
        wait_vmcnt<16>();  // stage t landed; stages t+1, t+2 may be in flight
        wait_lgkmcnt0();   // this wave's reads of stage t-1 are done
        fenced_barrier();
        issue(t + kSTStages - 1);
        const HK_LDS i32x4* pa = buf_a(t) + arow * kChunks;
        const HK_LDS i32x4* pb = buf_b(t) + brow * kChunks;
        i32x4 a0[4], a1[4], b0[4], b1[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a0[i] = pa[i * 16 * kChunks + fo0];
            b0[i] = pb[i * 16 * kChunks + fo0];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a1[i] = pa[i * 16 * kChunks + fo1];
            b1[i] = pb[i * 16 * kChunks + fo1];
        }
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                if constexpr (kFp8) {
                    acc[mb][nb] = mfma_fp8_16x16x128(
                        __builtin_shufflevector(b0[nb], b1[nb], 0, 1, 2, 3, 4, 5, 6, 7),
                        __builtin_shufflevector(a0[mb], a1[mb], 0, 1, 2, 3, 4, 5, 6, 7),
                        acc[mb][nb]);
                } else {
                    acc[mb][nb] = mfma_bf16_16x16x32(b0[nb], a0[mb], acc[mb][nb]);
                }
            }
        if constexpr (!kFp8) {
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                for (int nb = 0; nb < 4; ++nb)
                    acc[mb][nb] = mfma_bf16_16x16x32(b1[nb], a1[mb], acc[mb][nb]);
        }
    }
    wait_all();  // no LDS write may outlive the workgroup

    // ---- epilogue: lane holds C[m][n..n+3] of block (mb, nb)
    const int32_t mrow = m0 + (int32_t)(arow + r16);
    const int32_t ncol = n0 + (int32_t)(brow + g4 * 4u);
    const float sc = kFp8 ? fp8_scale(g) : 1.0f;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
        const int32_t m = mrow + mb * 16;
        if (m < g.M) {
            uint16_t* crow = g.C + (int64_t)m * g.ldc;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const int32_t n = ncol + nb * 16;
                if (n < g.N) {
                    f32x4 v = acc[mb][nb];
                    if constexpr (kFp8) v *= sc;
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
                if (am < g.M && k < g.K)
                    va = g.a_t ? g.A[k * g.lda_b + am] : g.A[(int64_t)am * g.lda_b + k];
                if (bn < g.N && k < g.K)
                    vb = g.b_t ? g.B[k * g.ldb_b + bn] : g.B[(int64_t)bn * g.ldb_b + k];
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
                if (am < g.M && k < g.K) va = g.a_t ? A16[k * lda + am] : A16[(int64_t)am * lda + k];
                if (bn < g.N && k < g.K) vb = g.b_t ? B16[k * ldb + bn] : B16[(int64_t)bn * ldb + k];
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
                    acc[mb][nb] = mfma_fp8_16x16x128(
                        __builtin_shufflevector(bfr[nb][0], bfr[nb][1], 0, 1, 2, 3, 4, 5, 6, 7),
                        __builtin_shufflevector(af[mb][0], af[mb][1], 0, 1, 2, 3, 4, 5, 6, 7),
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
    const float sc = kFp8 ? fp8_scale(g) : 1.0f;
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
                    if constexpr (kFp8) v *= sc;
                    store_bf16x4(crow + n, n, g.N, v, g.c_align);
                }
            }
        }
    }
}

}  // namespace hk
