// hk_device.hpp -- gfx950 device primitives used by the GEMM kernels.
//
// Vector types, buffer resources, direct HBM->LDS loads, LDS fragment reads,
// the two matrix-core instructions, schedule fences and the bf16 store path.
// Everything here is a thin, fixed-shape wrapper over a clang builtin; the
// kernels decide layout and schedule.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hk {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// Four dwords at a dword-aligned address: the vector memory unit takes a
// 16-byte access at any dword alignment, so C rows whose start is only
// 4-byte aligned (an even ldc) still get one store per 8 bf16.
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

#define HK_LDS __attribute__((address_space(3)))

// ---------------------------------------------------------------- buffers
//
// A raw buffer resource: base address, size in bytes, no stride.  Loads whose
// byte offset is at or beyond `bytes` return zero without touching memory;
// the kernels use that to zero-fill rows past the matrix edge and (with an
// offset of 0x80000000) K chunks past the end of a row.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    // dword3 0x00020000: 32-bit data format, no swizzle, raw addressing.
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

constexpr uint32_t kOobOffset = 0x80000000u;

// The same resource as four dwords, for the hand-issued direct loads below.
__device__ __forceinline__ i32x4 make_rsrc_words(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    return i32x4{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xFFFFu), (int)bytes, 0x00020000};
}

// One 16-byte direct load from a buffer into LDS: lane i of the wave writes
// its 16 bytes to lds_wave_base + 16*i (lds_wave_base is wave-uniform and goes
// through M0), fetched from byte voffset + soffset of the buffer.  Issued as
// inline assembly so that the compiler does not track the LDS write: the
// kernels order these writes against their LDS reads with explicit
// s_waitcnt vmcnt and workgroup barriers, and a compiler-inserted wait would
// serialise the loads they deliberately keep in flight.  M0 is an input
// operand ("{m0}"): the compiler writes it before the statement and knows it
// holds that value, so nothing it generates can be disturbed by the load.
// A direct load needs one wait state after M0 is written (the s_nop), which
// the compiler cannot see inside the statement.
__device__ __forceinline__ void load_lds_b128(i32x4 rsrc, HK_LDS void* lds_wave_base,
                                              uint32_t voffset, uint32_t soffset) {
    const uint32_t m0v = (uint32_t)(uintptr_t)lds_wave_base;
    asm volatile(
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %0, %1, %2 offen lds"
        :
        : "v"(voffset), "s"(rsrc), "s"(soffset), "{m0}"(m0v)
        : "memory");
}

// The same direct load through the global path: lane i fetches 16 bytes at
// base + voffset, with no range check.  The address path of these is cheaper
// than the buffer form's (measured: the sequencer's address FIFO toward the
// texture unit was full 19 times less often in the BF16 GEMM), so the 4-wave
// kernel uses them where every row and K chunk it loads lies inside the
// operand; base is wave-uniform.
__device__ __forceinline__ void load_lds_global_b128(const void* base, HK_LDS void* lds_wave_base,
                                                     uint32_t voffset) {
    const uint32_t m0v = (uint32_t)(uintptr_t)lds_wave_base;
    asm volatile(
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, %1"
        :
        : "v"(voffset), "s"(base), "{m0}"(m0v)
        : "memory");
}

// ------------------------------------------------------------ MFMA wrappers
//
// 16x16x32 bf16: each lane supplies 8 bf16 of one row of the 16 x 32 "A"
// operand and 8 of one column of the 32 x 16 "B" operand; lanes 16g..16g+15
// hold K positions 8g..8g+7.  The result lane l holds rows 4*(l/16)+v,
// column l%16 (v = 0..3).
__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(i32x4 a, i32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 16x16x128 with both operands in OCP E4M3 (format code 0) and unit block
// scales (E8M0 exponent 127 = 2^0): each lane supplies 32 bytes of K.
__device__ __forceinline__ f32x4 mfma_fp8_16x16x128(i32x8 a, i32x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// 32x32x16 bf16: lane l supplies 8 bf16 of row l%32 of the 32 x 16 "A"
// operand (K positions 8*(l/32) .. +7) and likewise of column l%32 of "B".
// The result lane l holds column l%32, rows 8j + 4*(l/32) + v in element
// 4j + v (j, v = 0..3).
__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(i32x4 a, i32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 32x32x64 with both operands in OCP E4M3 (format code 0) and unit block
// scales: lane l supplies 32 bytes of K of row (column) l%32; same result
// layout as the bf16 32x32 form.
__device__ __forceinline__ f32x16 mfma_fp8_32x32x64(i32x8 a, i32x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// The same instruction with the accumulator pinned to the accumulation
// registers (AGPRs): for kernels that keep 256 accumulators per lane, the
// compiler otherwise splits them between register files and copies them back
// and forth inside the loop.  Issued as inline assembly, so the compiler
// inserts no wait states for it: callers leave room between writing acc with
// ordinary instructions and this, and between this and reading acc
// (acc_settle below).  The compiler still waits for the loads that produce
// a and b, which are ordinary register operands.
__device__ __forceinline__ void mfma_bf16_16x16x32_pinned(f32x4& acc, i32x4 a, i32x4 b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// 16x16x128 E4M3 with unit block scales (`one` holds E8M0 127), accumulator
// pinned to the AGPRs like the BF16 form above.
__device__ __forceinline__ void mfma_fp8_16x16x128_pinned(f32x4& acc, i32x8 a, i32x8 b,
                                                          uint32_t one) {
    asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0]"
                 : "+a"(acc)
                 : "v"(a), "v"(b), "v"(one));
}

// 16x16x128 E4M3 with per-lane E8M0 block scales (byte 0 of sa for the "A"
// operand, of sb for "B"), accumulator pinned to the AGPRs.  Lane l's scale
// multiplies the 32 K-values of row l%16 in block l/16 of the instruction's
// 128: K 32g..32g+31 of the operand layout above, where lane group g holds
// K 16g..16g+15 in registers 0-3 and K 64+16g..64+16g+15 in registers 4-7
// (so block g's 32 values sit in lane groups 2(g%2) and 2(g%2)+1, register
// half g/2).  Measured on gfx950 with single-instruction probes.
__device__ __forceinline__ void mfma_mxfp8_16x16x128_pinned(f32x4& acc, i32x8 a, i32x8 b,
                                                            uint32_t sa, uint32_t sb) {
    asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
                 : "+a"(acc)
                 : "v"(a), "v"(b), "v"(sa), "v"(sb));
}

// Wait states that cover a matrix-core result (or an accumulator written by
// ordinary instructions) before its next reader: 4 x 8 idle cycles, more
// than the longest dependency the instructions above need.
__device__ __forceinline__ void acc_settle() {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}

// Half c (0 = low 16 bytes, 1 = high 16 bytes) of a 32-byte fragment.
__device__ __forceinline__ i32x4 half_of(i32x8 v, int c) {
    return c == 0 ? __builtin_shufflevector(v, v, 0, 1, 2, 3)
                  : __builtin_shufflevector(v, v, 4, 5, 6, 7);
}

// ------------------------------------------------------ schedule control
//
// A workgroup barrier that the compiler may not move any instruction across:
// the empty asm statements stop IR passes from moving memory accesses over it,
// sched_barrier stops the machine scheduler from moving anything.
__device__ __forceinline__ void fenced_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
}

// Make v look read and rewritten at this point, so that the instructions
// computing it stay before it (matrix-core intrinsics have no side effects
// and could otherwise be sunk past later barriers).
__device__ __forceinline__ void pin(f32x4& v) { asm volatile("" : "+v"(v)); }
template <int kM, int kN>
__device__ __forceinline__ void pin_all(f32x4 (&acc)[kM][kN]) {
#pragma unroll
    for (int i = 0; i < kM; ++i)
#pragma unroll
        for (int j = 0; j < kN; ++j) pin(acc[i][j]);
}

// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] at bits 3:0 and vmcnt[5:4]
// at 15:14, expcnt at 6:4, lgkmcnt at 11:8); a field at its maximum waits
// for nothing.
template <int kVm>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(kVm >= 0 && kVm < 64, "vmcnt is a 6-bit counter");
    __builtin_amdgcn_s_waitcnt((kVm & 15) | ((kVm >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_vmcnt0() { wait_vmcnt<0>(); }
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
__device__ __forceinline__ void wait_all() { __builtin_amdgcn_s_waitcnt(0x0070); }

// ------------------------------------------------------------- epilogue
//
// Two fp32 values -> two bf16 (round to nearest even) packed in one dword.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Store four consecutive bf16 of one C row, packed in two dwords (lo holds
// columns n, n+1), starting at column n and touching only columns < N.
// align is the guaranteed byte alignment of every 4-column group start
// (16, 8, 4 or 2).
__device__ __forceinline__ void store_packed4(uint16_t* p, int32_t n, int32_t N, uint32_t lo,
                                              uint32_t hi, int32_t align) {
    if (n + 4 <= N) {
        if (align >= 8) {
            *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
        } else if (align >= 4) {
            reinterpret_cast<uint32_t*>(p)[0] = lo;
            reinterpret_cast<uint32_t*>(p)[1] = hi;
        } else {
            p[0] = (uint16_t)lo;
            p[1] = (uint16_t)(lo >> 16);
            p[2] = (uint16_t)hi;
            p[3] = (uint16_t)(hi >> 16);
        }
    } else {
        if (n + 0 < N) p[0] = (uint16_t)lo;
        if (n + 1 < N) p[1] = (uint16_t)(lo >> 16);
        if (n + 2 < N) p[2] = (uint16_t)hi;
    }
}

// The same from four fp32 values (rounded to nearest even).
__device__ __forceinline__ void store_bf16x4(uint16_t* p, int32_t n, int32_t N, f32x4 v,
                                             int32_t align) {
    store_packed4(p, n, N, pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w), align);
}

// The lane's index in its wave, computed where it is called: as a volatile
// statement it is not hoisted out of a loop, so nothing holds it live across
// one (the 4-wave kernels use all 256 VGPRs there).
__device__ __forceinline__ uint32_t lane_id_here() {
    uint32_t l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// Optional clock record of a launch: the first workgroup dealt to each of the
// 8 chiplets (workgroups 0-7) writes the shader-clock counter (s_memtime,
// which advances with the chiplet's clock) and the constant-rate counter
// (s_memrealtime) at its start to stamps[4 * workgroup ..] and at its end to
// stamps[4 * workgroup + 2 ..].  stamps == nullptr writes nothing.  The end's
// address waits in an LDS slot, so no register holds it across the kernel.
__device__ __forceinline__ uint64_t** clock_slot() {
    __shared__ uint64_t* slot;
    return &slot;
}
__device__ __forceinline__ void clock_stamp_begin(uint64_t* stamps) {
    if (threadIdx.x == 0u) {
        uint64_t* p = nullptr;
        if (stamps != nullptr && blockIdx.x < 8u) {
            p = stamps + 4u * blockIdx.x;
            const uint64_t t = __builtin_amdgcn_s_memtime();
            const uint64_t r = __builtin_amdgcn_s_memrealtime();
            *reinterpret_cast<ulonglong2*>(p) = make_ulonglong2(t, r);
            p += 2;
        }
        *clock_slot() = p;
    }
}
// Called by every wave once its work (stores included) has completed; wave
// is the wave's index in the workgroup.
__device__ __forceinline__ void clock_stamp_end(uint32_t wave) {
    if (wave == 0u && lane_id_here() == 0u) {
        uint64_t* p = *clock_slot();
        if (p != nullptr) {
            const uint64_t t = __builtin_amdgcn_s_memtime();
            const uint64_t r = __builtin_amdgcn_s_memrealtime();
            *reinterpret_cast<ulonglong2*>(p) = make_ulonglong2(t, r);
        }
    }
}

// Swap between lane groups: rows of 16 lanes pair up as (0, 1) and (2, 3);
// the odd rows of x trade places with the even rows of y.  Afterwards a lane
// of an even row holds its own x and its partner's x in y; a lane of an odd
// row holds its partner's y in x and its own y.  The s_nop gives the two
// wait states a VALU write needs before the permute reads it.
__device__ __forceinline__ void swap_row_pairs(uint32_t& x, uint32_t& y) {
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(x), "+v"(y));
}

// Store one 16-row block of a wave's C sub-tile.  Lane (r, g) (r = lane % 16,
// g = lane / 16) holds, for blocks j = 0..kNB-1, C[m][c0 + 16j + 4g .. +3] in
// a[j] (times s); m is the lane's row, ok whether it lies inside C.  Whenever
// the 8-column groups are at least dword aligned (align 16, 8 or 4) each pair
// of blocks (j, j+1) goes out as one 16-byte store per lane: lane groups g
// and g+1 trade their halves (swap_row_pairs), so that even groups hold
// columns c0 + 16j + 4g .. +7 and odd groups c0 + 16(j+1) + 4(g-1) .. +7.
// Half the store instructions of 8-byte stores and a quarter of 4-byte ones,
// each covering 64 bytes of a row.  c0 is a multiple of 16 columns, so every
// group starts a multiple of 16 bytes into its row.
template <int kNB>
__device__ __forceinline__ void store_c_rows(uint16_t* crow, bool ok, int32_t c0, uint32_t g,
                                             int32_t N, const f32x4 (&a)[kNB], float s,
                                             int32_t align) {
    static_assert(kNB % 2 == 0, "blocks are stored in pairs");
    // an opaque copy of the lane group: the column offsets below are then
    // computed here, not hoisted out of the tile loop and kept live (spilled)
    // across it
    asm volatile("" : "+v"(g));
    if (align >= 4) {
#pragma unroll
        for (int j = 0; j < kNB; j += 2) {
            const f32x4 u = a[j] * s, v = a[j + 1] * s;
            uint32_t x0 = pack_bf16x2(u.x, u.y), x1 = pack_bf16x2(u.z, u.w);
            uint32_t y0 = pack_bf16x2(v.x, v.y), y1 = pack_bf16x2(v.z, v.w);
            swap_row_pairs(x0, y0);
            swap_row_pairs(x1, y1);
            const int32_t c = c0 + ((g & 1u) ? 16 * (j + 1) + 4 * (int32_t)(g - 1)
                                             : 16 * j + 4 * (int32_t)g);
            if (ok) {
                if (c + 8 <= N) {
                    const u32x4_a4 w = {x0, x1, y0, y1};
                    *reinterpret_cast<u32x4_a4*>(crow + c) = w;
                } else {
                    store_packed4(crow + c, c, N, x0, x1, align);
                    store_packed4(crow + c + 4, c + 4, N, y0, y1, align);
                }
            }
        }
    } else if (ok) {
#pragma unroll
        for (int j = 0; j < kNB; ++j) {
            const int32_t n = c0 + 16 * j + 4 * (int32_t)g;
            if (n < N) store_bf16x4(crow + n, n, N, a[j] * s, align);
        }
    }
}

}  // namespace hk
