// Device helpers shared by the attention kernels (forward and backward).
#pragma once

#include "sra_internal.h"

namespace sra {
namespace kc {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;

// Reductions across the two 32-lane halves of a wavefront (lane l and l ^ 32).
// v_permlane32_swap exchanges the upper half of its first operand with the
// lower half of its second; with x in both, each lane receives {own, partner}
// in its two results (in an order that depends on the half), so a symmetric
// combination of the two is the two-lane reduction in every lane.
__device__ __forceinline__ float halves_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// A value the compiler cannot prove wave-uniform (it went through vector
// registers) but that is: move it to scalar registers.
__device__ __forceinline__ uint64_t uniform_u64(uint64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ int64_t uniform_i64(int64_t x) { return (int64_t)uniform_u64((uint64_t)x); }

// Low (high) 16-bit halves of a and b packed as {a, b}: one v_perm_b32 each.
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

// Buffer resource over (what is left of) one device's slab of one head:
// loads at offsets past `bytes` read as zero, so tile loads need neither
// clamping nor branches.
constexpr int kBufferFlags = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slab_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kBufferFlags);
}

// ------------------------------------------------- loads straight into LDS --

// Workgroup barrier without a memory fence. Loads that write LDS directly
// complete asynchronously; a fenced barrier would make every wave wait for
// all of its loads in flight, which is exactly what a deep prefetch avoids.
// Ordering is explicit instead: a loading wave waits for its own loads of a
// tile (vmcnt) before the barrier that precedes the tile's first read, and
// LDS reads are complete (lgkmcnt) before the barriers after which their
// buffer can be refilled.
__device__ __forceinline__ void bar() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
// s_waitcnt immediates (gfx9 encoding): vmcnt in bits 3:0 and 15:14,
// expcnt in 6:4, lgkmcnt in 11:8; a field at its maximum is not waited on.
constexpr int kWaitLgkm0 = 0xC07F;   // lgkmcnt(0)

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource for `bytes` bytes at `base` (raw buffer: offsets at or
// past `bytes` read as zero), as four scalar words. Both arguments must be
// wave-uniform; readfirstlane keeps them in scalar registers even where the
// compiler cannot prove it.
__device__ __forceinline__ i32x4 raw_rsrc(uint64_t base, int bytes) {
    const int lo = __builtin_amdgcn_readfirstlane((int)(uint32_t)base);
    const int hi = __builtin_amdgcn_readfirstlane((int)(uint32_t)(base >> 32)) & 0xFFFF;
    return i32x4{lo, hi, __builtin_amdgcn_readfirstlane(bytes), kBufferFlags};
}

// One buffer_load_dwordx4 ... lds: lane l's 16 bytes at buffer offset voff go
// to LDS byte lds + 16 l (LDS base in M0). Issued from inline assembly so that
// the compiler's wait insertion, which would otherwise make every later LDS
// read wait for all loads in flight, leaves the loads alone; their
// completion is awaited explicitly (vmcnt) before the barrier that publishes
// the tile.
__device__ __forceinline__ void load_lds_b128(i32x4 rsrc, int voff, uint32_t lds) {
    asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voff), "s"(rsrc), "{m0}"(lds) : "memory");
}
// The same with 4 bytes per lane (LDS byte lds + 4 l).
__device__ __forceinline__ void load_lds_b32(i32x4 rsrc, int voff, uint32_t lds) {
    asm volatile("buffer_load_dword %0, %1, 0 offen lds" : : "v"(voff), "s"(rsrc), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
#define SRA_LDS4(p) ((__attribute__((address_space(3))) s16x4*)(p))

// ds_read_b64_tr_b16 pair: within each 16-lane group, lane i receives
// element i % 4 of the 8-byte pieces named by lanes 4v + i / 4 (v = 0..3);
// `p` and `p + row8` name two pieces, giving 8 values per lane.
__device__ __forceinline__ bf16x8 read_tr8(const bf16* p, int row8) {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(SRA_LDS4(p));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(SRA_LDS4(p + row8));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <bool B>
struct BoolTag {
    static constexpr bool value = B;
};

// Live keys of local query row j (int32 form of live_keys; |delta| <= L + 1).
__device__ __forceinline__ int live32(int j, int delta, int L) { return min(max(j + delta, 0), L); }

__device__ __forceinline__ int clamp_delta(int64_t dl, int L) {
    return (int)(dl < -(int64_t)L - 1 ? -(int64_t)L - 1 : (dl > (int64_t)L + 1 ? (int64_t)L + 1 : dl));
}

// Work item of a workgroup: tile index `tile` (0 = the heaviest of a group)
// within group (b, h, d). Workgroups are dealt to the 8 XCDs round-robin
// (hardware block i runs on XCD i mod 8) and each XCD has its own L2. When
// the group count G = B*H*nd is a multiple of 8, XCD x owns groups
// [x*G/8, (x+1)*G/8) -- devices of a head adjacent, so an XCD's workgroups
// stream the same slabs through its L2 -- and hands them out heaviest tile
// first, which makes the hardware's greedy dispatch a longest-job-first
// schedule. When an XCD owns an even number of groups it hands out all tiles
// of the first half of its groups before those of the second half (heaviest
// first within each half): the workgroups resident at one time then read
// fewer distinct K/V slabs (one head instead of two when an XCD owns two),
// which raises L2 reuse, and the greedy dispatch still pairs a CU's light
// first-half tile with a heavy second-half one. Otherwise blocks map in plain
// order.
struct WorkItem {
    int64_t b, h, d, heavy_rank;
};
__device__ __forceinline__ WorkItem decode_work(int64_t ntiles, int64_t B, int64_t H, int64_t nd, int64_t dev_lo,
                                                bool group_major = false) {
    const int64_t G = B * H * nd;
    const int64_t i = blockIdx.x;
    int64_t qi, g;
    if (group_major && (G & 7) == 0) {
        // One group at a time per XCD, its tiles heaviest first: the
        // workgroups resident on an XCD then all read the one key/value slab
        // of their group and share it through L2 (for launches whose groups
        // read different slabs, such as one ring round of every device).
        const int64_t gx = G >> 3;
        const int64_t m = i >> 3;
        qi = m % ntiles;
        g = (i & 7) * gx + m / ntiles;
    } else if ((G & 7) == 0 && ((G >> 3) & 1) == 0) {
        const int64_t gx = G >> 3, hx = gx >> 1;
        const int64_t m = i >> 3;
        const int64_t half = hx * ntiles;
        const int64_t mm = m < half ? m : m - half;
        qi = mm / hx;
        g = (i & 7) * gx + (m < half ? 0 : hx) + mm % hx;
    } else if ((G & 7) == 0) {
        const int64_t gx = G >> 3;
        const int64_t m = i >> 3;
        qi = m / gx;
        g = (i & 7) * gx + m % gx;
    } else {
        qi = i % ntiles;
        g = i / ntiles;
    }
    WorkItem w;
    w.d = uniform_i64(dev_lo + g % nd);
    g /= nd;
    w.h = uniform_i64(g % H);
    w.b = uniform_i64(g / H);
    w.heavy_rank = uniform_i64(qi);
    return w;
}

}  // namespace kc
}  // namespace sra
