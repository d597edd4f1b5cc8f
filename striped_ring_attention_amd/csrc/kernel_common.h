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
// first across all of its groups, which makes the hardware's greedy dispatch
// a longest-job-first schedule. Otherwise blocks map in plain order.
struct WorkItem {
    int64_t b, h, d, heavy_rank;
};
__device__ __forceinline__ WorkItem decode_work(int64_t ntiles, int64_t B, int64_t H, int64_t nd, int64_t dev_lo) {
    const int64_t G = B * H * nd;
    const int64_t i = blockIdx.x;
    int64_t qi, g;
    if ((G & 7) == 0) {
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
