// Rotary position embedding of model inputs, fused with the stripe gather.
//
// The striped layout is applied once, to the model's inputs before the first
// layer (Striped Attention summary page, research.elamur.ai, "Summary" ¶2 and
// "Key points: Striped layout"). A position-dependent encoding must still see
// each token's original position, so the rotation uses the position of the
// token in the original sequence (or an explicit position id), whatever slot
// it lands in. Rotate-half form: pair (c, c + D/2), c < D/2, of a head vector
// at position p turns by a_c = p * base^(-2c/D):
//   y_c = x_c cos a_c - x_{c+D/2} sin a_c,   y_{c+D/2} = x_c sin a_c + x_{c+D/2} cos a_c.
//
// One workgroup per output token row (b, slot): the D/2 angles of the row are
// reduced modulo 2*pi in fp64 and turned into (cos, sin) in fp32 once, in LDS,
// then every thread rotates four pairs of one head (coalesced: the threads of
// a head read the two halves of its row as contiguous runs). HBM-bound: each
// element is read once and written once.
#include "kernel_common.h"
#include "rope_internal.h"

namespace sra {
namespace {

using namespace kc;

constexpr int kRopeThreads = 256;

// 2*pi split into a double and its remainder (Cody-Waite reduction): for
// |a| < 2^40 the reduced angle a - k*2*pi is exact to a few ulps of fp64.
constexpr double kTwoPiHi = 6.283185307179586232;
constexpr double kTwoPiLo = 2.4492935982947063545e-16;
constexpr double kInvTwoPi = 0.15915494309189534561;

template <typename T>
struct Vec4;
template <>
struct Vec4<bf16> {
    using type = bf16x4;   // 8 bytes
};
template <>
struct Vec4<float> {
    using type = f32x4;    // 16 bytes
};

template <typename T>
__global__ void __launch_bounds__(kRopeThreads) rope_gather(RopeArgs a) {
    __shared__ float2 cs[kRopeMaxHalf];
    using V4 = typename Vec4<T>::type;
    const int64_t row = blockIdx.x;           // (b, slot) of the output
    const int64_t b = row / a.S;
    const int64_t slot = row - b * a.S;
    // Original position of the token in this slot.
    const int64_t t = a.strided ? (slot % a.L) * a.N + slot / a.L : slot;
    const int half = a.D / 2;

    if ((int)threadIdx.x < half) {
        const int c = threadIdx.x;
        const double p = a.pos != nullptr ? (double)a.pos[b * a.S + t] : (double)t;
        const double ang = p * a.inv_freq[c];
        const double k = rint(ang * kInvTwoPi);
        const double r = fma(-k, kTwoPiLo, fma(-k, kTwoPiHi, ang));
        float s, co;
        sincosf((float)r, &s, &co);
        cs[c] = float2{co, s};
    }
    __syncthreads();

    const T* xr = (const T*)a.x + (b * a.S + t) * a.H * a.D;
    T* yr = (T*)a.y + row * a.H * a.D;
    const int groups = half / 4;              // threads per head vector
    const int work = (int)a.H * groups;
    for (int i = threadIdx.x; i < work; i += kRopeThreads) {
        const int h = i / groups, c0 = 4 * (i - h * groups);
        // Each value is read and written once: non-temporal accesses keep the
        // stream from displacing cached data.
        const V4 lo = __builtin_nontemporal_load((const V4*)(xr + h * a.D + c0));
        const V4 hi = __builtin_nontemporal_load((const V4*)(xr + h * a.D + half + c0));
        V4 ylo, yhi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float2 w = cs[c0 + e];
            const float xl = (float)lo[e], xh = (float)hi[e];
            ylo[e] = (T)__builtin_fmaf(xl, w.x, -xh * w.y);
            yhi[e] = (T)__builtin_fmaf(xl, w.y, xh * w.x);
        }
        __builtin_nontemporal_store(ylo, (V4*)(yr + h * a.D + c0));
        __builtin_nontemporal_store(yhi, (V4*)(yr + h * a.D + half + c0));
    }
}

}  // namespace

hipError_t launch_rope(const RopeArgs& a, bool bf16_data, hipStream_t stream) {
    const int64_t rows = a.B * a.S;
    if (rows == 0) return hipSuccess;
    if (bf16_data)
        hipLaunchKernelGGL(rope_gather<bf16>, dim3((unsigned)rows), dim3(kRopeThreads), 0, stream, a);
    else
        hipLaunchKernelGGL(rope_gather<float>, dim3((unsigned)rows), dim3(kRopeThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace sra
