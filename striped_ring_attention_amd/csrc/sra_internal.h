// Internal declarations shared by the libsra sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sra {

// Liveness in local coordinates.
//
// Positions: striped pos(dev, i) = i*N + dev; contiguous pos(dev, i) = dev*L + i
// (device dev's i-th token; "Summary" ¶1-2 of the Striped Attention summary
// page). Key k of source device s is live for query j of device d iff
// pos(s, k) <= pos(d, j). Both layouts reduce this to a shifted causal mask
//     k < j + delta,   delta = delta(layout, d, s),
// because pos is affine in the local index with the same slope on both sides:
//   striped:    k*N + s <= j*N + d  <=>  k <= j + (d - s)/N, and |d - s| < N,
//               so delta = 1 if s <= d, else 0 (strict diagonal);
//   contiguous: s*L + k <= d*L + j  <=>  k <= j + (d - s)*L,
//               so delta = 1 + (d - s)*L (all keys if s < d, none if s > d).
// The number of live keys of query row j is clamp(j + delta, 0, L), which is
// nondecreasing in j; a key tile [k0, k1) is therefore FULL for query rows
// [j0, j1) iff k1 <= clamp(j0 + delta, 0, L) and EMPTY iff
// k0 >= clamp(j1 - 1 + delta, 0, L).
__host__ __device__ inline int64_t live_delta(int layout, int64_t n_dev, int64_t L, int64_t d, int64_t s) {
    if (layout == 1) return s <= d ? 1 : 0;
    return 1 + (d - s) * L;
}

__host__ __device__ inline int64_t live_keys(int64_t j, int64_t delta, int64_t L) {
    int64_t c = j + delta;
    return c < 0 ? 0 : (c > L ? L : c);
}

// Memory slot (row along the sequence axis) of device d's j-th token: d*L + j
// in device layout, and also in original order with the contiguous layout;
// j*N + d in original order with the striped layout ("strided": a device's
// tokens are every N-th row).
__host__ __device__ inline int64_t mem_slot(bool strided, int64_t N, int64_t L, int64_t d, int64_t j) {
    return strided ? j * N + d : d * L + j;
}

// Launchers (each returns hipSuccess or the launch error). Tensors are
// [B, S, H, Dh] with device d's j-th token at slot mem_slot(...); see sra.h
// for argument meaning.
struct RoundArgs {
    const void* q;
    const void* k;
    const void* v;
    float* o_acc;        // fp32 [B,S,H,Dh]: partial output, or merge accumulator
    float* lse_acc;      // fp32 [B,S,H]
    void* o_final;       // output in the input dtype (last round of the driver), or null
    int64_t* live_counts;
    int64_t B, S, H, L;
    int32_t N, layout, round, dev_lo, dev_hi;   // query devices [dev_lo, dev_hi)
    float scale;         // softmax scale
    float scale_log2;    // softmax scale * log2(e)
    int32_t strided;     // 1: tensors in original order with the striped layout (see mem_slot)
    int32_t mode;        // 0: write the partial to (o_acc, lse_acc); 1: merge it into them;
                         // 2: merge and write the output to o_final (dtype) and lse_acc;
                         // 3: write the partial as the output (o_final, lse_acc)
};

// start / stop: optional events recorded by the dispatch at the kernel's start and end.
hipError_t launch_round_bf16_d128(const RoundArgs& a, bool fused, hipStream_t stream, hipEvent_t start = nullptr,
                                  hipEvent_t stop = nullptr);

// Backward of the whole ring (every round), bf16 with head dim 128.
struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const float* lse;     // fp32 [B,S,H], natural log
    const void* dout;
    float* stats;         // fp32 [B,H,S,2] workspace: per memory slot (LSE * log2 e, rowsum(dO * O))
    void* dq;
    void* dk;
    void* dv;
    int64_t B, S, H, L;
    int32_t N, layout;
    int32_t strided;      // 1: tensors in original order with the striped layout (see mem_slot)
    float scale;
    float scale_log2;
};

hipError_t launch_bwd_bf16_d128(const BwdArgs& a, hipStream_t stream);

// Bytes of the library-held backward statistics array (one per GPU): 8 bytes
// per (b, s, h) row, so at most 33,554,432 rows.
constexpr size_t kBwdScratchBytes = (size_t)256 << 20;
// Device address of that array on the current device (looked up on the
// first call per device).
hipError_t bwd_scratch(void** ptr);
hipError_t launch_round_f32(const RoundArgs& a, int64_t head_dim, hipStream_t stream);

hipError_t launch_permute(const void* x, void* y, int64_t outer, int64_t seq, int64_t row_bytes,
                          int32_t n_dev, bool inverse, hipStream_t stream);

hipError_t launch_lse_merge(float* o_acc, float* lse_acc, const float* o_part, const float* lse_part,
                            int64_t rows, int64_t head_dim, hipStream_t stream);

constexpr int kBf16TileQ = 256;
constexpr int kBf16TileK = 64;
constexpr int kF32TileQ = 64;
constexpr int kF32TileK = 16;

}  // namespace sra
