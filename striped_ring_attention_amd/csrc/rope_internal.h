// Internal declarations of the rotary-embedding gather (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sra {

constexpr int kRopeMaxHalf = 128;   // head_dim <= 256

// Output row (b, slot) of y holds the input token at original position t
// (t = (slot % L) * N + slot / L when `strided`, else t = slot), rotated by
// its position: pos[b * S + t] if pos is non-null, else t. Tensors are
// [B, S, H, D]; inv_freq[c] = base^(-2c/D) for c < D/2.
struct RopeArgs {
    const void* x;
    void* y;
    const int64_t* pos;
    int64_t B, S, H, L;
    int32_t D, N;
    int32_t strided;
    double inv_freq[kRopeMaxHalf];
};

hipError_t launch_rope(const RopeArgs& a, bool bf16_data, hipStream_t stream);

}  // namespace sra
