// Stripe permutation (gather into striped device layout) and its inverse.
//
// Striped layout: device d holds every N-th token, positions d, d+N, d+2N, ...
// (Striped Attention summary page, "Summary" ¶2 and "Key points: Striped
// layout"; the permutation is applied once before the model). In device
// layout slot d*L + j holds position j*N + d, so
//   forward gather:  y[o, d*L + j, :] = x[o, j*N + d, :]
//   inverse gather:  x[o, j*N + d, :] = y[o, d*L + j, :]
// Both are pure row copies, HBM-bound: every byte is read once and written
// once.
//
// A workgroup owns a run of R consecutive tokens j0 .. j0+R-1 of one device d
// (and one outer slice, grid y), so the device index and the first token
// come from the block index once per workgroup, with no per-element
// division by the sequence length or the device count. Within the run the
// 256 threads take consecutive 16-byte chunks (4-byte words for rows that are
// not a multiple of 16 bytes) of the R rows, U per thread in flight before
// any store; the chunk's row within the run is a division by the chunks per
// row done with a multiply-high by a precomputed magic number. Measured on
// MI355X: U = 4 (16 KiB per workgroup pass) moves tensors of hundreds of MB
// at 6.2 TB/s with cold caches (5.4 with U = 8); U = 8 suits tensors of tens
// of MB (4.7 against 4.1 TB/s at 33 MB).
// Both the reads and the writes of a wavefront cover contiguous row
// segments. Non-temporal hints keep the streamed data from evicting other
// cache contents.
#include "sra_internal.h"

namespace sra {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr uint64_t kLargeBytes = (uint64_t)256 << 20;   // tensors at least this large take U = 4

// n / d for 32-bit n with an invariant divisor d (Granlund and Montgomery,
// "Division by invariant integers using multiplication", 1994): with
// l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1,
// n / d = (t + ((n - t) >> 1)) >> (l - 1), t = mulhi(m, n). l = 0 marks d = 1.
struct Div32 {
    uint32_t m;
    int32_t l;
    __device__ __forceinline__ uint32_t operator()(uint32_t n) const {
        if (l == 0) return n;
        const uint32_t t = __umulhi(m, n);
        return (t + ((n - t) >> 1)) >> (l - 1);
    }
};

Div32 make_div32(uint32_t d) {
    Div32 r{0u, 0};
    if (d <= 1) return r;
    int l = 0;
    while ((1ull << l) < d) ++l;
    r.l = l;
    r.m = (uint32_t)((((1ull << 32) * ((1ull << l) - d)) / d) + 1);
    return r;
}

// Copies the rows of token run (d, j0 .. j0+R-1) of outer slice blockIdx.y.
// `cpr` elements of type T per row; `bpd` workgroups per device; kUnroll
// elements per thread in flight. Consecutive workgroups take consecutive runs
// of one device (kDevMinor = false), or the same run of consecutive devices
// (kDevMinor = true). The second order makes the original-order rows j*N + d
// of neighbouring workgroups neighbours, so that side of the copy streams
// contiguously (the reads of the forward gather, the writes of the inverse):
// on a 6.4 GB tensor the forward gather moves 6.25 TB/s instead of 6.1 and the
// inverse 6.3 instead of 5.65. On tensors of tens of MB the first order is
// faster (inverse 3.3 against 3.1 TB/s at 33 MB).
template <typename T, bool kInverse, int kUnroll, bool kDevMinor>
__global__ void __launch_bounds__(kThreads) gather_run(const T* __restrict__ x, T* __restrict__ y, uint32_t seq,
                                                       uint32_t L, uint32_t N, uint32_t cpr, Div32 div_cpr,
                                                       uint32_t R, uint32_t bpd) {
    constexpr uint32_t kRunChunks = kThreads * kUnroll;   // chunks per workgroup pass
    const uint32_t d = kDevMinor ? blockIdx.x % N : blockIdx.x / bpd;
    const uint32_t j0 = (kDevMinor ? blockIdx.x / N : blockIdx.x - d * bpd) * R;
    const uint32_t rows = min(R, L - j0);
    const uint32_t total = rows * cpr;
    const uint64_t slice = (uint64_t)blockIdx.y * seq * cpr;
    // Source and destination row of local row r: device-layout slot d*L + j
    // and position j*N + d.
    const uint32_t dev_slot0 = d * L + j0;
    const uint32_t pos0 = j0 * N + d;
    for (uint32_t f0 = 0; f0 < total; f0 += kRunChunks) {
        T v[kUnroll];
        uint64_t dst[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const uint32_t f = f0 + u * kThreads + threadIdx.x;
            dst[u] = ~0ull;
            if (f < total) {
                const uint32_t r = div_cpr(f);
                const uint32_t c = f - r * cpr;
                const uint32_t slot = dev_slot0 + r, pos = pos0 + r * N;
                const uint32_t src_row = kInverse ? slot : pos;
                const uint32_t dst_row = kInverse ? pos : slot;
                v[u] = __builtin_nontemporal_load(&x[slice + (uint64_t)src_row * cpr + c]);
                dst[u] = slice + (uint64_t)dst_row * cpr + c;
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            if (dst[u] != ~0ull) __builtin_nontemporal_store(v[u], &y[dst[u]]);
    }
}

template <typename T, int kUnroll>
hipError_t launch_runs(const void* x, void* y, int64_t outer, int64_t seq, uint32_t cpr, int32_t n_dev, bool inverse,
                       hipStream_t stream) {
    constexpr uint32_t kRunChunks = kThreads * kUnroll;
    const uint32_t L = (uint32_t)(seq / n_dev);
    // Rows per workgroup: about kRunChunks chunks, at least one row.
    const uint32_t R = cpr >= kRunChunks ? 1u : kRunChunks / cpr;
    const uint32_t bpd = (L + R - 1) / R;
    const Div32 dv = make_div32(cpr);
    const uint64_t per_slice = (uint64_t)seq * cpr;
    // Grid y carries the outer index, at most 65535 slices per launch.
    for (int64_t o0 = 0; o0 < outer; o0 += 65535) {
        const unsigned ny = (unsigned)(outer - o0 < 65535 ? outer - o0 : 65535);
        const T* xs = (const T*)x + (uint64_t)o0 * per_slice;
        T* ys = (T*)y + (uint64_t)o0 * per_slice;
        const dim3 grid((unsigned)((uint64_t)n_dev * bpd), ny);
        // Large tensors (kUnroll = 4) go device-minor.
        if (inverse)
            hipLaunchKernelGGL((gather_run<T, true, kUnroll, kUnroll == 4>), grid, dim3(kThreads), 0, stream, xs, ys,
                               (uint32_t)seq, L, (uint32_t)n_dev, cpr, dv, R, bpd);
        else
            hipLaunchKernelGGL((gather_run<T, false, kUnroll, kUnroll == 4>), grid, dim3(kThreads), 0, stream, xs, ys,
                               (uint32_t)seq, L, (uint32_t)n_dev, cpr, dv, R, bpd);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_permute(const void* x, void* y, int64_t outer, int64_t seq, int64_t row_bytes,
                          int32_t n_dev, bool inverse, hipStream_t stream) {
    const bool large = (uint64_t)outer * (uint64_t)seq * (uint64_t)row_bytes >= kLargeBytes;
    if (row_bytes % 16 == 0 && ((uintptr_t)x % 16 == 0) && ((uintptr_t)y % 16 == 0)) {
        const uint32_t cpr = (uint32_t)(row_bytes / 16);
        return large ? launch_runs<u32x4, 4>(x, y, outer, seq, cpr, n_dev, inverse, stream)
                     : launch_runs<u32x4, 8>(x, y, outer, seq, cpr, n_dev, inverse, stream);
    }
    const uint32_t wpr = (uint32_t)(row_bytes / 4);
    return large ? launch_runs<uint32_t, 4>(x, y, outer, seq, wpr, n_dev, inverse, stream)
                 : launch_runs<uint32_t, 8>(x, y, outer, seq, wpr, n_dev, inverse, stream);
}

}  // namespace sra
