// Stripe permutation (gather into striped device layout) and its inverse.
//
// Striped layout: device d holds every N-th token, positions d, d+N, d+2N, ...
// (Striped Attention summary page, "Summary" ¶2 and "Key points: Striped
// layout"; the permutation is applied once before the model). In device
// layout slot t = d*L + j holds position p = j*N + d, so
//   forward gather:  y[o, t, :] = x[o, (t mod L)*N + t div L, :]
//   inverse gather:  x[o, p, :] = y[o, (p mod N)*L + p div N, :]
// Both are pure row gathers, HBM-bound: every byte is read once and written
// once. Each thread moves 16-byte chunks; consecutive threads take
// consecutive chunks of one row, so both the read and the write of a
// wavefront cover contiguous row segments. Non-temporal hints keep the
// streamed data from evicting other cache contents.
#include "sra_internal.h"

namespace sra {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct IndexMap {
    uint32_t n_dev, L;
    int n_shift, l_shift;   // log2 when a power of two, else -1
    bool inverse;

    __device__ __forceinline__ uint32_t src_row(uint32_t t) const {
        // t is the output row within one outer slice.
        uint32_t a_div, a_mod;   // forward: t = d*L + j -> (d, j); inverse: p = j*N + d -> (j, d)
        if (!inverse) {
            if (l_shift >= 0) { a_div = t >> l_shift; a_mod = t & (L - 1); }
            else { a_div = t / L; a_mod = t - a_div * L; }
            return a_mod * n_dev + a_div;             // j*N + d
        } else {
            if (n_shift >= 0) { a_div = t >> n_shift; a_mod = t & (n_dev - 1); }
            else { a_div = t / n_dev; a_mod = t - a_div * n_dev; }
            return a_mod * L + a_div;                 // d*L + j
        }
    }
};

// Rows of 16-byte chunks; chunks per row = 1 << cpr_shift when cpr_shift >= 0.
__global__ void __launch_bounds__(256) gather_rows16(const u32x4* __restrict__ x, u32x4* __restrict__ y,
                                                     uint64_t total_chunks, uint32_t seq, uint32_t cpr,
                                                     int cpr_shift, IndexMap map) {
    uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t c = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total_chunks; c += stride) {
        uint64_t row;
        uint32_t chunk;
        if (cpr_shift >= 0) { row = c >> cpr_shift; chunk = (uint32_t)(c & (cpr - 1)); }
        else { row = c / cpr; chunk = (uint32_t)(c - row * cpr); }
        uint64_t outer = row / seq;
        uint32_t t = (uint32_t)(row - outer * seq);
        uint64_t src = (outer * seq + map.src_row(t)) * cpr + chunk;
        u32x4 v = __builtin_nontemporal_load(&x[src]);
        __builtin_nontemporal_store(v, &y[c]);
    }
}

// Same with 4-byte elements (rows whose size is not a multiple of 16 bytes).
__global__ void __launch_bounds__(256) gather_rows4(const uint32_t* __restrict__ x, uint32_t* __restrict__ y,
                                                    uint64_t total_words, uint32_t seq, uint32_t wpr,
                                                    IndexMap map) {
    uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t c = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total_words; c += stride) {
        uint64_t row = c / wpr;
        uint32_t w = (uint32_t)(c - row * wpr);
        uint64_t outer = row / seq;
        uint32_t t = (uint32_t)(row - outer * seq);
        y[c] = x[(outer * seq + map.src_row(t)) * wpr + w];
    }
}

int log2_exact(uint64_t v) {
    if (v == 0 || (v & (v - 1))) return -1;
    int s = 0;
    while ((1ull << s) != v) ++s;
    return s;
}

}  // namespace

hipError_t launch_permute(const void* x, void* y, int64_t outer, int64_t seq, int64_t row_bytes,
                          int32_t n_dev, bool inverse, hipStream_t stream) {
    IndexMap map;
    map.n_dev = (uint32_t)n_dev;
    map.L = (uint32_t)(seq / n_dev);
    map.n_shift = log2_exact(map.n_dev);
    map.l_shift = log2_exact(map.L);
    map.inverse = inverse;
    const int threads = 256;
    const uint64_t max_blocks = 256ull * 64;   // enough waves in flight on every CU; grid-stride beyond
    if (row_bytes % 16 == 0 && ((uintptr_t)x % 16 == 0) && ((uintptr_t)y % 16 == 0)) {
        uint32_t cpr = (uint32_t)(row_bytes / 16);
        uint64_t total = (uint64_t)outer * seq * cpr;
        uint64_t blocks = (total + threads - 1) / threads;
        if (blocks > max_blocks) blocks = max_blocks;
        hipLaunchKernelGGL(gather_rows16, dim3((unsigned)blocks), dim3(threads), 0, stream,
                           (const u32x4*)x, (u32x4*)y, total, (uint32_t)seq, cpr, log2_exact(cpr), map);
    } else {
        uint32_t wpr = (uint32_t)(row_bytes / 4);
        uint64_t total = (uint64_t)outer * seq * wpr;
        uint64_t blocks = (total + threads - 1) / threads;
        if (blocks > max_blocks) blocks = max_blocks;
        hipLaunchKernelGGL(gather_rows4, dim3((unsigned)blocks), dim3(threads), 0, stream,
                           (const uint32_t*)x, (uint32_t*)y, total, (uint32_t)seq, wpr, map);
    }
    return hipGetLastError();
}

}  // namespace sra
