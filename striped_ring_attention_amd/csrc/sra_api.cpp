// Host side of the libsra C ABI: argument validation, the ring-round driver
// and the host-only census functions. Declarations and contracts: sra.h.
#include "../../include/sra.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "rope_internal.h"
#include "sra_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return status;
}

int hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return SRA_OK;
    return fail(SRA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

constexpr int64_t kMaxSeq = (int64_t)1 << 30;

// Shape checks common to every descriptor-based call.
int check_layout(int64_t seq, int32_t n_dev, int32_t layout) {
    if (layout != SRA_LAYOUT_CONTIGUOUS && layout != SRA_LAYOUT_STRIPED)
        return fail(SRA_ERR_INVALID_ARG, "layout %d is neither contiguous (0) nor striped (1)", layout);
    if (seq < 1 || seq > kMaxSeq) return fail(SRA_ERR_INVALID_ARG, "seq %lld out of range [1, 2^30]", (long long)seq);
    if (n_dev < 1 || n_dev > seq)
        return fail(SRA_ERR_INVALID_ARG, "n_dev %d out of range [1, seq=%lld]", n_dev, (long long)seq);
    if (seq % n_dev != 0)
        return fail(SRA_ERR_INVALID_ARG, "seq %lld is not a multiple of n_dev %d", (long long)seq, n_dev);
    return SRA_OK;
}

int check_desc(const sra_desc* d) {
    if (d == nullptr) return fail(SRA_ERR_INVALID_ARG, "desc is NULL");
    int st = check_layout(d->seq, d->n_dev, d->layout);
    if (st) return st;
    if (d->batch < 1 || d->heads < 1 || d->head_dim < 1)
        return fail(SRA_ERR_INVALID_ARG, "batch, heads and head_dim must be >= 1");
    if (d->dtype != SRA_DTYPE_F32 && d->dtype != SRA_DTYPE_BF16)
        return fail(SRA_ERR_INVALID_ARG, "dtype %d is neither f32 (0) nor bf16 (1)", d->dtype);
    if (d->schedule != SRA_SCHEDULE_PER_ROUND && d->schedule != SRA_SCHEDULE_FUSED)
        return fail(SRA_ERR_INVALID_ARG, "schedule %d unknown", d->schedule);
    if (d->order != SRA_ORDER_DEVICE && d->order != SRA_ORDER_ORIGINAL)
        return fail(SRA_ERR_INVALID_ARG, "order %d is neither device (0) nor original (1)", d->order);
    if (!(d->scale >= 0.f) || std::isinf(d->scale))
        return fail(SRA_ERR_INVALID_ARG, "scale must be finite and >= 0 (0 = 1/sqrt(head_dim))");
    // Element counts must fit comfortably in int64 and the grid in 32 bits.
    const double elems = (double)d->batch * (double)d->seq * (double)d->heads * (double)d->head_dim;
    if (elems > 9.0e18 / 8) return fail(SRA_ERR_INVALID_ARG, "tensor too large");
    const bool ok = (d->dtype == SRA_DTYPE_BF16 && d->head_dim == 128) ||
                    (d->dtype == SRA_DTYPE_F32 && (d->head_dim == 64 || d->head_dim == 128));
    if (!ok)
        return fail(SRA_ERR_UNSUPPORTED, "no kernel for dtype %d with head_dim %lld (supported: bf16/128, f32/64, f32/128)",
                    d->dtype, (long long)d->head_dim);
    const int64_t L = d->seq / d->n_dev;
    // Kernels address one device's slab of one head with 32-bit byte offsets
    // (including one tile of look-ahead past its end).
    const double slab = (double)(L + 2 * sra::kBf16TileK) * (double)d->heads * (double)d->head_dim * 4.0;
    if (slab > 2147483647.0) return fail(SRA_ERR_UNSUPPORTED, "a device slab of %lld tokens x %lld heads is too large for 32-bit offsets",
                                         (long long)L, (long long)d->heads);
    // In original order a device's consecutive tokens are N rows apart: one
    // key tile (plus a tile of look-ahead) must still span < 2^31 bytes.
    const double tile_span = (double)(2 * sra::kBf16TileK + 1) * (double)d->n_dev * (double)d->heads *
                             (double)d->head_dim * 4.0;
    if (d->order == SRA_ORDER_ORIGINAL && tile_span > 2147483647.0)
        return fail(SRA_ERR_UNSUPPORTED, "in original order %d devices x %lld heads is too wide for 32-bit tile offsets",
                    d->n_dev, (long long)d->heads);
    const int64_t tq = d->dtype == SRA_DTYPE_BF16 ? sra::kBf16TileQ : sra::kF32TileQ;
    const double blocks = (double)((L + tq - 1) / tq) * (double)d->heads * (double)d->n_dev * (double)d->batch;
    if (blocks > 2147483647.0) return fail(SRA_ERR_INVALID_ARG, "problem needs more than 2^31 workgroups per round");
    return SRA_OK;
}

float eff_scale(const sra_desc* d) { return d->scale > 0.f ? d->scale : (float)(1.0 / std::sqrt((double)d->head_dim)); }

sra::RoundArgs make_args(const sra_desc* d, const void* q, const void* k, const void* v) {
    sra::RoundArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.B = d->batch;
    a.S = d->seq;
    a.H = d->heads;
    a.L = d->seq / d->n_dev;
    a.N = d->n_dev;
    a.layout = d->layout;
    a.strided = d->order == SRA_ORDER_ORIGINAL && d->layout == SRA_LAYOUT_STRIPED;
    a.scale = eff_scale(d);
    a.scale_log2 = (float)((double)a.scale * 1.4426950408889634074);
    return a;
}

// Launch one round (or, fused, all of them). With events: the bf16 kernels
// have the dispatch record them at the kernel's start and end; the fp32
// kernels are bracketed by event records on the stream.
hipError_t launch_round(const sra_desc* d, const sra::RoundArgs& a, hipStream_t s, bool fused = false,
                        hipEvent_t start = nullptr, hipEvent_t stop = nullptr) {
    if (d->dtype == SRA_DTYPE_BF16) return sra::launch_round_bf16_d128(a, fused, s, start, stop);
    if (start != nullptr) {
        const hipError_t e = hipEventRecord(start, s);
        if (e != hipSuccess) return e;
    }
    const hipError_t e = sra::launch_round_f32(a, d->head_dim, s);
    if (e != hipSuccess || stop == nullptr) return e;
    return hipEventRecord(stop, s);
}

int64_t elem_bytes(const sra_desc* d) { return d->dtype == SRA_DTYPE_BF16 ? 2 : 4; }

// A byte range [p, p + bytes) named for error messages; bytes == 0 is empty.
struct Span {
    const void* p;
    size_t bytes;
    const char* name;
};

bool overlap(const Span& a, const Span& b) {
    if (a.p == nullptr || b.p == nullptr || a.bytes == 0 || b.bytes == 0) return false;
    const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
    return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

// Written buffers must be disjoint from every read buffer and from each other.
int check_disjoint(const Span* outs, int n_out, const Span* ins, int n_in) {
    for (int i = 0; i < n_out; ++i) {
        for (int j = 0; j < n_in; ++j)
            if (overlap(outs[i], ins[j]))
                return fail(SRA_ERR_INVALID_ARG, "%s overlaps the input %s", outs[i].name, ins[j].name);
        for (int j = i + 1; j < n_out; ++j)
            if (overlap(outs[i], outs[j]))
                return fail(SRA_ERR_INVALID_ARG, "outputs %s and %s overlap", outs[i].name, outs[j].name);
    }
    return SRA_OK;
}

}  // namespace

extern "C" {

int sra_abi_version(void) { return SRA_ABI_VERSION; }

const char* sra_status_str(int status) {
    switch (status) {
        case SRA_OK: return "SRA_OK";
        case SRA_ERR_INVALID_ARG: return "SRA_ERR_INVALID_ARG";
        case SRA_ERR_UNSUPPORTED: return "SRA_ERR_UNSUPPORTED";
        case SRA_ERR_HIP: return "SRA_ERR_HIP";
        case SRA_ERR_WORKSPACE: return "SRA_ERR_WORKSPACE";
        default: return "SRA_ERR_UNKNOWN";
    }
}

const char* sra_last_error(void) { return g_err; }

int sra_stripe_index(int64_t seq, int32_t n_dev, int32_t layout, int64_t* perm) {
    int st = check_layout(seq, n_dev, layout);
    if (st) return st;
    if (perm == nullptr) return fail(SRA_ERR_INVALID_ARG, "perm is NULL");
    const int64_t L = seq / n_dev;
    for (int64_t dv = 0; dv < n_dev; ++dv)
        for (int64_t j = 0; j < L; ++j) perm[dv * L + j] = layout == SRA_LAYOUT_STRIPED ? j * n_dev + dv : dv * L + j;
    return SRA_OK;
}

int sra_count_live_tiles(const sra_desc* desc, int64_t tile_q, int64_t tile_k, int64_t* live, int64_t* full,
                         int64_t* partial) {
    if (desc == nullptr) return fail(SRA_ERR_INVALID_ARG, "desc is NULL");
    int st = check_layout(desc->seq, desc->n_dev, desc->layout);
    if (st) return st;
    if (tile_q < 1 || tile_k < 1) return fail(SRA_ERR_INVALID_ARG, "tile sizes must be >= 1");
    if (live == nullptr) return fail(SRA_ERR_INVALID_ARG, "live is NULL");
    const int64_t N = desc->n_dev, L = desc->seq / N;
    const int64_t nk = (L + tile_k - 1) / tile_k;
    for (int64_t r = 0; r < N; ++r) {
        for (int64_t dv = 0; dv < N; ++dv) {
            const int64_t s = ((dv - r) % N + N) % N;
            const int64_t delta = sra::live_delta(desc->layout, N, L, dv, s);
            int64_t nl = 0, nf = 0;
            for (int64_t j0 = 0; j0 < L; j0 += tile_q) {
                const int64_t j1 = j0 + tile_q < L ? j0 + tile_q : L;
                const int64_t c_last = sra::live_keys(j1 - 1, delta, L);    // keys live for the last row
                const int64_t c_first = sra::live_keys(j0, delta, L);       // keys live for every row
                nl += (c_last + tile_k - 1) / tile_k;
                nf += c_first == L ? nk : c_first / tile_k;
            }
            live[r * N + dv] = nl;
            if (full) full[r * N + dv] = nf;
            if (partial) partial[r * N + dv] = nl - nf;
        }
    }
    return SRA_OK;
}

int sra_count_live_pairs(const sra_desc* desc, int64_t* pairs) {
    if (desc == nullptr) return fail(SRA_ERR_INVALID_ARG, "desc is NULL");
    int st = check_layout(desc->seq, desc->n_dev, desc->layout);
    if (st) return st;
    if (pairs == nullptr) return fail(SRA_ERR_INVALID_ARG, "pairs is NULL");
    const int64_t N = desc->n_dev, L = desc->seq / N;
    for (int64_t r = 0; r < N; ++r)
        for (int64_t dv = 0; dv < N; ++dv) {
            const int64_t s = ((dv - r) % N + N) % N;
            const int64_t delta = sra::live_delta(desc->layout, N, L, dv, s);
            int64_t n = 0;
            for (int64_t j = 0; j < L; ++j) n += sra::live_keys(j, delta, L);
            pairs[r * N + dv] = n;
        }
    return SRA_OK;
}

int sra_kernel_tiles(const sra_desc* desc, int32_t* tile_q, int32_t* tile_k) {
    int st = check_desc(desc);
    if (st) return st;
    if (tile_q == nullptr || tile_k == nullptr) return fail(SRA_ERR_INVALID_ARG, "tile_q/tile_k is NULL");
    *tile_q = desc->dtype == SRA_DTYPE_BF16 ? sra::kBf16TileQ : sra::kF32TileQ;
    *tile_k = desc->dtype == SRA_DTYPE_BF16 ? sra::kBf16TileK : sra::kF32TileK;
    return SRA_OK;
}

static int permute_common(const void* src, void* dst, int64_t outer, int64_t seq, int64_t row_bytes, int32_t n_dev,
                          bool inverse, void* stream) {
    int st = check_layout(seq, n_dev, SRA_LAYOUT_STRIPED);
    if (st) return st;
    if (src == nullptr || dst == nullptr) return fail(SRA_ERR_INVALID_ARG, "null tensor pointer");
    if (outer < 1) return fail(SRA_ERR_INVALID_ARG, "outer must be >= 1");
    if (row_bytes < 4 || row_bytes % 4 != 0) return fail(SRA_ERR_INVALID_ARG, "row_bytes must be a positive multiple of 4");
    // The gather indexes the elements of one row with 32 bits.
    if (row_bytes > ((int64_t)1 << 31)) return fail(SRA_ERR_INVALID_ARG, "row_bytes must be <= 2^31");
    if (((uintptr_t)src & 3u) || ((uintptr_t)dst & 3u)) return fail(SRA_ERR_INVALID_ARG, "tensors must be 4-byte aligned");
    const double total = (double)outer * (double)seq * (double)row_bytes;
    if (total > 4.0e18) return fail(SRA_ERR_INVALID_ARG, "tensor too large");
    const uintptr_t a0 = (uintptr_t)src, a1 = a0 + (uintptr_t)total, b0 = (uintptr_t)dst, b1 = b0 + (uintptr_t)total;
    if (a0 < b1 && b0 < a1) return fail(SRA_ERR_INVALID_ARG, "input and output overlap (in-place is not supported)");
    return hip_status(sra::launch_permute(src, dst, outer, seq, row_bytes, n_dev, inverse, (hipStream_t)stream),
                      inverse ? "unstripe launch" : "stripe_permute launch");
}

int sra_stripe_permute(const void* x, void* y, int64_t outer, int64_t seq, int64_t row_bytes, int32_t n_dev,
                       void* stream) {
    return permute_common(x, y, outer, seq, row_bytes, n_dev, false, stream);
}

int sra_unstripe(const void* y, void* x, int64_t outer, int64_t seq, int64_t row_bytes, int32_t n_dev, void* stream) {
    return permute_common(y, x, outer, seq, row_bytes, n_dev, true, stream);
}

int sra_ring_round_attn(const sra_desc* desc, int32_t round, int32_t device, const void* q, const void* k,
                        const void* v, float* o_part, float* lse_part, int64_t* live_counts, void* stream) {
    int st = check_desc(desc);
    if (st) return st;
    if (round < 0 || round >= desc->n_dev)
        return fail(SRA_ERR_INVALID_ARG, "round %d out of range [0, %d)", round, desc->n_dev);
    if (device < -1 || device >= desc->n_dev)
        return fail(SRA_ERR_INVALID_ARG, "device %d out of range [-1, %d)", device, desc->n_dev);
    if (!q || !k || !v || !o_part || !lse_part) return fail(SRA_ERR_INVALID_ARG, "null tensor pointer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o_part))
        return fail(SRA_ERR_INVALID_ARG, "q, k, v and o_part must be 16-byte aligned");
    if (((uintptr_t)lse_part & 3u) || ((uintptr_t)live_counts & 7u))
        return fail(SRA_ERR_INVALID_ARG, "lse_part / live_counts misaligned");
    sra::RoundArgs a = make_args(desc, q, k, v);
    a.o_acc = o_part;
    a.lse_acc = lse_part;
    a.o_final = nullptr;
    a.live_counts = live_counts;
    a.round = round;
    a.dev_lo = device < 0 ? 0 : device;
    a.dev_hi = device < 0 ? desc->n_dev : device + 1;
    a.mode = 0;
    return hip_status(launch_round(desc, a, (hipStream_t)stream), "ring_round_attn launch");
}

int sra_lse_merge(float* o_acc, float* lse_acc, const float* o_part, const float* lse_part, int64_t rows,
                  int64_t head_dim, void* stream) {
    if (!o_acc || !lse_acc || !o_part || !lse_part) return fail(SRA_ERR_INVALID_ARG, "null tensor pointer");
    if (rows < 0) return fail(SRA_ERR_INVALID_ARG, "rows must be >= 0");
    const int64_t q = head_dim / 4;
    if (head_dim < 4 || head_dim > 256 || head_dim % 4 || (q & (q - 1)))
        return fail(SRA_ERR_INVALID_ARG, "head_dim must be a power of two in [4, 256]");
    if (!aligned16(o_acc) || !aligned16(o_part)) return fail(SRA_ERR_INVALID_ARG, "o_acc / o_part must be 16-byte aligned");
    if (((uintptr_t)lse_acc & 3u) || ((uintptr_t)lse_part & 3u)) return fail(SRA_ERR_INVALID_ARG, "LSE misaligned");
    if ((double)rows * (double)head_dim > 4.0e18) return fail(SRA_ERR_INVALID_ARG, "tensor too large");
    return hip_status(sra::launch_lse_merge(o_acc, lse_acc, o_part, lse_part, rows, head_dim, (hipStream_t)stream),
                      "lse_merge launch");
}

size_t sra_fwd_workspace_bytes(const sra_desc* desc) {
    if (check_desc(desc)) return 0;
    // fp32 accumulates in o itself; one round or the fused schedule needs no accumulator.
    if (desc->dtype == SRA_DTYPE_F32 || desc->n_dev == 1 || desc->schedule == SRA_SCHEDULE_FUSED) return 0;
    return (size_t)(desc->batch * desc->seq * desc->heads * desc->head_dim) * sizeof(float);
}

int sra_ring_attn_fwd(const sra_desc* desc, const void* q, const void* k, const void* v, void* o, float* lse,
                      void* workspace, size_t workspace_bytes, int64_t* live_counts, void* const* round_events,
                      void* stream) {
    int st = check_desc(desc);
    if (st) return st;
    if (!q || !k || !v || !o || !lse) return fail(SRA_ERR_INVALID_ARG, "null tensor pointer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return fail(SRA_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
    if (((uintptr_t)lse & 3u) || ((uintptr_t)live_counts & 7u))
        return fail(SRA_ERR_INVALID_ARG, "lse / live_counts misaligned");
    if (desc->schedule == SRA_SCHEDULE_FUSED && desc->dtype != SRA_DTYPE_BF16)
        return fail(SRA_ERR_UNSUPPORTED, "the fused all-rounds schedule is built for bf16 only");
    const size_t need = sra_fwd_workspace_bytes(desc);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need))
        return fail(SRA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
    if (need > 0 && !aligned16(workspace)) return fail(SRA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    // Every buffer the driver writes (o, lse, the workspace) is written while
    // later rounds still read q, k and v, and the per-round schedule reads its
    // accumulator back: no written buffer may overlap an input or another
    // written buffer.
    const size_t nbytes = (size_t)(desc->batch * desc->seq * desc->heads * desc->head_dim * elem_bytes(desc));
    const size_t lbytes = (size_t)(desc->batch * desc->seq * desc->heads) * sizeof(float);
    const Span outs[3] = {{o, nbytes, "o"}, {lse, lbytes, "lse"}, {workspace, need, "workspace"}};
    const Span ins[3] = {{q, nbytes, "q"}, {k, nbytes, "k"}, {v, nbytes, "v"}};
    st = check_disjoint(outs, 3, ins, 3);
    if (st) return st;
    hipStream_t s = (hipStream_t)stream;
    sra::RoundArgs a = make_args(desc, q, k, v);
    a.live_counts = live_counts;
    a.dev_lo = 0;
    a.dev_hi = desc->n_dev;
    a.lse_acc = lse;
    const int N = desc->n_dev;
    const bool bf16 = desc->dtype == SRA_DTYPE_BF16;
    a.o_acc = bf16 ? (float*)workspace : (float*)o;
    a.o_final = o;
    if (desc->schedule == SRA_SCHEDULE_FUSED) {
        a.round = 0;
        a.mode = 3;
        hipError_t e = launch_round(desc, a, s, true, round_events ? (hipEvent_t)round_events[0] : nullptr,
                                    round_events ? (hipEvent_t)round_events[1] : nullptr);
        if (e != hipSuccess) return hip_status(e, "fused ring launch");
        return SRA_OK;
    }
    for (int r = 0; r < N; ++r) {
        a.round = r;
        if (bf16) a.mode = r == 0 ? (N == 1 ? 3 : 0) : (r == N - 1 ? 2 : 1);
        else a.mode = r == 0 ? 0 : 1;   // fp32: the accumulator is the output
        hipError_t e = launch_round(desc, a, s, false, round_events ? (hipEvent_t)round_events[2 * r] : nullptr,
                                    round_events ? (hipEvent_t)round_events[2 * r + 1] : nullptr);
        if (e != hipSuccess) return hip_status(e, "ring round launch");
    }
    return SRA_OK;
}

size_t sra_bwd_workspace_bytes(const sra_desc* desc) {
    if (check_desc(desc)) return 0;
    return (size_t)(desc->batch * desc->seq * desc->heads) * 2 * sizeof(float);
}

}  // extern "C"

namespace {

// Validation shared by the two backward entry points; `workspace` null with
// need_ws false skips the workspace checks (the allocation-free form uses the
// library's own array).
int bwd_check(const sra_desc* desc, const void* q, const void* k, const void* v, const void* o, const float* lse,
              const void* dout, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, bool need_ws) {
    int st = check_desc(desc);
    if (st) return st;
    if (desc->dtype != SRA_DTYPE_BF16)
        return fail(SRA_ERR_UNSUPPORTED, "the backward is built for bf16 with head_dim 128 only");
    if ((uint64_t)(desc->batch * desc->seq * desc->heads) >= (1ull << 32))
        return fail(SRA_ERR_UNSUPPORTED, "the backward indexes rows with 32 bits: batch * seq * heads < 2^32");
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv)
        return fail(SRA_ERR_INVALID_ARG, "null tensor pointer");
    for (const void* p : std::initializer_list<const void*>{q, k, v, o, dout, dq, dk, dv})
        if (!aligned16(p)) return fail(SRA_ERR_INVALID_ARG, "tensors must be 16-byte aligned");
    if ((uintptr_t)lse & 3u) return fail(SRA_ERR_INVALID_ARG, "lse misaligned");
    const size_t need = sra_bwd_workspace_bytes(desc);
    if (need_ws) {
        if (workspace == nullptr || workspace_bytes < need)
            return fail(SRA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace_bytes);
        if ((uintptr_t)workspace & 15u) return fail(SRA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    }
    // The gradients and the workspace (written by the first kernel, read by
    // the later ones) must not overlap any input or one another.
    const size_t nbytes = (size_t)(desc->batch * desc->seq * desc->heads * desc->head_dim * 2);
    const size_t lbytes = (size_t)(desc->batch * desc->seq * desc->heads) * sizeof(float);
    const Span outs[4] = {{dq, nbytes, "dq"}, {dk, nbytes, "dk"}, {dv, nbytes, "dv"},
                          {need_ws ? workspace : nullptr, need, "workspace"}};
    const Span ins[6] = {{q, nbytes, "q"}, {k, nbytes, "k"}, {v, nbytes, "v"},
                         {o, nbytes, "o"}, {dout, nbytes, "dout"}, {lse, lbytes, "lse"}};
    return check_disjoint(outs, 4, ins, 6);
}

sra::BwdArgs bwd_args(const sra_desc* desc, const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, void* dq, void* dk, void* dv, float* stats) {
    sra::BwdArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.dout = dout;
    a.stats = stats;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.B = desc->batch;
    a.S = desc->seq;
    a.H = desc->heads;
    a.L = desc->seq / desc->n_dev;
    a.N = desc->n_dev;
    a.layout = desc->layout;
    a.strided = desc->order == SRA_ORDER_ORIGINAL && desc->layout == SRA_LAYOUT_STRIPED;
    a.scale = eff_scale(desc);
    a.scale_log2 = (float)((double)a.scale * 1.4426950408889634074);
    return a;
}

}  // namespace

extern "C" {

int sra_ring_attn_bwd(const sra_desc* desc, const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, void* dq, void* dk, void* dv, void* workspace,
                      size_t workspace_bytes, void* stream) {
    const int st = bwd_check(desc, q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes, true);
    if (st) return st;
    const sra::BwdArgs a = bwd_args(desc, q, k, v, o, lse, dout, dq, dk, dv, (float*)workspace);
    return hip_status(sra::launch_bwd_bf16_d128(a, (hipStream_t)stream), "ring backward launch");
}

int sra_ring_attn_bwd_noalloc(const sra_desc* desc, const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dout, void* dq, void* dk, void* dv, void* stream) {
    const int st = bwd_check(desc, q, k, v, o, lse, dout, dq, dk, dv, nullptr, 0, false);
    if (st) return st;
    const size_t need = sra_bwd_workspace_bytes(desc);
    if (need > sra::kBwdScratchBytes)
        return fail(SRA_ERR_WORKSPACE,
                    "batch * seq * heads = %lld rows need %zu bytes of statistics; the allocation-free backward "
                    "holds %zu bytes (at most %zu rows)",
                    (long long)(desc->batch * desc->seq * desc->heads), need, sra::kBwdScratchBytes,
                    sra::kBwdScratchBytes / 8);
    void* stats = nullptr;
    const hipError_t e = sra::bwd_scratch(&stats);
    if (e != hipSuccess) return hip_status(e, "scratch address lookup");
    const sra::BwdArgs a = bwd_args(desc, q, k, v, o, lse, dout, dq, dk, dv, (float*)stats);
    return hip_status(sra::launch_bwd_bf16_d128(a, (hipStream_t)stream), "ring backward launch");
}

int sra_rope_permute(const sra_desc* desc, const void* x, void* y, const int64_t* pos, double base, void* stream) {
    if (desc == nullptr) return fail(SRA_ERR_INVALID_ARG, "desc is NULL");
    int st = check_layout(desc->seq, desc->n_dev, desc->layout);
    if (st) return st;
    if (desc->batch < 1 || desc->heads < 1) return fail(SRA_ERR_INVALID_ARG, "batch and heads must be >= 1");
    if (desc->dtype != SRA_DTYPE_F32 && desc->dtype != SRA_DTYPE_BF16)
        return fail(SRA_ERR_INVALID_ARG, "dtype %d is neither f32 (0) nor bf16 (1)", desc->dtype);
    if (desc->order != SRA_ORDER_DEVICE && desc->order != SRA_ORDER_ORIGINAL)
        return fail(SRA_ERR_INVALID_ARG, "order %d is neither device (0) nor original (1)", desc->order);
    if (desc->head_dim < 8 || desc->head_dim > 2 * sra::kRopeMaxHalf || desc->head_dim % 8 != 0)
        return fail(SRA_ERR_UNSUPPORTED, "rotary embedding needs head_dim a multiple of 8 in [8, %d], got %lld",
                    2 * sra::kRopeMaxHalf, (long long)desc->head_dim);
    if (!(base > 1.0) || std::isinf(base)) return fail(SRA_ERR_INVALID_ARG, "base must be finite and > 1");
    if (!x || !y) return fail(SRA_ERR_INVALID_ARG, "null tensor pointer");
    if (!aligned16(x) || !aligned16(y)) return fail(SRA_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
    if ((uintptr_t)pos & 7u) return fail(SRA_ERR_INVALID_ARG, "pos misaligned");
    const double rows = (double)desc->batch * (double)desc->seq;
    if (rows > 2147483647.0) return fail(SRA_ERR_INVALID_ARG, "batch * seq must be < 2^31");
    const bool strided = desc->order == SRA_ORDER_DEVICE && desc->layout == SRA_LAYOUT_STRIPED;
    const double total = rows * (double)desc->heads * (double)desc->head_dim * (desc->dtype == SRA_DTYPE_BF16 ? 2 : 4);
    if (total > 4.0e18) return fail(SRA_ERR_INVALID_ARG, "tensor too large");
    const uintptr_t a0 = (uintptr_t)x, a1 = a0 + (uintptr_t)total, b0 = (uintptr_t)y, b1 = b0 + (uintptr_t)total;
    // In place is allowed when no row moves (every element is read and
    // written by the same thread); any other overlap is rejected.
    if (a0 < b1 && b0 < a1 && !(a0 == b0 && !strided))
        return fail(SRA_ERR_INVALID_ARG, "x and y overlap (in place is allowed only when nothing is permuted)");
    sra::RopeArgs a{};
    a.x = x;
    a.y = y;
    a.pos = pos;
    a.B = desc->batch;
    a.S = desc->seq;
    a.H = desc->heads;
    a.L = desc->seq / desc->n_dev;
    a.D = (int32_t)desc->head_dim;
    a.N = desc->n_dev;
    a.strided = strided;
    for (int c = 0; c < a.D / 2; ++c) a.inv_freq[c] = std::pow(base, -2.0 * c / (double)a.D);
    return hip_status(sra::launch_rope(a, desc->dtype == SRA_DTYPE_BF16, (hipStream_t)stream), "rope_permute launch");
}

}  // extern "C"
