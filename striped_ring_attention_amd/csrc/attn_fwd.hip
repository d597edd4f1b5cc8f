// Ring-round causal attention kernels for gfx950 (CDNA4, wave64).
//
// One launch computes one ring round for a set of query devices: device d's
// queries attend to the K/V block of device s = (d - r) mod N (Striped
// Attention summary page, "Summary" ¶1: K/V blocks circulate around the
// ring). Tiles with no live pair are skipped and only partially live tiles
// are masked ("Summary" ¶1-2: with contiguous chunks a device's work in a
// round is all live or all masked; with stripes every device skips about
// half in every round). The mask is the shifted causal mask k < j + delta
// (see live_delta in sra_internal.h).
//
// The epilogue optionally merges the round's partial result into a running
// accumulator with the log-sum-exp rule (exact combination of partial
// softmax results over disjoint key sets) and, on the driver's last round,
// writes the output in the input dtype.
//
// bf16 kernel (Dh = 128): 4 wavefronts x 32 query rows = 128 rows per
// workgroup, 64 keys per step.
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: K is the A operand (32 keys x
//    16 dims from LDS), Q^T the B operand (held in registers for the whole
//    kernel). In the 32x32 accumulator a lane owns one query (column l%32)
//    and 16 keys, so a query's row max and row sum are in-lane reductions
//    plus one exchange between the two wave halves (v_permlane32_swap).
//  * O^T = V^T P^T on the same instruction: P^T comes straight from the S^T
//    accumulator registers (converted to bf16); V^T is the A operand read
//    from an LDS copy of the V tile stored dimension-major, with the keys of
//    each 16-key group ordered [0-3, 8-11, 4-7, 12-15] so that one 16-byte
//    LDS read gives the 8 keys a lane's P^T registers hold. The O^T
//    accumulator keeps one query per lane, so the softmax rescale is
//    per-lane too.
//  * Softmax runs in the log2 domain with v_exp_f32. The running offset is
//    only raised when a tile's max exceeds it by more than 2^8 (the result
//    does not depend on the offset; it only bounds p <= 256), so the
//    64-register rescale of O is rare.
//  * K and V tiles are double-buffered in LDS (row pitches padded so the
//    16-byte reads of 8 consecutive lanes hit distinct banks); the next
//    tile's global loads are in flight while the current tile computes.
#include "sra_internal.h"

namespace sra {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kFlagMerge = 1;   // merge with (o_acc, lse_acc) instead of overwriting them
constexpr int kFlagFinal = 2;   // write the (merged) output to o_final in the input dtype

constexpr float kLn2 = 0.693147180559945309f;


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

// Log-sum-exp merge weights (natural-log LSEs).
__device__ __forceinline__ void merge_weights(float la, float lb, float& wa, float& wb, float& l) {
    float M = fmaxf(la, lb);
    if (M == -INFINITY) { wa = 0.f; wb = 0.f; l = -INFINITY; return; }
    float ea = __expf(la - M);
    float eb = __expf(lb - M);
    float tot = ea + eb;
    l = M + __logf(tot);
    float inv = 1.0f / tot;
    wa = ea * inv;
    wb = eb * inv;
}

// A value the compiler cannot prove wave-uniform (it went through vector
// registers) but that is: move it to scalar registers.
__device__ __forceinline__ uint64_t uniform_u64(uint64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ int64_t uniform_i64(int64_t x) { return (int64_t)uniform_u64((uint64_t)x); }

struct Decoded {
    int64_t b, h, d, s, qt, delta;
};

__device__ __forceinline__ Decoded decode_block(const RoundArgs& a, int64_t nqt) {
    // Block order: query tiles fastest and heaviest first (the last query
    // tile of a device has the most live keys), then heads, devices, batch.
    int64_t bid = blockIdx.x;
    Decoded o;
    int64_t qi = bid % nqt; bid /= nqt;
    o.h = bid % a.H; bid /= a.H;
    int64_t nd = a.dev_hi - a.dev_lo;
    o.d = a.dev_lo + bid % nd; bid /= nd;
    o.b = bid;
    o.qt = nqt - 1 - qi;
    o.s = (o.d - a.round + a.N) % a.N;
    o.delta = live_delta(a.layout, a.N, a.L, o.d, o.s);
    // The 64-bit divisions above are expanded on the vector ALU; the results
    // are per-workgroup constants, so move them back to scalar registers.
    o.b = uniform_i64(o.b);
    o.h = uniform_i64(o.h);
    o.d = uniform_i64(o.d);
    o.s = uniform_i64(o.s);
    o.qt = uniform_i64(o.qt);
    o.delta = uniform_i64(o.delta);
    return o;
}

// ---------------------------------------------------------------- bf16 ----

constexpr int D = 128;
constexpr int BM = kBf16TileQ;   // 128 query rows per workgroup
constexpr int BN = kBf16TileK;   // 64 keys per step
constexpr int NT = 256;          // 4 wavefronts
constexpr int KP = D + 8;        // K tile row pitch in LDS (elements)
constexpr int VP = BN + 8;       // V^T tile row pitch in LDS (elements)
constexpr float kTau = 8.0f;     // lazy-rescale threshold (log2 units)

static_assert(BM == 128 && BN == 64 && NT == 256, "thread mappings below assume these");

struct __align__(16) SmemBf16 {
    bf16 k[2][BN * KP];
    bf16 vt[2][D * VP];
};

// Low (high) 16-bit halves of a and b packed as {a, b}: one v_perm_b32 each.
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

// Buffer resource over (what is left of) one device's K or V slab of one
// head: loads at offsets past `bytes` read as zero, so tile loads need
// neither clamping nor branches.
constexpr int kBufferFlags = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t slab_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, kBufferFlags);
}

template <bool B>
struct BoolTag {
    static constexpr bool value = B;
};

__global__ void __launch_bounds__(NT, 2) round_fwd_bf16_d128(RoundArgs a, int flags) {
    __shared__ SmemBf16 sm;

    const int64_t nqt = (a.L + BM - 1) / BM;
    const Decoded blk = decode_block(a, nqt);
    const int L = (int)a.L;   // the host bounds L * H * D so that in-slab offsets fit in 32 bits
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, c32 = lane & 31, h2 = lane >> 5;

    const int j0 = (int)blk.qt * BM;
    const int j1 = min(j0 + BM, L);
    const int k_end = (int)live_keys(j1 - 1, blk.delta, L);
    const int n_tiles = (k_end + BN - 1) / BN;

    if (a.live_counts != nullptr && tid == 0 && n_tiles > 0)
        atomicAdd((unsigned long long*)&a.live_counts[(int64_t)a.round * a.N + blk.d], (unsigned long long)n_tiles);

    if (n_tiles == 0 && (flags & kFlagMerge) && !(flags & kFlagFinal)) return;   // merging nothing

    const int rs = (int)(a.H * D);   // elements between consecutive slots
    const bf16* __restrict__ qp0 = (const bf16*)a.q + ((blk.b * a.S + blk.d * a.L) * a.H + blk.h) * D;
    const bf16* __restrict__ kp0 = (const bf16*)a.k + ((blk.b * a.S + blk.s * a.L) * a.H + blk.h) * D;
    const bf16* __restrict__ vp0 = (const bf16*)a.v + ((blk.b * a.S + blk.s * a.L) * a.H + blk.h) * D;

    // This wave's rows and live-key bounds (live keys of a row form a prefix).
    const int jw0 = j0 + w * 32;
    const int j = jw0 + c32;
    const bool row_ok = j < L;
    const int kw_end = jw0 < L ? (int)live_keys(min(jw0 + 31, L - 1), blk.delta, L) : 0;
    const int kw_full = jw0 < L ? (int)live_keys(jw0, blk.delta, L) : 0;
    const int c_row = row_ok ? (int)live_keys(j, blk.delta, L) : 0;

    // Q^T operand: lane holds query c32, dims kk*16 + 8*h2 .. +7. Rows past
    // the end read a valid row; they are fully masked and never written.
    bf16x8 qreg[8];
    {
        const bf16x8* qp = (const bf16x8*)(qp0 + min(j, L - 1) * rs) + h2;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) qreg[kk] = qp[2 * kk];
    }

    f32x16 oacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};
    float m_run = -INFINITY;   // running offset (log2 domain), equal in both halves
    float l_part = 0.f;        // this half's share of the row sum
    const float sl = a.scale_log2;

    // Global -> register staging of one K/V tile through buffer loads. Each
    // tile gets its own buffer resource (base advanced to the tile's first
    // row, size cut to what is left of the slab, both scalar), so the
    // per-lane offsets are loop-invariant and rows past the slab end read
    // as zero (their scores are masked and their V rows get weight 0).
    //  K: thread -> (key row kr, 32-dim chunk kc), four 16-byte loads.
    //  V: thread -> (key quad kq, 8-dim chunk dc), one 16-byte load per key
    //     of the quad; each group of 16 lanes covers all 16 quads of one dim
    //     chunk, so the transposed LDS writes of a group fill one V^T row.
    const int kr = tid >> 2, kc = tid & 3;
    const int kq = tid & 15, dc = tid >> 4;
    const int row_bytes = rs * 2;
    const int slab_bytes = __builtin_amdgcn_readfirstlane((L - 1) * row_bytes + D * 2);
    const int k_voff = kr * row_bytes + kc * 64;
    const int v_voff = 4 * kq * row_bytes + dc * 16;
    const uint64_t kbase = uniform_u64((uint64_t)kp0), vbase = uniform_u64((uint64_t)vp0);
    u32x4 kreg[4], vreg[4];

    auto load_tile = [&](int it) {
        const int tile_off = it * BN * row_bytes;
        const int left = slab_bytes - tile_off > 0 ? slab_bytes - tile_off : 0;
        const __amdgpu_buffer_rsrc_t krs = slab_rsrc((const void*)(kbase + tile_off), left);
        const __amdgpu_buffer_rsrc_t vrs = slab_rsrc((const void*)(vbase + tile_off), left);
#pragma unroll
        for (int i = 0; i < 4; ++i) kreg[i] = __builtin_amdgcn_raw_buffer_load_b128(krs, k_voff + 16 * i, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) vreg[r] = __builtin_amdgcn_raw_buffer_load_b128(vrs, v_voff + r * row_bytes, 0, 0);
    };
    // V^T column of key quad kq: within each 16-key group the quads are
    // stored in the order [0, 2, 1, 3] (keys [0-3, 8-11, 4-7, 12-15]).
    const int vt_col = 16 * (kq >> 2) + 4 * ((kq & 1) * 2 + ((kq >> 1) & 1));
    auto store_tile = [&](int buf) {
        bf16* kd = &sm.k[buf][kr * KP + kc * 32];
#pragma unroll
        for (int i = 0; i < 4; ++i) *(u32x4*)(kd + 8 * i) = kreg[i];
        // vreg[r][p] holds dims (2p, 2p+1) of key 4*kq + r.
        bf16* vd = &sm.vt[buf][(8 * dc) * VP + vt_col];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            uint2 lo = {pack_lo(vreg[0][p], vreg[1][p]), pack_lo(vreg[2][p], vreg[3][p])};
            uint2 hi = {pack_hi(vreg[0][p], vreg[1][p]), pack_hi(vreg[2][p], vreg[3][p])};
            *(uint2*)(vd + (2 * p) * VP) = lo;
            *(uint2*)(vd + (2 * p + 1) * VP) = hi;
        }
    };

    // One step over the tile in LDS buffer `cur` for this wave's 32 rows.
    // kMasked: the tile is not fully live for every row of the wave.
    auto step = [&](auto masked_tag, int cur, int k0) {
        constexpr bool kMasked = decltype(masked_tag)::value;
        const bf16* ks = sm.k[cur] + c32 * KP + 8 * h2;
        f32x16 s0, s1;
        {
            bf16x8 kf[8];
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) kf[kk] = *(const bf16x8*)(ks + kk * 16);
            s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[0], qreg[0], f32x16{}, 0, 0, 0);
#pragma unroll
            for (int kk = 1; kk < 8; ++kk) s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qreg[kk], s0, 0, 0, 0);
        }
        {
            bf16x8 kf[8];
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) kf[kk] = *(const bf16x8*)(ks + 32 * KP + kk * 16);
            s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[0], qreg[0], f32x16{}, 0, 0, 0);
#pragma unroll
            for (int kk = 1; kk < 8; ++kk) s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk], qreg[kk], s1, 0, 0, 0);
        }
        if constexpr (kMasked) {
            // key offset in the tile of accumulator element i of block kb is
            // kb*32 + 8*(i/4) + 4*h2 + i%4; live iff key < c_row.
            const int lim = c_row - k0 - 4 * h2;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int off = 8 * (i >> 2) + (i & 3);
                if (off >= lim) s0[i] = -INFINITY;
                if (off + 32 >= lim) s1[i] = -INFINITY;
            }
        }
        // Row max over this tile (raw scores; scale > 0 keeps the order).
        float mx = fmaxf(fmaxf(s0[0], s1[0]), s0[1]);
#pragma unroll
        for (int i = 1; i < 15; i += 2) mx = fmaxf(fmaxf(mx, s1[i]), fmaxf(s0[i + 1], s1[i + 1]));
        mx = fmaxf(fmaxf(mx, s1[15]), s0[15]);
        mx = halves_max(mx);
        const float m_tile = mx * sl;
        const bool need = m_tile > m_run + kTau;
        if (__builtin_amdgcn_ballot_w64(need) != 0) {
            const float m_new = need ? fmaxf(m_run, m_tile) : m_run;
            const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
#pragma unroll
            for (int db = 0; db < 4; ++db) oacc[db] *= alpha;
            l_part *= alpha;
            m_run = m_new;
        }
        const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
        // p = 2^(s*scale*log2e - m), summed in fp32 and rounded to bf16 for P^T.
        bf16x8 pop[2][2];
        float lsum0 = 0.f, lsum1 = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[i], sl, -m_use));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[i], sl, -m_use));
            lsum0 += p0;
            lsum1 += p1;
            pop[0][i >> 3][i & 7] = (bf16)p0;
            pop[1][i >> 3][i & 7] = (bf16)p1;
        }
        l_part += lsum0 + lsum1;
        const bf16* vts = sm.vt[cur] + c32 * VP + 8 * h2;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int kk2 = 0; kk2 < 2; ++kk2) {
                bf16x8 vf[4];
#pragma unroll
                for (int db = 0; db < 4; ++db) vf[db] = *(const bf16x8*)(vts + db * 32 * VP + kb * 32 + kk2 * 16);
#pragma unroll
                for (int db = 0; db < 4; ++db)
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db], pop[kb][kk2], oacc[db], 0, 0, 0);
            }
        }
    };

    if (n_tiles > 0) {
        load_tile(0);
        store_tile(0);
    }
    // Every global load issued so far (Q and tile 0) has landed before the
    // loop, so waits inside the loop only ever cover the prefetch.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int it = 0; it < n_tiles; ++it) {
        const int cur = it & 1;
        // Prefetch the next tile (past the last tile the loads read zeros
        // into the idle buffer; no branch needed).
        load_tile(it + 1);
        const int k0 = it * BN;
        if (k0 < kw_end) {
            if (k0 + BN <= kw_full) step(BoolTag<false>{}, cur, k0);
            else step(BoolTag<true>{}, cur, k0);
        }
        store_tile(cur ^ 1);
        __syncthreads();
    }

    // Finish the row: l = both halves' sums; O = O / l; lse in natural log.
    const float l_tot = halves_sum(l_part);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    const float lse_b = l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
    if (!row_ok) return;

    const int64_t row = (blk.b * a.S + blk.d * a.L + j) * a.H + blk.h;   // (b, slot, h) row index
    float wa = 0.f, wb = 1.f, l_out = lse_b;
    if (flags & kFlagMerge) {
        const float la = a.lse_acc[row];
        merge_weights(la, lse_b, wa, wb, l_out);
    }
    wb *= inv;   // fold the normalisation into the partial's weight
    float* oa = a.o_acc + row * D;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int dcol = db * 32 + 8 * g + 4 * h2;
            f32x4 ob = {oacc[db][4 * g], oacc[db][4 * g + 1], oacc[db][4 * g + 2], oacc[db][4 * g + 3]};
            f32x4 r = f32x4{0.f, 0.f, 0.f, 0.f};
            if (wb != 0.f) r = wb * ob;
            if ((flags & kFlagMerge) && wa != 0.f) r += wa * *(const f32x4*)(oa + dcol);
            if (flags & kFlagFinal) {
                bf16x4 rb = {(bf16)r[0], (bf16)r[1], (bf16)r[2], (bf16)r[3]};
                *(bf16x4*)((bf16*)a.o_final + row * D + dcol) = rb;
            } else {
                *(f32x4*)(oa + dcol) = r;
            }
        }
    }
    if (h2 == 0) a.lse_acc[row] = l_out;
}

// ---------------------------------------------------------------- fp32 ----
// Plain fp32 kernel: one wavefront of 64 query rows (one row per lane),
// keys staged through LDS 16 at a time, exact online softmax in fp32 with
// accurate expf/logf. Used for fp32 inputs (small shapes).

template <int DH>
__global__ void __launch_bounds__(64) round_fwd_f32(RoundArgs a, int flags) {
    constexpr int BMf = kF32TileQ, BNf = kF32TileK;
    __shared__ float ks[BNf][DH];
    __shared__ float vs[BNf][DH];
    const int64_t L = a.L, S = a.S, H = a.H;
    const int64_t nqt = (L + BMf - 1) / BMf;
    const Decoded blk = decode_block(a, nqt);
    const int lane = threadIdx.x;
    const int64_t j0 = blk.qt * BMf;
    const int64_t j1 = (j0 + BMf < L) ? j0 + BMf : L;
    const int64_t k_end = live_keys(j1 - 1, blk.delta, L);
    const int n_chunks = (int)((k_end + BNf - 1) / BNf);
    if (a.live_counts != nullptr && lane == 0 && n_chunks > 0)
        atomicAdd((unsigned long long*)&a.live_counts[(int64_t)a.round * a.N + blk.d], (unsigned long long)n_chunks);
    if (n_chunks == 0 && (flags & kFlagMerge) && !(flags & kFlagFinal)) return;

    const float* __restrict__ q = (const float*)a.q;
    const float* __restrict__ kg = (const float*)a.k;
    const float* __restrict__ vg = (const float*)a.v;
    const int64_t row_stride = H * DH;
    const int64_t kv_base = ((blk.b * S + blk.s * L) * H + blk.h) * DH;
    const int64_t j = j0 + lane;
    const bool row_ok = j < L;
    const int64_t c_row = row_ok ? live_keys(j, blk.delta, L) : 0;
    const int64_t row = (blk.b * S + blk.d * L + (row_ok ? j : 0)) * H + blk.h;

    float qr[DH], o[DH];
#pragma unroll
    for (int c = 0; c < DH; ++c) {
        qr[c] = row_ok ? q[row * DH + c] : 0.f;
        o[c] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    for (int ch = 0; ch < n_chunks; ++ch) {
        __syncthreads();
        for (int e = lane; e < BNf * DH; e += 64) {
            const int kk = e / DH, c = e % DH;
            const int64_t key = (int64_t)ch * BNf + kk;
            ks[kk][c] = key < L ? kg[kv_base + key * row_stride + c] : 0.f;
            vs[kk][c] = key < L ? vg[kv_base + key * row_stride + c] : 0.f;
        }
        __syncthreads();
        for (int kk = 0; kk < BNf; ++kk) {
            const int64_t key = (int64_t)ch * BNf + kk;
            if (key >= c_row) break;   // live keys of a row are a prefix
            float s = 0.f;
#pragma unroll
            for (int c = 0; c < DH; ++c) s = fmaf(qr[c], ks[kk][c], s);
            s *= a.scale;
            const float m_new = fmaxf(m, s);
            const float alpha = (m == -INFINITY) ? 0.f : expf(m - m_new);
            const float p = expf(s - m_new);
            l = l * alpha + p;
#pragma unroll
            for (int c = 0; c < DH; ++c) o[c] = o[c] * alpha + p * vs[kk][c];
            m = m_new;
        }
    }
    if (!row_ok) return;
    const float lse_b = l > 0.f ? m + logf(l) : -INFINITY;
    const float inv = l > 0.f ? 1.0f / l : 0.f;
    float wa = 0.f, wb = 1.f, l_out = lse_b;
    if (flags & kFlagMerge) {
        const float la = a.lse_acc[row];
        const float M = fmaxf(la, lse_b);
        if (M == -INFINITY) { wa = 0.f; wb = 0.f; l_out = -INFINITY; }
        else {
            const float ea = expf(la - M), eb = expf(lse_b - M);
            const float tot = ea + eb;
            l_out = M + logf(tot);
            wa = ea / tot;
            wb = eb / tot;
        }
    }
    wb *= inv;
    float* dst = (flags & kFlagFinal) ? (float*)a.o_final : a.o_acc;
#pragma unroll
    for (int c = 0; c < DH; ++c) {
        float r = 0.f;
        if (wb != 0.f) r = wb * o[c];
        if ((flags & kFlagMerge) && wa != 0.f) r += wa * a.o_acc[row * DH + c];
        dst[row * DH + c] = r;
    }
    a.lse_acc[row] = l_out;
}

int flags_of(const RoundArgs& a) {
    return a.mode == 0 ? 0 : (a.mode == 1 ? kFlagMerge : (a.mode == 2 ? kFlagMerge | kFlagFinal : kFlagFinal));
}

}  // namespace

hipError_t launch_round_bf16_d128(const RoundArgs& a, hipStream_t stream) {
    const int64_t nqt = (a.L + BM - 1) / BM;
    const int64_t blocks = nqt * a.H * (a.dev_hi - a.dev_lo) * a.B;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(round_fwd_bf16_d128, dim3((unsigned)blocks), dim3(NT), 0, stream, a, flags_of(a));
    return hipGetLastError();
}

hipError_t launch_round_f32(const RoundArgs& a, int64_t head_dim, hipStream_t stream) {
    const int64_t nqt = (a.L + kF32TileQ - 1) / kF32TileQ;
    const int64_t blocks = nqt * a.H * (a.dev_hi - a.dev_lo) * a.B;
    if (blocks == 0) return hipSuccess;
    if (head_dim == 64)
        hipLaunchKernelGGL(round_fwd_f32<64>, dim3((unsigned)blocks), dim3(64), 0, stream, a, flags_of(a));
    else
        hipLaunchKernelGGL(round_fwd_f32<128>, dim3((unsigned)blocks), dim3(64), 0, stream, a, flags_of(a));
    return hipGetLastError();
}

}  // namespace sra
