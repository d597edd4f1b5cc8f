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


__device__ __forceinline__ float swap_halves(float x) {
    // Exchange a value between lane l and lane l ^ 32.
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]);
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

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }

__global__ void __launch_bounds__(NT, 2) round_fwd_bf16_d128(RoundArgs a, int flags) {
    __shared__ SmemBf16 sm;

    const int64_t L = a.L, S = a.S, H = a.H;
    const int64_t nqt = (L + BM - 1) / BM;
    const Decoded blk = decode_block(a, nqt);
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, c32 = lane & 31, h2 = lane >> 5;

    const int64_t j0 = blk.qt * BM;
    const int64_t j1 = (j0 + BM < L) ? j0 + BM : L;
    const int64_t k_end = live_keys(j1 - 1, blk.delta, L);
    const int n_tiles = (int)((k_end + BN - 1) / BN);

    if (a.live_counts != nullptr && tid == 0 && n_tiles > 0)
        atomicAdd((unsigned long long*)&a.live_counts[(int64_t)a.round * a.N + blk.d], (unsigned long long)n_tiles);

    if (n_tiles == 0 && (flags & kFlagMerge) && !(flags & kFlagFinal)) return;   // merging nothing

    const bf16* __restrict__ q = (const bf16*)a.q;
    const bf16* __restrict__ kg = (const bf16*)a.k;
    const bf16* __restrict__ vg = (const bf16*)a.v;
    const int64_t row_stride = H * D;   // elements between consecutive slots
    const int64_t q_base = ((blk.b * S + blk.d * L) * H + blk.h) * D;
    const int64_t kv_base = ((blk.b * S + blk.s * L) * H + blk.h) * D;

    // This wave's rows and live-key bounds.
    const int64_t jw0 = j0 + w * 32;
    const int64_t j = jw0 + c32;
    const bool row_ok = j < L;
    const int64_t jw_last = (jw0 + 31 < L) ? jw0 + 31 : L - 1;
    const int64_t kw_end = (jw0 < L) ? live_keys(jw_last, blk.delta, L) : 0;
    const int64_t kw_full = (jw0 < L) ? live_keys(jw0, blk.delta, L) : 0;
    const int64_t c_row = row_ok ? live_keys(j, blk.delta, L) : 0;

    // Q^T operand: lane holds query c32, dims kk*16 + 8*h2 .. +7.
    bf16x8 qreg[8];
    if (row_ok) {
        const bf16x8* qp = (const bf16x8*)(q + q_base + j * row_stride);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) qreg[kk] = qp[2 * kk + h2];
    } else {
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) qreg[kk] = bf16x8{};
    }

    f32x16 oacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};
    float m_run = -INFINITY;   // running offset (log2 domain), same in both halves
    float l_part = 0.f;        // this half's share of the row sum
    const float sl = a.scale_log2;

    // Global -> register staging of one K/V tile.
    const int kr = tid >> 2, kc = tid & 3;        // K: key row, 32-dim chunk
    const int vdp = tid & 63, vkg = tid >> 6;      // V: dim pair, 16-key group
    bf16x8 kreg[4];
    uint32_t vreg[16];

    auto load_tile = [&](int it) {
        const int64_t k0 = (int64_t)it * BN;
        const int64_t key = k0 + kr;
        if (key < L) {
            const bf16x8* kp = (const bf16x8*)(kg + kv_base + key * row_stride + kc * 32);
#pragma unroll
            for (int i = 0; i < 4; ++i) kreg[i] = kp[i];
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) kreg[i] = bf16x8{};
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int64_t vkey = k0 + vkg * 16 + i;
            vreg[i] = (vkey < L) ? *(const uint32_t*)(vg + kv_base + vkey * row_stride + 2 * vdp) : 0u;
        }
    };
    auto store_tile = [&](int buf) {
        bf16* kd = &sm.k[buf][kr * KP + kc * 32];
#pragma unroll
        for (int i = 0; i < 4; ++i) *(bf16x8*)(kd + 8 * i) = kreg[i];
        // V^T rows 2*vdp (low halves) and 2*vdp+1 (high halves); within the
        // 16-key group the order is [0-3, 8-11 | 4-7, 12-15].
        u32x4 lo_a = {pack_lo(vreg[0], vreg[1]), pack_lo(vreg[2], vreg[3]), pack_lo(vreg[8], vreg[9]), pack_lo(vreg[10], vreg[11])};
        u32x4 lo_b = {pack_lo(vreg[4], vreg[5]), pack_lo(vreg[6], vreg[7]), pack_lo(vreg[12], vreg[13]), pack_lo(vreg[14], vreg[15])};
        u32x4 hi_a = {pack_hi(vreg[0], vreg[1]), pack_hi(vreg[2], vreg[3]), pack_hi(vreg[8], vreg[9]), pack_hi(vreg[10], vreg[11])};
        u32x4 hi_b = {pack_hi(vreg[4], vreg[5]), pack_hi(vreg[6], vreg[7]), pack_hi(vreg[12], vreg[13]), pack_hi(vreg[14], vreg[15])};
        bf16* v0 = &sm.vt[buf][(2 * vdp) * VP + vkg * 16];
        bf16* v1 = v0 + VP;
        *(u32x4*)(v0) = lo_a;
        *(u32x4*)(v0 + 8) = lo_b;
        *(u32x4*)(v1) = hi_a;
        *(u32x4*)(v1 + 8) = hi_b;
    };

    if (n_tiles > 0) {
        load_tile(0);
        store_tile(0);
        __syncthreads();
    }

    for (int it = 0; it < n_tiles; ++it) {
        const int cur = it & 1;
        const bool has_next = it + 1 < n_tiles;
        if (has_next) load_tile(it + 1);

        const int64_t k0 = (int64_t)it * BN;
        // Live 32-key blocks of this tile for this wave (0, 1 or 2); wave-uniform.
        const int64_t rem = kw_end - k0;
        const int n_kb = rem <= 0 ? 0 : (rem > 32 ? 2 : 1);
        if (n_kb > 0) {
            const bf16* ks = sm.k[cur];
            const bf16* vts = sm.vt[cur];
            f32x16 sacc[2];
            sacc[0] = f32x16{};
            sacc[1] = f32x16{};
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (kb < n_kb) {
#pragma unroll
                    for (int kk = 0; kk < 8; ++kk) {
                        bf16x8 kop = *(const bf16x8*)(ks + (kb * 32 + c32) * KP + kk * 16 + 8 * h2);
                        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qreg[kk], sacc[kb], 0, 0, 0);
                    }
                }
            }
            // Mask: only when the tile is not fully live for every row of the wave.
            if (k0 + BN > kw_full) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    if (kb < n_kb) {
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int64_t key = k0 + kb * 32 + 8 * (i >> 2) + 4 * h2 + (i & 3);
                            if (key >= c_row) sacc[kb][i] = -INFINITY;
                        }
                    }
                }
            }
            // Row max over this tile (raw scores; scale > 0 keeps the order).
            float mx = sacc[0][0];
#pragma unroll
            for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sacc[0][i]);
            if (n_kb > 1) {
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[1][i]);
            }
            mx = fmaxf(mx, swap_halves(mx));
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
            // p = 2^(s*scale*log2e - m); P^T operands for the PV product.
            bf16x8 pop[2][2];
            float lsum = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (kb < n_kb) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][i], sl, -m_use));
                        lsum += p;
                        pop[kb][i >> 3][i & 7] = (bf16)p;
                    }
                }
            }
            l_part += lsum;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (kb < n_kb) {
#pragma unroll
                    for (int kk2 = 0; kk2 < 2; ++kk2) {
#pragma unroll
                        for (int db = 0; db < 4; ++db) {
                            bf16x8 vop = *(const bf16x8*)(vts + (db * 32 + c32) * VP + kb * 32 + kk2 * 16 + 8 * h2);
                            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop[kb][kk2], oacc[db], 0, 0, 0);
                        }
                    }
                }
            }
        }

        if (has_next) store_tile(cur ^ 1);
        __syncthreads();
    }

    // Finish the row: l = both halves' sums; O = O / l; lse in natural log.
    const float l_tot = l_part + swap_halves(l_part);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    const float lse_b = l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
    if (!row_ok) return;

    const int64_t row = (blk.b * S + blk.d * L + j) * H + blk.h;   // (b, slot, h) row index
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
