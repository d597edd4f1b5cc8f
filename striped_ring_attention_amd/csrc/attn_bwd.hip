// Backward pass of striped ring attention for gfx950: dQ, dK, dV (bf16,
// head dim 128).
//
// Ring attention computes exact causal attention (abstract of the Striped
// Attention paper, pith.science/paper/2311.09431), so its gradient is the
// gradient of exact attention, taken with the saved final log-sum-exp:
//   P_ik  = exp(s_ik - lse_i) on live pairs,  Delta_i = dO_i . O_i,
//   dV_k  = sum_i P_ik dO_i,  dP_ik = dO_i . V_k,
//   dS_ik = P_ik (dP_ik - Delta_i),
//   dQ_i  = scale sum_k dS_ik K_k,  dK_k = scale sum_i dS_ik Q_i.
// Decomposed over the ring (Striped Attention summary page, "Summary" ¶1:
// K/V blocks circulate): in round r the K/V block of device s meets the
// queries of device (s + r) mod N; dK/dV of a block sum over rounds (they
// travel with the block and return to its owner on a real ring) and dQ of a
// device sums over the blocks it met. Both kernels below walk every round in
// one launch, with the same shifted causal mask as the forward, skipping
// empty tiles and masking only partial ones.
//
//  * bwd_delta:  Delta = rowsum(dO * O) in fp32.
//  * bwd_dq:     a workgroup owns 128 query rows (4 waves x 32) and walks
//                the (round, 64-key tile) pairs in ring order. Per 32-key
//                block: S^T = K Q^T and dP^T = V dO^T on MFMA (Q^T and dO^T
//                held in registers, K and V row-major in LDS), then
//                dS^T = P^T (dP^T - Delta) scale, and dQ^T += K^T dS^T with
//                K^T read from a dimension-major LDS copy whose 16-key groups
//                are ordered [0-3, 8-11, 4-7, 12-15] (the order in which a
//                lane's accumulator registers hold keys).
//  * bwd_dkdv:   a workgroup owns 128 keys (4 waves x 32) of one source
//                device and walks the 32-row query tiles of every device that
//                meets the block, round by round. S = Q K^T and dP = dO V^T
//                (K and V held in registers, Q and dO row-major in LDS), then
//                dV^T += dO^T P and dK^T += Q^T dS, with Q^T and dO^T read
//                from dimension-major LDS copies in the same permuted order.
// No atomics: each gradient accumulates in the registers of the workgroup
// that owns its rows, so results are deterministic. S and dP are computed in
// both kernels (seven tile products per live tile instead of five).
#include "kernel_common.h"

namespace sra {
namespace {

using namespace kc;

constexpr int D = 128;
constexpr int KP = D + 8;     // row-major tile pitch in LDS (elements)

// ------------------------------------------------------------------ Delta --

// Row statistics of the backward, one float pair per row in a head-major
// layout [B, H, S, 2]: (LSE * log2 e, Delta), Delta = sum_c dO[c] * O[c] in
// fp32. The rows of one head are contiguous, so the 32 rows of a query tile
// are 256 contiguous bytes. Sixteen lanes per (b, slot, h) row, each taking
// 8 consecutive elements (16-byte loads: a wave reads four whole 256-byte
// rows of O and of dO), then a 16-lane butterfly sum.
__global__ void __launch_bounds__(256) bwd_delta(const bf16* __restrict__ o, const bf16* __restrict__ dout,
                                                 const float* __restrict__ lse, float* __restrict__ stats,
                                                 uint32_t rows, uint32_t S, uint32_t H) {
    const uint32_t stride = (gridDim.x * blockDim.x) >> 4;
    const int c = threadIdx.x & 15;
    for (uint32_t r = (blockIdx.x * blockDim.x + threadIdx.x) >> 4; r < rows; r += stride) {
        const bf16x8 x = *(const bf16x8*)(o + (uint64_t)r * D + 8 * c);
        const bf16x8 y = *(const bf16x8*)(dout + (uint64_t)r * D + 8 * c);
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s = __builtin_fmaf((float)x[e], (float)y[e], s);
#pragma unroll
        for (int m = 8; m >= 1; m >>= 1) s += __shfl_xor(s, m, 16);
        if (c == 0) {
            const uint32_t h = r % H, bs = r / H, b = bs / S, slot = bs % S;
            const uint64_t i = ((uint64_t)b * H + h) * S + slot;
            *(float2*)(stats + 2 * i) = float2{lse[r] * kLog2e, s};
        }
    }
}

// -------------------------------------------------------------------- dQ --

constexpr int QBM = 128;          // query rows per workgroup
constexpr int QBN = 64;           // keys per tile
constexpr int QVP = QBN + 8;      // K^T tile pitch (elements)

struct __align__(16) SmemDq {
    bf16 kr[QBN * KP];    // K tile, row-major
    bf16 kt[D * QVP];     // K tile, dimension-major, permuted key order
    bf16 vr[QBN * KP];    // V tile, row-major
};

__global__ void __launch_bounds__(256, 2) bwd_dq(BwdArgs a) {
    __shared__ SmemDq sm;
    const int L = (int)a.L;
    const int64_t nqt = (a.L + QBM - 1) / QBM;
    const WorkItem wi = decode_work(nqt, a.B, a.H, a.N, 0);
    const int d = (int)wi.d;
    const int qt = (int)uniform_i64(nqt - 1 - wi.heavy_rank);
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, c32 = lane & 31, h2 = lane >> 5;
    const int j0 = qt * QBM;
    const int j1 = min(j0 + QBM, L);

    const int rs = (int)(a.H * D);
    const int row_bytes = rs * 2;
    // Device t's j-th token sits at slot mem_slot(t, j); consecutive tokens of
    // a device are rstride bytes apart.
    const bool strided = a.strided != 0;
    const int rstride = (int)(strided ? a.N : 1) * row_bytes;
    const uint64_t k_head = uniform_u64((uint64_t)((const bf16*)a.k + (wi.b * a.S * a.H + wi.h) * D));
    const uint64_t v_head = uniform_u64((uint64_t)((const bf16*)a.v + (wi.b * a.S * a.H + wi.h) * D));
    auto slot_bytes = [&](int t) { return (uint64_t)mem_slot(strided, a.N, a.L, t, 0) * (uint64_t)row_bytes; };
    const int64_t span_bytes = (int64_t)(L - 1) * rstride + D * 2;

    // Rounds: in round r device d holds the block of device (d - r) mod N.
    auto source = [&](int r) { return (d - r + a.N) % a.N; };
    auto delta_of = [&](int r) { return clamp_delta(live_delta(a.layout, a.N, L, d, source(r)), L); };
    auto tiles_of = [&](int r) { return (live32(j1 - 1, delta_of(r), L) + QBN - 1) / QBN; };
    int n_tiles = 0;
    for (int r = 0; r < a.N; ++r) n_tiles += tiles_of(r);

    // This wave's rows.
    const int jw0 = j0 + 32 * w;
    const int j = jw0 + c32;
    const bool row_ok = j < L;
    const bool wave_live = jw0 < L;
    const int jw_last = min(jw0 + 31, L - 1);
    const int64_t row = (wi.b * a.S + mem_slot(strided, a.N, a.L, d, min(j, L - 1))) * a.H + wi.h;

    // Q^T and dO^T operands (lane: query c32, dims kk*16 + 8*h2 .. +7).
    bf16x8 qreg[8], doreg[8];
    {
        const bf16x8* qp = (const bf16x8*)((const bf16*)a.q + row * D) + h2;
        const bf16x8* dp = (const bf16x8*)((const bf16*)a.dout + row * D) + h2;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            qreg[kk] = qp[2 * kk];
            doreg[kk] = dp[2 * kk];
        }
    }
    const int64_t srow = (wi.b * a.H + wi.h) * a.S + mem_slot(strided, a.N, a.L, d, min(j, L - 1));
    const float2 st2 = *(const float2*)(a.stats + 2 * srow);
    const float lse_l2 = row_ok ? st2.x : 0.f;
    const float dlt = row_ok ? st2.y : 0.f;
    __builtin_amdgcn_s_waitcnt(0);   // row operands land before any tile load is issued

    f32x16 dqacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) dqacc[db] = f32x16{};
    const float sl = a.scale_log2;
    const float scale = a.scale;

    // Tile staging: K as (key quad kq, 8-dim chunk dc) -- four keys x 16 bytes
    // per thread, written row-major and transposed; V as (key row kr, 32-dim
    // chunk kc) -- four 16-byte loads per thread, written row-major.
    const int kq = tid & 15, dc = tid >> 4;
    const int kr = tid >> 2, kcc = tid & 3;
    const int k_voff = 4 * kq * rstride + dc * 16;
    const int v_voff = kr * rstride + kcc * 64;
    const int kt_col = 16 * (kq >> 2) + 4 * ((kq & 1) * 2 + ((kq >> 1) & 1));
    u32x4 kst[4], vst[4];

    auto load_tile = [&](int s, int kt, bool valid) {
        const int64_t tile_off = (int64_t)kt * QBN * rstride;
        const int64_t left64 = span_bytes - tile_off;
        const int left = (valid && left64 > 0) ? (int)min(left64, (int64_t)QBN * rstride) : 0;
        const uint64_t so = slot_bytes(s) + (uint64_t)tile_off;
        const __amdgpu_buffer_rsrc_t krs = slab_rsrc((const void*)(k_head + so), left);
        const __amdgpu_buffer_rsrc_t vrs = slab_rsrc((const void*)(v_head + so), left);
#pragma unroll
        for (int i = 0; i < 4; ++i) kst[i] = __builtin_amdgcn_raw_buffer_load_b128(krs, k_voff + i * rstride, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) vst[i] = __builtin_amdgcn_raw_buffer_load_b128(vrs, v_voff + 16 * i, 0, 0);
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int i = 0; i < 4; ++i) *(u32x4*)&sm.kr[(4 * kq + i) * KP + 8 * dc] = kst[i];
        bf16* ktd = &sm.kt[(8 * dc) * QVP + kt_col];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            uint2 lo = {pack_lo(kst[0][p], kst[1][p]), pack_lo(kst[2][p], kst[3][p])};
            uint2 hi = {pack_hi(kst[0][p], kst[1][p]), pack_hi(kst[2][p], kst[3][p])};
            *(uint2*)(ktd + (2 * p) * QVP) = lo;
            *(uint2*)(ktd + (2 * p + 1) * QVP) = hi;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) *(u32x4*)&sm.vr[kr * KP + kcc * 32 + 8 * i] = vst[i];
    };

    // Tile cursor (round, key tile), in ring order.
    int cr = 0, ck = 0, cnt = tiles_of(0);
    auto settle = [&](int& r, int& k, int& nt) {
        while (k >= nt && r + 1 < a.N) {
            ++r;
            k = 0;
            nt = tiles_of(r);
        }
    };
    settle(cr, ck, cnt);
    int lr = cr, lk = ck, lnt = cnt;   // loader cursor

    if (n_tiles > 0) load_tile(source(lr), lk, true);
    for (int t = 0; t < n_tiles; ++t) {
        __syncthreads();   // every wave is done with the previous tile
        store_tile();
        __syncthreads();
        ++lk;
        settle(lr, lk, lnt);
        load_tile(source(lr), lk, t + 1 < n_tiles);   // next tile, in flight during compute

        const int delta = delta_of(cr);
        const int k0 = ck * QBN;
        const int kw_end = wave_live ? live32(jw_last, delta, L) : 0;
        const bool masked = k0 + QBN > live32(jw0, delta, L);
        const int c_row = row_ok ? live32(j, delta, L) : 0;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (k0 + 32 * kb >= kw_end) continue;   // no live key for this wave
            const bf16* ks = &sm.kr[(32 * kb + c32) * KP + 8 * h2];
            const bf16* vs = &sm.vr[(32 * kb + c32) * KP + 8 * h2];
            f32x16 s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)ks, qreg[0], f32x16{}, 0, 0, 0);
            f32x16 dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)vs, doreg[0], f32x16{}, 0, 0, 0);
#pragma unroll
            for (int kk = 1; kk < 8; ++kk) {
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(ks + 16 * kk), qreg[kk], s, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(vs + 16 * kk), doreg[kk], dp, 0, 0, 0);
            }
            if (masked) {
                const int lim = c_row - (k0 + 32 * kb) - 4 * h2;
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (8 * (i >> 2) + (i & 3) >= lim) s[i] = -INFINITY;
            }
            bf16x8 dsb[2];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], sl, -lse_l2));
                dsb[i >> 3][i & 7] = (bf16)(p * (dp[i] - dlt) * scale);
            }
#pragma unroll
            for (int kk2 = 0; kk2 < 2; ++kk2) {
                const bf16* kts = &sm.kt[c32 * QVP + 32 * kb + 16 * kk2 + 8 * h2];
#pragma unroll
                for (int db = 0; db < 4; ++db)
                    dqacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(kts + db * 32 * QVP), dsb[kk2],
                                                                       dqacc[db], 0, 0, 0);
            }
        }
        ++ck;
        settle(cr, ck, cnt);
    }

    if (!row_ok) return;
    bf16* dqp = (bf16*)a.dq + row * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const bf16x4 v4 = {(bf16)dqacc[db][4 * g], (bf16)dqacc[db][4 * g + 1], (bf16)dqacc[db][4 * g + 2],
                               (bf16)dqacc[db][4 * g + 3]};
            *(bf16x4*)(dqp + db * 32 + 8 * g + 4 * h2) = v4;
        }
}

// ----------------------------------------------------------------- dK/dV --

constexpr int KBM = 128;          // keys per workgroup (4 waves x 32)
constexpr int KBQ = 32;           // query rows per tile
constexpr int DK_NS = 4;          // LDS stages
constexpr int DK_AHEAD = 3;       // tiles in flight ahead of the one computed
constexpr int kWaitVm10 = 0x0F7A; // vmcnt(10): the two newest tiles (5 loads each per wave) may be in flight

// Q and dO tiles are stored row-major with 256-byte rows and no padding
// (they are loaded straight into LDS); 16-byte chunk c of row r sits in slot
// c ^ swz(r), swz(r) = 4 (r % 4) + (r / 4) % 4. This one swizzle keeps both
// read patterns conflict-free: 16 lanes reading one chunk of 16 consecutive
// rows (the MFMA row operand) hit 16 different slots, and a transposing read
// (4 consecutive rows x 4 consecutive chunks per 32 lanes) hits 16 as well.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

struct __align__(16) SmemDkdv {
    bf16 q[DK_NS][KBQ * D];       // Q tiles
    bf16 dout[DK_NS][KBQ * D];    // dO tiles
    float st[DK_NS][4][64];       // row statistics (LSE log2 e, Delta) of the tile's 32 rows; one copy per wave
};

// A workgroup owns 128 keys (4 waves x 32) of one source device and walks,
// round by round, the 32-row query tiles of the device that meets the block
// in that round (from the first tile with a live pair). Per tile:
// S = Q K^T and dP = dO V^T on MFMA (Q and dO rows from LDS, K and V held in
// registers), P = 2^(S scale log2 e - LSE log2 e), dS = P (dP - Delta) scale,
// then dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T read from the same
// row-major tiles through ds_read_b64_tr_b16. Tiles stream into a 4-stage
// LDS ring three tiles ahead; one barrier per tile.
__global__ void __launch_bounds__(256, 1) bwd_dkdv(BwdArgs a) {
    __shared__ SmemDkdv sm;
    const int L = (int)a.L;
    const int64_t nkt = (a.L + KBM - 1) / KBM;
    const WorkItem wi = decode_work(nkt, a.B, a.H, a.N, 0);
    const int s = (int)wi.d;                               // the key block's owner
    const int ktile = (int)wi.heavy_rank;                  // early keys meet the most queries
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, c32 = lane & 31, h2 = lane >> 5;
    const int k0 = ktile * KBM;

    const int rs = (int)(a.H * D);
    const int row_bytes = rs * 2;
    const uint64_t q_head = uniform_u64((uint64_t)((const bf16*)a.q + (wi.b * a.S * a.H + wi.h) * D));
    const uint64_t do_head = uniform_u64((uint64_t)((const bf16*)a.dout + (wi.b * a.S * a.H + wi.h) * D));
    const uint64_t st_head = uniform_u64((uint64_t)(a.stats + 2 * (wi.b * a.H + wi.h) * a.S));
    // Device t's j-th token sits at slot mem_slot(t, j); consecutive tokens of
    // a device are rstep slots (rstride bytes) apart.
    const bool strided = a.strided != 0;
    const int rstep = strided ? a.N : 1;
    const int rstride = rstep * row_bytes;
    const int64_t span_bytes = (int64_t)(L - 1) * rstride + D * 2;
    const int nqt = (L + KBQ - 1) / KBQ;

    // Rounds: in round r the block of device s meets the queries of device
    // (s + r) mod N. Query rows that see any key of this workgroup start at
    // k0 - delta + 1 (the live keys of row j are those < j + delta).
    auto qdev = [&](int r) {
        const int x = s + r;
        return x >= a.N ? x - a.N : x;
    };
    auto delta_of = [&](int r) { return clamp_delta(live_delta(a.layout, a.N, L, qdev(r), s), L); };
    auto first_tile = [&](int r) { return min(max(k0 - delta_of(r) + 1, 0), L) / KBQ; };
    int n_tiles = 0;
    for (int r = 0; r < a.N; ++r) n_tiles += nqt - first_tile(r);

    // This wave's keys.
    const int kw0 = k0 + 32 * w;
    const int kw = kw0 + c32;
    const bool key_ok = kw < L;
    const bool wave_live = kw0 < L;
    const int64_t krow = (wi.b * a.S + mem_slot(strided, a.N, a.L, s, min(kw, L - 1))) * a.H + wi.h;

    // K^T and V^T operands (lane: key c32, dims kk*16 + 8*h2 .. +7).
    bf16x8 kreg[8], vreg[8];
    {
        const bf16x8* kp = (const bf16x8*)((const bf16*)a.k + krow * D) + h2;
        const bf16x8* vp = (const bf16x8*)((const bf16*)a.v + krow * D) + h2;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            kreg[kk] = kp[2 * kk];
            vreg[kk] = vp[2 * kk];
        }
    }
    __builtin_amdgcn_s_waitcnt(0);

    f32x16 dkacc[4], dvacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        dkacc[db] = f32x16{};
        dvacc[db] = f32x16{};
    }
    const float sl = a.scale_log2;
    const float scale = a.scale;

    // Loads: wave w issues instructions w and w + 4 of each 8-instruction
    // (8 KiB) tile of Q and of dO, instruction i covering rows 4i .. 4i+3;
    // lane l writes row 4i + l/16, slot l % 16, loading the chunk that slot
    // holds (for these rows swz = 4 (l/16) + w). Each wave also loads the
    // tile's 64 statistics floats into its own copy.
    const int ld_voff = (4 * w + (lane >> 4)) * rstride + 16 * ((lane & 15) ^ (((lane >> 4) << 2) | w));
    const int ld_step = 16 * rstride;
    const int st_voff = (lane >> 1) * rstep * 8 + (lane & 1) * 4;   // lane: row lane/2, (LSE, Delta)[lane % 2]
    auto load_tile = [&](int r, int tq, bool valid, int stage) {
        const int dq = qdev(r);
        const int64_t tile_off = (int64_t)tq * KBQ * rstride;
        const int64_t left64 = span_bytes - tile_off;
        const int left = (valid && left64 > 0) ? (int)min(left64, (int64_t)KBQ * rstride) : 0;
        const uint64_t off = (uint64_t)mem_slot(strided, a.N, a.L, dq, 0) * (uint64_t)row_bytes + (uint64_t)tile_off;
        const i32x4 rq = raw_rsrc(q_head + off, left);
        const i32x4 rd = raw_rsrc(do_head + off, left);
        const int64_t srow0 = mem_slot(strided, a.N, a.L, dq, tq * KBQ);   // slot of the tile's first row
        const int64_t st64 = (a.S - srow0) * 8;
        const int st_left = valid ? (int)min(st64, (int64_t)KBQ * rstep * 8) : 0;
        const i32x4 rst = raw_rsrc(st_head + (uint64_t)srow0 * 8, st_left);
        const uint32_t dsq = lds_addr(&sm.q[stage][512 * w]);
        const uint32_t dsd = lds_addr(&sm.dout[stage][512 * w]);
        load_lds_b128(rq, ld_voff, dsq);
        load_lds_b128(rq, ld_voff + ld_step, dsq + 4096);
        load_lds_b128(rd, ld_voff, dsd);
        load_lds_b128(rd, ld_voff + ld_step, dsd + 4096);
        load_lds_b32(rst, st_voff, lds_addr(&sm.st[stage][w][0]));
    };

    // Transposing-read addressing (lane (g, j) names key row 16 kk2 + 8 rd +
    // 4 (g / 2) + j / 4, dims 32 db + 16 (g % 2) + 4 (j % 4) .. +3).
    const int tg = lane >> 4, tj = lane & 15;
    const int tr_row = 4 * (tg >> 1) + (tj >> 2);
    const int tr_c = 2 * (tg & 1) + ((tj & 3) >> 1);      // chunk within the 4-chunk group of a dim block
    auto tr_ptr = [&](const bf16* tile, int kk2, int rd, int db) {
        const int row = 16 * kk2 + 8 * rd + tr_row;
        const int slot = (4 * db + tr_c) ^ swz(row);
        return tile + row * D + 8 * slot + 4 * (tj & 1);
    };
    auto read_t = [&](const bf16* tile, int kk2, int db) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(SRA_LDS4(tr_ptr(tile, kk2, 0, db)));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(SRA_LDS4(tr_ptr(tile, kk2, 1, db)));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    int cr = 0, cq = first_tile(0);
    auto settle = [&](int& r, int& tq) {
        while (tq >= nqt && r + 1 < a.N) {
            ++r;
            tq = first_tile(r);
        }
    };
    settle(cr, cq);
    int lr = cr, lq = cq;

    // Zero LDS once (rows past a slab end are never loaded), then tiles 0..2.
    {
        u32x4* z = (u32x4*)&sm;
        for (int i = tid; i < (int)(sizeof(SmemDkdv) / 16); i += 256) z[i] = u32x4{0u, 0u, 0u, 0u};
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        bar();
    }
#pragma unroll
    for (int u = 0; u < DK_AHEAD; ++u) {
        load_tile(lr, lq, u < n_tiles, u);
        ++lq;
        settle(lr, lq);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm10);   // tile 0 is in
    bar();

    for (int t = 0; t < n_tiles; ++t) {
        load_tile(lr, lq, t + DK_AHEAD < n_tiles, (t + DK_AHEAD) & (DK_NS - 1));
        ++lq;
        settle(lr, lq);

        const int stg = t & (DK_NS - 1);
        const bf16* qs = sm.q[stg];
        const bf16* ds = sm.dout[stg];
        const int delta = delta_of(cr);
        const int jq0 = cq * KBQ;
        const int jq_last = min(jq0 + KBQ - 1, L - 1);
        // Live pairs for this wave: its first key is live for the tile's last row.
        if (wave_live && kw0 < live32(jq_last, delta, L)) {
            f32x16 sacc, dp;
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const int slot = (2 * kk + h2) ^ swz(c32);
                const bf16x8 qf = *(const bf16x8*)&qs[c32 * D + 8 * slot];
                const bf16x8 df = *(const bf16x8*)&ds[c32 * D + 8 * slot];
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf, kreg[kk], kk == 0 ? f32x16{} : sacc, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(df, vreg[kk], kk == 0 ? f32x16{} : dp, 0, 0, 0);
            }
            // Accumulator element i of this lane is query jq0 + 8*(i/4) + 4*h2 + i%4
            // against key kw. The tile is fully live when all its rows are in
            // range and the wave's last key is live for the tile's first row.
            const bool full = jq0 + KBQ <= L && kw0 + 31 < L && kw0 + 31 < jq0 + delta;
            if (!full) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int jj = jq0 + 8 * (i >> 2) + 4 * h2 + (i & 3);
                    if (!(jj < L && key_ok && kw < jj + delta)) sacc[i] = -INFINITY;
                }
            }
            bf16x8 pb[2], dsb[2];
            const float* stt = sm.st[stg][0];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                // (LSE log2 e, Delta) of rows 8g + 4h2 .. +3
                const f32x4 s01 = *(const f32x4*)&stt[2 * (8 * g + 4 * h2)];
                const f32x4 s23 = *(const f32x4*)&stt[2 * (8 * g + 4 * h2) + 4];
                const float lz[4] = {s01[0], s01[2], s23[0], s23[2]};
                const float dz[4] = {s01[1], s01[3], s23[1], s23[3]};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 4 * g + e;
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i], sl, -lz[e]));
                    pb[i >> 3][i & 7] = (bf16)p;
                    dsb[i >> 3][i & 7] = (bf16)(p * (dp[i] - dz[e]) * scale);
                }
            }
#pragma unroll
            for (int kk2 = 0; kk2 < 2; ++kk2) {
#pragma unroll
                for (int db = 0; db < 4; ++db) {
                    dvacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_t(ds, kk2, db), pb[kk2], dvacc[db], 0, 0, 0);
                    dkacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(read_t(qs, kk2, db), dsb[kk2], dkacc[db], 0, 0, 0);
                }
            }
        }
        ++cq;
        settle(cr, cq);
        __builtin_amdgcn_s_waitcnt(kWaitVm10);   // tile t+1 is in
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        bar();
    }
    __builtin_amdgcn_s_waitcnt(0);   // no load may still be writing LDS when the workgroup ends

    if (!key_ok) return;
    bf16* dkp = (bf16*)a.dk + krow * D;
    bf16* dvp = (bf16*)a.dv + krow * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int dcol = db * 32 + 8 * g + 4 * h2;
            const bf16x4 k4 = {(bf16)dkacc[db][4 * g], (bf16)dkacc[db][4 * g + 1], (bf16)dkacc[db][4 * g + 2],
                               (bf16)dkacc[db][4 * g + 3]};
            const bf16x4 v4 = {(bf16)dvacc[db][4 * g], (bf16)dvacc[db][4 * g + 1], (bf16)dvacc[db][4 * g + 2],
                               (bf16)dvacc[db][4 * g + 3]};
            *(bf16x4*)(dkp + dcol) = k4;
            *(bf16x4*)(dvp + dcol) = v4;
        }
}

}  // namespace

hipError_t launch_bwd_bf16_d128(const BwdArgs& a, hipStream_t stream) {
    const uint64_t rows = (uint64_t)(a.B * a.S * a.H);
    uint64_t blocks = (rows + 15) / 16;   // 16 rows per 256-thread block
    if (blocks > 256ull * 64) blocks = 256ull * 64;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(bwd_delta, dim3((unsigned)blocks), dim3(256), 0, stream, (const bf16*)a.o, (const bf16*)a.dout,
                       a.lse, a.stats, (uint32_t)rows, (uint32_t)a.S, (uint32_t)a.H);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nq = (a.L + QBM - 1) / QBM * a.H * a.N * a.B;
    hipLaunchKernelGGL(bwd_dq, dim3((unsigned)nq), dim3(256), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nk = (a.L + KBM - 1) / KBM * a.H * a.N * a.B;
    hipLaunchKernelGGL(bwd_dkdv, dim3((unsigned)nk), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace sra
