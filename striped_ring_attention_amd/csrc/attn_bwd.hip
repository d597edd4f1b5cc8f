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

// Sixteen lanes per (b, slot, h) row, each taking 8 consecutive elements
// (16-byte loads, so a wave reads four whole 256-byte rows of O and of dO),
// then a 16-lane butterfly sum: Delta = sum_c dO[c] * O[c] in fp32.
__global__ void __launch_bounds__(256) bwd_delta(const bf16* __restrict__ o, const bf16* __restrict__ dout,
                                                 float* __restrict__ delta, uint64_t rows) {
    const uint64_t stride = ((uint64_t)gridDim.x * blockDim.x) >> 4;
    const int c = threadIdx.x & 15;
    for (uint64_t r = ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 4; r < rows; r += stride) {
        const bf16x8 x = *(const bf16x8*)(o + r * D + 8 * c);
        const bf16x8 y = *(const bf16x8*)(dout + r * D + 8 * c);
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) s = __builtin_fmaf((float)x[e], (float)y[e], s);
#pragma unroll
        for (int m = 8; m >= 1; m >>= 1) s += __shfl_xor(s, m, 16);
        if (c == 0) delta[r] = s;
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
    const int64_t slot0 = wi.b * a.S + (int64_t)d * a.L;   // first slot of device d
    const uint64_t k_head = uniform_u64((uint64_t)((const bf16*)a.k + (wi.b * a.S * a.H + wi.h) * D));
    const uint64_t v_head = uniform_u64((uint64_t)((const bf16*)a.v + (wi.b * a.S * a.H + wi.h) * D));
    const uint64_t slab_stride = (uint64_t)a.L * (uint64_t)row_bytes;
    const int slab_bytes = __builtin_amdgcn_readfirstlane((L - 1) * row_bytes + D * 2);

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
    const int64_t row = (slot0 + min(j, L - 1)) * a.H + wi.h;

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
    const float lse_l2 = row_ok ? a.lse[row] * kLog2e : 0.f;
    const float dlt = row_ok ? a.delta[row] : 0.f;
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
    const int k_voff = 4 * kq * row_bytes + dc * 16;
    const int v_voff = kr * row_bytes + kcc * 64;
    const int kt_col = 16 * (kq >> 2) + 4 * ((kq & 1) * 2 + ((kq >> 1) & 1));
    u32x4 kst[4], vst[4];

    auto load_tile = [&](int s, int kt, bool valid) {
        const int tile_off = kt * QBN * row_bytes;
        int left = slab_bytes - tile_off;
        left = (valid && left > 0) ? left : 0;
        const uint64_t so = (uint64_t)s * slab_stride + (uint64_t)tile_off;
        const __amdgpu_buffer_rsrc_t krs = slab_rsrc((const void*)(k_head + so), left);
        const __amdgpu_buffer_rsrc_t vrs = slab_rsrc((const void*)(v_head + so), left);
#pragma unroll
        for (int i = 0; i < 4; ++i) kst[i] = __builtin_amdgcn_raw_buffer_load_b128(krs, k_voff + i * row_bytes, 0, 0);
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

constexpr int KBM = 128;          // keys per workgroup
constexpr int KBQ = 32;           // query rows per tile
constexpr int QTP = KBQ + 8;      // Q^T / dO^T tile pitch (elements)

struct __align__(16) SmemDkdv {
    bf16 qr[KBQ * KP];    // Q tile, row-major
    bf16 dor[KBQ * KP];   // dO tile, row-major
    bf16 qt[D * QTP];     // Q tile, dimension-major, permuted query order
    bf16 dot[D * QTP];    // dO tile, dimension-major, permuted query order
    float lse[KBQ];       // log2-scaled LSE of the tile's rows
    float dl[KBQ];        // Delta of the tile's rows
};

__global__ void __launch_bounds__(256, 1) bwd_dkdv(BwdArgs a) {
    __shared__ SmemDkdv sm;
    const int L = (int)a.L;
    const int64_t nkt = (a.L + KBM - 1) / KBM;
    const WorkItem wi = decode_work(nkt, a.B, a.H, a.N, 0);
    const int s = (int)wi.d;                               // the key block's owner
    const int ktile = (int)wi.heavy_rank;                  // early keys meet the most queries
    const int tid = threadIdx.x;
    const int w = tid >> 6, lane = tid & 63, c32 = lane & 31, h2 = lane >> 5;
    const int k0 = ktile * KBM;

    const int rs = (int)(a.H * D);
    const int row_bytes = rs * 2;
    const uint64_t q_head = uniform_u64((uint64_t)((const bf16*)a.q + (wi.b * a.S * a.H + wi.h) * D));
    const uint64_t do_head = uniform_u64((uint64_t)((const bf16*)a.dout + (wi.b * a.S * a.H + wi.h) * D));
    const uint64_t slab_stride = (uint64_t)a.L * (uint64_t)row_bytes;
    const int slab_bytes = __builtin_amdgcn_readfirstlane((L - 1) * row_bytes + D * 2);
    const int nqt = (L + KBQ - 1) / KBQ;

    // Rounds: in round r the block of device s meets the queries of device
    // (s + r) mod N. Query rows that see any key of this workgroup start at
    // k0 - delta + 1 (the live keys of row j are those < j + delta).
    auto qdev = [&](int r) { return (s + r) % a.N; };
    auto delta_of = [&](int r) { return clamp_delta(live_delta(a.layout, a.N, L, qdev(r), s), L); };
    auto first_tile = [&](int r) { return min(max(k0 - delta_of(r) + 1, 0), L) / KBQ; };
    int n_tiles = 0;
    for (int r = 0; r < a.N; ++r) n_tiles += nqt - first_tile(r);

    // This wave's keys.
    const int kw0 = k0 + 32 * w;
    const int kw = kw0 + c32;
    const bool key_ok = kw < L;
    const bool wave_live = kw0 < L;
    const int64_t krow = (wi.b * a.S + (int64_t)s * a.L + min(kw, L - 1)) * a.H + wi.h;

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

    // Tile staging: threads 0-127 stage Q, 128-255 stage dO, as (query quad
    // qq, 8-dim chunk dc): four rows x 16 bytes, written row-major and
    // transposed. Threads 0-31 / 32-63 also fetch the tile's LSE / Delta.
    const int half = tid >> 7, lt = tid & 127;
    const int qq = lt & 7, dc = lt >> 3;
    const int st_voff = 4 * qq * row_bytes + dc * 16;
    const uint64_t st_head = uniform_u64(half == 0 ? q_head : do_head);   // wave-uniform
    const int qt_col = 16 * (qq >> 2) + 4 * ((qq & 1) * 2 + ((qq >> 1) & 1));
    u32x4 st[4];
    float sc_val = 0.f;

    auto load_tile = [&](int r, int tq, bool valid) {
        const int dq = qdev(r);
        const int tile_off = tq * KBQ * row_bytes;
        int left = slab_bytes - tile_off;
        left = (valid && left > 0) ? left : 0;
        const __amdgpu_buffer_rsrc_t rsrc =
            slab_rsrc((const void*)(st_head + (uint64_t)dq * slab_stride + (uint64_t)tile_off), left);
#pragma unroll
        for (int i = 0; i < 4; ++i) st[i] = __builtin_amdgcn_raw_buffer_load_b128(rsrc, st_voff + i * row_bytes, 0, 0);
        if (tid < 64) {
            const int jr = tq * KBQ + (tid & 31);
            const int64_t srow = (wi.b * a.S + (int64_t)dq * a.L + min(jr, L - 1)) * a.H + wi.h;
            sc_val = (valid && jr < L) ? (tid < 32 ? a.lse[srow] * kLog2e : a.delta[srow]) : 0.f;
        }
    };
    auto store_tile = [&]() {
        bf16* rm = half == 0 ? sm.qr : sm.dor;
        bf16* tr = half == 0 ? sm.qt : sm.dot;
#pragma unroll
        for (int i = 0; i < 4; ++i) *(u32x4*)&rm[(4 * qq + i) * KP + 8 * dc] = st[i];
        bf16* td = &tr[(8 * dc) * QTP + qt_col];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            uint2 lo = {pack_lo(st[0][p], st[1][p]), pack_lo(st[2][p], st[3][p])};
            uint2 hi = {pack_hi(st[0][p], st[1][p]), pack_hi(st[2][p], st[3][p])};
            *(uint2*)(td + (2 * p) * QTP) = lo;
            *(uint2*)(td + (2 * p + 1) * QTP) = hi;
        }
        if (tid < 32) sm.lse[tid] = sc_val;
        else if (tid < 64) sm.dl[tid - 32] = sc_val;
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

    if (n_tiles > 0) load_tile(lr, lq, true);
    for (int t = 0; t < n_tiles; ++t) {
        __syncthreads();
        store_tile();
        __syncthreads();
        ++lq;
        settle(lr, lq);
        load_tile(lr, lq, t + 1 < n_tiles);

        const int delta = delta_of(cr);
        const int jq0 = cq * KBQ;
        const int jq_last = min(jq0 + KBQ - 1, L - 1);
        // Live pairs for this wave: its first key is live for the tile's last row.
        if (wave_live && kw0 < live32(jq_last, delta, L)) {
            f32x16 sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)&sm.qr[c32 * KP + 8 * h2], kreg[0],
                                                                  f32x16{}, 0, 0, 0);
            f32x16 dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)&sm.dor[c32 * KP + 8 * h2], vreg[0],
                                                                f32x16{}, 0, 0, 0);
#pragma unroll
            for (int kk = 1; kk < 8; ++kk) {
                sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)&sm.qr[c32 * KP + 16 * kk + 8 * h2],
                                                               kreg[kk], sacc, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)&sm.dor[c32 * KP + 16 * kk + 8 * h2],
                                                             vreg[kk], dp, 0, 0, 0);
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
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 l4 = *(const f32x4*)&sm.lse[8 * g + 4 * h2];
                const f32x4 d4 = *(const f32x4*)&sm.dl[8 * g + 4 * h2];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int i = 4 * g + e;
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i], sl, -l4[e]));
                    pb[i >> 3][i & 7] = (bf16)p;
                    dsb[i >> 3][i & 7] = (bf16)(p * (dp[i] - d4[e]) * scale);
                }
            }
#pragma unroll
            for (int kk2 = 0; kk2 < 2; ++kk2) {
#pragma unroll
                for (int db = 0; db < 4; ++db) {
                    const int off = (db * 32 + c32) * QTP + 16 * kk2 + 8 * h2;
                    dvacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)&sm.dot[off], pb[kk2], dvacc[db], 0, 0, 0);
                    dkacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)&sm.qt[off], dsb[kk2], dkacc[db], 0, 0, 0);
                }
            }
        }
        ++cq;
        settle(cr, cq);
    }

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
                       a.delta, rows);
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
