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
//  * bwd_dkdv:   a workgroup owns 128 keys (4 groups x 32) of one source
//                device and walks the 32-row query tiles of every device that
//                meets the block, round by round. Two waves per 32-key group:
//                one computes S = Q K^T, P and dV^T += dO^T P (K held in
//                registers), the other dP = dO V^T, dS and dK^T += Q^T dS (V
//                held in registers), P passing between them through LDS; Q and
//                dO are read from row-major LDS tiles, directly and through
//                transposing reads.
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

}  // namespace

// The dK/dV kernel lives in attn_bwd_dkdv.hip (built with its own flags).
hipError_t launch_bwd_dkdv_bf16_d128(const BwdArgs& a, hipStream_t stream);

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
    return launch_bwd_dkdv_bf16_d128(a, stream);
}

}  // namespace sra
