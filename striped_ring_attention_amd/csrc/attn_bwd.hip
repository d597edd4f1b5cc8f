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
//  * bwd_dq:     a workgroup owns 256 query rows (8 waves x 32) and walks
//                the (round, 64-key tile) pairs, taking the rounds in the
//                same source order on every device. Per 32-key
//                block: S^T = K Q^T and dP^T = V dO^T on MFMA (Q^T and dO^T
//                held in registers, K and V row-major in LDS), then
//                dS^T = P^T (dP^T - Delta) scale, and dQ^T += K^T dS^T with
//                K^T read from the row-major K tile by transposing LDS reads
//                (ds_read_b64_tr_b16).
//  * bwd_dkdv:   a workgroup owns 128 keys (4 groups x 32) of one source
//                device and walks the 32-row query tiles of every device that
//                meets the block, round by round (query devices in the same
//                order for every key block). Two waves per 32-key group:
//                one computes S = Q K^T, P and dV^T += dO^T P (K held in
//                registers), the other dP = dO V^T, dS and dK^T += Q^T dS (V
//                held in registers), P passing between them through LDS; Q and
//                dO are read from row-major LDS tiles, directly and through
//                transposing reads.
// No atomics: each gradient accumulates in the registers of the workgroup
// that owns its rows, so results are deterministic. S and dP are computed in
// both kernels (seven tile products per live tile instead of five).
#include <mutex>

#include "kernel_common.h"

namespace sra {

// Backward statistics storage for callers that cannot allocate: one array
// per GPU, held by the library for the life of the process. Host code never
// passes `scratch` itself (in host code that name is only a stand-in for the
// symbol); it passes the device address that hipGetSymbolAddress returns.
static __device__ __align__(256) float scratch[kBwdScratchBytes / sizeof(float)];

namespace {

using namespace kc;

constexpr int D = 128;

// ------------------------------------------------------------------ Delta --

// Row statistics of the backward, one float pair per row in a head-major
// layout [B, H, S, 2]: (LSE * log2 e, Delta), Delta = sum_c dO[c] * O[c] in
// fp32. The rows of one head are contiguous, so the 32 rows of a query tile
// are 256 contiguous bytes. A workgroup takes 16 slots x up to 64 heads of one
// batch: sixteen lanes per (b, slot, h) row, each taking 8 consecutive
// elements (16-byte loads; consecutive rows of a pass are consecutive heads
// of one slot, so a wave reads four whole 256-byte rows of O and of dO), a
// 16-lane butterfly sum, and the pair parked in LDS as [head][slot]. The
// pairs then go out head by head, 16 slots = 128 contiguous bytes, instead of
// one 8-byte store per row across the head-major array.
constexpr int kDeltaSlots = 16;
constexpr int kDeltaHeads = 64;
__global__ void __launch_bounds__(256) bwd_delta(const bf16* __restrict__ o, const bf16* __restrict__ dout,
                                                 const float* __restrict__ lse, float* __restrict__ stats,
                                                 uint32_t S, uint32_t H) {
    __shared__ float2 tile[kDeltaHeads][kDeltaSlots];
    const uint32_t n_sb = (S + kDeltaSlots - 1) / kDeltaSlots, n_hb = (H + kDeltaHeads - 1) / kDeltaHeads;
    const uint32_t hb = blockIdx.x % n_hb, sb = (blockIdx.x / n_hb) % n_sb, b = blockIdx.x / n_hb / n_sb;
    const uint32_t s0 = sb * kDeltaSlots, h0 = hb * kDeltaHeads;
    const uint32_t ns = min((uint32_t)kDeltaSlots, S - s0), nh = min((uint32_t)kDeltaHeads, H - h0);
    const int c = threadIdx.x & 15;
    for (uint32_t i = threadIdx.x >> 4; i < ns * nh; i += 16) {
        const uint32_t si = i / nh, hk = i - si * nh;
        const uint64_t r = ((uint64_t)b * S + s0 + si) * H + h0 + hk;
        const bf16x8 x = *(const bf16x8*)(o + r * D + 8 * c);
        const bf16x8 y = *(const bf16x8*)(dout + r * D + 8 * c);
        float sum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) sum = __builtin_fmaf((float)x[e], (float)y[e], sum);
#pragma unroll
        for (int m = 8; m >= 1; m >>= 1) sum += __shfl_xor(sum, m, 16);
        if (c == 0) tile[hk][si] = float2{lse[r] * kLog2e, sum};
    }
    __syncthreads();
    for (uint32_t i = threadIdx.x; i < nh * kDeltaSlots; i += 256) {
        const uint32_t hk = i / kDeltaSlots, si = i % kDeltaSlots;
        if (si < ns) *(float2*)(stats + 2 * (((uint64_t)b * H + h0 + hk) * S + s0 + si)) = tile[hk][si];
    }
}

// -------------------------------------------------------------------- dQ --

constexpr int QBM = 256;          // query rows per workgroup (8 waves x 32)
constexpr int QBN = 64;           // keys per tile
constexpr int DQ_NT = 512;
constexpr int DQ_NS = 4;          // LDS stages, tiles loaded three ahead
constexpr int kWaitVm8 = 0x0F78;  // vmcnt(8): the two newest tiles (4 loads each per wave) may be in flight

// K and V tiles are stored row-major with 256-byte rows and no padding (they
// are loaded straight into LDS); 16-byte chunk c of key row r sits in slot
// c ^ swz(r), swz(r) = 4 (r % 4) + (r / 4) % 4, which keeps both the row
// reads of the S and dP products and the transposing K^T reads of the dQ
// product free of bank conflicts.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

struct __align__(16) SmemDq {
    bf16 k[DQ_NS][QBN * D];   // K tiles
    bf16 v[DQ_NS][QBN * D];   // V tiles
};

// A workgroup owns 256 query rows (8 waves x 32) of one device and walks the
// (round, 64-key tile) pairs, the rounds in source-device order (see
// source() below). Per 32-key block: S^T = K Q^T
// and dP^T = V dO^T on MFMA (Q^T and dO^T held in registers, K and V rows
// from LDS), dS^T = P^T (dP^T - Delta) with P^T = 2^(S^T scale log2 e - LSE
// log2 e), then dQ^T += K^T dS^T with K^T read transposed from the
// row-major K tile through ds_read_b64_tr_b16; dQ takes the softmax scale
// once at the end (one multiply per output instead of one per score). Waves
// 0-3 load K tiles and waves 4-7 V tiles straight into a 4-stage LDS ring,
// three tiles ahead; one barrier per tile.
__global__ void __launch_bounds__(DQ_NT, 1) bwd_dq(BwdArgs a) {
    __shared__ SmemDq sm;
    const int L = (int)a.L;
    const int64_t nqt = (a.L + QBM - 1) / QBM;
    const WorkItem wi = decode_work(nqt, a.B, a.H, a.N, 0);
    const int d = (int)wi.d;
    const int qt = (int)uniform_i64(nqt - 1 - wi.heavy_rank);   // late query tiles meet the most keys
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, c32 = lane & 31, h2 = lane >> 5;
    const int j0 = qt * QBM;
    const int j1 = min(j0 + QBM, L);

    const int row_bytes = (int)(a.H * D) * 2;
    // Device t's j-th token sits at slot mem_slot(t, j); consecutive tokens of
    // a device are rstride bytes apart.
    const bool strided = a.strided != 0;
    const int rstride = (int)(strided ? a.N : 1) * row_bytes;
    const uint64_t k_head = uniform_u64((uint64_t)((const bf16*)a.k + (wi.b * a.S * a.H + wi.h) * D));
    const uint64_t v_head = uniform_u64((uint64_t)((const bf16*)a.v + (wi.b * a.S * a.H + wi.h) * D));
    auto slot_bytes = [&](int t) { return (uint64_t)mem_slot(strided, a.N, a.L, t, 0) * (uint64_t)row_bytes; };
    const int64_t span_bytes = (int64_t)(L - 1) * rstride + D * 2;

    // Rounds: in round r device d holds the block of device (d - r) mod N.
    // Walk step u visits source device u (round (d - u) mod N): every device
    // of a head walks the sources in the same order, so the workgroups of a
    // head read the same K/V slab at the same time and share it through L2.
    // The sum over rounds is the same in any order up to rounding.
    auto source = [&](int u) { return u; };
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

    // Q^T and dO^T operands (lane: query c32, dims kk*16 + 8*h2 .. +7) and the
    // row statistics; awaited together with the first tiles below.
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

    f32x16 dqacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) dqacc[db] = f32x16{};
    const float sl = a.scale_log2;
    const float scale = a.scale;

    // Loads: group 0 (waves 0-3) loads K tiles, group 1 V tiles; wave wg of a
    // group issues four instructions per tile, instruction q covering key rows
    // 4 wg + 16 q .. +3. Lane l writes row 4 wg + 16 q + l/16, LDS slot l % 16,
    // loading the chunk that slot holds (for these rows swz = 4 (l/16) + wg).
    // Each tile gets its own buffer resource (base at the tile's first row,
    // size cut to what is left of the slab), so rows past the slab end are not
    // read.
    const int grp = w >> 2, wg = w & 3;
    const int ld_voff = (4 * wg + (lane >> 4)) * rstride + 16 * ((lane & 15) ^ (((lane >> 4) << 2) | wg));
    const int ld_step = 16 * rstride;
    const uint64_t ld_head = uniform_u64(grp == 0 ? k_head : v_head);
    const uint32_t ld_lds0 = lds_addr(grp == 0 ? &sm.k[0][0] : &sm.v[0][0]) + 1024 * wg;
    auto load_tile = [&](int s, int kt, bool valid, int stage) {
        const int64_t tile_off = (int64_t)kt * QBN * rstride;
        const int64_t left64 = span_bytes - tile_off;
        const int left = (valid && left64 > 0) ? (int)min(left64, (int64_t)QBN * rstride) : 0;
        const i32x4 rsrc = raw_rsrc(ld_head + slot_bytes(s) + (uint64_t)tile_off, left);
        const uint32_t dst = ld_lds0 + stage * (QBN * D * 2);
#pragma unroll
        for (int q = 0; q < 4; ++q) load_lds_b128(rsrc, ld_voff + q * ld_step, dst + 4096 * q);
    };

    // Transposing-read addressing for K^T: lane (g = l / 16, i = l % 16) names
    // key row 16 kk2 + 8 rd + 4 (g / 2) + i / 4 of a 32-key block, dims
    // 32 db + 16 (g % 2) + 4 (i % 4) .. +3, so lane l collects dim 32 db + l % 32
    // of keys 16 kk2 + 4 h2 + 0..3 and 16 kk2 + 8 + 4 h2 + 0..3 -- the keys its
    // dS^T registers hold. The swizzle of such a row does not depend on the
    // block or kk2.
    const int tg = lane >> 4, tj = lane & 15;
    const int tr_row = 4 * (tg >> 1) + (tj >> 2);
    const int tr_c = 2 * (tg & 1) + ((tj & 3) >> 1);
    auto tr_off = [&](int rd, int db) {
        const int r = 8 * rd + tr_row;
        return r * D + 8 * ((4 * db + tr_c) ^ swz(r)) + 4 * (tj & 1);
    };
    auto row_off = [&](int kk) { return c32 * D + 8 * ((2 * kk + h2) ^ swz(c32)); };

    // Tile cursor (walk step, key tile); walk step u visits source u.
    int cr = 0, ck = 0, cnt = tiles_of(0);
    auto settle = [&](int& r, int& k, int& nt) {
        while (k >= nt && r + 1 < a.N) {
            ++r;
            k = 0;
            nt = tiles_of(r);
        }
        r = __builtin_amdgcn_readfirstlane(r);
        k = __builtin_amdgcn_readfirstlane(k);
        nt = __builtin_amdgcn_readfirstlane(nt);
    };
    settle(cr, ck, cnt);
    int lr = cr, lk = ck, lnt = cnt;   // loader cursor

    // When a slab ends inside a key tile, zero the stages once (rows past the
    // end are never loaded and must hold finite values). Then tiles 0..2.
    if (L % QBN != 0) {
        u32x4* z = (u32x4*)&sm;
        for (int i = tid; i < (int)(sizeof(SmemDq) / 16); i += DQ_NT) z[i] = u32x4{0u, 0u, 0u, 0u};
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        bar();
    }
#pragma unroll 1
    for (int u = 0; u < 3; ++u) {
        load_tile(source(lr), lk, u < n_tiles, u);
        ++lk;
        settle(lr, lk, lnt);
    }
    __builtin_amdgcn_s_waitcnt(0);   // Q, dO, statistics and tiles 0..2 are in
    bar();
    const float lse_l2 = row_ok ? st2.x : 0.f;
    const float dlt = row_ok ? st2.y : 0.f;

    for (int t = 0; t < n_tiles; ++t) {
        // Tile t+3 into the stage of tile t-1 (every wave finished it before
        // the barrier that ended step t-1).
        load_tile(source(lr), lk, t + 3 < n_tiles, (t + 3) & (DQ_NS - 1));
        ++lk;
        settle(lr, lk, lnt);

        const bf16* ks = sm.k[t & (DQ_NS - 1)];
        const bf16* vs = sm.v[t & (DQ_NS - 1)];
        const int delta = delta_of(cr);
        const int k0 = ck * QBN;
        const int kw_end = wave_live ? live32(jw_last, delta, L) : 0;
        const bool masked = k0 + QBN > live32(jw0, delta, L);
        const int c_row = row_ok ? live32(j, delta, L) : 0;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (k0 + 32 * kb >= kw_end) continue;   // no live key for this wave
            const bf16* kb_s = ks + 32 * kb * D;
            const bf16* vb_s = vs + 32 * kb * D;
            bf16x8 kr[8], vr[8];
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                kr[kk] = *(const bf16x8*)&kb_s[row_off(kk)];
                vr[kk] = *(const bf16x8*)&vb_s[row_off(kk)];
            }
            f32x16 s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[0], qreg[0], f32x16{}, 0, 0, 0);
            f32x16 dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[0], doreg[0], f32x16{}, 0, 0, 0);
#pragma unroll
            for (int kk = 1; kk < 8; ++kk) {
                s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[kk], qreg[kk], s, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[kk], doreg[kk], dp, 0, 0, 0);
            }
            // K^T operands of this block, read while the S and dP MFMAs run.
            bf16x8 kt[2][4];
#pragma unroll
            for (int kk2 = 0; kk2 < 2; ++kk2)
#pragma unroll
                for (int db = 0; db < 4; ++db) {
                    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(SRA_LDS4(kb_s + 16 * kk2 * D + tr_off(0, db)));
                    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(SRA_LDS4(kb_s + 16 * kk2 * D + tr_off(1, db)));
                    kt[kk2][db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                }
            // Accumulator element i of this lane is key k0 + 32 kb + 8 (i/4) + 4 h2 + i%4
            // against query c32.
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
                dsb[i >> 3][i & 7] = (bf16)(p * (dp[i] - dlt));
            }
#pragma unroll
            for (int kk2 = 0; kk2 < 2; ++kk2)
#pragma unroll
                for (int db = 0; db < 4; ++db)
                    dqacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kt[kk2][db], dsb[kk2], dqacc[db], 0, 0, 0);
        }
        ++ck;
        settle(cr, ck, cnt);
        __builtin_amdgcn_s_waitcnt(kWaitVm8);   // tile t+1 is in
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        bar();
    }
    __builtin_amdgcn_s_waitcnt(0);   // no load may still be writing LDS when the workgroup ends

    if (!row_ok) return;
    bf16* dqp = (bf16*)a.dq + row * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            // dQ carries the softmax scale once here (its dS operands leave it out).
            const bf16x4 v4 = {(bf16)(dqacc[db][4 * g] * scale), (bf16)(dqacc[db][4 * g + 1] * scale),
                               (bf16)(dqacc[db][4 * g + 2] * scale), (bf16)(dqacc[db][4 * g + 3] * scale)};
            *(bf16x4*)(dqp + db * 32 + 8 * g + 4 * h2) = v4;
        }
}

}  // namespace

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and cached.
hipError_t bwd_scratch(void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

// The dK/dV kernel lives in attn_bwd_dkdv.hip (built with its own flags).
hipError_t launch_bwd_dkdv_bf16_d128(const BwdArgs& a, hipStream_t stream);

hipError_t launch_bwd_bf16_d128(const BwdArgs& a, hipStream_t stream) {
    const uint64_t blocks = (uint64_t)a.B * ((a.S + kDeltaSlots - 1) / kDeltaSlots) *
                            ((a.H + kDeltaHeads - 1) / kDeltaHeads);
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(bwd_delta, dim3((unsigned)blocks), dim3(256), 0, stream, (const bf16*)a.o, (const bf16*)a.dout,
                       a.lse, a.stats, (uint32_t)a.S, (uint32_t)a.H);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nq = (a.L + QBM - 1) / QBM * a.H * a.N * a.B;
    hipLaunchKernelGGL(bwd_dq, dim3((unsigned)nq), dim3(DQ_NT), 0, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_bwd_dkdv_bf16_d128(a, stream);
}

}  // namespace sra
