// Backward pass of striped ring attention for gfx950: the dK/dV kernel (bf16,
// head dim 128). The gradient formulas and the ring decomposition are stated
// in attn_bwd.hip, which also runs the Delta and dQ kernels before this one.
#include "kernel_common.h"

namespace sra {
namespace {

using namespace kc;

constexpr int D = 128;

constexpr int KBM = 128;          // keys per workgroup (4 key groups x 32)
constexpr int KBQ = 32;           // query rows per tile
constexpr int DK_NT = 512;        // 8 waves: two per key group
constexpr int DK_NS = 7;          // LDS stages
constexpr int DK_AHEAD = 5;       // tiles in flight ahead of the one computed
constexpr int kWaitVm12 = 0x0F7C; // vmcnt(12): the four newest tiles (3 loads each, the statistics wave) may be in flight
constexpr int kWaitVm8 = 0x0F78;  // vmcnt(8): the same for the other waves (2 loads each)
constexpr int kStWave = 4;        // the wave that loads each tile's row statistics

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
    float st[DK_NS][64];          // LSE log2 e of the tile's 32 rows, then their Delta
    f32x4 p[2][4][4][64];         // P of tiles t (slot t % 2) and t-1: [slot][group][register quad][lane]
};

// A workgroup owns 128 keys of one source device and walks, round by round,
// the 32-row query tiles of the device that meets the block in that round
// (from the first tile with a live pair). Each 32-key group has two waves on
// one SIMD (waves g and g + 4):
//   the P wave holds K^T and dV: S = Q K^T, P = 2^(S scale log2 e - LSE log2 e),
//     dV^T += dO^T P;
//   the dS wave holds V^T and dK: dP = dO V^T, dS = P (dP - Delta),
//     dK^T += Q^T dS, times the softmax scale once at the end,
// with P (fp32) handed over through LDS. In tile step t the two waves of a
// SIMD do their matrix and vector work in opposite order, so that one's
// vector work runs under the other's MFMAs:
//   P wave:  dV += (tile t-1), S of tile t (16 MFMAs); then P of tile t (vector)
//   dS wave: dS of tile t-1 from P and dP (vector); then dK += (tile t-1),
//            dP of tile t (16 MFMAs)
// P is double-buffered in LDS (tile t in slot t % 2), so the dS wave reads
// P of tile t-1 while the P wave writes P of tile t, and one barrier per step
// (for the tile ring and P) suffices. Each wave holds half the accumulators
// a single wave would need. Q and dO
// rows are read from LDS as MFMA row operands and, for dV and dK, transposed
// through ds_read_b64_tr_b16. Tiles stream into a 7-stage LDS ring five
// tiles ahead; tiles t-1 and t are read during step t.
__global__ void __launch_bounds__(DK_NT, 1) bwd_dkdv(BwdArgs a) {
    __shared__ SmemDkdv sm;
    const int L = (int)a.L;
    const int N = a.N;
    const int64_t nkt = (a.L + KBM - 1) / KBM;
    const WorkItem wi = decode_work(nkt, a.B, a.H, N, 0);
    const int s = (int)wi.d;                               // the key block's owner
    const int ktile = (int)wi.heavy_rank;                  // early keys meet the most queries
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, c32 = lane & 31, h2 = lane >> 5;
    const int kg = w & 3;          // key group
    const bool ds_wave = w >= 4;   // the dS wave of the group (else the P wave)
    const int k0 = ktile * KBM;

    const int row_bytes = (int)(a.H * D) * 2;
    const uint64_t q_head = uniform_u64((uint64_t)((const bf16*)a.q + (wi.b * a.S * a.H + wi.h) * D));
    const uint64_t do_head = uniform_u64((uint64_t)((const bf16*)a.dout + (wi.b * a.S * a.H + wi.h) * D));
    const uint64_t st_head = uniform_u64((uint64_t)(a.stats + 2 * (wi.b * a.H + wi.h) * a.S));
    // Device t's j-th token sits at slot mem_slot(t, j); consecutive tokens of
    // a device are rstep slots (rstride bytes) apart.
    const bool strided = a.strided != 0;
    const int rstep = strided ? N : 1;
    const int rstride = rstep * row_bytes;
    const int64_t span_bytes = (int64_t)(L - 1) * rstride + D * 2;
    const int nqt = (L + KBQ - 1) / KBQ;

    // Rounds: in round r the block of device s meets the queries of device
    // (s + r) mod N. Query rows that see any key of this workgroup start at
    // k0 - delta + 1 (the live keys of row j are those < j + delta).
    // Walk step u visits the queries of device u (round (u - s) mod N): the
    // key blocks of every device of a head walk the query devices in the same
    // order, so they read the same Q/dO slab at the same time and share it
    // through L2. The sum over rounds is the same in any order up to rounding.
    auto qdev = [&](int u) { return u; };
    auto delta_of = [&](int r) { return clamp_delta(live_delta(a.layout, N, L, qdev(r), s), L); };
    auto first_tile = [&](int r) { return min(max(k0 - delta_of(r) + 1, 0), L) / KBQ; };
    int n_tiles = 0;
    for (int r = 0; r < N; ++r) n_tiles += nqt - first_tile(r);
    // Move a (round, tile) cursor past the rounds it has finished; true if it moved.
    auto settle = [&](int& r, int& tq) {
        if (tq < nqt || r + 1 >= N) return false;
        do {
            ++r;
            tq = first_tile(r);
        } while (tq >= nqt && r + 1 < N);
        r = __builtin_amdgcn_readfirstlane(r);
        tq = __builtin_amdgcn_readfirstlane(tq);
        return true;
    };

    // This group's keys.
    const int kw0 = k0 + 32 * kg;
    const int kw = kw0 + c32;
    const bool key_ok = kw < L;
    const bool wave_live = kw0 < L;
    const int64_t krow = (wi.b * a.S + mem_slot(strided, N, a.L, s, min(kw, L - 1))) * a.H + wi.h;

    // K^T (P wave) or V^T (dS wave) operand: lane holds key c32, dims
    // kk*16 + 8*h2 .. +7. Issued before the first tile loads and awaited
    // together with them (one memory round trip before the loop).
    bf16x8 kvreg[8];
    {
        const bf16x8* kp = (const bf16x8*)((const bf16*)(ds_wave ? a.v : a.k) + krow * D) + h2;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) kvreg[kk] = kp[2 * kk];
    }

    // Loads: wave w issues instruction w of each 8-instruction (8 KiB) tile of
    // Q and of dO, covering rows 4w .. 4w+3: lane l writes row 4w + l/16,
    // slot l % 16, loading the chunk that slot holds (for these rows
    // swz = 4 (l/16) + w % 4). Wave kStWave also loads the tile's statistics
    // into the one copy every wave reads: lane l takes row l % 32, LSE for
    // l < 32 and Delta above. Each wave waits for its own loads of a tile
    // before the barrier that precedes the tile's first read.
    const int ld_voff = (4 * w + (lane >> 4)) * rstride + 16 * ((lane & 15) ^ (((lane >> 4) << 2) | kg));
    const int st_voff = (lane & 31) * rstep * 8 + (lane >> 5) * 4;
    const uint32_t lds_q = lds_addr(&sm.q[0][0]) + 1024 * w;
    const uint32_t lds_do = lds_addr(&sm.dout[0][0]) + 1024 * w;
    const uint32_t lds_st = lds_addr(&sm.st[0][0]);
    constexpr uint32_t kTileBytes = KBQ * D * 2;
    constexpr uint32_t kStBytes = 64 * 4;
    // Loader cursor (round lr, query tile lq) and, for its tile, the
    // addresses of its first Q and dO rows and of its first statistics slot.
    // Every round's slab has L rows, so only a round's last tile can be
    // partial: its Q/dO loads may read kLastRec bytes (rows past the slab
    // read as zero) and its statistics load st_last bytes (up to the end of
    // the head's statistics), every other tile kFullRec and kStFull. Per tile
    // the loader only adds strides; the round change happens apart from the
    // loads (ld_settle).
    const int kFullRec = KBQ * rstride;
    const int kLastRec = (int)(span_bytes - (int64_t)(nqt - 1) * KBQ * rstride);
    const int kStFull = KBQ * rstep * 8;
    int lr = 0, lq = first_tile(0);
    settle(lr, lq);
    uint64_t ld_q = 0, ld_do = 0, ld_st = 0;
    int st_last = 0;
    auto ld_enter = [&]() {
        const int dq = qdev(lr);
        const int64_t off = mem_slot(strided, N, a.L, dq, 0) * (int64_t)row_bytes + (int64_t)lq * KBQ * rstride;
        const int64_t st_row = mem_slot(strided, N, a.L, dq, (int64_t)lq * KBQ);
        ld_q = uniform_u64(q_head + (uint64_t)off);
        ld_do = uniform_u64(do_head + (uint64_t)off);
        ld_st = uniform_u64(st_head + (uint64_t)st_row * 8);
        const int64_t st_row_last = mem_slot(strided, N, a.L, dq, (int64_t)(nqt - 1) * KBQ);
        st_last = __builtin_amdgcn_readfirstlane((int)min((a.S - st_row_last) * 8, (int64_t)kStFull));
    };
    ld_enter();
    auto ld_settle = [&]() {
        if (settle(lr, lq)) ld_enter();
    };
    // The three loads of the loader's tile (all reading zero when !valid),
    // then the cursor moved to the next tile of the round.
    auto load_q = [&](bool valid, int stage) {
        const int rec = valid ? (lq == nqt - 1 ? kLastRec : kFullRec) : 0;
        load_lds_b128(raw_rsrc(ld_q, rec), ld_voff, lds_q + stage * kTileBytes);
    };
    auto load_do = [&](bool valid, int stage) {
        const int rec = valid ? (lq == nqt - 1 ? kLastRec : kFullRec) : 0;
        load_lds_b128(raw_rsrc(ld_do, rec), ld_voff, lds_do + stage * kTileBytes);
    };
    auto load_st = [&](bool valid, int stage) {
        const int rec = valid ? (lq == nqt - 1 ? st_last : kStFull) : 0;
        if (w == kStWave) load_lds_b32(raw_rsrc(ld_st, rec), st_voff, lds_st + stage * kStBytes);
    };
    auto ld_advance = [&]() {
        ++lq;
        ld_q += (uint64_t)kFullRec;
        ld_do += (uint64_t)kFullRec;
        ld_st += (uint64_t)kStFull;
    };
    auto load_tile = [&](bool valid, int stage) {
        load_q(valid, stage);
        load_do(valid, stage);
        load_st(valid, stage);
        ld_advance();
    };

    // Transposing-read addressing (lane (g, j) names query row 16 kk2 + 8 rd +
    // 4 (g / 2) + j / 4, dims 32 db + 16 (g % 2) + 4 (j % 4) .. +3). The
    // swizzle of such a row does not depend on kk2.
    const int tg = lane >> 4, tj = lane & 15;
    const int tr_row = 4 * (tg >> 1) + (tj >> 2);
    const int tr_c = 2 * (tg & 1) + ((tj & 3) >> 1);      // chunk within the 4-chunk group of a dim block
    auto tr_off = [&](int rd, int db) {
        const int row = 8 * rd + tr_row;
        return row * D + 8 * ((4 * db + tr_c) ^ swz(row)) + 4 * (tj & 1);
    };
    // Row-operand addressing: lane (c32, h2) reads chunk 2 kk + h2 of row c32.
    auto row_off = [&](int kk) { return c32 * D + 8 * ((2 * kk + h2) ^ swz(c32)); };

    // When a slab ends inside a query tile, zero LDS once (rows past a slab
    // end are never loaded and must hold finite values). Then tiles 0..4.
    if (L % KBQ != 0) {
        u32x4* z = (u32x4*)&sm;
        for (int i = tid; i < (int)(sizeof(SmemDkdv) / 16); i += DK_NT) z[i] = u32x4{0u, 0u, 0u, 0u};
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        bar();
    }
#pragma unroll 1
    for (int u = 0; u < DK_AHEAD; ++u) {
        load_tile(u < n_tiles, u);
        ld_settle();
    }
    __builtin_amdgcn_s_waitcnt(0);   // the K/V operands and tiles 0..4 are in
    bar();

    const float sl = a.scale_log2;
    const float scale = a.scale;
    auto pex = [&](int t) { return sm.p[t & 1][kg][0] + lane; };   // this lane's P quads of tile t: [64 g]
    auto next_stage = [](int x) { return x + 1 == DK_NS ? 0 : x + 1; };

    // Operand reads. Transposed: 8 operands (two 16-row halves x 4 dim
    // blocks) of Y^T from a row-major tile. Rows: the 8 row operands of X.
    auto read_yt = [&](const bf16* ys, bf16x8 (&yt)[2][4]) {
#pragma unroll
        for (int kk2 = 0; kk2 < 2; ++kk2)
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(SRA_LDS4(ys + 16 * kk2 * D + tr_off(0, db)));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(SRA_LDS4(ys + 16 * kk2 * D + tr_off(1, db)));
                yt[kk2][db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
    };
    auto read_rows = [&](const bf16* xs, bf16x8 (&xr)[8]) {
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) xr[kk] = *(const bf16x8*)&xs[row_off(kk)];
    };
    f32x16 acc[4];   // dV^T (P wave) or dK^T (dS wave): dims 32 db + .., key c32
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[db] = f32x16{};
    // acc += Y^T op (Y^T operands already read).
    auto acc_t = [&](const bf16x8 (&yt)[2][4], const bf16x8 (&op)[2]) {
#pragma unroll
        for (int kk2 = 0; kk2 < 2; ++kk2)
#pragma unroll
            for (int db = 0; db < 4; ++db)
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(yt[kk2][db], op[kk2], acc[db], 0, 0, 0);
    };
    // X K^T or X V^T (row operands already read). Element i of a lane is
    // query jq0 + 8*(i/4) + 4*h2 + i%4 against key kw.
    auto rows_kv = [&](const bf16x8 (&xr)[8]) {
        f32x16 x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xr[0], kvreg[0], f32x16{}, 0, 0, 0);
#pragma unroll
        for (int kk = 1; kk < 8; ++kk) x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xr[kk], kvreg[kk], x, 0, 0, 0);
        return x;
    };

    // The two waves of a group run the same tile walk and barriers with their
    // own halves of the work. Tile t is in LDS from the start of step t, so
    // each wave reads its operands a phase ahead where registers allow:
    // the P wave reads dO^T of tile t while it computes P, and Q rows and LSE
    // of tile t at the start of step t; the dS wave reads P and Delta of tile
    // t-1 and dO rows of tile t at the start of step t, and Q^T of tile t-1
    // while its dP MFMAs run. Reads are issued whether or not the tile has
    // work for the group (every address is valid), which keeps the compiler's
    // LDS wait counting exact. Only the P wave's writes need an LDS wait before
    // the step's barrier; every other read is consumed before its stage is
    // refilled two steps later. (Phase A and B below name the two halves of
    // each wave's step.)
    int cr = 0, cq = first_tile(0);
    settle(cr, cq);
    // Per round of the compute cursor: the group has live pairs in tile cq
    // iff its first key is live for the tile's last row, i.e. iff
    // cq >= c_act; the tile is fully live for the group (every row in range
    // and the group's last key live for the tile's first row) iff
    // c_full_lo <= cq < c_full_hi.
    constexpr int kNever = 1 << 30;
    int c_delta = 0, c_act = kNever, c_full_lo = kNever;
    const int c_full_hi = kw0 + 31 < L ? L / KBQ : 0;
    auto c_enter = [&]() {
        c_delta = delta_of(cr);
        const int need = kw0 - c_delta + 1;   // the tile's last row must be at least this
        c_act = __builtin_amdgcn_readfirstlane(wave_live && need <= L - 1 ? max(need, 0) / KBQ : kNever);
        const int m = kw0 + 31 - c_delta;     // the tile's first row must exceed this
        c_full_lo = __builtin_amdgcn_readfirstlane(m < 0 ? 0 : m / KBQ + 1);
    };
    c_enter();
    int stg = 0, stg_prev = 0, stg_ld = DK_AHEAD;
    bool act_prev = false;
    f32x16 x;        // S of tile t (P wave) or dP of tile t-1 (dS wave)
    bf16x8 opb[2];   // P of tile t-1 (P wave) or dS of tile t-1 (dS wave), bf16 MFMA operand
    auto step_end = [&](int t, bool act) {
        if (t < n_tiles) {
            ++cq;
            if (settle(cr, cq)) c_enter();
        }
        act_prev = act;
        stg_prev = stg;
        stg = next_stage(stg);
        stg_ld = next_stage(stg_ld);
        ld_settle();
        if (w == kStWave)   // tile t+1 is in
            __builtin_amdgcn_s_waitcnt(kWaitVm12);
        else
            __builtin_amdgcn_s_waitcnt(kWaitVm8);
    };

    if (!ds_wave) {
        // dO^T of tile t-1 and P of tile t-1: the dV product runs every step,
        // on zero P when that tile had no work for the group (adding zero
        // products leaves dV as it is), so both start at zero.
        bf16x8 yt[2][4];
#pragma unroll
        for (int kk2 = 0; kk2 < 2; ++kk2) {
            opb[kk2] = bf16x8{};
#pragma unroll
            for (int db = 0; db < 4; ++db) yt[kk2][db] = bf16x8{};
        }
        for (int t = 0; t <= n_tiles; ++t) {
            const bool act = t < n_tiles && cq >= c_act;
            const bool ld_valid = t + DK_AHEAD < n_tiles;
            const int jq0 = cq * KBQ;
            // Phase A: Q rows and LSE of tile t read; dV^T += dO^T P (tile
            // t-1) with the step's three tile loads (into the stage of tile
            // t-2) and the loader's advance issued between its MFMAs; S of
            // tile t.
            bf16x8 xr[8];
            f32x4 lz[4];   // LSE log2 e of rows 8g + 4h2 .. +3
            read_rows(sm.q[stg], xr);
            {
                const float* stt = sm.st[stg];
#pragma unroll
                for (int g = 0; g < 4; ++g) lz[g] = *(const f32x4*)&stt[8 * g + 4 * h2];
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int kk2 = 0; kk2 < 2; ++kk2)
#pragma unroll
                for (int db = 0; db < 4; ++db) {
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(yt[kk2][db], opb[kk2], acc[db], 0, 0, 0);
                    __builtin_amdgcn_sched_barrier(0);
                    if (kk2 == 0 && db == 0) load_q(ld_valid, stg_ld);
                    if (kk2 == 0 && db == 1) load_do(ld_valid, stg_ld);
                    if (kk2 == 0 && db == 2) load_st(ld_valid, stg_ld);
                    if (kk2 == 0 && db == 3) ld_advance();
                    __builtin_amdgcn_sched_barrier(0);
                }
            if (act) x = rows_kv(xr);
            // Phase B: P of tile t, written for the dS wave; dO^T of tile t read.
            read_yt(sm.dout[stg], yt);
            __builtin_amdgcn_sched_barrier(0);
            if (act) {
                if (!(cq >= c_full_lo && cq < c_full_hi)) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int jj = jq0 + 8 * (i >> 2) + 4 * h2 + (i & 3);
                        if (!(jj < L && key_ok && kw < jj + c_delta)) x[i] = -INFINITY;
                    }
                }
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    f32x4 pq;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = 4 * g + e;
                        pq[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], sl, -lz[g][e]));
                        opb[i >> 3][i & 7] = (bf16)pq[e];
                    }
                    pex(t)[64 * g] = pq;
                }
            } else {
                opb[0] = bf16x8{};
                opb[1] = bf16x8{};
            }
            step_end(t, act);
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);   // P is in LDS
            bar();
        }
    } else {
        for (int t = 0; t <= n_tiles; ++t) {
            load_tile(t + DK_AHEAD < n_tiles, stg_ld);   // into the stage of tile t-2
            const bool act = t < n_tiles && cq >= c_act;
            // Phase A: dS of tile t-1 from P, dP and Delta; dO rows of tile t read.
            f32x4 pq[4], dz[4];
            bf16x8 xr[8];
            {
                const float* stp = sm.st[stg_prev];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    pq[g] = pex(t - 1)[64 * g];
                    dz[g] = *(const f32x4*)&stp[32 + 8 * g + 4 * h2];
                }
            }
            read_rows(sm.dout[stg], xr);
            __builtin_amdgcn_sched_barrier(0);
            if (act_prev) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    opb[i >> 3][i & 7] = (bf16)(pq[i >> 2][i & 3] * (x[i] - dz[i >> 2][i & 3]));
            }
            // Phase B: dP of tile t, dK^T += Q^T dS (tile t-1); the Q^T reads
            // land while the dP MFMAs run.
            bf16x8 yt[2][4];
            read_yt(sm.q[stg_prev], yt);
            __builtin_amdgcn_sched_barrier(0);
            if (act) x = rows_kv(xr);
            if (act_prev) acc_t(yt, opb);
            step_end(t, act);
            bar();
        }
    }
    __builtin_amdgcn_s_waitcnt(0);   // no load may still be writing LDS when the workgroup ends

    if (!key_ok) return;
    // dK carries the softmax scale once here (its dS operands leave it out).
    const float osc = ds_wave ? scale : 1.0f;
    bf16* outp = (bf16*)(ds_wave ? a.dk : a.dv) + krow * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int dcol = db * 32 + 8 * g + 4 * h2;
            const bf16x4 v4 = {(bf16)(acc[db][4 * g] * osc), (bf16)(acc[db][4 * g + 1] * osc),
                               (bf16)(acc[db][4 * g + 2] * osc), (bf16)(acc[db][4 * g + 3] * osc)};
            *(bf16x4*)(outp + dcol) = v4;
        }
}

}  // namespace

hipError_t launch_bwd_dkdv_bf16_d128(const BwdArgs& a, hipStream_t stream) {
    const int64_t nk = (a.L + KBM - 1) / KBM * a.H * a.N * a.B;
    if (nk == 0) return hipSuccess;
    hipLaunchKernelGGL(bwd_dkdv, dim3((unsigned)nk), dim3(DK_NT), 0, stream, a);
    return hipGetLastError();
}

}  // namespace sra
