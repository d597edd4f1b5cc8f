// Ring-round causal attention kernels for gfx950 (CDNA4, wave64).
//
// One launch computes one ring round for a set of query devices: device d's
// queries attend to the K/V block of device s = (d - r) mod N (Striped
// Attention summary page, "Summary" ¶1: K/V blocks circulate around the
// ring). Tiles with no live pair are skipped and only partially live tiles
// are masked ("Summary" ¶1-2: with contiguous chunks a device's block in a
// round is either entirely live or entirely masked, while the striped layout
// leaves every device a near-triangular, roughly half-live block in each
// round). The mask is the shifted causal mask k < j + delta
// (see live_delta in sra_internal.h).
//
// The epilogue optionally merges the round's partial result into a running
// accumulator with the log-sum-exp rule (exact combination of partial
// softmax results over disjoint key sets) and, on the driver's last round,
// writes the output in the input dtype.
//
// bf16 kernel (Dh = 128): 8 wavefronts x 32 query rows = 256 rows per
// workgroup, 64 keys per step.
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: K is the A operand (32 keys x
//    16 dims from LDS), Q^T the B operand (held in registers for the whole
//    kernel). In the 32x32 accumulator a lane owns one query (column l%32)
//    and 16 keys, so a query's row max and row sum are in-lane reductions
//    plus one exchange between the two wave halves (v_permlane32_swap).
//  * O^T = V^T P^T on the same instruction: P^T comes straight from the S^T
//    accumulator registers (converted to bf16); the V^T operand is read from
//    the key-major V tile with ds_read_b64_tr_b16, which transposes 16-bit
//    elements across groups of 16 lanes, so each lane receives the keys its
//    P^T registers hold for one head dimension. The O^T accumulator keeps one
//    query per lane, so the softmax rescale is per-lane too.
//  * Softmax runs in the log2 domain with v_exp_f32. The running offset is
//    only raised when a tile's max exceeds it by more than 2^8 (the result
//    does not depend on the offset; it only bounds p <= 256), so the
//    64-register rescale of O is rare. The weights are taken against the
//    current offset first and the row max is only computed when some
//    lane's weights sum past 2^8 (which any weight past 2^8 implies), so
//    the common step has no max at all.
//  * K and V tiles go from HBM straight into a 4-stage LDS ring
//    (buffer_load ... lds, no register staging), K three tiles and V two
//    tiles ahead of the step that first reads them;
//    16-byte chunks are XOR-swizzled per row so both MFMA operand read
//    patterns are bank-conflict-free.
#include <hip/hip_ext.h>

#include <type_traits>

#include "kernel_common.h"

namespace sra {
namespace {

using namespace kc;

constexpr int kFlagMerge = 1;   // merge with (o_acc, lse_acc) instead of overwriting them
constexpr int kFlagFinal = 2;   // write the (merged) output to o_final in the input dtype

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

__device__ __forceinline__ Decoded decode_block(const RoundArgs& a, int64_t nqt, bool group_major = false) {
    // Query tile heavy_rank 0 is the device's last (most live keys).
    const WorkItem wi = decode_work(nqt, a.B, a.H, a.dev_hi - a.dev_lo, a.dev_lo, group_major);
    Decoded o;
    o.b = wi.b;
    o.h = wi.h;
    o.d = wi.d;
    o.qt = uniform_i64(nqt - 1 - wi.heavy_rank);
    o.s = uniform_i64((o.d - a.round + a.N) % a.N);
    o.delta = uniform_i64(live_delta(a.layout, a.N, a.L, o.d, o.s));
    return o;
}

// ---------------------------------------------------------------- bf16 ----

constexpr int D = 128;
constexpr int BM = kBf16TileQ;   // 256 query rows per workgroup: 8 wavefronts x 32
constexpr int BN = kBf16TileK;   // 64 keys per tile
constexpr int NT = 512;          // 8 wavefronts in two groups of 4: one wave of each group per SIMD
constexpr int NS = 4;             // K/V tile stages in LDS
constexpr float kTau = 8.0f;     // lazy-rescale threshold (log2 units)
constexpr float kSumCap = 256.0f;  // 2^kTau: a lane's weights sum past this only if one of them does

static_assert(BM == 256 && BN == 64 && NT == 512 && D == 128, "thread mappings below assume these");

// K and V tiles, key-major (256-byte rows, no padding: the loads write LDS
// directly), with the 16-byte chunks of each row XOR-swizzled so that the
// MFMA operand reads are bank-conflict-free:
//   K: chunk c of key row r sits in slot c ^ (r & 15)
//   V: chunk c of key row r sits in slot c ^ (4 * (r & 3))
struct __align__(16) SmemBf16 {
    bf16 k[NS][BN * D];
    bf16 v[NS][BN * D];
};

constexpr int kWaitVm4 = 0x0F74;   // vmcnt(4)
constexpr int kWaitVm8 = 0x0F78;   // vmcnt(8)

// Walks the (round, key tile) pairs one workgroup visits: the rounds
// r_lo .. r_hi-1 (see RoundGeom for their order), and within a round the key
// tiles of the source device that hold at least one live key for the
// workgroup's last query row. All fields are wave-uniform.
struct TileCursor {
    int r, kt, nt;        // walk step, key tile within its round, tiles in the round
    int s, delta;         // source device of the round, live-key shift
};

struct RoundGeom {
    int L, N, layout, d, j_last, r_hi;
    int slab_walk;   // 1: step c.r of the walk visits source device s = c.r
    // Enter step c.r of the walk. In ring order (one launch per round) step
    // r is round r, whose source is s = (d - r) mod N, found with 32-bit
    // scalar arithmetic and no division (0 <= d, r < N). The all-rounds
    // launch visits the sources in the same order on every device instead
    // (step u: source u, i.e. round (d - u) mod N): at any moment the
    // workgroups of all devices of a head then read the same K/V slab, which
    // they share through L2, while in ring order they would read N different
    // slabs. The rounds' partial results combine the same way in any order
    // (the log-sum-exp merge is exact), so only rounding differs.
    // The shift is only ever used through live32(j, delta, L) with
    // 0 <= j < L, so with a contiguous layout it is reduced to what that
    // sees: a source after d has no live key for any query (-L-1), one before
    // d has all of them (L+1), and s = d is the causal block (1).
    __device__ __forceinline__ void enter(TileCursor& c) const {
        int s = c.r;
        if (!slab_walk) {
            s = d - c.r;
            if (s < 0) s += N;
        }
        const int dl = layout == 1 ? (s <= d ? 1 : 0) : (s == d ? 1 : (s < d ? L + 1 : -L - 1));
        c.s = __builtin_amdgcn_readfirstlane(s);
        c.delta = __builtin_amdgcn_readfirstlane(dl);
        c.nt = __builtin_amdgcn_readfirstlane((int)((unsigned)(live32(j_last, c.delta, L) + BN - 1) / BN));
        c.kt = 0;
    }
    // Move to the first tile at or after the cursor's position.
    __device__ __forceinline__ void settle(TileCursor& c) const {
        while (c.kt >= c.nt && c.r + 1 < r_hi) {
            ++c.r;
            enter(c);
        }
    }
    __device__ __forceinline__ void advance(TileCursor& c) const {
        ++c.kt;
        settle(c);
    }
};

// kFused = false: one ring round per launch (a.round), with the epilogue
//   writing, merging or finishing per a.mode.
// kFused = true: all N rounds in one launch, visiting the source devices in
//   the same order on every device (RoundGeom); the online softmax carries the
//   running (O, max, sum) across rounds, which is the log-sum-exp merge of
//   the per-round partial results, and the epilogue writes the output.
//
// Schedule: the tile sequence runs in steps, one workgroup barrier per step.
// X(t) is a wave's MFMA work -- O += P V for tile t-1, then S = K Q^T for
// tile t -- and Y(t) its softmax of tile t on the vector ALU. In step t group
// 0 runs X(t) then Y(t), and group 1 runs Y(t-1) then X(t). Waves w and w+4
// share a SIMD, so every step starts with one wave of each SIMD on the MFMA
// unit and the other on the vector ALU, and the two swap roles half-way; the
// wave in X runs at raised issue priority. Group 0 loads K three tiles ahead
// (in Y(t), K(t+3)), group 1 V two tiles ahead (at the start of its step,
// V(t+2)). The loop body holds four steps, one per LDS stage, so that every
// stage offset is a compile-time immediate.
template <bool kFused>
__global__ void __launch_bounds__(NT, 1) round_fwd_bf16_d128(RoundArgs a, int flags) {
    __shared__ SmemBf16 sm;

    const int64_t nqt = (a.L + BM - 1) / BM;
    // One launch per round: every device of a head reads a different source
    // slab, so with enough query tiles per device the workgroups go group by
    // group (shared slab per XCD). With few tiles per device the interleaved
    // heaviest-first order packs the CUs better. The all-rounds launch keeps
    // the interleaved order: there all devices of a head read the same slab.
    const Decoded blk = decode_block(a, nqt, !kFused && nqt >= 16);
    const int L = (int)a.L;   // the host bounds L * H * D so that in-slab offsets fit in 32 bits
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, c32 = lane & 31, h2 = lane >> 5;
    const int grp = w >> 2;

    const int j0 = (int)blk.qt * BM;
    const int j1 = min(j0 + BM, L);
    const int d = (int)blk.d;
    const RoundGeom geo{L, a.N, a.layout, d, j1 - 1, kFused ? a.N : a.round + 1, kFused ? 1 : 0};

    // Tiles per round; device-side live-tile census.
    int n_tiles = 0;
    {
        TileCursor c;
        for (c.r = kFused ? 0 : a.round; c.r < geo.r_hi; ++c.r) {
            geo.enter(c);
            n_tiles += c.nt;
            if (a.live_counts != nullptr && tid == 0 && c.nt > 0)
                atomicAdd((unsigned long long*)&a.live_counts[(int64_t)(c.s <= d ? d - c.s : d - c.s + a.N) * a.N + d],
                          (unsigned long long)c.nt);
        }
    }
    if (!kFused && n_tiles == 0 && (flags & kFlagMerge) && !(flags & kFlagFinal)) return;   // merging nothing

    const int rs = (int)(a.H * D);   // elements between consecutive slots
    const int row_bytes = rs * 2;
    // Device t's j-th token sits at slot mem_slot(t, j): consecutive tokens of
    // a device are rstep slots (rstride bytes) apart.
    const bool strided = a.strided != 0;
    const int64_t rstep = strided ? a.N : 1;
    const int rstride = (int)rstep * row_bytes;   // the host bounds a key tile's span below 2^31
    const bf16* __restrict__ qp0 =
        (const bf16*)a.q + ((blk.b * a.S + mem_slot(strided, a.N, a.L, blk.d, 0)) * a.H + blk.h) * D;
    // Device s's tokens of this (b, h) start at kv_head + slot_bytes(s).
    const uint64_t kv_head_k = uniform_u64((uint64_t)((const bf16*)a.k + (blk.b * a.S * a.H + blk.h) * D));
    const uint64_t kv_head_v = uniform_u64((uint64_t)((const bf16*)a.v + (blk.b * a.S * a.H + blk.h) * D));
    auto slot_bytes = [&](int s) { return (uint64_t)mem_slot(strided, a.N, a.L, s, 0) * (uint64_t)row_bytes; };
    const int64_t span_bytes = (int64_t)(L - 1) * rstride + D * 2;   // first to last token of a device

    // This wave's 32 rows and live-key bounds (live keys of a row form a prefix).
    const int jw0 = j0 + w * 32;
    const int j = jw0 + c32;
    const bool row_ok = j < L;
    const bool wave_live = jw0 < L;
    const int jw_last = min(jw0 + 31, L - 1);

    // Q^T operand: lane holds query c32, dims kk*16 + 8*h2 .. +7. Rows past
    // the end read a valid row; they are fully masked and never written.
    bf16x8 qreg[8];
    {
        const bf16x8* qp = (const bf16x8*)(qp0 + (int64_t)min(j, L - 1) * rstep * rs) + h2;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) qreg[kk] = qp[2 * kk];
        // Let the Q loads land before any K/V load is issued: later waits on
        // the K/V prefetch then never hold up the MFMAs that read Q.
        __builtin_amdgcn_s_waitcnt(0);
    }

    f32x16 oacc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db) oacc[db] = f32x16{};
    // Running offset (log2 domain), equal in both halves. Rows past the end
    // are fully masked; they start at offset 0 so they never ask for the max.
    float m_run = row_ok ? -INFINITY : 0.f;
    float l_part = 0.f;        // this half's share of the row sum
    float neg_m = 0.f;         // minus the offset the weights are taken against (0 while it is unset)
    bool rows_set = false;     // every row of the wave has an offset (wave-uniform)
    const float sl = a.scale_log2;

    // K/V staging: each tile is loaded straight into LDS (buffer_load ...
    // lds: lane l of an instruction writes bytes [16 l, 16 l + 16) after the
    // instruction's LDS base, from any global address the lane names). Group 0
    // loads K tiles and group 1 V tiles; wave wg of a group issues four
    // instructions per tile, instruction q covering key rows 4 wg + 16 q .. +3.
    // Lane l writes key row 4 wg + 16 q + l/16, LDS slot l % 16, so it loads
    // the global chunk that the slot holds under the swizzle. Each tile gets
    // its own buffer resource (base at the tile's first row, size cut to what
    // is left of the slab): the lane offsets are loop-invariant and rows past
    // the slab end are not read (their scores are masked and their V rows get
    // weight 0; LDS is zeroed once at the start so such rows hold finite data).
    const int wg = w & 3;
    const int ld_row = 4 * wg + (lane >> 4);
    const int ld_sw = grp == 0 ? (ld_row & 15) : 4 * (lane >> 4);
    const int ld_voff = ld_row * rstride + 16 * ((lane & 15) ^ ld_sw);
    const int ld_step = 16 * rstride;
    const uint64_t ld_head = uniform_u64(grp == 0 ? kv_head_k : kv_head_v);
    bf16* const ld_lds0 = (grp == 0 ? &sm.k[0][0] : &sm.v[0][0]) + 512 * wg;

    auto load_tile = [&](const TileCursor& c, bool valid, int stage) {
        const int64_t tile_off = (int64_t)c.kt * BN * rstride;
        const int64_t left64 = span_bytes - tile_off;
        const int left = (valid && left64 > 0) ? (int)min(left64, (int64_t)BN * rstride) : 0;
        const uint64_t base = ld_head + slot_bytes(c.s) + (uint64_t)tile_off;
        const i32x4 rsrc = raw_rsrc(base, left);
        const uint32_t dst = lds_addr(ld_lds0 + stage * (BN * D));
#pragma unroll
        for (int q = 0; q < 4; ++q) load_lds_b128(rsrc, ld_voff + q * ld_step, dst + 4096 * q);
    };

    // S^T = K Q^T over the K tile in `stage`: sacc[kb] holds keys
    // kb*32 .. kb*32+31 of the tile against this wave's 32 queries. Lane
    // (c32, h2) reads chunk 2 kk + h2 of key row 32 kb + c32.
    f32x16 sacc[2];
    auto compute_s = [&](int stage) {
        const bf16* ks = sm.k[stage] + c32 * D;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
            const int slot = (2 * kk + h2) ^ (c32 & 15);
            const bf16x8 k0f = *(const bf16x8*)(ks + 8 * slot);
            const bf16x8 k1f = *(const bf16x8*)(ks + 32 * D + 8 * slot);
            sacc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0f, qreg[kk], kk == 0 ? f32x16{} : sacc[0], 0, 0, 0);
            sacc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1f, qreg[kk], kk == 0 ? f32x16{} : sacc[1], 0, 0, 0);
        }
    };

    // O^T += V^T P^T over the V tile in `stage`, after applying the pending
    // rescale of O (rare: only when the running offset was raised).
    // The V^T operand comes from the key-major tile through ds_read_b64_tr_b16:
    // within each 16-lane group, lane i receives element i % 4 of the 8-byte
    // pieces named by lanes 4v + i / 4 (v = 0..3). Lane (g = l / 16, j = l % 16)
    // names key 16 kk + 8 rd + 4 (g / 2) + j / 4, dims 32 db + 16 (g % 2) +
    // 4 (j % 4) .. +3, so lane l collects dim 32 db + l % 32 of keys
    // 16 kk + 8 rd + 4 h2 + 0..3 -- the keys its P^T registers hold
    // (16-key step kk uses keys 16 kk + [4 h2 .. 4 h2 + 3] and
    // 16 kk + 8 + [4 h2 .. 4 h2 + 3] of the S^T accumulator).
    bf16x8 pop[2][2];
    bool resc = false;
    float alpha_p = 1.f;
    const int tg = lane >> 4, tj = lane & 15;
    const int tr_row = 4 * (tg >> 1) + (tj >> 2);
    const int tr_lo = 8 * (2 * (tg & 1) + ((tj & 3) >> 1)) + 4 * (tj & 1);   // element offset in the slot group
    auto compute_pv = [&](int stage) {
        if (resc) {
#pragma unroll
            for (int db = 0; db < 4; ++db) oacc[db] *= alpha_p;
        }
        const bf16* vs = sm.v[stage] + tr_row * D + tr_lo;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            bf16x8 vf[4];
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                const bf16* p = vs + 32 * (db ^ (tj >> 2)) + kk * 16 * D;
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(SRA_LDS4(p));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(SRA_LDS4(p + 8 * D));
                const s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                vf[db] = __builtin_bit_cast(bf16x8, both);
            }
#pragma unroll
            for (int db = 0; db < 4; ++db)
                oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[db], pop[kk >> 1][kk & 1], oacc[db], 0, 0, 0);
        }
    };

    // Softmax of the tile at cursor c: mask (only if not fully live for the
    // wave's first row), row max, lazy rescale, p = 2^(s*scale*log2e - m),
    // fp32 row sum, bf16 P^T operands.
    auto softmax = [&](const TileCursor& c) {
        const int k0 = c.kt * BN;
        const int live_first = live32(jw0, c.delta, L);   // fewest live keys of the wave's rows
        if (k0 + BN > live_first) {
            const int lim = (row_ok ? live32(j, c.delta, L) : 0) - k0 - 4 * h2;
            // The first 32 keys need no mask when every row of the wave has them.
            if (k0 + 32 > live_first) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (8 * (i >> 2) + (i & 3) >= lim) sacc[0][i] = -INFINITY;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (8 * (i >> 2) + (i & 3) + 32 >= lim) sacc[1][i] = -INFINITY;
        }
        // Weights against the current offset first. Only when some weight of
        // the wave exceeds 2^kTau (its lane's partial sum then does too), or
        // some row of the wave has no offset yet, does the wave take the exact
        // path below: the row max, the raised offset and the weights again.
        // Otherwise the offset stays, exactly as the max test would have
        // decided.
        float ls0, ls1;
        auto weights = [&]() {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[0][i], sl, neg_m));
                const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[1][i], sl, neg_m));
                ls0 = i == 0 ? p0 : ls0 + p0;
                ls1 = i == 0 ? p1 : ls1 + p1;
                pop[0][i >> 3][i & 7] = (bf16)p0;
                pop[1][i >> 3][i & 7] = (bf16)p1;
            }
        };
        weights();
        resc = false;
        if (!rows_set || __builtin_amdgcn_ballot_w64(!(ls0 + ls1 <= kSumCap)) != 0) {
            float mx = fmaxf(fmaxf(sacc[0][0], sacc[1][0]), sacc[0][1]);
#pragma unroll
            for (int i = 1; i < 15; i += 2) mx = fmaxf(fmaxf(mx, sacc[1][i]), fmaxf(sacc[0][i + 1], sacc[1][i + 1]));
            mx = fmaxf(fmaxf(mx, sacc[1][15]), sacc[0][15]);
            const float m_tile = halves_max(mx) * sl;   // raw max times scale (> 0 keeps the order)
            const bool need = m_tile > m_run + kTau;
            // The O rescale this implies is applied in the next MFMA phase, just
            // before this tile's P V is accumulated (keeps O's registers in place).
            resc = __builtin_amdgcn_ballot_w64(need) != 0;
            const float m_new = need ? fmaxf(m_run, m_tile) : m_run;
            alpha_p = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
            l_part *= alpha_p;
            m_run = m_new;
            neg_m = (m_run == -INFINITY) ? 0.f : -m_run;
            rows_set = __builtin_amdgcn_ballot_w64(m_run == -INFINITY) == 0;
            weights();
        }
        l_part += ls0 + ls1;
    };

    // Does this wave have a live key in the tile at cursor c?
    auto wave_active = [&](const TileCursor& c) {
        return wave_live && c.kt * BN < live32(jw_last, c.delta, L);
    };

    TileCursor c0;
    c0.r = kFused ? 0 : a.round;
    geo.enter(c0);
    geo.settle(c0);
    TileCursor c1 = c0;
    geo.advance(c1);
    TileCursor c2 = c1;
    geo.advance(c2);
    // Group 0 loads K three tiles ahead, group 1 V two tiles ahead.
    TileCursor ld = c1;
    if (grp == 0) geo.advance(ld);
    geo.advance(ld);

    // Zero the stages once (rows past a slab end are never loaded), then put
    // K(0..2) and V(0..1) in flight and wait for K(0). V(0) is first read in
    // step 1; group 1 waits for it in step 0.
    {
        u32x4* z = (u32x4*)&sm;
        for (int i = tid; i < (int)(sizeof(SmemBf16) / 16); i += NT) z[i] = u32x4{0u, 0u, 0u, 0u};
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        bar();
    }
    load_tile(c0, n_tiles > 0, 0);
    load_tile(c1, n_tiles > 1, 1);
    if (grp == 0) {
        load_tile(c2, n_tiles > 2, 2);
        __builtin_amdgcn_s_waitcnt(kWaitVm8);
    }
    bar();

    // Main loop, step t (tile t's K is read in step t, its V in step t+1).
    // Loads: group 0 starts K(t+3) into the stage of tile t-1, whose K was
    // last read in step t-1; group 1 starts V(t+2) into the stage of tile
    // t-2, whose V was last read in step t-1. Before that each waits for the
    // oldest of its two tiles in flight (K(t+1), V(t)), which the next step
    // reads. Every wave drains its LDS reads before the step's barrier, so a
    // stage is never refilled while read, and a tile is complete before the
    // barrier that precedes its first use. The cursor of the next tile and
    // whether this wave is active in it are worked out next to the softmax,
    // off the MFMA work.
    TileCursor cur = c0;
    bool act_prev = false;
    bool act = n_tiles > 0 && wave_active(cur);
    // One step; kSt = t mod NS is a compile-time constant (the loop below runs
    // NS steps per iteration), so every LDS stage offset is an immediate.
    auto step = [&](int t, auto kst) {
        constexpr int kSt = decltype(kst)::value;
        if (grp == 1) {
            if (t > 0) {
                if (act_prev) softmax(cur);
                geo.advance(cur);
                act = t < n_tiles && wave_active(cur);
            }
            __builtin_amdgcn_s_waitcnt(kWaitVm4);
            load_tile(ld, t + 2 < n_tiles, (kSt + 2) & (NS - 1));
            geo.advance(ld);
        }
        __builtin_amdgcn_s_setprio(1);
        if (act_prev) compute_pv((kSt + NS - 1) & (NS - 1));
        if (act) compute_s(kSt);
        __builtin_amdgcn_s_setprio(0);
        if (grp == 0) {
            if (t < n_tiles) {
                if (act) softmax(cur);
                act_prev = act;
                geo.advance(cur);
                act = t + 1 < n_tiles && wave_active(cur);
                __builtin_amdgcn_s_waitcnt(kWaitVm4);
                load_tile(ld, t + 3 < n_tiles, (kSt + 3) & (NS - 1));
                geo.advance(ld);
            }
        } else {
            act_prev = act;
        }
        if (t == n_tiles) return true;
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        bar();
        return false;
    };
    static_assert(NS == 4, "the loop below runs one step per stage");
    for (int t = 0;; t += NS) {
        if (step(t, std::integral_constant<int, 0>{})) break;
        if (step(t + 1, std::integral_constant<int, 1>{})) break;
        if (step(t + 2, std::integral_constant<int, 2>{})) break;
        if (step(t + 3, std::integral_constant<int, 3>{})) break;
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_waitcnt(0);   // no load may still be writing LDS when the workgroup ends

    // Finish the row: l = both halves' sums; O = O / l; lse in natural log.
    const float l_tot = halves_sum(l_part);
    const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
    const float lse_b = l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
    if (!row_ok) return;

    const int64_t row = (blk.b * a.S + mem_slot(strided, a.N, a.L, blk.d, j)) * a.H + blk.h;   // (b, slot, h) row
    float wa = 0.f, wb = 1.f, l_out = lse_b;
    if (!kFused && (flags & kFlagMerge)) {
        const float la = a.lse_acc[row];
        merge_weights(la, lse_b, wa, wb, l_out);
    }
    wb *= inv;   // fold the normalisation into the partial's weight
    float* oa = a.o_acc + row * D;
    const bool final_out = kFused || (flags & kFlagFinal);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int dcol = db * 32 + 8 * g + 4 * h2;
            f32x4 ob = {oacc[db][4 * g], oacc[db][4 * g + 1], oacc[db][4 * g + 2], oacc[db][4 * g + 3]};
            f32x4 r = f32x4{0.f, 0.f, 0.f, 0.f};
            if (wb != 0.f) r = wb * ob;
            if (!kFused && (flags & kFlagMerge) && wa != 0.f) r += wa * *(const f32x4*)(oa + dcol);
            if (final_out) {
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
    const bool strided = a.strided != 0;
    const int64_t row_stride = (strided ? a.N : 1) * H * DH;   // between consecutive keys of a device
    const int64_t kv_base = ((blk.b * S + mem_slot(strided, a.N, L, blk.s, 0)) * H + blk.h) * DH;
    const int64_t j = j0 + lane;
    const bool row_ok = j < L;
    const int64_t c_row = row_ok ? live_keys(j, blk.delta, L) : 0;
    const int64_t row = (blk.b * S + mem_slot(strided, a.N, L, blk.d, row_ok ? j : 0)) * H + blk.h;

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

hipError_t launch_round_bf16_d128(const RoundArgs& a, bool fused, hipStream_t stream, hipEvent_t start,
                                  hipEvent_t stop) {
    const int64_t nqt = (a.L + BM - 1) / BM;
    const int64_t blocks = nqt * a.H * (a.dev_hi - a.dev_lo) * a.B;
    if (blocks == 0) {
        // Nothing to launch: the events still mark this point of the stream.
        if (start != nullptr) {
            const hipError_t e = hipEventRecord(start, stream);
            if (e != hipSuccess) return e;
        }
        return stop != nullptr ? hipEventRecord(stop, stream) : hipSuccess;
    }
    // With events, the dispatch itself records them at the kernel's start and
    // end (no separate marker packets around the launch).
    const dim3 grid((unsigned)blocks), block(NT);
    if (start != nullptr || stop != nullptr) {
        if (fused)
            hipExtLaunchKernelGGL(round_fwd_bf16_d128<true>, grid, block, 0, stream, start, stop, 0, a, 0);
        else
            hipExtLaunchKernelGGL(round_fwd_bf16_d128<false>, grid, block, 0, stream, start, stop, 0, a, flags_of(a));
    } else if (fused) {
        hipLaunchKernelGGL(round_fwd_bf16_d128<true>, grid, block, 0, stream, a, 0);
    } else {
        hipLaunchKernelGGL(round_fwd_bf16_d128<false>, grid, block, 0, stream, a, flags_of(a));
    }
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
