/*
 * sra.h -- C ABI of libsra, striped ring attention for AMD MI355X (gfx950).
 *
 * The method ("Striped Attention: Faster Ring Attention for Causal
 * Transformers"; summary page at research.elamur.ai, "Summary" ¶1-2 and
 * "Key points"): exact causal attention computed by ring attention over N
 * devices, where each device holds either one contiguous chunk of the
 * sequence or -- the striped layout -- every N-th token, so that the causal
 * work per device is about equal in every ring round. Here the N ring
 * devices are simulated on one GPU: device d is a slice of one buffer and
 * "receiving a K/V block" in round r is reading the slice of device
 * (d - r) mod N.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Tensors are row-major [B, S, H, Dh] (batch, sequence, heads, head dim);
 * LSE tensors are fp32 [B, S, H]. A "row" of [B, S, H, Dh] is one
 * (b, s, h) triple with Dh contiguous values.
 *
 * Device layout: the ring entry points take and return tensors in device
 * layout, in which slot d*L + j (L = S / N) holds device d's j-th token:
 *   contiguous (SRA_LAYOUT_CONTIGUOUS): position d*L + j (original order);
 *   striped    (SRA_LAYOUT_STRIPED):    position j*N + d.
 * sra_stripe_permute converts original order to striped device layout once,
 * before the ring (the pages apply the permutation once, before the first
 * layer; "Key points: Striped layout"), and sra_unstripe converts back.
 * With desc->order = SRA_ORDER_ORIGINAL the ring entry points instead take
 * and return tensors in original token order and address device d's j-th
 * token at its position directly (row j*N + d when striped): the
 * permutation is folded into the kernels' row addressing and no permuted
 * copy exists. Results are bit-identical to the device-layout call followed
 * by sra_unstripe.
 *
 * Causality: key slot k of device s is live for query slot j of device d
 * when position(s, k) <= position(d, j) (diagonal included). Scores are
 * scale * q.k with scale = 1/sqrt(Dh) unless the descriptor gives one. LSE
 * is the natural log of the sum of exp(score) over live keys; a row with no
 * live key has O = 0 and LSE = -inf.
 *
 * Pointers: names ending in nothing are device pointers (HIP global memory)
 * unless the comment says "host". Device tensors must be 16-byte aligned and
 * densely packed. The caller owns every buffer; the library never allocates
 * or frees memory, never synchronises, and enqueues all device work on
 * `stream` (a hipStream_t; NULL = the null stream). Inputs are read-only.
 *
 * Errors: every function returns an int status (SRA_OK = 0). Arguments are
 * validated on the host before any HIP call, so an invalid call has no side
 * effect. sra_last_error() returns a message for the calling thread's most
 * recent failing call. A HIP launch error returns SRA_ERR_HIP.
 */
#ifndef SRA_H
#define SRA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SRA_ABI_VERSION 2

enum sra_status {
    SRA_OK = 0,
    SRA_ERR_INVALID_ARG = 1, /* null pointer, bad size, misalignment, out-of-range index */
    SRA_ERR_UNSUPPORTED = 2, /* valid request the library has no kernel for (dtype/head_dim) */
    SRA_ERR_HIP = 3,         /* a HIP call or kernel launch failed */
    SRA_ERR_WORKSPACE = 4    /* workspace missing or smaller than the query function says */
};

enum sra_layout { SRA_LAYOUT_CONTIGUOUS = 0, SRA_LAYOUT_STRIPED = 1 };
enum sra_dtype { SRA_DTYPE_F32 = 0, SRA_DTYPE_BF16 = 1 };
enum sra_order {
    SRA_ORDER_DEVICE = 0,   /* tensors in device layout (slot d*L + j) */
    SRA_ORDER_ORIGINAL = 1  /* tensors in original token order (slot = position) */
};
enum sra_schedule {
    SRA_SCHEDULE_PER_ROUND = 0, /* one kernel launch per ring round, LSE merge fused in its epilogue */
    SRA_SCHEDULE_FUSED = 1      /* all rounds in one launch, merged online (no partial traffic) */
};

/* Problem descriptor. Supported (dtype, head_dim): (BF16, 128), (F32, 64),
 * (F32, 128). bf16 inputs are multiplied on matrix cores with fp32
 * accumulation and fp32 softmax; fp32 inputs are computed in fp32. */
typedef struct sra_desc {
    int64_t batch;     /* B >= 1 */
    int64_t seq;       /* S >= 1, a multiple of n_dev */
    int64_t heads;     /* H >= 1 */
    int64_t head_dim;  /* Dh */
    int32_t n_dev;     /* N virtual ring devices, 1 <= N <= S */
    int32_t layout;    /* enum sra_layout */
    int32_t dtype;     /* enum sra_dtype: element type of q, k, v and o */
    int32_t schedule;  /* enum sra_schedule (sra_ring_attn_fwd only) */
    float scale;       /* softmax scale; 0 selects 1/sqrt(head_dim) */
    int32_t order;     /* enum sra_order: how q, k, v, o, lse (and gradients) are ordered */
} sra_desc;

/* Library ABI version (SRA_ABI_VERSION of the build). */
int sra_abi_version(void);

/* Static string naming a status code. */
const char* sra_status_str(int status);

/* Message for the calling thread's last failing call ("" if none). */
const char* sra_last_error(void);

/* ---------------------------------------------------------------- host ---
 * Host-only functions: they make no HIP call and need no GPU. */

/* perm[slot] = original position held by device-layout `slot`, for
 * slot in [0, seq) (host array of seq int64). Defines the layouts above
 * ("Summary" ¶2: every N-th token per device). */
int sra_stripe_index(int64_t seq, int32_t n_dev, int32_t layout, int64_t* perm);

/* Tile census of the ring (imbalance accounting; "Key points: Imbalance"
 * and the notes page at phantomic12.github.io ¶1: the slowest device sets
 * the pace of each round). Queries of each device are cut into tiles of
 * tile_q rows and keys of the source device into tiles of tile_k (ragged
 * last tiles allowed). A tile is FULL if all its pairs are live, PARTIAL if
 * some are, EMPTY if none; live = FULL + PARTIAL. Host arrays of N*N
 * int64 indexed [r*N + d] (round r, query device d); `full` and `partial`
 * may be NULL. Only seq, n_dev and layout of desc are read; counts are per
 * (b, h) pair (multiply by B*H for all heads). */
int sra_count_live_tiles(const sra_desc* desc, int64_t tile_q, int64_t tile_k,
                         int64_t* live, int64_t* full, int64_t* partial);

/* Live (query, key) pairs per (round, device), per (b, h): host array of
 * N*N int64 indexed [r*N + d]. Their sum is S(S+1)/2. */
int sra_count_live_pairs(const sra_desc* desc, int64_t* pairs);

/* The (query rows, keys) tile the ring-round kernel for this descriptor
 * processes per step; its device-side live counters count these tiles. */
int sra_kernel_tiles(const sra_desc* desc, int32_t* tile_q, int32_t* tile_k);

/* -------------------------------------------------------------- device ---*/

/* Gather into striped device layout: viewing x and y as [outer, seq, row]
 * with `row_bytes` bytes per row, y[o, d*L + j, :] = x[o, j*N + d, :].
 * Bit-exact copy; x and y must not overlap; row_bytes % 4 == 0 and
 * row_bytes <= 2^31; x and y 4-byte aligned (16-byte aligned with row_bytes
 * % 16 == 0 takes the 16-byte path). outer >= 1; seq and n_dev as in
 * sra_stripe_index. Errors: SRA_ERR_INVALID_ARG before any work is
 * enqueued; SRA_ERR_HIP if the launch fails. */
int sra_stripe_permute(const void* x, void* y, int64_t outer, int64_t seq,
                       int64_t row_bytes, int32_t n_dev, void* stream);

/* Inverse of sra_stripe_permute: x[o, j*N + d, :] = y[o, d*L + j, :]. */
int sra_unstripe(const void* y, void* x, int64_t outer, int64_t seq,
                 int64_t row_bytes, int32_t n_dev, void* stream);

/* Rotary position embedding of a model input (Q or K), fused with the stripe
 * gather. The pages stripe the inputs once, before the first layer
 * ("Summary" ¶2; "Key points: Striped layout"); they say nothing about
 * positional encodings, and a rotary encoding must see every token's
 * original position whatever slot the token lands in. Each head vector of the
 * token at original position t is rotated in "rotate half" form: pair
 * (c, c + D/2), c < D/2, turns by a_c = p * base^(-2c/D), with p = pos[b*S + t]
 * (device int64 [B, S] in original order) or p = t when pos is NULL:
 *   y_c = x_c cos a_c - x_{c+D/2} sin a_c,  y_{c+D/2} = x_c sin a_c + x_{c+D/2} cos a_c.
 * Angles are reduced modulo 2*pi in fp64 and evaluated in fp32; the rotation
 * is computed in fp32 and stored in the dtype (bf16 rounded to nearest even).
 * x: [B, S, H, D] in original order; y: same shape, in striped device layout
 * (slot d*L + j holds the token at j*N + d) when desc->order is
 * SRA_ORDER_DEVICE and the layout striped, else in original order (plain
 * rotary embedding; in that case y may equal x, any other overlap is an
 * error). Reads batch, seq, heads, head_dim, n_dev, layout, dtype and order of
 * desc; head_dim a multiple of 8 up to 256; base finite and > 1 (10000 is
 * the usual value). Token ids and any other per-token row are striped with
 * sra_stripe_permute. */
int sra_rope_permute(const sra_desc* desc, const void* x, void* y, const int64_t* pos, double base,
                     void* stream);

/* One ring round (round r in [0, N)) for query device `device` (or all
 * devices if device == -1): device d's queries attend to the K/V block of
 * device (d - r) mod N under the causal mask above, skipping tiles with no
 * live pair and masking only tiles that are partially live ("Summary" ¶1-2).
 * q, k, v: [B, S, H, Dh] in device layout (dtype of desc).
 * o_part: fp32 [B, S, H, Dh], lse_part: fp32 [B, S, H]; only the rows of the
 * selected device(s) are written, each normalised over this round's keys.
 * live_counts: NULL or device int64 [N*N] indexed [r*N + d]; the number of
 * kernel tiles (sra_kernel_tiles) processed is ADDED (all heads, batches).
 * desc->schedule is ignored. */
int sra_ring_round_attn(const sra_desc* desc, int32_t round, int32_t device,
                        const void* q, const void* k, const void* v,
                        float* o_part, float* lse_part, int64_t* live_counts,
                        void* stream);

/* Log-sum-exp merge of a partial result into an accumulator, in place,
 * over `rows` rows of `head_dim` fp32 values:
 *   M = max(lse_acc, lse_part); lse = M + log(exp(lse_acc-M) + exp(lse_part-M));
 *   o_acc = exp(lse_acc-lse) o_acc + exp(lse_part-lse) o_part.
 * A side with LSE = -inf contributes nothing; both -inf gives o = 0,
 * LSE = -inf. Passage: each device attends to one circulating K/V block per
 * round ("Summary" ¶1) and the ring computes attention exactly, not an
 * approximation of it (abstract, pith.science/paper/2311.09431; "Summary"
 * ¶2); softmax partial results over disjoint key
 * sets combine exactly by this rule, which is how the per-round results of
 * one device become its attention over every key.
 * o_acc, o_part: device fp32 [rows, head_dim], 16-byte aligned; lse_acc,
 * lse_part: device fp32 [rows]. o_acc/lse_acc are read and overwritten;
 * o_part/lse_part are read only and must not overlap them. head_dim a
 * power of two in [4, 256]; rows >= 0 (0 is a no-op). Errors:
 * SRA_ERR_INVALID_ARG for a null pointer, bad head_dim or misalignment (no
 * work enqueued); SRA_ERR_HIP if the launch fails. */
int sra_lse_merge(float* o_acc, float* lse_acc, const float* o_part,
                  const float* lse_part, int64_t rows, int64_t head_dim,
                  void* stream);

/* Bytes of workspace sra_ring_attn_fwd needs for desc (may be 0). */
size_t sra_fwd_workspace_bytes(const sra_desc* desc);

/* The whole ring forward: all N rounds for all N devices, merged.
 * Passage: "Summary" ¶1 (each device keeps its queries while the K/V blocks
 * travel around the ring, one block per round, until every device has met
 * every block; tiles that are entirely masked are skipped) and ¶2 (with the
 * striped layout every device does about half of each round's work, and the
 * result is exact). With SRA_SCHEDULE_PER_ROUND round r is one launch whose
 * epilogue merges into the running result (sra_lse_merge's rule); with
 * SRA_SCHEDULE_FUSED one launch walks every round per query tile and
 * carries the online softmax across rounds, visiting the source devices in
 * the same order on every device (only the rounding order differs).
 * q, k, v: [B, S, H, Dh] in device layout (dtype of desc);
 * o: [B, S, H, Dh] in device layout, dtype of desc (bf16 rounded to nearest
 * even); lse: fp32 [B, S, H]. workspace: device memory of at least
 * sra_fwd_workspace_bytes(desc) bytes (contents undefined on entry/exit).
 * live_counts: NULL or device int64 [N*N]; tiles are ADDED as above.
 * round_events: NULL, or a host array of hipEvent_t (passed as void*): with
 * SRA_SCHEDULE_PER_ROUND 2*N events bracketing each round's kernel, with
 * SRA_SCHEDULE_FUSED 2 events bracketing the one launch. For bf16 the
 * dispatch itself records them at the kernel's start and end; for fp32 they
 * are recorded on `stream` before and after the launch. A launch with no
 * work still records both. The events must have been created by the caller,
 * with timing enabled.
 * o, lse and the workspace are written while q, k, v are still read: none
 * of them may overlap q, k, v or one another (SRA_ERR_INVALID_ARG).
 * Errors: SRA_ERR_INVALID_ARG / SRA_ERR_UNSUPPORTED / SRA_ERR_WORKSPACE
 * before any work is enqueued; SRA_ERR_HIP if a launch fails. */
int sra_ring_attn_fwd(const sra_desc* desc, const void* q, const void* k,
                      const void* v, void* o, float* lse, void* workspace,
                      size_t workspace_bytes, int64_t* live_counts,
                      void* const* round_events, void* stream);

/* Bytes of workspace sra_ring_attn_bwd needs for desc: fp32 [B, H, S, 2],
 * per row the log2-scaled LSE and Delta = rowsum(dout * o). */
size_t sra_bwd_workspace_bytes(const sra_desc* desc);

/* Gradient of the ring forward: every round for every device, bf16 with
 * head_dim 128. Inputs in device layout: q, k, v, the forward's output o
 * (dtype of desc), its fp32 lse, and the upstream gradient dout. Outputs dq,
 * dk, dv (dtype of desc, device layout; fully overwritten). The pages train
 * causal transformers with the method ("Key points": A100 and TPU results),
 * which takes this pass: with P = exp(scale q.k - lse) on live pairs and
 * Delta = rowsum(dout * o), dv = P^T dout, ds = P (dout v^T - Delta),
 * dq = scale ds k, dk = scale ds^T q. In round r the K/V block of device s
 * meets the queries of device (s + r) mod N; dk and dv of a block sum over
 * rounds, dq of a device over the blocks it meets. Deterministic (no
 * atomics). workspace: at least sra_bwd_workspace_bytes(desc) bytes.
 * desc->schedule is ignored. Returns SRA_ERR_UNSUPPORTED for fp32. dq, dk,
 * dv and the workspace must not overlap any input or one another
 * (SRA_ERR_INVALID_ARG). */
int sra_ring_attn_bwd(const sra_desc* desc, const void* q, const void* k,
                      const void* v, const void* o, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv,
                      void* workspace, size_t workspace_bytes, void* stream);

/* sra_ring_attn_bwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). The per-row statistics go to an array
 * the library holds on each GPU it runs on (256 MiB, kept until the process
 * ends), so batch * seq * heads must be at most 33,554,432 rows; a larger
 * descriptor returns SRA_ERR_WORKSPACE before any work is enqueued. The
 * call makes no allocation; its first call on a device (the current device)
 * looks up the array's address there. Every call on one GPU uses that GPU's
 * one array: calls that overlap in time on the same GPU (other streams, other
 * threads) race and give undefined results; calls on one stream are
 * ordered. Arguments, results and errors are otherwise those of
 * sra_ring_attn_bwd (same kernels, bit-identical outputs). */
int sra_ring_attn_bwd_noalloc(const sra_desc* desc, const void* q,
                              const void* k, const void* v, const void* o,
                              const float* lse, const void* dout, void* dq,
                              void* dk, void* dv, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SRA_H */
