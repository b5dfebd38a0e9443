/*
 * pasa_attn.h -- C ABI of the PASA forward pass for AMD Instinct MI355X (gfx950).
 *
 * The operation.  "Online Pseudo-average Shifting Attention (PASA) for Robust
 * Low-precision LLM Inference", Abstract: PASA computes attention
 *     O = softmax(scale * Q K^T) V
 * blockwise, Flash-Attention style, with the score tiles, the exponentials and
 * the running softmax statistics held in half precision.  Each key block's
 * scores are shifted by a per-row pseudo-average (online pseudo-average
 * shifting) so the half-precision tile stays below the fp16 maximum 65504, and
 * an epilogue (global recovering) re-applies the removed shifts so the softmax
 * normalisation and the log-sum-exp are exact up to rounding.  The result is
 * mathematically equivalent to plain softmax attention.
 *
 * Conventions shared by every entry point
 *  - Pointers are DEVICE pointers (HIP global memory) unless stated otherwise.
 *    The caller owns every buffer.  The library allocates nothing, never
 *    synchronises, keeps no global state (each host thread only remembers its
 *    last prefill shape's item-shape choice) and is safe to call from several
 *    host threads on different streams.
 *  - Work is enqueued on `stream` (0 = the null stream) and runs asynchronously;
 *    the return code reports argument validation and launch errors only.
 *  - Element types: q, k, v, o are IEEE binary16 (fp16); lse is fp32.
 *  - Layout: contiguous BSHD.  q, o are [batch, seqlen_q, num_heads_q, head_dim];
 *    k, v are [batch, seqlen_kv, num_heads_q / gqa_group, head_dim];
 *    lse is [batch, num_heads_q, seqlen_q].  Query head h reads key/value head
 *    h / gqa_group.
 *  - lse holds ln(sum_j exp(softmax_scale * q_i . k_j)) over the visible keys,
 *    natural logarithm; a row with no visible key gets o = 0 and lse = -inf.
 *  - Causal masking is aligned to the bottom-right corner: key j is visible to
 *    query i iff j <= i + seqlen_kv - seqlen_q.
 *  - On any error nothing is enqueued and no output byte is written.
 *  - Supported: head_dim 64 or 128; num_heads_q % gqa_group == 0; any
 *    batch >= 1 and sequence lengths from 1 to 2^31 - 512 (ragged tails are
 *    masked), within the per-call limits each entry point lists.  The running
 *    softmax sum is an fp16 (hi, lo) pair over each segment of 32768 keys, and
 *    the completed segments' sums are carried in fp32, so the key count has no
 *    fp16 bound.
 */
#ifndef PASA_ATTN_H
#define PASA_ATTN_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PASA_OK = 0,
    PASA_ERR_INVALID = -1,     /* null pointer, non-positive size, bad GQA group */
    PASA_ERR_UNSUPPORTED = -2, /* valid but outside what the kernels implement */
    PASA_ERR_WORKSPACE = -3,   /* decode workspace missing or too small */
    PASA_ERR_HIP = -4          /* the HIP runtime reported a launch error */
} pasa_status;

/*
 * PASA prefill / full forward pass ("Online Pseudo-average Shifting Attention
 * (PASA) ...", Abstract: online pseudo-average shifting, half-precision
 * softmax, global recovering).
 *   q, k, v   device, fp16, layouts above.       o   device, fp16, written.
 *   lse       device fp32 [B,Hq,Sq], written; may be NULL (not computed).
 *   softmax_scale  multiplies q.k before the softmax (e.g. 1/sqrt(head_dim)).
 *   causal    0 or 1 (bottom-right aligned).
 * Errors: PASA_ERR_INVALID for a null q/k/v/o, a size < 1, a causal flag
 * other than 0 or 1, or num_heads_q % gqa_group != 0; PASA_ERR_UNSUPPORTED
 * for head_dim not in {64,128}, a sequence length above 2^31 - 512, a
 * non-finite or non-positive softmax_scale, sizes whose element count
 * overflows 64-bit indexing, one head's K or V slab of one sequence above
 * 4 GiB (seqlen_kv * (num_heads_q / gqa_group) * head_dim * 2 bytes), or more
 * than 2^31 - 1 work items of 256 query rows of one head (batch * num_heads_q *
 * ceil(seqlen_q / 256)).
 */
int pasa_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                  int batch, int seqlen_q, int seqlen_kv, int num_heads_q, int gqa_group,
                  int head_dim, float softmax_scale, int causal, hipStream_t stream);

/*
 * PASA forward with all of the per-row bookkeeping in fp16 ("Online
 * Pseudo-average Shifting Attention (PASA) ...", Abstract: the Flash-Attention
 * process runs in half precision throughout).  pasa_attn_fwd keeps the
 * running maximum R and the block offset in fp32 and everything tile-shaped
 * (scores, exponentials, block maxima and sums, rescale factors) plus the
 * running sum in fp16; this variant also rounds R and the offset to fp16 where
 * they are formed.  It is exposed so that its error can be measured beside the
 * default.  Usable while |softmax_scale * q.k| * log2(e) stays below about
 * 3.2e4: beyond that the fp16 rounding of R (a step of 16 there) lets the
 * exponentials of a block exceed 1 by up to 2^8 and the fp16 running sum can
 * overflow.  Arguments, layouts and errors as pasa_attn_fwd.
 */
int pasa_attn_fwd_strict(const void* q, const void* k, const void* v, void* o, float* lse,
                         int batch, int seqlen_q, int seqlen_kv, int num_heads_q, int gqa_group,
                         int head_dim, float softmax_scale, int causal, hipStream_t stream);

/*
 * PASA forward with 8-bit queries and keys: q and k hold OCP fp8 e4m3 values
 * (1 byte each, largest finite 448, no infinities) with one dequantisation
 * scale per tensor, v stays fp16.  The score is
 *     S_ij = q_scale * k_scale * sum_d q8_id * k8_jd
 * formed on the fp8 matrix cores with fp32 accumulation; everything after the
 * score -- the pseudo-average shift, the fp16 tile, exponentials, statistics,
 * P V and the epilogue -- is pasa_attn_fwd's.  The method's fp16 range
 * argument ("Online Pseudo-average Shifting Attention (PASA) ...", Abstract:
 * overflow above 65504) is unchanged: the dot products of e4m3 inputs can
 * still exceed it.  Producing the e4m3 inputs (rounding, saturation, scale
 * choice) is the caller's.
 *   q  device e4m3 [batch, seqlen_q, num_heads_q, head_dim]
 *   k  device e4m3 [batch, seqlen_kv, num_heads_q / gqa_group, head_dim]
 *   v, o, lse, softmax_scale, causal, stream: as pasa_attn_fwd.
 *   q_scale, k_scale  positive finite dequantisation factors.
 * Errors: as pasa_attn_fwd, plus PASA_ERR_UNSUPPORTED for a non-positive or
 * non-finite q_scale, k_scale or product with softmax_scale.
 */
int pasa_attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                      int batch, int seqlen_q, int seqlen_kv, int num_heads_q, int gqa_group,
                      int head_dim, float softmax_scale, float q_scale, float k_scale, int causal,
                      hipStream_t stream);

/*
 * Naive fp16 Flash-Attention forward: the same blockwise kernel WITHOUT the
 * pseudo-average shift.  The unscaled score tile QK^T is rounded to fp16 and
 * then multiplied by the scale in fp16, as a plain half-precision Flash
 * Attention would; scores above 65504 become +-inf and the output turns to
 * inf/NaN.  It exists to exhibit the overflow the PASA page describes
 * ("Online Pseudo-average Shifting Attention (PASA) ...", Abstract: overflow
 * above 65504 caused by a large sequence-dimension bias and by query/key
 * resonance).  Arguments, layouts and errors as pasa_attn_fwd.
 */
int pasa_naive_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                        int batch, int seqlen_q, int seqlen_kv, int num_heads_q,
                        int gqa_group, int head_dim, float softmax_scale, int causal,
                        hipStream_t stream);

/*
 * Split-KV decode: one query token per sequence against a KV cache.
 * The keys [0, seqlen_kv) are cut into num_splits contiguous ranges; each range
 * yields a normalised partial (o_s, lse_s) computed with the PASA tile numerics,
 * and a combine step merges them.  Partials over disjoint key ranges compose
 * exactly once each is re-weighted by its own log-sum-exp ("Block Sparse Flash
 * Attention" topic page, FoldAttention card: softmax is invariant to a common
 * shift; additive partials compose split KV).
 *   q        device fp16 [batch, 1, num_heads_q, head_dim]
 *   k_cache, v_cache  device fp16 [batch, seqlen_kv, num_heads_q/gqa_group, head_dim]
 *   o        device fp16 [batch, 1, num_heads_q, head_dim], written
 *   lse      device fp32 [batch, num_heads_q], written; may be NULL
 *   num_splits  >= 1, or 0 to let the library choose (pasa_attn_decode_splits).
 *   workspace   device memory of at least
 *               pasa_attn_decode_workspace_bytes(batch, num_heads_q, head_dim, n)
 *               bytes (n = the split count actually used), 256-byte aligned.
 *               It holds the fp32 partials: o_part [batch, num_heads_q, n, head_dim]
 *               followed, at the next 256-byte boundary, by
 *               lse_part [batch, num_heads_q, n].  Its contents on return are
 *               the partials of this call.
 * Launches the split kernel and the combine kernel on `stream`, in order.
 * Errors: the argument checks of pasa_attn_fwd (without the prefill
 * work-item limit), plus PASA_ERR_WORKSPACE for a null,
 * misaligned or too-small workspace, PASA_ERR_INVALID for num_splits < 0, and
 * PASA_ERR_UNSUPPORTED for more
 * than 65535 splits, or when the split grid (batch * kv heads *
 * ceil(gqa_group / 32) * splits waves) or the combine grid (batch *
 * num_heads_q workgroups) exceeds 2^31 - 1.  More splits than 32-key
 * sub-tiles are clamped to the number of sub-tiles.
 */
int pasa_attn_decode(const void* q, const void* k_cache, const void* v_cache, void* o,
                     float* lse, int batch, int seqlen_kv, int num_heads_q, int gqa_group,
                     int head_dim, float softmax_scale, int num_splits, void* workspace,
                     size_t workspace_bytes, hipStream_t stream);

/*
 * pasa_attn_decode for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * operation, arguments, split choice, kernels and results are pasa_attn_decode's
 * (bit for bit, for the same num_splits); only the fp32 partials live in a
 * scratch area the library reserves statically: PASA_DECODE_SCRATCH_BYTES
 * (16 MiB) of device memory per GPU, held from the library's load until the
 * process ends.  The call itself allocates nothing and frees nothing.
 * Limit: the partials of the split count used,
 * pasa_attn_decode_workspace_bytes(batch, num_heads_q, head_dim, n), must fit
 * the scratch area (the decode workload of 64 sequences x 28 query heads x
 * head_dim 128 at 2 splits takes 1.8 MB).
 * Every call on one GPU uses that GPU's one scratch area: calls that overlap in
 * time on one GPU (different streams or host threads without ordering between
 * them) race and may return wrong results; calls on one stream are ordered and
 * safe.  The area keeps the last call's partials; each call writes every
 * partial it reads, so nothing needs clearing.
 * Errors: as pasa_attn_decode, with PASA_ERR_WORKSPACE when the partials exceed
 * PASA_DECODE_SCRATCH_BYTES, and PASA_ERR_HIP if the scratch area's device
 * address cannot be obtained.
 */
#define PASA_DECODE_SCRATCH_BYTES (16u << 20)
int pasa_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o,
                             float* lse, int batch, int seqlen_kv, int num_heads_q, int gqa_group,
                             int head_dim, float softmax_scale, int num_splits,
                             hipStream_t stream);

/*
 * Split-KV decode over a paged KV cache (one query token per sequence).  The
 * operation is pasa_attn_decode's: the same PASA tile numerics per split and
 * the same merge of the normalised partials ("Block Sparse Flash Attention"
 * topic page, FoldAttention card); only the cache layout differs, and that
 * layout is this library's choice, not the pages'.
 *   k_pages, v_pages  device fp16 [num_pages, page_size, num_heads_q/gqa_group,
 *                     head_dim]: a pool of pages of page_size keys each.
 *   block_table  device int32 [batch, max_pages_per_seq]: key j of sequence b
 *                is row j % page_size of page block_table[b][j / page_size].
 *   seq_lens     device int32 [batch]: key count of each sequence, read on the
 *                device (no host synchronisation); values are clamped to
 *                [0, page_size * max_pages_per_seq].  A sequence of length 0
 *                gets o = 0 and lse = -inf.
 *   q, o, lse, softmax_scale, num_splits, workspace, stream: as
 *                pasa_attn_decode, with page_size * max_pages_per_seq standing
 *                for seqlen_kv (the splits are cut from that bound; splits past
 *                a sequence's end contribute nothing).
 * page_size must be a multiple of 32.  Entries of block_table that a sequence's
 * keys use must lie in [0, num_pages); an entry outside that range reads as
 * zero keys and values instead of faulting.
 * Errors: as pasa_attn_decode, plus PASA_ERR_INVALID for a null block_table or
 * seq_lens or a page_size, num_pages or max_pages_per_seq < 1, and
 * PASA_ERR_UNSUPPORTED for a page_size that is not a multiple of 32.
 */
int pasa_attn_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                           const int* block_table, const int* seq_lens, void* o, float* lse,
                           int batch, int num_heads_q, int gqa_group, int head_dim, int page_size,
                           int num_pages, int max_pages_per_seq, float softmax_scale,
                           int num_splits, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* Whether the prefill entry points (pasa_attn_fwd and its strict, fp8 and naive
 * variants) run a problem as key-split work items on num_cus compute units
 * (host function, no device work; the entry points pass the current device's
 * count, 256 on an MI355X).  A key-split item is 128 query rows whose two groups
 * of waves take the two halves of the key range, merged in fp32 by the
 * log-sum-exp rule ("Block Sparse Flash Attention" topic page, FoldAttention
 * card: partials over disjoint key ranges compose).  The results differ from
 * the 256-row items only by rounding.  Non-causal problems take it when the
 * 256-row items would leave the last round of work items partly idle; causal
 * problems when an estimate of the makespan of the items dealt longest first
 * favours it by at least 5 % (short sequences or few heads, where the longest
 * causal items set the time).
 * Returns 1 (key split) or 0; PASA_ERR_INVALID for a size < 1, a causal flag
 * other than 0 or 1, or num_cus outside [1, 65536]; PASA_ERR_UNSUPPORTED for a
 * head_dim other than 64 or 128. */
int pasa_attn_fwd_key_split(int batch, int seqlen_q, int seqlen_kv, int num_heads_q, int head_dim,
                            int causal, int num_cus);

/* The split count pasa_attn_decode and pasa_attn_decode_paged use for
 * num_splits = 0 (host function, no device work): enough (sequence, key/value
 * head, split) work items for two waves per compute unit at head_dim 128; at
 * head_dim 64 six per compute unit when there are at least 256 (sequence,
 * key/value head) pairs and three otherwise; clamped to the number of 32-key
 * sub-tiles.  Returns 0 on invalid sizes, including a head_dim other than 64
 * or 128. */
int pasa_attn_decode_splits(int batch, int seqlen_kv, int num_heads_q, int gqa_group,
                            int head_dim);

/* Workspace size in bytes for pasa_attn_decode with num_splits splits (host
 * function).  Returns 0 on invalid sizes. */
size_t pasa_attn_decode_workspace_bytes(int batch, int num_heads_q, int head_dim,
                                        int num_splits);

/*
 * Combine step alone (global recovering across splits):
 *   M = max_s lse_s,  lse = M + ln sum_s exp(lse_s - M),
 *   o = sum_s exp(lse_s - lse) * o_s      (fp32 arithmetic, o rounded to fp16).
 * Partials with lse_s = -inf carry no weight; if every partial is empty the
 * row gets o = 0 and lse = -inf.
 *   o_part    device fp32 [batch, num_heads_q, num_splits, head_dim]
 *   lse_part  device fp32 [batch, num_heads_q, num_splits]
 *   o         device fp16 [batch, 1, num_heads_q, head_dim], written
 *   lse       device fp32 [batch, num_heads_q], written; may be NULL
 * Errors: PASA_ERR_INVALID for null o_part/lse_part/o or sizes < 1;
 * PASA_ERR_UNSUPPORTED for head_dim not in {64,128}.
 */
int pasa_attn_decode_combine(const float* o_part, const float* lse_part, void* o,
                             float* lse, int batch, int num_heads_q, int head_dim,
                             int num_splits, hipStream_t stream);

/* Human-readable text for a pasa_status value (static storage). */
const char* pasa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PASA_ATTN_H */
