// Argument validation of the C ABI (include/pasa_attn.h): every check an entry
// point makes before it enqueues anything.  Plain host C++ with no device code
// and no HIP runtime calls, so that it can also be compiled on its own (with the
// host compiler and its sanitizers) and driven with edge-case sizes.
#pragma once

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <functional>
#include <queue>
#include <vector>

#include "../../include/pasa_attn.h"

namespace pasa {
namespace validate {

constexpr int kDecodeBlock = 32;         // keys per decode sub-tile; splits are whole sub-tiles
constexpr int kFwdRows = 256;            // query rows per prefill work item (at most)
// Longest sequence: the kernels index rows as int, and a work item's last row
// (its first row + 255) must not overflow.
constexpr int kMaxSeq = 0x7FFFFFFF - 511;

inline bool supported_dim(int d) { return d == 64 || d == 128; }

// Element counts must stay below 2^62 so 64-bit indexing cannot overflow.
inline bool fits(int64_t a, int64_t b, int64_t c, int64_t d) {
    const double p = (double)a * (double)b * (double)c * (double)d;
    return p < 4.0e18;
}

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Causal prefill: time, in key-block intervals, of dealing the work items
// longest first to n_cu compute units (one workgroup per unit).  An item of
// `rows` query rows takes its key blocks (64 keys at head_dim 128, 128 at 64)
// plus one interval of pipeline fill; with the key split its two halves run
// side by side.  Every (batch, head) has the same items, and a later query
// tile never sees fewer keys, so the tiles are dealt from the last one down.
inline double causal_makespan(int batch, int seqlen_q, int seqlen_kv, int num_heads_q, int head_dim,
                              int rows, bool split, int n_cu) {
    const int64_t kbc = head_dim == 64 ? 128 : 64;
    const int64_t copies = (int64_t)batch * num_heads_q;
    const int64_t shift = (int64_t)seqlen_kv - seqlen_q;
    std::priority_queue<double, std::vector<double>, std::greater<double>> cu;
    for (int i = 0; i < n_cu; ++i) cu.push(0.0);
    double end = 0.0;
    for (int64_t t = ((int64_t)seqlen_q + rows - 1) / rows - 1; t >= 0; --t) {
        const int64_t last = std::min<int64_t>((int64_t)seqlen_q - 1, t * rows + rows - 1);
        const int64_t kv_end = std::max<int64_t>(0, std::min<int64_t>(seqlen_kv, last + shift + 1));
        const int64_t nb = (kv_end + kbc - 1) / kbc;
        const double len = (double)((split ? (nb + 1) / 2 : nb) + 1);
        for (int64_t c = 0; c < copies; ++c) {
            const double t0 = cu.top();
            cu.pop();
            cu.push(t0 + len);
            end = std::max(end, t0 + len);
        }
    }
    return end;
}

// Whether a prefill takes the key split (128-row items whose two ping-pong
// groups take the two halves of the key range) on n_cu compute units.
//  * Non-causal: when the 256-row items leave the last round of workgroups
//    partly idle: ceil(n128 / CUs) half-length rounds against ceil(n256 / CUs)
//    full ones.
//  * Causal: when the estimate above for the split items, with an interval of
//    the split kernel priced at 1.2 of one of the other (twice the tile loads,
//    and every diagonal block in one half), is at least 5 % lower.  Calibrated
//    on eight causal shapes (head_dim 64 and 128, 1024 to 32768 keys), where it
//    picks the faster kernel every time.  Only problems of at most 8 * n_cu
//    split items are considered: beyond that the items balance and the split
//    loses.
constexpr int kMaxCus = 65536;   // compute units the choice accepts (the simulation keeps one entry each)

inline bool fwd_key_split(int batch, int seqlen_q, int seqlen_kv, int num_heads_q, int head_dim,
                          int causal, int n_cu) {
    if (batch < 1 || seqlen_q < 1 || seqlen_kv < 1 || num_heads_q < 1 || n_cu < 1 || n_cu > kMaxCus ||
        !supported_dim(head_dim))
        return false;
    const int64_t heads = (int64_t)batch * num_heads_q;
    const int64_t n256 = heads * (((int64_t)seqlen_q + kFwdRows - 1) / kFwdRows);
    const int64_t n128 = heads * (((int64_t)seqlen_q + kFwdRows / 2 - 1) / (kFwdRows / 2));
    if (n128 > 0x7FFFFFFFLL) return false;
    if (causal) {
        if (n128 > 8 * (int64_t)n_cu) return false;
        return 1.2 * causal_makespan(batch, seqlen_q, seqlen_kv, num_heads_q, head_dim, kFwdRows / 2, true, n_cu) <
               0.95 * causal_makespan(batch, seqlen_q, seqlen_kv, num_heads_q, head_dim, kFwdRows, false, n_cu);
    }
    return (n128 + n_cu - 1) / n_cu < 2 * ((n256 + n_cu - 1) / n_cu);
}

// pasa_attn_fwd_key_split: 1 or 0, or the status for invalid arguments.
inline int fwd_key_split_query(int batch, int seqlen_q, int seqlen_kv, int num_heads_q, int head_dim,
                               int causal, int num_cus) {
    if (batch < 1 || seqlen_q < 1 || seqlen_kv < 1 || num_heads_q < 1 || (causal != 0 && causal != 1) ||
        num_cus < 1 || num_cus > kMaxCus)
        return PASA_ERR_INVALID;
    if (!supported_dim(head_dim)) return PASA_ERR_UNSUPPORTED;
    return fwd_key_split(batch, seqlen_q, seqlen_kv, num_heads_q, head_dim, causal, num_cus) ? 1 : 0;
}

// Checks shared by the forward and decode entry points.
inline int common(const void* q, const void* k, const void* v, const void* o, int batch,
                  int seqlen_q, int seqlen_kv, int num_heads_q, int gqa_group, int head_dim,
                  float softmax_scale) {
    if (!q || !k || !v || !o) return PASA_ERR_INVALID;
    if (batch < 1 || seqlen_q < 1 || seqlen_kv < 1 || num_heads_q < 1 || gqa_group < 1 ||
        head_dim < 1)
        return PASA_ERR_INVALID;
    if (num_heads_q % gqa_group != 0) return PASA_ERR_INVALID;
    if (!supported_dim(head_dim)) return PASA_ERR_UNSUPPORTED;
    if (seqlen_q > kMaxSeq || seqlen_kv > kMaxSeq) return PASA_ERR_UNSUPPORTED;
    if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale)) return PASA_ERR_UNSUPPORTED;
    if (!fits(batch, seqlen_q, num_heads_q, head_dim) ||
        !fits(batch, seqlen_kv, num_heads_q, head_dim))
        return PASA_ERR_UNSUPPORTED;
    // one head's K/V slab of one sequence is addressed through a buffer
    // descriptor: 32-bit byte offsets
    if ((int64_t)seqlen_kv * (num_heads_q / gqa_group) * head_dim * 2 > 0xFFFFFFFFLL)
        return PASA_ERR_UNSUPPORTED;
    return PASA_OK;
}

// pasa_attn_fwd and its variants.
inline int fwd(const void* q, const void* k, const void* v, const void* o, int batch,
               int seqlen_q, int seqlen_kv, int num_heads_q, int gqa_group, int head_dim,
               float softmax_scale, int causal) {
    const int rc = common(q, k, v, o, batch, seqlen_q, seqlen_kv, num_heads_q, gqa_group, head_dim,
                          softmax_scale);
    if (rc != PASA_OK) return rc;
    if (causal != 0 && causal != 1) return PASA_ERR_INVALID;
    // the prefill's work items (up to 256 query rows of one head) are counted in int
    if ((int64_t)batch * num_heads_q * (((int64_t)seqlen_q + kFwdRows - 1) / kFwdRows) >
        0x7FFFFFFFLL)
        return PASA_ERR_UNSUPPORTED;
    return PASA_OK;
}

// The dequantisation scales of pasa_attn_fwd_fp8.
inline int fp8_scales(float q_scale, float k_scale, float softmax_scale) {
    if (!(q_scale > 0.0f) || !isfinite(q_scale) || !(k_scale > 0.0f) || !isfinite(k_scale))
        return PASA_ERR_UNSUPPORTED;
    const float dq = q_scale * k_scale;
    if (!(dq > 0.0f) || !isfinite(dq) || !isfinite(softmax_scale * dq)) return PASA_ERR_UNSUPPORTED;
    return PASA_OK;
}

// pasa_attn_decode_splits: waves on 256 CUs, measured: at head_dim 128 two
// per CU (LDS would hold three, but fewer and longer key streams per sequence
// read the cache faster); at head_dim 64 six per CU (the LDS limit) when there
// are at least 256 (sequence, key/value head) units, else three.
inline int decode_splits(int batch, int seqlen_kv, int num_heads_q, int gqa_group, int head_dim) {
    if (batch < 1 || seqlen_kv < 1 || num_heads_q < 1 || gqa_group < 1 ||
        num_heads_q % gqa_group != 0 || (head_dim != 64 && head_dim != 128))
        return 0;
    const int64_t units = (int64_t)batch * (num_heads_q / gqa_group) * ((gqa_group + 31) / 32);
    const int64_t target = head_dim == 64 ? (units >= 256 ? 1536 : 768) : 512;
    int64_t n = (target + units - 1) / units;
    const int64_t blocks = ((int64_t)seqlen_kv + kDecodeBlock - 1) / kDecodeBlock;
    if (n > blocks) n = blocks;
    if (n > 65535) n = 65535;
    return (int)(n < 1 ? 1 : n);
}

inline size_t workspace_bytes(int batch, int num_heads_q, int head_dim, int num_splits) {
    if (batch < 1 || num_heads_q < 1 || head_dim < 1 || num_splits < 1) return 0;
    const size_t rows = (size_t)batch * num_heads_q * num_splits;
    return align256(rows * head_dim * sizeof(float)) + align256(rows * sizeof(float));
}

// The decode launches one wave per (sequence, key/value head, chunk of 32
// query heads, split) and one combine workgroup per (sequence, query head),
// each a 1-D grid indexed by int.
inline bool decode_grids_fit(int batch, int num_heads_q, int gqa_group, int n) {
    const int64_t waves = (int64_t)batch * (num_heads_q / gqa_group) * ((gqa_group + 31) / 32) * n;
    return waves <= 0x7FFFFFFFLL && (int64_t)batch * num_heads_q <= 0x7FFFFFFFLL;
}

// The split count a decode call uses (num_splits, or the library's choice for
// 0, clamped to the number of 32-key sub-tiles), and the checks on it.  On
// success *n_used holds the count.
inline int decode_split_count(int batch, int seqlen_kv, int num_heads_q, int gqa_group,
                              int head_dim, int num_splits, int* n_used) {
    if (num_splits < 0) return PASA_ERR_INVALID;
    int n = num_splits == 0 ? decode_splits(batch, seqlen_kv, num_heads_q, gqa_group, head_dim)
                            : num_splits;
    const int blocks = (int)(((int64_t)seqlen_kv + kDecodeBlock - 1) / kDecodeBlock);
    if (n > blocks) n = blocks;
    if (n < 1 || n > 65535 || !decode_grids_fit(batch, num_heads_q, gqa_group, n))
        return PASA_ERR_UNSUPPORTED;
    *n_used = n;
    return PASA_OK;
}

// A caller's decode workspace for n splits: present, 256-byte aligned, large enough.
inline int decode_workspace(const void* workspace, size_t workspace_bytes_given, int batch,
                            int num_heads_q, int head_dim, int n) {
    const size_t need = workspace_bytes(batch, num_heads_q, head_dim, n);
    if (workspace == nullptr || ((uintptr_t)workspace & 255) != 0 || workspace_bytes_given < need)
        return PASA_ERR_WORKSPACE;
    return PASA_OK;
}

// pasa_attn_decode: shapes and the split count (the workspace is checked
// separately).
inline int decode(const void* q, const void* k, const void* v, const void* o, int batch,
                  int seqlen_kv, int num_heads_q, int gqa_group, int head_dim, float softmax_scale,
                  int num_splits, int* n_used) {
    const int rc = common(q, k, v, o, batch, 1, seqlen_kv, num_heads_q, gqa_group, head_dim,
                          softmax_scale);
    if (rc != PASA_OK) return rc;
    return decode_split_count(batch, seqlen_kv, num_heads_q, gqa_group, head_dim, num_splits, n_used);
}

// pasa_attn_decode_paged: the paging arguments, then the checks of the
// contiguous decode with page_size * max_pages_per_seq keys.
inline int decode_paged(const void* q, const void* k_pages, const void* v_pages,
                        const int* block_table, const int* seq_lens, const void* o, int batch,
                        int num_heads_q, int gqa_group, int head_dim, int page_size, int num_pages,
                        int max_pages_per_seq, float softmax_scale, int num_splits, int* n_used) {
    if (!block_table || !seq_lens) return PASA_ERR_INVALID;
    if (page_size < 1 || num_pages < 1 || max_pages_per_seq < 1) return PASA_ERR_INVALID;
    if (page_size % kDecodeBlock != 0) return PASA_ERR_UNSUPPORTED;
    const int64_t max_keys = (int64_t)page_size * max_pages_per_seq;
    if (max_keys > 0x7fffffff) return PASA_ERR_UNSUPPORTED;
    const int seqlen_kv = (int)max_keys;
    int rc = common(q, k_pages, v_pages, o, batch, 1, seqlen_kv, num_heads_q, gqa_group, head_dim,
                    softmax_scale);
    if (rc != PASA_OK) return rc;
    if (!fits(num_pages, page_size, num_heads_q / gqa_group, head_dim)) return PASA_ERR_UNSUPPORTED;
    if ((int64_t)batch * max_pages_per_seq > 0x7fffffff) return PASA_ERR_UNSUPPORTED;
    return decode_split_count(batch, seqlen_kv, num_heads_q, gqa_group, head_dim, num_splits, n_used);
}

// pasa_attn_decode_combine.
inline int combine(const float* o_part, const float* lse_part, const void* o, int batch,
                   int num_heads_q, int head_dim, int num_splits) {
    if (!o_part || !lse_part || !o) return PASA_ERR_INVALID;
    if (batch < 1 || num_heads_q < 1 || head_dim < 1 || num_splits < 1) return PASA_ERR_INVALID;
    if (!supported_dim(head_dim)) return PASA_ERR_UNSUPPORTED;
    if ((int64_t)batch * num_heads_q > 0x7fffffff) return PASA_ERR_UNSUPPORTED;
    return PASA_OK;
}

}  // namespace validate
}  // namespace pasa
