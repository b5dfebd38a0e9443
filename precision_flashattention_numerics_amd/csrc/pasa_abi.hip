// C ABI of the PASA library: argument validation and dispatch to the kernels.
// The declarations, with the passages each operation follows, are in
// include/pasa_attn.h.

#include <math.h>
#include <stdint.h>

#include "../../include/pasa_attn.h"
#include "kernels.hpp"

namespace {

constexpr int kMaxFp16Sum = 65504;   // fp16 running sum: at most this many keys

bool supported_dim(int d) { return d == 64 || d == 128; }

// Element counts must stay below 2^62 so 64-bit indexing cannot overflow.
bool fits(int64_t a, int64_t b, int64_t c, int64_t d) {
    const double p = (double)a * (double)b * (double)c * (double)d;
    return p < 4.0e18;
}

int check_common(const void* q, const void* k, const void* v, const void* o, int batch,
                 int seqlen_q, int seqlen_kv, int num_heads_q, int gqa_group, int head_dim,
                 float softmax_scale) {
    if (!q || !k || !v || !o) return PASA_ERR_INVALID;
    if (batch < 1 || seqlen_q < 1 || seqlen_kv < 1 || num_heads_q < 1 || gqa_group < 1 ||
        head_dim < 1)
        return PASA_ERR_INVALID;
    if (num_heads_q % gqa_group != 0) return PASA_ERR_INVALID;
    if (!supported_dim(head_dim)) return PASA_ERR_UNSUPPORTED;
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

// The decode launches one wave per (sequence, key/value head, chunk of 32
// query heads, split) and one combine workgroup per (sequence, query head),
// each a 1-D grid indexed by int.
bool decode_grids_fit(int batch, int num_heads_q, int gqa_group, int n) {
    const int64_t waves = (int64_t)batch * (num_heads_q / gqa_group) * ((gqa_group + 31) / 32) * n;
    return waves <= 0x7FFFFFFFLL && (int64_t)batch * num_heads_q <= 0x7FFFFFFFLL;
}

int fwd_common(int variant, const void* q, const void* k, const void* v, void* o, float* lse,
               int batch, int seqlen_q, int seqlen_kv, int num_heads_q, int gqa_group,
               int head_dim, float softmax_scale, int causal, hipStream_t stream,
               float qk_dequant = 1.0f) {
    int rc = check_common(q, k, v, o, batch, seqlen_q, seqlen_kv, num_heads_q, gqa_group,
                          head_dim, softmax_scale);
    if (rc != PASA_OK) return rc;
    if (causal != 0 && causal != 1) return PASA_ERR_INVALID;
    if (seqlen_kv > kMaxFp16Sum) return PASA_ERR_UNSUPPORTED;
    // the prefill's work items (256 query rows of one head) are counted in int
    if ((int64_t)batch * num_heads_q * ((seqlen_q + 255) / 256) > 0x7FFFFFFFLL)
        return PASA_ERR_UNSUPPORTED;
    pasa::FwdArgs a{q, k, v, o, lse, batch, seqlen_q, seqlen_kv, num_heads_q, gqa_group,
                    head_dim, softmax_scale, causal, qk_dequant};
    return pasa::launch_fwd(a, variant, stream) == hipSuccess ? PASA_OK : PASA_ERR_HIP;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

extern "C" {

int pasa_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int batch,
                  int seqlen_q, int seqlen_kv, int num_heads_q, int gqa_group, int head_dim,
                  float softmax_scale, int causal, hipStream_t stream) {
    return fwd_common(pasa::kVarPasa, q, k, v, o, lse, batch, seqlen_q, seqlen_kv, num_heads_q,
                      gqa_group, head_dim, softmax_scale, causal, stream);
}

int pasa_attn_fwd_strict(const void* q, const void* k, const void* v, void* o, float* lse,
                         int batch, int seqlen_q, int seqlen_kv, int num_heads_q, int gqa_group,
                         int head_dim, float softmax_scale, int causal, hipStream_t stream) {
    return fwd_common(pasa::kVarStrict, q, k, v, o, lse, batch, seqlen_q, seqlen_kv, num_heads_q,
                      gqa_group, head_dim, softmax_scale, causal, stream);
}

int pasa_attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                      int batch, int seqlen_q, int seqlen_kv, int num_heads_q, int gqa_group,
                      int head_dim, float softmax_scale, float q_scale, float k_scale, int causal,
                      hipStream_t stream) {
    if (!(q_scale > 0.0f) || !isfinite(q_scale) || !(k_scale > 0.0f) || !isfinite(k_scale))
        return PASA_ERR_UNSUPPORTED;
    const float dq = q_scale * k_scale;
    if (!(dq > 0.0f) || !isfinite(dq) || !isfinite(softmax_scale * dq)) return PASA_ERR_UNSUPPORTED;
    return fwd_common(pasa::kVarFp8, q, k, v, o, lse, batch, seqlen_q, seqlen_kv, num_heads_q,
                      gqa_group, head_dim, softmax_scale, causal, stream, dq);
}

int pasa_naive_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                        int batch, int seqlen_q, int seqlen_kv, int num_heads_q, int gqa_group,
                        int head_dim, float softmax_scale, int causal, hipStream_t stream) {
    return fwd_common(pasa::kVarNaive, q, k, v, o, lse, batch, seqlen_q, seqlen_kv, num_heads_q,
                      gqa_group, head_dim, softmax_scale, causal, stream);
}

int pasa_attn_decode_splits(int batch, int seqlen_kv, int num_heads_q, int gqa_group,
                            int head_dim) {
    if (batch < 1 || seqlen_kv < 1 || num_heads_q < 1 || gqa_group < 1 ||
        num_heads_q % gqa_group != 0 || (head_dim != 64 && head_dim != 128))
        return 0;
    const int64_t units = (int64_t)batch * (num_heads_q / gqa_group) * ((gqa_group + 31) / 32);
    // waves on 256 CUs, measured: at head_dim 128 two per CU (LDS would hold
    // three, but fewer and longer key streams per sequence read the cache
    // faster); at head_dim 64 three per CU (of the six LDS holds)
    const int64_t target = head_dim == 64 ? 768 : 512;
    int64_t n = (target + units - 1) / units;
    const int64_t blocks = (seqlen_kv + pasa::kDecodeBlock - 1) / pasa::kDecodeBlock;
    if (n > blocks) n = blocks;
    if (n > 65535) n = 65535;
    return (int)(n < 1 ? 1 : n);
}

size_t pasa_attn_decode_workspace_bytes(int batch, int num_heads_q, int head_dim,
                                        int num_splits) {
    if (batch < 1 || num_heads_q < 1 || head_dim < 1 || num_splits < 1) return 0;
    const size_t rows = (size_t)batch * num_heads_q * num_splits;
    return align256(rows * head_dim * sizeof(float)) + align256(rows * sizeof(float));
}

int pasa_attn_decode(const void* q, const void* k_cache, const void* v_cache, void* o,
                     float* lse, int batch, int seqlen_kv, int num_heads_q, int gqa_group,
                     int head_dim, float softmax_scale, int num_splits, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
    int rc = check_common(q, k_cache, v_cache, o, batch, 1, seqlen_kv, num_heads_q, gqa_group,
                          head_dim, softmax_scale);
    if (rc != PASA_OK) return rc;
    if (num_splits < 0) return PASA_ERR_INVALID;
    int n = num_splits == 0 ? pasa_attn_decode_splits(batch, seqlen_kv, num_heads_q, gqa_group, head_dim)
                            : num_splits;
    const int blocks = (seqlen_kv + pasa::kDecodeBlock - 1) / pasa::kDecodeBlock;
    if (n > blocks) n = blocks;
    if (n > 65535 || !decode_grids_fit(batch, num_heads_q, gqa_group, n)) return PASA_ERR_UNSUPPORTED;
    // every split sums at most 65504 keys in fp16
    const int per_split = (blocks + n - 1) / n * pasa::kDecodeBlock;
    if (per_split > kMaxFp16Sum) return PASA_ERR_UNSUPPORTED;
    const size_t need = pasa_attn_decode_workspace_bytes(batch, num_heads_q, head_dim, n);
    if (workspace == nullptr || ((uintptr_t)workspace & 255) != 0 || workspace_bytes < need)
        return PASA_ERR_WORKSPACE;
    const size_t rows = (size_t)batch * num_heads_q * n;
    float* o_part = (float*)workspace;
    float* lse_part = (float*)((char*)workspace + align256(rows * head_dim * sizeof(float)));
    pasa::DecodeArgs a{q, k_cache, v_cache, o_part, lse_part, batch, seqlen_kv, num_heads_q,
                       gqa_group, head_dim, softmax_scale, n};
    if (pasa::launch_decode_split(a, stream) != hipSuccess) return PASA_ERR_HIP;
    if (pasa::launch_decode_combine(o_part, lse_part, o, lse, batch, num_heads_q, head_dim, n,
                                    stream) != hipSuccess)
        return PASA_ERR_HIP;
    return PASA_OK;
}

int pasa_attn_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                           const int* block_table, const int* seq_lens, void* o, float* lse,
                           int batch, int num_heads_q, int gqa_group, int head_dim, int page_size,
                           int num_pages, int max_pages_per_seq, float softmax_scale,
                           int num_splits, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
    if (!block_table || !seq_lens) return PASA_ERR_INVALID;
    if (page_size < 1 || num_pages < 1 || max_pages_per_seq < 1) return PASA_ERR_INVALID;
    if (page_size % pasa::kDecodeBlock != 0) return PASA_ERR_UNSUPPORTED;
    const int64_t max_keys = (int64_t)page_size * max_pages_per_seq;
    if (max_keys > 0x7fffffff) return PASA_ERR_UNSUPPORTED;
    const int seqlen_kv = (int)max_keys;
    // the shape checks of the contiguous decode, with the pool as one "sequence"
    int rc = check_common(q, k_pages, v_pages, o, batch, 1, seqlen_kv, num_heads_q, gqa_group,
                          head_dim, softmax_scale);
    if (rc != PASA_OK) return rc;
    if (!fits(num_pages, page_size, num_heads_q / gqa_group, head_dim)) return PASA_ERR_UNSUPPORTED;
    if ((int64_t)batch * max_pages_per_seq > 0x7fffffff) return PASA_ERR_UNSUPPORTED;
    if (num_splits < 0) return PASA_ERR_INVALID;
    int n = num_splits == 0 ? pasa_attn_decode_splits(batch, seqlen_kv, num_heads_q, gqa_group, head_dim)
                            : num_splits;
    const int blocks = (seqlen_kv + pasa::kDecodeBlock - 1) / pasa::kDecodeBlock;
    if (n > blocks) n = blocks;
    if (n > 65535 || !decode_grids_fit(batch, num_heads_q, gqa_group, n)) return PASA_ERR_UNSUPPORTED;
    const int per_split = (blocks + n - 1) / n * pasa::kDecodeBlock;
    if (per_split > kMaxFp16Sum) return PASA_ERR_UNSUPPORTED;
    const size_t need = pasa_attn_decode_workspace_bytes(batch, num_heads_q, head_dim, n);
    if (workspace == nullptr || ((uintptr_t)workspace & 255) != 0 || workspace_bytes < need)
        return PASA_ERR_WORKSPACE;
    const size_t rows = (size_t)batch * num_heads_q * n;
    float* o_part = (float*)workspace;
    float* lse_part = (float*)((char*)workspace + align256(rows * head_dim * sizeof(float)));
    pasa::DecodeArgs a{q, k_pages, v_pages, o_part, lse_part, batch, seqlen_kv, num_heads_q,
                       gqa_group, head_dim, softmax_scale, n};
    if (pasa::launch_decode_split_paged(a, block_table, seq_lens, page_size, max_pages_per_seq,
                                        num_pages, stream) != hipSuccess)
        return PASA_ERR_HIP;
    if (pasa::launch_decode_combine(o_part, lse_part, o, lse, batch, num_heads_q, head_dim, n,
                                    stream) != hipSuccess)
        return PASA_ERR_HIP;
    return PASA_OK;
}

int pasa_attn_decode_combine(const float* o_part, const float* lse_part, void* o, float* lse,
                             int batch, int num_heads_q, int head_dim, int num_splits,
                             hipStream_t stream) {
    if (!o_part || !lse_part || !o) return PASA_ERR_INVALID;
    if (batch < 1 || num_heads_q < 1 || head_dim < 1 || num_splits < 1) return PASA_ERR_INVALID;
    if (!supported_dim(head_dim)) return PASA_ERR_UNSUPPORTED;
    if ((int64_t)batch * num_heads_q > 0x7fffffff) return PASA_ERR_UNSUPPORTED;
    return pasa::launch_decode_combine(o_part, lse_part, o, lse, batch, num_heads_q, head_dim,
                                       num_splits, stream) == hipSuccess
               ? PASA_OK
               : PASA_ERR_HIP;
}

const char* pasa_status_string(int status) {
    switch (status) {
        case PASA_OK: return "ok";
        case PASA_ERR_INVALID: return "invalid argument";
        case PASA_ERR_UNSUPPORTED: return "unsupported configuration";
        case PASA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case PASA_ERR_HIP: return "HIP launch error";
        default: return "unknown status";
    }
}

}  // extern "C"
