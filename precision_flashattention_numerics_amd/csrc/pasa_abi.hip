// C ABI of the PASA library: argument validation (pasa_validate.hpp) and
// dispatch to the kernels.  The declarations, with the passages each operation
// follows, are in include/pasa_attn.h.

#include <stdint.h>

#include <mutex>

#include "../../include/pasa_attn.h"
#include "kernels.hpp"
#include "pasa_validate.hpp"

static_assert(pasa::validate::kDecodeBlock == pasa::kDecodeBlock, "one decode sub-tile size");

namespace V = pasa::validate;

namespace {

int fwd_common(int variant, const void* q, const void* k, const void* v, void* o, float* lse,
               int batch, int seqlen_q, int seqlen_kv, int num_heads_q, int gqa_group,
               int head_dim, float softmax_scale, int causal, hipStream_t stream,
               float qk_dequant = 1.0f) {
    const int rc = V::fwd(q, k, v, o, batch, seqlen_q, seqlen_kv, num_heads_q, gqa_group, head_dim,
                          softmax_scale, causal);
    if (rc != PASA_OK) return rc;
    pasa::FwdArgs a{q, k, v, o, lse, batch, seqlen_q, seqlen_kv, num_heads_q, gqa_group,
                    head_dim, softmax_scale, causal, qk_dequant};
    return pasa::launch_fwd(a, variant, stream) == hipSuccess ? PASA_OK : PASA_ERR_HIP;
}

// Split + combine into a caller's workspace (already validated for n splits).
int decode_launch(const void* q, const void* k, const void* v, void* o, float* lse, int batch,
                  int seqlen_kv, int num_heads_q, int gqa_group, int head_dim, float softmax_scale,
                  int n, void* workspace, const int* block_table, const int* seq_lens,
                  int page_size, int max_pages, int num_pages, hipStream_t stream) {
    const size_t rows = (size_t)batch * num_heads_q * n;
    float* o_part = (float*)workspace;
    float* lse_part = (float*)((char*)workspace + V::align256(rows * head_dim * sizeof(float)));
    pasa::DecodeArgs a{q, k, v, o_part, lse_part, batch, seqlen_kv, num_heads_q,
                       gqa_group, head_dim, softmax_scale, n};
    const hipError_t e = block_table != nullptr
        ? pasa::launch_decode_split_paged(a, block_table, seq_lens, page_size, max_pages,
                                          num_pages, stream)
        : pasa::launch_decode_split(a, stream);
    if (e != hipSuccess) return PASA_ERR_HIP;
    if (pasa::launch_decode_combine(o_part, lse_part, o, lse, batch, num_heads_q, head_dim, n,
                                    stream) != hipSuccess)
        return PASA_ERR_HIP;
    return PASA_OK;
}

// Decode partials for callers that cannot allocate (pasa_attn_decode_noalloc):
// a file-scope device array, one copy per GPU, held until the process ends.
// Host code never passes `scratch` itself to a kernel (on the host it is only
// a stand-in for the symbol); it resolves each device's address once, with
// that device current, and uses that address.
constexpr size_t kScratchBytes = PASA_DECODE_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 256;
std::mutex scratch_mu;
void* scratch_addr[kMaxDevices] = {};

// The current device's copy of the scratch array, or nullptr on a HIP error.
void* device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (scratch_addr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
            return nullptr;
        scratch_addr[dev] = p;
    }
    return scratch_addr[dev];
}

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
    const int rc = V::fp8_scales(q_scale, k_scale, softmax_scale);
    if (rc != PASA_OK) return rc;
    return fwd_common(pasa::kVarFp8, q, k, v, o, lse, batch, seqlen_q, seqlen_kv, num_heads_q,
                      gqa_group, head_dim, softmax_scale, causal, stream, q_scale * k_scale);
}

int pasa_naive_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                        int batch, int seqlen_q, int seqlen_kv, int num_heads_q, int gqa_group,
                        int head_dim, float softmax_scale, int causal, hipStream_t stream) {
    return fwd_common(pasa::kVarNaive, q, k, v, o, lse, batch, seqlen_q, seqlen_kv, num_heads_q,
                      gqa_group, head_dim, softmax_scale, causal, stream);
}

int pasa_attn_fwd_key_split(int batch, int seqlen_q, int seqlen_kv, int num_heads_q, int head_dim,
                            int causal, int num_cus) {
    return V::fwd_key_split_query(batch, seqlen_q, seqlen_kv, num_heads_q, head_dim, causal, num_cus);
}

int pasa_attn_decode_splits(int batch, int seqlen_kv, int num_heads_q, int gqa_group,
                            int head_dim) {
    return V::decode_splits(batch, seqlen_kv, num_heads_q, gqa_group, head_dim);
}

size_t pasa_attn_decode_workspace_bytes(int batch, int num_heads_q, int head_dim,
                                        int num_splits) {
    return V::workspace_bytes(batch, num_heads_q, head_dim, num_splits);
}

int pasa_attn_decode(const void* q, const void* k_cache, const void* v_cache, void* o,
                     float* lse, int batch, int seqlen_kv, int num_heads_q, int gqa_group,
                     int head_dim, float softmax_scale, int num_splits, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
    int n = 0;
    int rc = V::decode(q, k_cache, v_cache, o, batch, seqlen_kv, num_heads_q, gqa_group, head_dim,
                       softmax_scale, num_splits, &n);
    if (rc != PASA_OK) return rc;
    rc = V::decode_workspace(workspace, workspace_bytes, batch, num_heads_q, head_dim, n);
    if (rc != PASA_OK) return rc;
    return decode_launch(q, k_cache, v_cache, o, lse, batch, seqlen_kv, num_heads_q, gqa_group,
                         head_dim, softmax_scale, n, workspace, nullptr, nullptr, 0, 0, 0, stream);
}

int pasa_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o,
                             float* lse, int batch, int seqlen_kv, int num_heads_q, int gqa_group,
                             int head_dim, float softmax_scale, int num_splits,
                             hipStream_t stream) {
    int n = 0;
    const int rc = V::decode(q, k_cache, v_cache, o, batch, seqlen_kv, num_heads_q, gqa_group,
                             head_dim, softmax_scale, num_splits, &n);
    if (rc != PASA_OK) return rc;
    if (V::workspace_bytes(batch, num_heads_q, head_dim, n) > kScratchBytes)
        return PASA_ERR_WORKSPACE;
    void* ws = device_scratch();
    if (ws == nullptr) return PASA_ERR_HIP;
    // every partial the combine reads is written by this call's split kernel
    // (an empty split writes o = 0, lse = -inf), so nothing is cleared first
    return decode_launch(q, k_cache, v_cache, o, lse, batch, seqlen_kv, num_heads_q, gqa_group,
                         head_dim, softmax_scale, n, ws, nullptr, nullptr, 0, 0, 0, stream);
}

int pasa_attn_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                           const int* block_table, const int* seq_lens, void* o, float* lse,
                           int batch, int num_heads_q, int gqa_group, int head_dim, int page_size,
                           int num_pages, int max_pages_per_seq, float softmax_scale,
                           int num_splits, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
    int n = 0;
    int rc = V::decode_paged(q, k_pages, v_pages, block_table, seq_lens, o, batch, num_heads_q,
                             gqa_group, head_dim, page_size, num_pages, max_pages_per_seq,
                             softmax_scale, num_splits, &n);
    if (rc != PASA_OK) return rc;
    rc = V::decode_workspace(workspace, workspace_bytes, batch, num_heads_q, head_dim, n);
    if (rc != PASA_OK) return rc;
    return decode_launch(q, k_pages, v_pages, o, lse, batch, page_size * max_pages_per_seq,
                         num_heads_q, gqa_group, head_dim, softmax_scale, n, workspace,
                         block_table, seq_lens, page_size, max_pages_per_seq, num_pages, stream);
}

int pasa_attn_decode_combine(const float* o_part, const float* lse_part, void* o, float* lse,
                             int batch, int num_heads_q, int head_dim, int num_splits,
                             hipStream_t stream) {
    const int rc = V::combine(o_part, lse_part, o, batch, num_heads_q, head_dim, num_splits);
    if (rc != PASA_OK) return rc;
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
