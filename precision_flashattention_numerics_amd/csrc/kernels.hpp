// Host-side launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace pasa {

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int batch, seqlen_q, seqlen_kv, num_heads_q, gqa_group, head_dim;
    float softmax_scale;
    int causal;
    float qk_dequant = 1.0f;   // fp8 variant: q_scale * k_scale
};

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    float* o_part;     // [batch, num_heads_q, num_splits, head_dim]
    float* lse_part;   // [batch, num_heads_q, num_splits]
    int batch, seqlen_kv, num_heads_q, gqa_group, head_dim;
    float softmax_scale;
    int num_splits;
};

// Forward variants: PASA, PASA with fp16 running maximum and offset, the
// naive fp16 Flash-Attention overflow exhibit, and PASA with e4m3 Q and K.
enum { kVarPasa = 0, kVarStrict = 1, kVarNaive = 2, kVarFp8 = 3 };
hipError_t launch_fwd_d64(const FwdArgs& a, int variant, hipStream_t stream);
hipError_t launch_fwd_d128(const FwdArgs& a, int variant, hipStream_t stream);
inline hipError_t launch_fwd(const FwdArgs& a, int variant, hipStream_t stream) {
    return a.head_dim == 128 ? launch_fwd_d128(a, variant, stream) : launch_fwd_d64(a, variant, stream);
}
hipError_t launch_decode_split(const DecodeArgs& a, hipStream_t stream);
// Same over a paged cache (a.k / a.v are the page pools, a.seqlen_kv the
// longest key count the block table can address).
hipError_t launch_decode_split_paged(const DecodeArgs& a, const int* block_table,
                                     const int* seq_lens, int page_size, int max_pages,
                                     int num_pages, hipStream_t stream);
hipError_t launch_decode_combine(const float* o_part, const float* lse_part, void* o, float* lse,
                                 int batch, int num_heads_q, int head_dim, int num_splits,
                                 hipStream_t stream);

// Keys per decode sub-tile; splits are whole multiples of it.
constexpr int kDecodeBlock = 32;

}  // namespace pasa
