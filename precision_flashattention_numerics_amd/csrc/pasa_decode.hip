// PASA split-KV decode for gfx950: one query token per sequence against a
// KV cache, and the combine step that merges the per-split partials.
//
// Method: the per-block half-precision softmax of "Online Pseudo-average
// Shifting Attention (PASA) for Robust Low-precision LLM Inference", Abstract
// (pasa_tile.hpp), applied to a contiguous key range per workgroup.  The
// partials over disjoint key ranges are merged with their log-sum-exp weights:
// the "Block Sparse Flash Attention" topic page, FoldAttention card, states
// that softmax is invariant to a common shift and that normalised partials
// over disjoint key ranges compose (split KV) without further rescaling.
//
// Split kernel: grid (num_splits, Hkv * head_chunks, batch), 4 waves.
//   The workgroup owns keys [s*L, min((s+1)*L, Skv)) of one key/value head, L a
//   multiple of 128.  The up to 32 query heads sharing that key/value head are
//   the 32 query columns of S^T = K Q^T (unused columns are zero).  Each
//   128-key block is staged into LDS by all 256 threads (K row-major, V
//   transposed); wave w takes keys [32w, 32w+32) of every block with its own
//   online-softmax state, and the four states are merged at the end in fp32.
//   The next block's global loads are in flight while the current one is
//   processed; decode is bound by streaming the KV cache from HBM.
// Combine kernel: one workgroup per (batch, query head), one thread per
//   head-dim column.

#include "kernels.hpp"
#include "pasa_tile.hpp"

namespace pasa {

namespace {

constexpr int kThreads = 256;
constexpr int kBK = kDecodeBlock;   // keys per staged block (32 per wave)

template <int D>
using DecStager = Stager<D, kBK, kThreads>;

template <int D>
constexpr int dec_smem_bytes() {
    constexpr int stage = DecStager<D>::STAGE_HALVES * 2;
    constexpr int merge = (4 * 32 * (D + 4) + 2 * 4 * 32) * 4;   // acc, R, L of the 4 waves
    return stage > merge ? stage : merge;
}

template <int D>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(
    const _Float16* __restrict__ q, const _Float16* __restrict__ k,
    const _Float16* __restrict__ v, float* __restrict__ o_part, float* __restrict__ lse_part,
    int Skv, int Hq, int group, float c, int split_len, int head_chunks) {
    using ST = DecStager<D>;
    constexpr int KK = D / 16;
    constexpr int DT = D / 32;
    extern __shared__ __attribute__((aligned(16))) _Float16 smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int hh = lane >> 5;
    const int n = lane & 31;

    const int split = blockIdx.x;
    const int nsplit = gridDim.x;
    const int hkv = blockIdx.y / head_chunks;
    const int hc = blockIdx.y % head_chunks;
    const int b = blockIdx.z;
    const int Hkv = Hq / group;
    const int hloc = 32 * hc + n;             // query head within the group
    const bool row_valid = hloc < group;
    const int hq = hkv * group + hloc;

    const int64_t kv_stride = (int64_t)Hkv * D;
    const _Float16* kb = k + ((int64_t)b * Skv * Hkv + hkv) * D;
    const _Float16* vb = v + ((int64_t)b * Skv * Hkv + hkv) * D;

    const int kbeg = min(split * split_len, Skv);
    const int kend = min(kbeg + split_len, Skv);
    const int nblocks = (kend - kbeg + kBK - 1) / kBK;

    h8 qreg[KK];
    const _Float16* qrow = q + ((int64_t)b * Hq + hq) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
        qreg[kk] = row_valid ? *(const h8*)(qrow + 16 * kk + 8 * hh) : (h8){};

    ST stager;
    RowState st;
    f16v acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = (f16v){};

    if (nblocks > 0) stager.load(kb, vb, kv_stride, kbeg, kend, tid);
    for (int blk = 0; blk < nblocks; ++blk) {
        stager.store(smem, tid);
        __syncthreads();
        if (blk + 1 < nblocks) stager.load(kb, vb, kv_stride, kbeg + (blk + 1) * kBK, kend, tid);

        const int wbase = kbeg + blk * kBK + 32 * w;   // first key of this wave's slice
        if (wbase < kend) {
            const _Float16* Ks = smem;
            const _Float16* Vt = smem + ST::K_HALVES;
            f16v S[1];
            S[0] = qk_subtile<D, ST::KPAD>(Ks, 32 * w, qreg, n, hh);
            const bool full = wbase + 32 <= kend;
            const int cnt = full ? 32 : kend - wbase;
            auto vis = [&](int, int r) { return wbase + key_of(r, hh) < kend; };
            h2 P[8];
            const _Float16 alpha = softmax_block<1, false>(S, P, st, c, full, cnt, vis);
            if (wave_any(alpha != (_Float16)1)) {
                const float af = (float)alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) acc[dt] *= af;
            }
            pv_chunks<D, ST::VPAD, 2>(Vt, 2 * w, P, acc, n, hh);
        }
        __syncthreads();
    }

    // ---- merge the four wave states (fp32), write this split's partial
    constexpr int MD = D + 4;                   // padded row stride (bank spread)
    float* macc = (float*)smem;                 // [4][32][MD]
    float* mR = macc + 4 * 32 * MD;             // [4][32]
    float* mL = mR + 4 * 32;                    // [4][32]
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int d = 32 * dt + 8 * (r >> 2) + 4 * hh + (r & 3);
            macc[(w * 32 + n) * MD + d] = acc[dt][r];
        }
    if (hh == 0) {
        mR[w * 32 + n] = st.R;
        mL[w * 32 + n] = row_sum<false>(st);
    }
    __syncthreads();
    const int ngroup_rows = min(32, group - 32 * hc);
    for (int idx = tid; idx < ngroup_rows * D; idx += kThreads) {
        const int row = idx / D, d = idx % D;
        float M = -__builtin_inff();
#pragma unroll
        for (int i = 0; i < 4; ++i) M = fmaxf(M, mR[i * 32 + row]);
        float L = 0.0f, val = 0.0f;
        if (M != -__builtin_inff()) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float wgt = __builtin_exp2f(mR[i * 32 + row] - M);
                L += wgt * mL[i * 32 + row];
                val += wgt * macc[(i * 32 + row) * MD + d];
            }
        }
        const int hq_out = hkv * group + 32 * hc + row;
        const int64_t prow = ((int64_t)b * Hq + hq_out) * nsplit + split;
        o_part[prow * D + d] = L > 0.0f ? val / L : 0.0f;
        if (d == 0) lse_part[prow] = L > 0.0f ? (M + __builtin_log2f(L)) * kLn2 : -__builtin_inff();
    }
}

__global__ __launch_bounds__(128) void decode_combine_kernel(
    const float* __restrict__ o_part, const float* __restrict__ lse_part,
    _Float16* __restrict__ o, float* __restrict__ lse, int D, int nsplit) {
    const int64_t row = blockIdx.x;   // b * Hq + hq
    const float* lp = lse_part + row * nsplit;
    float M = -__builtin_inff();
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, lp[s]);
    float sum = 0.0f;
    if (M != -__builtin_inff())
        for (int s = 0; s < nsplit; ++s) sum += expf(lp[s] - M);
    const float L = M != -__builtin_inff() ? M + logf(sum) : -__builtin_inff();
    const int d = threadIdx.x;
    if (d < D) {
        float val = 0.0f;
        if (M != -__builtin_inff())
            for (int s = 0; s < nsplit; ++s) {
                const float wgt = expf(lp[s] - L);
                val += wgt * o_part[(row * nsplit + s) * D + d];
            }
        o[row * D + d] = (_Float16)val;
    }
    if (lse != nullptr && d == 0) lse[row] = L;
}

template <int D>
hipError_t launch_split(const DecodeArgs& a, hipStream_t stream) {
    auto kern = decode_split_kernel<D>;
    constexpr int smem = dec_smem_bytes<D>();
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e != hipSuccess) return e;
    const int blocks = (a.seqlen_kv + kBK - 1) / kBK;
    const int per_split = (blocks + a.num_splits - 1) / a.num_splits;
    const int head_chunks = (a.gqa_group + 31) / 32;
    dim3 grid(a.num_splits, (a.num_heads_q / a.gqa_group) * head_chunks, a.batch);
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), smem, stream,
                       (const _Float16*)a.q, (const _Float16*)a.k, (const _Float16*)a.v,
                       a.o_part, a.lse_part, a.seqlen_kv, a.num_heads_q, a.gqa_group,
                       a.softmax_scale * kLog2e, per_split * kBK, head_chunks);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_split(const DecodeArgs& a, hipStream_t stream) {
    return a.head_dim == 128 ? launch_split<128>(a, stream) : launch_split<64>(a, stream);
}

hipError_t launch_decode_combine(const float* o_part, const float* lse_part, void* o, float* lse,
                                 int batch, int num_heads_q, int head_dim, int num_splits,
                                 hipStream_t stream) {
    dim3 grid((unsigned)((int64_t)batch * num_heads_q));
    hipLaunchKernelGGL(decode_combine_kernel, grid, dim3(128), 0, stream, o_part, lse_part,
                       (_Float16*)o, lse, head_dim, num_splits);
    return hipGetLastError();
}

}  // namespace pasa
