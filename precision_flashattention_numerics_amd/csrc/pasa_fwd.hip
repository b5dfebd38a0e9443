// PASA forward (prefill) kernel and the naive fp16 Flash-Attention kernel for
// gfx950 (AMD Instinct MI355X).
//
// Method: "Online Pseudo-average Shifting Attention (PASA) for Robust
// Low-precision LLM Inference", Abstract -- blockwise Flash-Attention in which
// the score tile, the exponentials and the softmax statistics are fp16; each
// key block's scores are shifted by a per-row pseudo-average so that the fp16
// tile stays inside the fp16 range (65504); the epilogue re-applies the removed
// shifts ("global recovering") so the normalisation and the log-sum-exp are
// exact up to rounding.
//
// Work decomposition (one workgroup = 4 waves = 128 query rows of one head):
//   * S^T = K Q^T on the matrix cores (v_mfma_f32_32x32x16_f16).  Q is the B
//     operand and stays in registers for the whole key loop; K rows come from
//     LDS.  With keys on the M side, each lane ends up holding 32 of the 64
//     scores of ONE query row per key block, so row max / sum / mean are
//     in-lane reductions plus a single exchange with the lane 32 apart.
//   * O^T += V^T P^T on the matrix cores.  The fp16 P tile produced by the
//     softmax is already laid out as the B operand (no LDS round trip): the K
//     rows are fed to the first product in a permuted order (bits 2 and 3 of
//     the row index swapped) so that every lane's scores are 8 consecutive
//     keys per 16-key chunk.
//   * K and V tiles go straight from HBM into LDS (buffer_load ... lds, no
//     staging registers; rows past the sequence end read as zero), stored
//     row-major with XOR-swizzled 16-byte chunks.  V is consumed through the
//     transposing LDS read of gfx950 (ds_read_b64_tr_b16), so it needs no
//     transpose on the way in.  Two LDS stages: the next block's loads are in
//     flight while the current block is processed.
//   * Blocks that every row of a wave sees in full take a branch-free path;
//     only the diagonal / ragged-tail blocks evaluate the mask.
//
// The per-block half-precision softmax (pseudo-average shift, refine, fp16
// exponentials and sums) lives in pasa_tile.hpp.

#include "kernels.hpp"
#include "pasa_tile.hpp"

namespace pasa {

namespace {

constexpr int kBR = 128;      // query rows per workgroup (32 per wave)
constexpr int kBC = 64;       // keys per block
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

template <int D>
constexpr int tile_halves() { return kBC * D; }
template <int D>
constexpr int fwd_smem_bytes() { return 2 /*stages*/ * 2 /*K,V*/ * tile_halves<D>() * 2; }

template <int D, bool CAUSAL, bool NAIVE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_kernel(
    const _Float16* __restrict__ q, const _Float16* __restrict__ k,
    const _Float16* __restrict__ v, _Float16* __restrict__ o, float* __restrict__ lse,
    int Sq, int Skv, int Hq, int group, float c, int n_qtiles) {
    constexpr int KK = D / 16;
    constexpr int DT = D / 32;
    extern __shared__ __attribute__((aligned(1024))) _Float16 smem[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int hh = lane >> 5;   // which half of the wave
    const int n = lane & 31;    // query column owned by this lane

    const int hq = blockIdx.x;
    const int tile = CAUSAL ? (n_qtiles - 1 - (int)blockIdx.y) : (int)blockIdx.y;
    const int b = blockIdx.z;
    const int Hkv = Hq / group;
    const int hkv = hq / group;
    const int q0 = tile * kBR;
    const int qi = q0 + 32 * w + n;

    const int64_t q_stride = (int64_t)Hq * D;
    const int64_t kv_stride = (int64_t)Hkv * D;
    const _Float16* qb = q + ((int64_t)b * Sq * Hq + hq) * D;
    const _Float16* kb = k + ((int64_t)b * Skv * Hkv + hkv) * D;
    const _Float16* vb = v + ((int64_t)b * Skv * Hkv + hkv) * D;
    const uint32_t slab_bytes = (uint32_t)(((int64_t)(Skv - 1) * kv_stride + D) * 2);
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(kb, slab_bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vb, slab_bytes);
    const uint32_t stride_b = (uint32_t)(kv_stride * 2);

    // ---- key range of this workgroup and of this lane's row
    const int64_t shift = (int64_t)Skv - Sq;   // bottom-right causal alignment
    int kv_end = Skv;
    if (CAUSAL) {
        const int64_t last = (int64_t)min(q0 + kBR - 1, Sq - 1) + shift;
        kv_end = last < 0 ? 0 : (int)min<int64_t>(Skv, last + 1);
    }
    const int nblocks = (kv_end + kBC - 1) / kBC;
    auto row_limit = [&](int row) -> int {   // keys [0, limit) are visible to row
        if (!CAUSAL) return Skv;
        const int64_t l = (int64_t)row + shift + 1;
        return (int)max<int64_t>(0, min<int64_t>(Skv, l));
    };
    const int lim = row_limit(qi);
    const int wave_lim_lo = row_limit(q0 + 32 * w);
    const int wave_lim_hi = row_limit(q0 + 32 * w + 31);

    auto stage_ptr = [&](int stage) { return smem + stage * 2 * tile_halves<D>(); };
    auto issue = [&](int blk) {
        _Float16* st = stage_ptr(blk & 1);
        stage_tile<D, kBC, kWaves, false>(krs, stride_b, blk * kBC, st, w, lane);
        stage_tile<D, kBC, kWaves, true>(vrs, stride_b, blk * kBC, st + tile_halves<D>(), w, lane);
    };
    if (nblocks > 0) issue(0);

    // ---- Q operand: lane holds Q[qi][16*kk + 8*hh .. +7]
    h8 qreg[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
        qreg[kk] = qi < Sq ? *(const h8*)(qb + (int64_t)qi * q_stride + 16 * kk + 8 * hh) : (h8){};

    RowState st;
    f16v acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = (f16v){};

    wait_vmem();
    __syncthreads();

    for (int blk = 0; blk < nblocks; ++blk) {
        if (blk + 1 < nblocks) issue(blk + 1);

        const int kbase = blk * kBC;
        if (kbase < wave_lim_hi) {   // some row of this wave sees a key of the block
            const _Float16* Ks = stage_ptr(blk & 1);
            const _Float16* Vs = Ks + tile_halves<D>();
            f16v S[2];
            S[0] = qk_subtile_sw<D>(Ks, 0, qreg, n, hh);
            S[1] = qk_subtile_sw<D>(Ks, 32, qreg, n, hh);

            h2 P[16];
            _Float16 alpha;
            if (kbase + kBC <= wave_lim_lo) {   // the whole block is visible to the wave
                alpha = softmax_block<2, NAIVE>(S, P, st, c, true, kBC, [](int, int) { return true; });
            } else {
                const int m = lim - kbase;        // keys [0, m) of the block are visible
                const int cnt = max(0, min(kBC, m));
                alpha = softmax_block<2, NAIVE>(S, P, st, c, false, cnt,
                                                [&](int t, int r) { return 32 * t + key_of(r, hh) < m; });
            }
            if (wave_any(alpha != (_Float16)1)) {
                const float af = (float)alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) acc[dt] *= af;
            }
            pv_chunks_tr<D, 4>(Vs, 0, P, acc, lane);
        }
        wait_vmem();
        __syncthreads();
    }

    // ---- epilogue: global recovering
    if (qi < Sq) {
        const float L = row_sum<NAIVE>(st);
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        _Float16* orow = o + ((int64_t)b * Sq + qi) * q_stride + (int64_t)hq * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const h4 t = {(_Float16)(acc[dt][4 * g + 0] * inv), (_Float16)(acc[dt][4 * g + 1] * inv),
                              (_Float16)(acc[dt][4 * g + 2] * inv), (_Float16)(acc[dt][4 * g + 3] * inv)};
                *(h4*)(orow + 32 * dt + 8 * g + 4 * hh) = t;
            }
        if (lse != nullptr && hh == 0)
            lse[((int64_t)b * Hq + hq) * Sq + qi] =
                L > 0.0f ? (st.R + __builtin_log2f(L)) * kLn2 : -__builtin_inff();
    }
}

template <int D, bool CAUSAL, bool NAIVE>
hipError_t launch_one(const FwdArgs& a, hipStream_t stream) {
    auto kern = fwd_kernel<D, CAUSAL, NAIVE>;
    constexpr int smem = fwd_smem_bytes<D>();
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e != hipSuccess) return e;
    const int n_qtiles = (a.seqlen_q + kBR - 1) / kBR;
    // x = query head, y = query tile: consecutive workgroups are the heads of
    // one tile, and for causal masking tiles are issued longest first.
    dim3 grid(a.num_heads_q, n_qtiles, a.batch);
    hipLaunchKernelGGL(kern, grid, dim3(kThreads), smem, stream,
                       (const _Float16*)a.q, (const _Float16*)a.k, (const _Float16*)a.v,
                       (_Float16*)a.o, a.lse, a.seqlen_q, a.seqlen_kv, a.num_heads_q,
                       a.gqa_group, a.softmax_scale * kLog2e, n_qtiles);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a, bool naive, hipStream_t stream) {
    if (a.head_dim == 128) {
        if (naive)
            return a.causal ? launch_one<128, true, true>(a, stream) : launch_one<128, false, true>(a, stream);
        return a.causal ? launch_one<128, true, false>(a, stream) : launch_one<128, false, false>(a, stream);
    }
    if (naive)
        return a.causal ? launch_one<64, true, true>(a, stream) : launch_one<64, false, true>(a, stream);
    return a.causal ? launch_one<64, true, false>(a, stream) : launch_one<64, false, false>(a, stream);
}

}  // namespace pasa
