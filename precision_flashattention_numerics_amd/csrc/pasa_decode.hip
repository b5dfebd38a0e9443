// PASA split-KV decode for gfx950: one query token per sequence against a
// KV cache, and the combine step that merges the per-split partials.
//
// Method: the per-block half-precision softmax of "Online Pseudo-average
// Shifting Attention (PASA) for Robust Low-precision LLM Inference", Abstract
// (pasa_tile.hpp), applied to a contiguous key range per wave.  The partials
// over disjoint key ranges are merged with their log-sum-exp weights: the
// "Block Sparse Flash Attention" topic page, FoldAttention card, states that
// softmax is invariant to a common shift and that normalised partials over
// disjoint key ranges compose (split KV) without further rescaling.
//
// Split kernel: one wave per workgroup; the wave owns keys [s*L, (s+1)*L) of
// one key/value head of one sequence (L a multiple of 32).  The up to 32
// query heads sharing that key/value head are the 32 query columns of
// S^T = K Q^T (unused columns are zero).  Decode reads every KV-cache byte
// once, so the kernel is bound by HBM: each wave streams its keys in 32-key
// sub-tiles straight from HBM into a private ring of LDS slots
// (buffer_load ... lds), keeping the next sub-tiles in flight while it
// computes on the current one; it synchronises only with itself
// (s_waitcnt vmcnt), never with other waves.  Every wave writes one fp32
// partial (o_s, lse_s).
// Paged variant (PAGED = true): the cache is a pool of pages of page_size
// keys ([num_pages, page_size, Hkv, D]); sequence b's key j lives in page
// block_table[b][j / page_size] at row j % page_size, and its length is
// seq_lens[b], read on the device.  page_size is a multiple of 32, so a
// sub-tile never straddles pages; each sub-tile gets its own buffer
// descriptor bounded by the sequence end, and an out-of-range page index
// reads as zeros instead of faulting.
// Combine kernel: one workgroup per (sequence, query head), one thread per
// head-dim column.

#include "kernels.hpp"
#include "pasa_tile.hpp"

namespace pasa {

namespace {

constexpr int kSub = kDecodeBlock;   // keys per sub-tile (one 32x32 product tile)
constexpr int kSlots = 3;            // LDS ring depth per wave

template <int D>
constexpr int sub_halves() { return kSub * D; }                     // one tensor, one sub-tile
template <int D>
constexpr int dec_smem_bytes() { return kSlots * 2 * sub_halves<D>() * 2; }
template <int D>
constexpr int dma_per_sub() { return 2 * (kSub * D / 8) / 64; }     // 16-byte-per-lane loads

struct Paging {
    const int* block_table;   // [batch, max_pages] page indices
    const int* seq_lens;      // [batch] key counts
    int page_size, max_pages, num_pages;
};

// At head_dim 64 the register budget is capped at 256 (two waves per SIMD):
// the kernel then needs 132 registers and keeps its accumulator in ordinary
// vector registers, where the uncapped build moved it through AGPRs on every
// sub-tile (batch 64, 28/4 heads, 8192 keys: 112.5 -> 98.3 us; batch 8,
// 32/8 heads, 16384 keys: 62.8 -> 55.9 us; bitwise-equal outputs).  At
// head_dim 128 the same cap measured slower on long caches and is not used.
template <int D, bool PAGED>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(D == 64 ? 2 : 1, D == 64 ? 2 : 10)))
void decode_split_kernel(
    const _Float16* __restrict__ q, const _Float16* __restrict__ k,
    const _Float16* __restrict__ v, float* __restrict__ o_part, float* __restrict__ lse_part,
    int Skv, int Hq, int group, float c, int split_len, int head_chunks, int nsplit, Paging pg) {
    constexpr int KK = D / 16;
    constexpr int DT = D / 32;
    constexpr int NL = dma_per_sub<D>();
    extern __shared__ __attribute__((aligned(1024))) _Float16 smem[];

    const int lane = threadIdx.x;
    const int hh = lane >> 5;
    const int n = lane & 31;

    // workgroup -> (split, head chunk, key/value head, sequence), split fastest
    int id = blockIdx.x;
    const int split = id % nsplit;
    id /= nsplit;
    const int hc = id % head_chunks;
    id /= head_chunks;
    const int Hkv = Hq / group;
    const int hkv = id % Hkv;
    const int b = id / Hkv;
    const int hloc = 32 * hc + n;             // query head within the group
    const bool row_valid = hloc < group;
    const int hq = hkv * group + hloc;

    const int64_t kv_stride = (int64_t)Hkv * D;
    const uint32_t stride_b = (uint32_t)(kv_stride * 2);
    if (PAGED) {   // this sequence's length, clamped to what its block table can address
        const int len = __builtin_amdgcn_readfirstlane(pg.seq_lens[b]);
        Skv = max(0, min(len, pg.max_pages * pg.page_size));
    }
    const _Float16* kb = k + ((int64_t)b * Skv * Hkv + hkv) * D;
    const _Float16* vb = v + ((int64_t)b * Skv * Hkv + hkv) * D;
    const uint32_t slab_bytes =
        PAGED ? 0u : (uint32_t)(((int64_t)(Skv - 1) * kv_stride + D) * 2);
    const i32x4 krs = make_rsrc(kb, slab_bytes);   // contiguous: the whole slab
    const i32x4 vrs = make_rsrc(vb, slab_bytes);

    const int kbeg = min(split * split_len, Skv);
    const int kend = min(kbeg + split_len, Skv);
    const int nsub = (kend - kbeg + kSub - 1) / kSub;

    // Paged: the split's page indices, 64 at a time, one per lane (lane l holds
    // entry pbase + 64 * pchunk + l of the sequence's block table; -1 past its
    // end), so that a sub-tile's page is a lane read, not a dependent memory
    // load in front of every DMA.
    const int pbase = PAGED ? kbeg / pg.page_size : 0;
    int pchunk = 0, pcache = -1;
    // The wait sits here, on the rare path: the compiler does not count the
    // ring's inline-asm DMA loads, so a wait it places for pcache lands after
    // this branch joins, as vmcnt(0) on every sub-tile, and drains the ring
    // (in-order 64-key pages 180 against 160 us).
    auto load_pages = [&](int ch) {
        const int idx = pbase + 64 * ch + lane;
        pcache = idx < pg.max_pages ? pg.block_table[(int64_t)b * pg.max_pages + idx] : -1;
        pchunk = ch;
        wait_vmem();
    };
    if (PAGED) load_pages(0);
    // the page (relative to pbase) and the sub-tile within it of the next
    // sub-tile to issue; sub-tiles are issued in order, so both advance by
    // counting instead of dividing by the page size
    const int subs_per_page = PAGED ? pg.page_size / kSub : 1;
    int next_page = 0, next_sub = PAGED ? (kbeg - pbase * pg.page_size) / kSub : 0;
    const int64_t page_elems = PAGED ? (int64_t)pg.page_size * kv_stride : 0;

    // paged: this wave's lane offsets inside a sub-tile and the segments'
    // offsets inside a slot, computed once (measured about 5 % faster than
    // forming them at each load, which the contiguous path does); the ring's
    // LDS byte address
    const TileDma<D, kSub, 1, false, false, true> kdma(stride_b, 0u, lane);
    const TileDma<D, kSub, 1, true, false, true> vdma(stride_b, 0u, lane);
    constexpr uint32_t kTileBytes = sub_halves<D>() * 2;   // one tensor's sub-tile
    const uint32_t ring = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)smem);

    auto slot_k = [&](int j) { return smem + (j % kSlots) * 2 * sub_halves<D>(); };
    auto issue = [&](int j) {
        const uint32_t slot = ring + (uint32_t)(j % kSlots) * (2 * kTileBytes);
        const int key0 = kbeg + j * kSub;
        if (PAGED) {
            // the sub-tile's page, and a descriptor over its rows that exist
            const int pl = next_page, sub = next_sub;
            if (++next_sub == subs_per_page) {
                next_sub = 0;
                ++next_page;
            }
            if ((pl >> 6) != pchunk) load_pages(pl >> 6);   // rare
            const int page = __builtin_amdgcn_readlane(pcache, pl & 63);
            const int rows = min(kSub, Skv - key0);
            const bool ok = page >= 0 && page < pg.num_pages;
            const int64_t base = (int64_t)(ok ? page : 0) * page_elems +
                                 (int64_t)(sub * kSub) * kv_stride + (int64_t)hkv * D;
            const uint32_t bytes = ok ? (uint32_t)(((int64_t)(rows - 1) * kv_stride + D) * 2) : 0u;
            kdma.issue(make_rsrc(k + base, bytes), slot);
            vdma.issue(make_rsrc(v + base, bytes), slot + kTileBytes);
        } else {
            _Float16* const sk = slot_k(j);
            stage_tile_nt<D, kSub, false>(krs, stride_b, key0, sk, lane);
            stage_tile_nt<D, kSub, true>(vrs, stride_b, key0, sk + sub_halves<D>(), lane);
        }
    };

    h8 qreg[KK];
    const _Float16* qrow = q + ((int64_t)b * Hq + hq) * D;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
        qreg[kk] = row_valid ? *(const h8*)(qrow + 16 * kk + 8 * hh) : (h8){};
    wait_vmem();

#pragma unroll
    for (int j = 0; j < kSlots - 1; ++j)
        if (j < nsub) issue(j);

    RowState st;
    f16v acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = (f16v){};

    for (int j = 0; j < nsub; ++j) {
        // sub-tiles j+1 .. j+kSlots-2 stay in flight while j is consumed
        if (j + kSlots - 1 < nsub) {
            issue(j + kSlots - 1);
            __builtin_amdgcn_s_waitcnt(vmcnt_imm((kSlots - 1) * NL));
        } else if (j + 1 < nsub) {
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(NL));
        } else {
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        }
        const _Float16* Ks = slot_k(j);
        const _Float16* Vs = Ks + sub_halves<D>();
        // every kSegKeys keys the fp16 running sum moves into the fp32 carry
        if (j > 0 && j % (kSegKeys / kSub) == 0) fold_segment(st);
        f16v S[1];
        S[0] = qk_subtile_sw<D>(Ks, 0, qreg, n, hh);
        xdl_fence(S[0]);   // the softmax's maxima read the product directly
        const int wbase = kbeg + j * kSub;
        const bool full = wbase + kSub <= kend;
        const int cnt = full ? kSub : kend - wbase;
        h2 P[8];
        _Float16 alpha;
        if (full)
            alpha = softmax_block<1, false>(S, P, st, c, true, kSub, [](int, int) { return true; });
        else
            alpha = softmax_block<1, false>(S, P, st, c, false, cnt,
                                            [&](int, int r) { return key_of(r, hh) < cnt; });
        if (wave_any(alpha != (_Float16)1)) {
            const float af = (float)alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc[dt] *= af;
            st.lc *= af;
        }
        pv_chunks_tr<D, 2>(Vs, 0, P, acc, lane);
    }

    // ---- this split's normalised partial (fp32)
    if (row_valid) {
        const float L = row_sum<false>(st);
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        const int64_t prow = ((int64_t)b * Hq + hq) * nsplit + split;
        float* orow = o_part + prow * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f4 t = {acc[dt][4 * g + 0] * inv, acc[dt][4 * g + 1] * inv,
                              acc[dt][4 * g + 2] * inv, acc[dt][4 * g + 3] * inv};
                *(f4*)(orow + 32 * dt + 8 * g + 4 * hh) = t;
            }
        if (hh == 0)
            lse_part[prow] = L > 0.0f ? (st.R + __builtin_log2f(L)) * kLn2 : -__builtin_inff();
    }
}

// Up to kFast splits per row are combined from registers: every partial of
// the row (its lse and this thread's o column) is loaded in one round of
// independent loads before any arithmetic; more splits take the general loop.
constexpr int kFast = 8;

__global__ __launch_bounds__(128) void decode_combine_kernel(
    const float* __restrict__ o_part, const float* __restrict__ lse_part,
    _Float16* __restrict__ o, float* __restrict__ lse, int D, int nsplit) {
    const int64_t row = blockIdx.x;   // b * Hq + hq
    const float* lp = lse_part + row * nsplit;
    const float* op = o_part + row * nsplit * D;
    const int d = threadIdx.x;
    const bool col = d < D;
    float M = -__builtin_inff(), L, val = 0.0f;
    if (nsplit <= kFast) {
        float lv[kFast], ov[kFast];
#pragma unroll
        for (int s = 0; s < kFast; ++s) {
            lv[s] = s < nsplit ? lp[s] : -__builtin_inff();
            ov[s] = (s < nsplit && col) ? op[s * D + d] : 0.0f;
        }
#pragma unroll
        for (int s = 0; s < kFast; ++s) M = fmaxf(M, lv[s]);
        float sum = 0.0f;
        if (M != -__builtin_inff())
#pragma unroll
            for (int s = 0; s < kFast; ++s) sum += s < nsplit ? expf(lv[s] - M) : 0.0f;
        L = M != -__builtin_inff() ? M + logf(sum) : -__builtin_inff();
        if (M != -__builtin_inff())
#pragma unroll
            for (int s = 0; s < kFast; ++s)
                if (s < nsplit) val += expf(lv[s] - L) * ov[s];
    } else {
        for (int s = 0; s < nsplit; ++s) M = fmaxf(M, lp[s]);
        float sum = 0.0f;
        if (M != -__builtin_inff())
            for (int s = 0; s < nsplit; ++s) sum += expf(lp[s] - M);
        L = M != -__builtin_inff() ? M + logf(sum) : -__builtin_inff();
        if (M != -__builtin_inff() && col)
            for (int s = 0; s < nsplit; ++s) val += expf(lp[s] - L) * op[s * D + d];
    }
    if (col) o[row * D + d] = (_Float16)val;
    if (lse != nullptr && d == 0) lse[row] = L;
}

template <int D, bool PAGED>
hipError_t launch_split(const DecodeArgs& a, const Paging& pg, hipStream_t stream) {
    auto kern = decode_split_kernel<D, PAGED>;
    constexpr int smem = dec_smem_bytes<D>();
    static_assert(smem <= 64 * 1024, "dynamic LDS above 64 KB would need an opt-in");
    // seqlen_kv is the (upper bound of the) key count the splits are cut from
    const int subs = (a.seqlen_kv + kSub - 1) / kSub;
    const int per_split = (subs + a.num_splits - 1) / a.num_splits;
    const int head_chunks = (a.gqa_group + 31) / 32;
    const int64_t waves = (int64_t)a.batch * (a.num_heads_q / a.gqa_group) * head_chunks * a.num_splits;
    hipLaunchKernelGGL(kern, dim3((unsigned)waves), dim3(64), smem, stream,
                       (const _Float16*)a.q, (const _Float16*)a.k, (const _Float16*)a.v,
                       a.o_part, a.lse_part, a.seqlen_kv, a.num_heads_q, a.gqa_group,
                       a.softmax_scale * kLog2e, per_split * kSub, head_chunks, a.num_splits, pg);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_split(const DecodeArgs& a, hipStream_t stream) {
    const Paging none{nullptr, nullptr, 0, 0, 0};
    return a.head_dim == 128 ? launch_split<128, false>(a, none, stream)
                             : launch_split<64, false>(a, none, stream);
}

hipError_t launch_decode_split_paged(const DecodeArgs& a, const int* block_table,
                                     const int* seq_lens, int page_size, int max_pages,
                                     int num_pages, hipStream_t stream) {
    const Paging pg{block_table, seq_lens, page_size, max_pages, num_pages};
    return a.head_dim == 128 ? launch_split<128, true>(a, pg, stream)
                             : launch_split<64, true>(a, pg, stream);
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
