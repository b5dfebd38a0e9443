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
// Work decomposition (one workgroup = 8 waves = 256 query rows of one head):
//   * Two groups of four waves (rows 0-127 and 128-255 of the tile) share the
//     K/V tiles in LDS and run in ping-pong: while one group issues its matrix
//     products for a key block (P V of the previous block, then S^T = K Q^T of
//     this one), the other group runs the half-precision softmax of its
//     current block, and at every phase boundary they swap (a barrier ends
//     every odd phase, and at head_dim 64 every phase).  Each SIMD holds one wave
//     of each group, so the matrix cores and the vector ALUs stay busy at the
//     same time; the wave in its matrix phase runs at raised priority.
//   * S^T = K Q^T on the matrix cores (v_mfma_f32_32x32x16_f16).  Q is the B
//     operand and stays in registers for the whole key loop; K rows come from
//     LDS.  With keys on the M side, each lane holds 32 of the 64 scores of ONE
//     query row per key block, so row reductions are in-lane plus a single
//     exchange with the lane 32 apart.
//   * O^T += V^T P^T on the matrix cores.  The fp16 P tile produced by the
//     softmax is already laid out as the B operand (no LDS round trip): the K
//     rows are fed to the first product in a permuted order (bits 2 and 3 of
//     the row index swapped) so that every lane's scores are 8 consecutive
//     keys per 16-key chunk.
//   * K and V tiles go straight from HBM into LDS (buffer_load ... lds, no
//     staging registers; rows past the sequence end read as zero), stored
//     row-major with XOR-swizzled 16-byte chunks.  V is consumed through the
//     transposing LDS read of gfx950 (ds_read_b64_tr_b16).  Two LDS stages per
//     tensor; a block's K loads have two phases to land, its V loads one.
//   * Workgroups are ordered so that each XCD (each with its own L2) works on
//     one key/value head at a time, and causal tiles are issued longest first.
//   * Blocks that every row of a wave sees in full take a branch-free path;
//     only the diagonal / ragged-tail blocks evaluate the mask.
//   * The epilogue stages each wave's normalised fp16 rows in the (by then
//     free) LDS stages and writes whole rows with 16-byte stores.
//
// The per-block half-precision softmax (pseudo-average shift, refine, fp16
// exponentials and sums) lives in pasa_tile.hpp.  Each head dim is compiled
// in its own translation unit (pasa_fwd_d64.hip, pasa_fwd_d128.hip), so that
// the build can give each its own compiler scheduling options.
#pragma once

#include "kernels.hpp"
#include "pasa_tile.hpp"
#include "pasa_validate.hpp"

namespace pasa {

namespace {

constexpr int kBR = 256;      // query rows per workgroup (32 per wave)
// keys per block: 64 at head_dim 128, 128 at head_dim 64 (the same K/V tile
// bytes; at head_dim 64 the matrix work per key halves, so the longer block
// spreads the per-block vector work over more keys)
template <int D>
constexpr int kBCof() { return D == 64 ? 128 : 64; }
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kXcds = 8;      // XCDs of an MI355X; workgroups are dealt round-robin

template <int D>
constexpr int tile_halves() { return kBCof<D>() * D; }
template <int D>
constexpr int fwd_smem_bytes() { return 2 /*stages*/ * 2 /*K,V*/ * tile_halves<D>() * 2; }

// Work item of workgroup L: (batch, query head, query tile).  Items are
// enumerated key/value head by key/value head, longest causal tile first,
// and dealt to XCDs so that each XCD holds one key/value head (or one slice
// of one) at a time when the counts allow it.  When they do not (the number
// of key/value units neither divides nor is a multiple of the XCD count),
// causal items go longest first across all units: with 12 units of the
// Qwen2-shaped causal prefill (batch 3) that took 394 us against 460 us
// unit by unit, bitwise-equal outputs.
struct Item { int b, hq, tile; };
__device__ __forceinline__ Item decode_item(int L, int N, int B, int Hq, int g, int nt, bool causal) {
    const int Hkv = Hq / g;
    const int U = B * Hkv;            // key/value units
    const int per_unit = g * nt;
    int unit, item;
    if (N % kXcds == 0 && kXcds % U == 0 && per_unit % (kXcds / U) == 0) {
        const int X = kXcds / U, xcd = L % kXcds, k = L / kXcds;
        unit = xcd / X;
        item = k * X + xcd % X;
    } else if (U % kXcds == 0) {
        const int xcd = L % kXcds, k = L / kXcds;
        unit = (k / per_unit) * kXcds + xcd;
        item = k % per_unit;
    } else if (causal) {
        // no XCD grouping fits: longest tile first across all units (unit by
        // unit, the last units' longest tiles would start last)
        const int rank = L / (U * g), rem = L % (U * g);
        unit = rem / g;
        item = rank * g + rem % g;
    } else {
        unit = L / per_unit;
        item = L % per_unit;
    }
    const int rank = item / g;
    Item it;
    it.b = unit / Hkv;
    it.hq = (unit % Hkv) * g + item % g;
    it.tile = causal ? nt - 1 - rank : rank;
    return it;
}

// KS (key split): a workgroup takes 128 query rows, and its two ping-pong
// groups hold the same rows and take the two halves of the key range, each
// staging its own K/V tiles; the epilogue merges the two partial results
// (running maximum, running sum, accumulator) in fp32 with the same
// log-sum-exp rule as the decode's combine (a half in which a row sees no key
// gets weight 0).  Twice the work items of half the length each: for problems
// whose 256-row items leave a partly idle last round of workgroups (e.g. 360
// items on 256 CUs), or whose longest causal items set the kernel's time.
template <int D, bool CAUSAL, int VAR, bool KS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_kernel(
    const _Float16* __restrict__ q, const _Float16* __restrict__ k,
    const _Float16* __restrict__ v, _Float16* __restrict__ o, float* __restrict__ lse,
    int B, int Sq, int Skv, int Hq, int group, float c, int n_qtiles) {
    constexpr bool NAIVE = VAR == kVarNaive;
    constexpr bool STRICT = VAR == kVarStrict;
    constexpr bool FP8 = VAR == kVarFp8;       // q and k are e4m3 bytes
    constexpr int EB = FP8 ? 1 : 2;            // bytes per q / k element
    constexpr int KK = D / 16;
    constexpr int DT = D / 32;
    constexpr int kBC = kBCof<D>();
    constexpr int NT = kBC / 32;               // 32-key sub-tiles per block
    // packed pairs whose exponentials the vector phase takes (the matrix phase
    // takes the rest): at head_dim 64 the matrix phase has half the products
    // per score, so all of them go to the vector phase
    constexpr int EV = D == 64 ? 8 * NT : 0;
    constexpr int kRows = KS ? kBR / 2 : kBR;   // query rows per workgroup
    constexpr int kGroupStages = KS ? 2 : 1;    // stage sets: one per group with KS
    __shared__ __attribute__((aligned(1024))) _Float16 smem[kGroupStages * fwd_smem_bytes<D>() / 2];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int grp = w >> 2;     // ping-pong group (wave-uniform)
    const int hh = lane >> 5;   // which half of the wave
    const int n = lane & 31;    // query column owned by this lane

    const Item it = decode_item(blockIdx.x, gridDim.x, B, Hq, group, n_qtiles, CAUSAL);
    const int hq = it.hq, b = it.b;
    const int Hkv = Hq / group;
    const int hkv = hq / group;
    const int q0 = it.tile * kRows;
    const int wr = KS ? (w & 3) : w;    // the wave's 32-row slot in the tile
    const int wrow0 = q0 + 32 * wr;     // first query row of this wave
    const int qi = wrow0 + n;

    const int64_t q_stride = (int64_t)Hq * D;
    const int64_t kv_stride = (int64_t)Hkv * D;
    const uint8_t* qb = (const uint8_t*)q + ((int64_t)b * Sq * Hq + hq) * D * EB;
    const uint8_t* kb = (const uint8_t*)k + ((int64_t)b * Skv * Hkv + hkv) * D * EB;
    const _Float16* vb = v + ((int64_t)b * Skv * Hkv + hkv) * D;
    const uint32_t slab_bytes = (uint32_t)(((int64_t)(Skv - 1) * kv_stride + D) * 2);
    const uint32_t stride_b = (uint32_t)(kv_stride * 2);

    // ---- key range of this workgroup and of this lane's row
    const int64_t shift = (int64_t)Skv - Sq;   // bottom-right causal alignment
    int kv_end = Skv;
    if (CAUSAL) {
        const int64_t last = (int64_t)min(q0 + kRows - 1, Sq - 1) + shift;
        kv_end = last < 0 ? 0 : (int)min<int64_t>(Skv, last + 1);
    }
    const int nblocks = (kv_end + kBC - 1) / kBC;
    // this wave's key blocks: [blk0, blk0 + nbl); with KS group 0 takes the
    // first half (the longer one when odd) and group 1 the rest
    const int nb0 = KS ? (nblocks + 1) / 2 : nblocks;
    const int blk0 = KS ? __builtin_amdgcn_readfirstlane(grp ? nb0 : 0) : 0;   // wave-uniform
    const int nbl = KS ? __builtin_amdgcn_readfirstlane(grp ? nblocks - nb0 : nb0) : nblocks;
    auto row_limit = [&](int row) -> int {   // keys [0, limit) are visible to row
        if (!CAUSAL) return Skv;
        const int64_t l = (int64_t)row + shift + 1;
        return (int)max<int64_t>(0, min<int64_t>(Skv, l));
    };
    const int lim = row_limit(qi);
    const int wave_lim_lo = row_limit(wrow0);
    const int wave_lim_hi = row_limit(wrow0 + 31);
    // local block index j of this wave's range
    auto active = [&](int j) { return j < nbl && (blk0 + j) * kBC < wave_lim_hi; };

    // 2 stages of K then 2 of V (with KS: per group, the group's own)
    const int sg = (KS && grp) ? 2 : 0;
    _Float16* const Kst = smem + sg * tile_halves<D>();
    _Float16* const Vst = smem + (2 * kGroupStages + sg) * tile_halves<D>();
    // LDS DMA constants of this wave, and the stages' LDS byte addresses.  A
    // phase's loads (with the key split, both groups' tiles) are issued by the
    // four waves of one group, by the group that has the time for it (each
    // choice measured against all eight waves issuing their own share, outputs
    // bitwise equal):
    //  * head_dim 128: the group entering its vector phase, so the group
    //    starting its products spends nothing on them (each wave runs both
    //    phases back to back; c2 0.5-1.4 %, key-split shapes 3-5 % faster);
    //  * head_dim 64: the group entering its matrix phase, which then waits
    //    about 1000 cycles at the barrier for the vector phase (c3 1.9 %, a
    //    non-split causal prefill 2.9 % faster).
    constexpr int kLoadWaves = kWaves / 2;
    const uint32_t w_u = __builtin_amdgcn_readfirstlane((uint32_t)(w & 3));
    const TileDma<D, kBC, kLoadWaves, false, FP8> kdma(FP8 ? (uint32_t)kv_stride : stride_b, w_u, lane);
    const TileDma<D, kBC, kLoadWaves, true> vdma(stride_b, w_u, lane);
    constexpr uint32_t kTileBytes = tile_halves<D>() * 2;
    const uint32_t k_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)Kst);
    const uint32_t v_lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)Vst);
    const uint32_t k_bytes = (uint32_t)(((int64_t)(Skv - 1) * kv_stride + D) * EB);
    // block b0 + j of the slab into stage j % 2 of the stage pair at klds / vlds
    auto load_k_at = [&](int b0, uint32_t klds, int j) {
        const uint32_t off = (uint32_t)((b0 + j) * kBC) * (uint32_t)(kv_stride * EB);   // < k_bytes
        kdma.issue(make_rsrc(kb + off, k_bytes - off), klds + (j & 1) * kTileBytes);
    };
    auto load_v_at = [&](int b0, uint32_t vlds, int j) {
        const uint32_t off = (uint32_t)((b0 + j) * kBC) * stride_b;
        vdma.issue(make_rsrc((const uint8_t*)vb + off, slab_bytes - off), vlds + (j & 1) * kTileBytes);
    };
    auto load_k = [&](int j) { load_k_at(blk0, k_lds, j); };   // local block j of this wave's range
    auto load_v = [&](int j) { load_v_at(blk0, v_lds, j); };
    // with the key split: the other group's range and stages
    constexpr bool kBothKS = KS;
    const int blk0_o = kBothKS ? __builtin_amdgcn_readfirstlane(grp ? 0 : nb0) : 0;
    const int nbl_o = kBothKS ? __builtin_amdgcn_readfirstlane(grp ? nb0 : nblocks - nb0) : 0;
    const uint32_t k_lds_o = kBothKS ? __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(lds_void*)(smem + (grp ? 0 : 2) * tile_halves<D>())) : 0;
    const uint32_t v_lds_o = kBothKS ? __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(lds_void*)(smem + (2 * kGroupStages + (grp ? 0 : 2)) * tile_halves<D>())) : 0;
    // block 0's K: with the key split each group its own, else group 0
    if (nbl > 0 && (KS || grp == 0)) load_k(0);

    // ---- Q operand: lane holds Q[qi][16*kk + 8*hh .. +7]
    h8 qreg[FP8 ? 1 : KK];
    v8i q8reg[FP8 ? D / 64 : 1];
    if constexpr (FP8) {
        // lane holds Q[qi][64*kk + 32*hh .. +31] (e4m3 bytes)
#pragma unroll
        for (int kk = 0; kk < D / 64; ++kk) {
            const uint8_t* src = qb + (int64_t)qi * q_stride + 64 * kk + 32 * hh;
            const u4 lo = qi < Sq ? *(const u4*)src : (u4){};
            const u4 hi = qi < Sq ? *(const u4*)(src + 16) : (u4){};
            q8reg[kk] = (v8i){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                              (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        }
    } else {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk)
            qreg[kk] = qi < Sq ? *(const h8*)((const _Float16*)qb + (int64_t)qi * q_stride + 16 * kk + 8 * hh)
                               : (h8){};
    }
    // S^T for the 32-key sub-tile at row0 of the staged K tile
    auto qk_sub = [&](const _Float16* Ks, int row0) __attribute__((always_inline)) {
        if constexpr (FP8)
            return qk_subtile_f8<D>((const uint8_t*)Ks, row0, q8reg, n, hh);
        else
            return qk_subtile_sw<D>(Ks, row0, qreg, n, hh);
    };

    RowState st;
    f16v acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = (f16v){};
    f16v S[NT];
    h2 P[8 * NT];          // exponent arguments X of a block, then its P in place
    _Float16 apend = 1;    // alpha of the block whose X is held in P

    // matrix phase of block j: S^T = K Q^T for block j with the exponentials
    // and row sums of block j-1 issued between the products, then P V for
    // block j-1, as one straight-line region whose LDS operand reads are kept
    // several products ahead of their use
    auto mphase_at = [&](int j, const _Float16* Ks, const _Float16* Vs) __attribute__((always_inline)) {
        __builtin_amdgcn_s_setprio(1);
        const bool pv = j >= 1 && active(j - 1);
        const bool qk = active(j);
        if constexpr (D == 128 && !FP8) {
            if (pv && qk) {
                // The same work as below, in slots placed by hand.  The kernel
                // holds all 256 registers, and with the key split the
                // compiler's own order kept only three K reads and one product
                // of V reads ahead, with the exponentials bunched in front of
                // the products (12 % slower; without the key split the slots
                // measure the same as its order).  Slot m issues the K read of
                // product m + 4 and S^T product m; slots 0-7 add four
                // exponentials of block j-1, ordered after the slot's product
                // by naming its result; the V reads run four products ahead,
                // from the last S^T slots on.  Products and exponentials are
                // the same as below, in the same order per accumulator.
                constexpr int NQ = NT * KK, NPV = 2 * NT * DT, AH = 4, AHV = 4;
                h8 kop[AH + 1], vop[AHV + 1];
                auto kread = [&](int m) { return k_operand<D>(Ks, 32 * (m / KK), m % KK, n, hh); };
                auto vread = [&](int p) { return v_operand_tr<D>(Vs, p / DT, p % DT, lane); };
#pragma unroll
                for (int m = 0; m < AH; ++m) kop[m] = kread(m);
                static_for<0, NQ>([&](auto mc) __attribute__((always_inline)) {
                    constexpr int m = decltype(mc)::value, t = m / KK, kk = m % KK;
                    if constexpr (m + AH < NQ) kop[(m + AH) % (AH + 1)] = kread(m + AH);
                    S[t] = mfma_32x32x16(kop[m % (AH + 1)], qreg[kk], kk == 0 ? (f16v){} : S[t]);
                    if constexpr (m < 4 * NT) hexp2_pk2_after(&P[2 * m], S[t]);
                    if constexpr (m >= NQ - AHV) vop[m - (NQ - AHV)] = vread(m - (NQ - AHV));
                    __builtin_amdgcn_sched_barrier(0);
                });
                softmax_exp<NT, NAIVE, 8 * NT>(P, st, apend);   // the row sum
                static_for<0, NPV>([&](auto pc) __attribute__((always_inline)) {
                    constexpr int p = decltype(pc)::value;
                    if constexpr (p + AHV < NPV) vop[(p + AHV) % (AHV + 1)] = vread(p + AHV);
                    acc[p % DT] = mfma_32x32x16(vop[p % (AHV + 1)], p_operand(P, p / DT), acc[p % DT]);
                    __builtin_amdgcn_sched_barrier(0);
                });
                __builtin_amdgcn_s_setprio(0);
                return;
            }
        }
        if (pv && qk) {
#pragma unroll
            for (int t = 0; t < NT; ++t) S[t] = qk_sub(Ks, 32 * t);
            softmax_exp<NT, NAIVE, EV>(P, st, apend);
            pv_chunks_tr<D, 2 * NT>(Vs, 0, P, acc, lane);
            // Operand reads are kept AHEADM products ahead of the product that
            // consumes them, across the boundary between the two products: the
            // V reads of the first P V products go out under the last S^T
            // products
            constexpr int NQKM = FP8 ? NT * (D / 64) : NT * (D / 16);   // S^T products
            constexpr int RQ = FP8 ? 2 : 1;                             // K reads per S^T product
            constexpr int NPV = 2 * NT * (D / 32);                      // P V products, 2 V reads each
            constexpr int AHEADM = 8;
            constexpr int FIRST = AHEADM <= NQKM ? AHEADM * RQ : NQKM * RQ + 2 * (AHEADM - NQKM);
            __builtin_amdgcn_sched_group_barrier(0x100, FIRST, 0);
#pragma unroll
            for (int m = 0; m < NQKM + NPV; ++m) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                const int nx = m + AHEADM;   // product whose operands are read next
                if (nx < NQKM) {
                    if (RQ == 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    else __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                } else if (nx < NQKM + NPV) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                }
            }
        } else {
            if (pv) {
                softmax_exp<NT, NAIVE, EV>(P, st, apend);
                pv_chunks_tr<D, 2 * NT>(Vs, 0, P, acc, lane);
            }
            if (qk) {
                // no P V products follow these (first block): fence the
                // results before the vector phase's maxima read them
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    S[t] = qk_sub(Ks, 32 * t);
                    xdl_fence(S[t]);
                }
            }
        }
        __builtin_amdgcn_s_setprio(0);
    };
    // one copy of the matrix phase per stage parity, so that the stages' LDS
    // addresses are constants of each copy
    auto mphase = [&](int j) {
        if (j & 1) mphase_at(j, Kst + tile_halves<D>(), Vst);
        else mphase_at(j, Kst, Vst + tile_halves<D>());
    };
    // vector phase of block j: the shift, the fp16 tile and its exponent
    // arguments; the accumulator rescale the new running maximum calls for
    // dma: the phase's loads when this wave's group issues them (at head_dim
    // 128), issued with the tile: in each of the three paths (no visible key,
    // whole block, diagonal block) the compiler puts them after the path's
    // tests and ahead of the maxima.  Issued there instead of ahead of the
    // phase's tests, c2 ran 1.7-2.2 % faster, c4 0.8-1.4 % (same process,
    // outputs bitwise equal).
    auto vphase = [&](int j, auto&& dma) {
        if (!active(j)) {
            dma();
            return;
        }
        // every kSegKeys keys the fp16 running sum (complete up to block j-1,
        // whose sum the matrix phase just added) moves into the fp32 carry
        if (!NAIVE && j > 0 && j % (kSegKeys / kBC) == 0) fold_segment(st);
        const int kbase = (blk0 + j) * kBC;
        _Float16 d;
        if (kbase + kBC <= wave_lim_lo) {   // the whole block is visible to the wave
            auto all = [](int, int) { return true; };
            d = softmax_tile<NT, NAIVE, decltype(all), STRICT>(S, P, st, c, true, kBC, all, dma);
        } else {
            const int m = lim - kbase;        // keys [0, m) of the block are visible
            const int cnt = max(0, min(kBC, m));
            auto vis = [&](int t, int r) { return 32 * t + key_of(r, hh) < m; };
            d = softmax_tile<NT, NAIVE, decltype(vis), STRICT>(S, P, st, c, false, cnt, vis, dma);
        }
        apend = hexp2(d);
        exp_pairs<0, EV>(P);
        if (wave_any(apend != (_Float16)1)) {
            const float af = (float)apend;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc[dt] *= af;
            st.lc *= af;
        }
    };

    wait_vmem();
    __syncthreads();

    // Phase p: group 0 runs mphase(p/2) on even p and vphase(p/2) on odd p;
    // group 1 runs one phase behind.  K(m+1) is loaded from phase 2m and V(m)
    // from phase 2m+1 (spreading the loads' issue over both phases), into the
    // stages freed by K(m-1) and V(m-2); both have landed by the barrier that
    // ends phase 2m+1, before either is read (the waves that issued them wait
    // for their loads before it).  The group in its matrix phase is group
    // p % 2; which group issues is chosen above.
    const int nphase = nb0 > 0 ? 2 * nb0 + 2 : 0;   // nb0: the longer of the ranges
    for (int p = 0; p < nphase; ++p) {
        auto dma = [&]() __attribute__((always_inline)) {
            const int m = p >> 1;
            if ((p & 1) == 0) {
                if (m + 1 < nbl) load_k(m + 1);
                if (kBothKS && m + 1 < nbl_o) load_k_at(blk0_o, k_lds_o, m + 1);
            } else {
                if (m < nbl) load_v(m);
                if (kBothKS && m < nbl_o) load_v_at(blk0_o, v_lds_o, m);
            }
        };
        const int pp = p - grp;   // this group's own phase index
        if constexpr (D == 128) {
            if (pp >= 0 && (pp & 1)) vphase(pp >> 1, dma);   // the issuing group: its loads go out with the tile
            else if (pp >= 0) mphase(pp >> 1);
            else dma();   // group 1's first phase: nothing to compute, the loads to issue
        } else {
            // head_dim 64: the vector-phase wave (the binding one) takes one
            // test; the loads go out from group p % 2, in its matrix phase.
            // In phase 0, group 1, still idle, issues the same loads as group
            // 0 (identical bytes into the same stage, which nobody reads
            // before the barrier that ends phase 1, where both have waited
            // for their loads).  Keeping it out with one more test lays the
            // loop out differently: 3-8 % slower against 5-6 % faster on the
            // key-split shapes (same process, outputs bitwise equal).
            if (pp >= 0 && (pp & 1)) {
                vphase(pp >> 1, NoPre{});
            } else {
                dma();
                if (pp >= 0) mphase(pp >> 1);
            }
        }
        // The barrier after an odd phase orders the LDS stages: the DMA into a
        // stage has landed before anyone reads it, and every read of a stage
        // is done before the next even phase refills it.  The barrier after an
        // even phase only keeps the two groups in step; at head_dim 128 the
        // groups stay in step on their own and the barrier costs more than it
        // saves (c2 138.4 -> 133.9 us), at head_dim 64 it pays.
        if (p & 1) {
            wait_vmem();
            __syncthreads();
        } else if (D == 64) {
            __syncthreads();
        }
    }

    // ---- epilogue: global recovering
    constexpr int NV = DT * 16 + 2;                        // floats per lane handed over with KS
    constexpr int kMergeHalves = KS ? 4 * NV * 64 * 2 : 0;  // LDS the hand-over takes (halves)
    float Lf = row_sum<NAIVE>(st);   // running sum, relative to 2^Rf
    float Rf = st.R;
    if constexpr (KS) {
        // merge the two key halves: group 1 hands its partial to its partner
        // wave of group 0 through LDS (the stages are free after the last
        // barrier), which rescales both to the larger maximum and adds them
        float* const mb = (float*)smem + (w & 3) * (NV * 64);
        if (grp == 1) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) mb[(16 * dt + r) * 64 + lane] = acc[dt][r];
            mb[(NV - 2) * 64 + lane] = Rf;
            mb[(NV - 1) * 64 + lane] = Lf;
        }
        __syncthreads();
        if (grp == 1) return;
        const float R1 = mb[(NV - 2) * 64 + lane];
        const float L1 = mb[(NV - 1) * 64 + lane];
        const float R = fmaxf(Rf, R1);
        const bool any = R != -__builtin_inff();
        const float a0 = any ? __builtin_amdgcn_exp2f(Rf - R) : 0.0f;   // 0 for a half with no key
        const float a1 = any ? __builtin_amdgcn_exp2f(R1 - R) : 0.0f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[dt][r] = acc[dt][r] * a0 + mb[(16 * dt + r) * 64 + lane] * a1;
        Lf = Lf * a0 + L1 * a1;
        Rf = R;
    }
    // The K/V stages are free after the last barrier, so each wave stages its
    // normalised fp16 rows in its own 32*D halves of LDS (16-byte chunks
    // XOR-swizzled by row) and then writes whole rows: 16-byte stores, D/8
    // lanes per row, instead of scattered 8-byte ones.
    {
        constexpr int C = D / 8;   // 16-byte chunks per row
        const float L = Lf;
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        _Float16* const stg = smem + kMergeHalves + wr * (32 * D);   // past the hand-over
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const h4 t = {(_Float16)(acc[dt][4 * g + 0] * inv), (_Float16)(acc[dt][4 * g + 1] * inv),
                              (_Float16)(acc[dt][4 * g + 2] * inv), (_Float16)(acc[dt][4 * g + 3] * inv)};
                const int ch = 4 * dt + g;   // columns 32*dt + 8*g .. +7; this lane's 4 at +4*hh
                *(h4*)(stg + n * D + 8 * (ch ^ (n & (C - 1))) + 4 * hh) = t;
            }
#pragma unroll
        for (int i = 0; i < C / 2; ++i) {
            const int slot = 64 * i + lane;
            const int row = slot / C, ch = slot % C;
            const h8 val = *(const h8*)(stg + row * D + 8 * (ch ^ (row & (C - 1))));
            if (wrow0 + row < Sq)
                *(h8*)(o + ((int64_t)b * Sq + wrow0 + row) * q_stride + (int64_t)hq * D + 8 * ch) = val;
        }
        if (lse != nullptr && hh == 0 && qi < Sq)
            lse[((int64_t)b * Hq + hq) * Sq + qi] =
                L > 0.0f ? (Rf + __builtin_log2f(L)) * kLn2 : -__builtin_inff();
    }
}

template <int D, bool CAUSAL, int VAR, bool KS>
hipError_t launch_one(const FwdArgs& a, hipStream_t stream) {
    auto kern = fwd_kernel<D, CAUSAL, VAR, KS>;
    static_assert((KS ? 2 : 1) * fwd_smem_bytes<D>() <= 160 * 1024, "LDS of one CU");
    constexpr int rows = KS ? kBR / 2 : kBR;
    const int n_qtiles = (int)(((int64_t)a.seqlen_q + rows - 1) / rows);   // item count checked by the ABI
    const int64_t n_items = (int64_t)a.batch * a.num_heads_q * n_qtiles;
    hipLaunchKernelGGL(kern, dim3((unsigned)n_items), dim3(kThreads), 0, stream,
                       (const _Float16*)a.q, (const _Float16*)a.k, (const _Float16*)a.v,
                       (_Float16*)a.o, a.lse, a.batch, a.seqlen_q, a.seqlen_kv, a.num_heads_q,
                       a.gqa_group, a.softmax_scale * a.qk_dequant * kLog2e, n_qtiles);
    return hipGetLastError();
}

// The item shape (pasa::validate::fwd_key_split) on this device's compute
// units.  A causal choice simulates the dealing of up to 8 * CUs items, about
// 20 us of host time, so each thread keeps the last shape's choice (and each
// device's unit count): a repeated launch costs a comparison.
struct SplitKey {
    int dev, b, sq, skv, hq, d, causal;
    bool operator==(const SplitKey& o) const {
        return dev == o.dev && b == o.b && sq == o.sq && skv == o.skv && hq == o.hq && d == o.d &&
               causal == o.causal;
    }
};
bool use_key_split(const FwdArgs& a) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    static thread_local SplitKey last = {-1, 0, 0, 0, 0, 0, 0};
    static thread_local bool last_split = false;
    const SplitKey key = {dev, a.batch, a.seqlen_q, a.seqlen_kv, a.num_heads_q, a.head_dim, a.causal};
    if (key == last) return last_split;
    static thread_local int cu_dev = -1, cu_count = 0;
    if (dev != cu_dev) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
            return false;
        cu_dev = dev;
        cu_count = n;
    }
    last_split = validate::fwd_key_split(a.batch, a.seqlen_q, a.seqlen_kv, a.num_heads_q, a.head_dim,
                                         a.causal, cu_count);
    last = key;
    return last_split;
}

template <int D, int VAR>
hipError_t launch_causal_or_not(const FwdArgs& a, hipStream_t stream) {
    const bool ks = use_key_split(a);
    if (a.causal) return ks ? launch_one<D, true, VAR, true>(a, stream) : launch_one<D, true, VAR, false>(a, stream);
    return ks ? launch_one<D, false, VAR, true>(a, stream) : launch_one<D, false, VAR, false>(a, stream);
}

template <int D>
hipError_t launch_var(const FwdArgs& a, int variant, hipStream_t stream) {
    if (variant == kVarNaive) return launch_causal_or_not<D, kVarNaive>(a, stream);
    if (variant == kVarStrict) return launch_causal_or_not<D, kVarStrict>(a, stream);
    if (variant == kVarFp8) return launch_causal_or_not<D, kVarFp8>(a, stream);
    return launch_causal_or_not<D, kVarPasa>(a, stream);
}

}  // namespace

}  // namespace pasa
