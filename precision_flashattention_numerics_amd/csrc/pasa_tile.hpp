// Building blocks shared by the PASA prefill and decode kernels: K/V staging
// into LDS, and the per-block half-precision softmax with online
// pseudo-average shifting.
//
// Method: "Online Pseudo-average Shifting Attention (PASA) for Robust
// Low-precision LLM Inference", Abstract (online pseudo-average shifting,
// half-precision Flash-Attention process, global recovering).  The page gives
// no equations; the per-row rules below are this library's reading of it:
//
//   mu    = mean of the row's visible scores S in the block         (fp32)
//   off   = c*mu on the row's first visible block, else max(c*mu, R) (fp32)
//   m_b   = fp16_rne(c*max_j S - off), the largest entry of the
//           shifted fp16 tile                                          (fp16)
//   if m_b > THETA (the tile's largest entries would sit where fp16 is
//   coarse, or overflow): off = max_j c*S over visible keys, and m_b is
//   taken relative to that instead
//   R'    = max(R, off + m_b)      running maximum, log2 units        (fp32)
//   s     = fp16(R' - off)                                            (fp16)
//   X     = fp16_rne(fp32(c*S - (off + s))), masked keys -> -inf
//   P     = exp2(X);  r = sum_j P                                     (fp16)
//   alpha = exp2(fp16(R - R'))                                        (fp16)
//   (l_hi, l_lo) <- compensated fp16 sum of alpha*(l_hi, l_lo) + r    (fp16)
//   every 32768 keys: l_c <- l_c + (l_hi + l_lo), (l_hi, l_lo) <- 0;
//   l_c <- alpha*l_c on every block                                    (fp32)
// where c = scale * log2(e).  X is the shifted tile fp16(c*S - off) moved
// down by s, formed straight from the fp32 score (s is known before the tile
// is formed).  Because X is taken against off + s, P = exp2(c*S - R') up to
// rounding whatever off was: the shift changes only which fp16 numbers are
// formed, never the softmax (a per-row shift leaves softmax unchanged).  The
// epilogue recovers the exact log-sum-exp as ln2 * (R + log2(L)) with
// L = l_c + l_hi + l_lo.
//
// The naive variant rounds the UNSCALED S to fp16, scales it in fp16 and
// keeps a plain running maximum: a half-precision Flash Attention without the
// shift, which overflows when |QK^T| > 65504.
#pragma once

#include "device_common.hpp"

namespace pasa {

constexpr float kTheta = 4.0f;   // refine threshold on the tile maximum (log2 units)

// Row permutation applied to K when it feeds S^T = K Q^T: swaps bits 2 and 3
// of the row index, so lane l's 16 scores of a 32-key sub-tile are the keys
// 16*(r/8) + 8*(l/32) + (r%8): two runs of 8 consecutive keys, which is the
// B-operand layout of the following P V product.
__device__ __forceinline__ int sigma(int n) {
    return (n & ~0xC) | ((n & 4) << 1) | ((n & 8) >> 1);
}

// Key offset (within a 32-key sub-tile) of accumulator register r of lane
// half hh (= lane / 32).
__device__ __forceinline__ int key_of(int r, int hh) {
    return 16 * (r >> 3) + 8 * hh + (r & 7);
}

// Compensated fp16 accumulation (hi, lo) <- alpha * (hi, lo) + r: a
// two-sum in fp16 carries the rounding error of each addition in lo.
__device__ __forceinline__ void comp_add(_Float16& hi, _Float16& lo, _Float16 alpha, _Float16 r) {
#pragma clang fp contract(off)
    _Float16 a = alpha * hi;
    _Float16 b = alpha * lo;
    _Float16 s = a + r;
    _Float16 bb = s - a;
    _Float16 err = (a - (s - bb)) + (r - bb);
    hi = s;
    lo = b + err;
}

struct RowState {
    float R = -__builtin_inff();   // running maximum of c*S (log2 units)
    _Float16 lhi = 0, llo = 0;     // running sum (PASA): compensated fp16 pair
    float lsum = 0.0f;             // running sum (naive): fp32
    float lc = 0.0f;               // PASA: the running sums of completed key segments
};

// Keys per segment of the PASA running sum.  The compensated fp16 pair sums at
// most this many exponentials (each at most 1 up to rounding, since every
// block is taken against its running maximum), then is folded into the fp32
// carry `lc`: partial sums over disjoint key ranges taken against one running
// maximum add ("Block Sparse Flash Attention" topic page, FoldAttention card:
// normalised partials over disjoint key ranges compose), so no sequence length
// can push the fp16 pair past 65504.  Each block's sum stays an fp16 sum.
constexpr int kSegKeys = 32768;

// Fold the compensated fp16 sum into the carry (at a segment boundary, when
// both hold sums against the same running maximum).
__device__ __forceinline__ void fold_segment(RowState& st) {
    st.lc += (float)st.lhi + (float)st.llo;
    st.lhi = 0;
    st.llo = 0;
}

// One key block of NT 32-key sub-tiles for the row held by this lane (and by
// the lane 32 apart, which holds the other half of the row's keys), in two
// steps that a kernel may run at different times:
//   softmax_tile  the shift and the fp16 exponent arguments X (the
//                 shifted tile less s); updates the running maximum and returns
//                 d = fp16(R - R') (0 when the row sees no key of the block)
//   softmax_exp   P = exp2(X) in place, the row sum r, and the running sum
//                 rescaled by alpha = exp2(d), the factor the caller also
//                 applies to its accumulator
// Arguments:
//   S       fp32 scores (unscaled q.k), register r of sub-tile t is key
//           32*t + key_of(r, hh) of the block
//   X / P   packed fp16 pairs, X[8*t + r/2] = keys r, r+1 of sub-tile t
//   full    every key of the block is visible to every row of the wave
//   cnt     number of keys of the block visible to this row
//   vis     vis(t, r) -> visibility of that key (used only when !full)
//
// The tile maximum m_b = max_j fp16(c*S_j - off) equals fp16(c*max_j S_j - off)
// because rounding to fp16 is monotone; it is therefore taken from one fp32
// max pass that runs beside the pseudo-average sum, and the refine decision
// (m_b > THETA -> centre at the row maximum) is made before any fp16 entry is
// formed, so the exponent arguments are formed exactly once and without a
// branch.
//
// STRICT (PASA only) also holds the running maximum R and the offset off in
// fp16: each is rounded to fp16 where it is formed, and R' = max(R, off + m_b)
// is an fp16 addition.  This is usable while |c * score| stays well inside
// the fp16 range (about 3.2e4): the rounding of R (ulp 16 there) moves the
// largest P of a block up to 2^8 above 1.
// pre: work of the caller issued with the tile (the prefill's vector-phase
// wave passes its phase's K/V loads); the compiler places it at the start of
// the tile's code, ahead of the maxima.
struct NoPre {
    __device__ __forceinline__ void operator()() const {}
};
template <int NT, bool NAIVE, typename Vis, bool STRICT = false, typename Pre = NoPre>
__device__ __forceinline__ _Float16 softmax_tile(const f16v (&S)[NT], h2 (&X)[8 * NT],
                                                 RowState& st, float c, bool full, int cnt,
                                                 Vis vis, Pre pre = {}) {
    static_assert(!(STRICT && NAIVE), "the strict variant is a PASA variant");
    auto r16 = [](float x) { return STRICT ? (float)(_Float16)x : x; };
    _Float16 mb;
    float off = 0.0f;
    if (!NAIVE) {
        // four independent partial maxima keep the dependency chains short;
        // each starts from the sub-tile's first scores
        float pm[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) pm[r] = (full || vis(0, r)) ? S[0][r] : -__builtin_inff();
        // maxima two scores at a time (v_max3_f32 on the raw products: no
        // NaN canonicalisation is needed for them)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            constexpr int NV = 4 * NT - 1;        // chain k: scores r = k mod 4 past the first
            float vv[NV];
            int nv = 0;
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int r = k; r < 16; r += 4) {
                    if (t == 0 && r == k) continue;
                    vv[nv++] = (full || vis(t, r)) ? S[t][r] : -__builtin_inff();
                }
#pragma unroll
            for (int i = 0; i + 1 < NV; i += 2) pm[k] = max3f(pm[k], vv[i], vv[i + 1]);
            if (NV & 1) pm[k] = max3f(pm[k], vv[NV - 1], vv[NV - 1]);
        }
        const float m32 = xmax32(max3f(pm[0], pm[1], max3f(pm[2], pm[3], pm[3])));
        // The pseudo-average never exceeds the block maximum, so max(c*mu, R)
        // is R wherever c*max <= R; the mean is formed only when some row of
        // the wave has c*max above R (the margin covers the rounding of the
        // mean's sum: at most 128 terms, each at most the maximum).  This
        // gives the same offsets as always forming it.  The strict variant's
        // fp16 rounding of c*mu can exceed c*max, so it always forms it.
        const float cm = c * m32;
        const bool may = cnt > 0 && !(cm + __builtin_fabsf(cm) * 0x1p-16f < st.R);
        if (STRICT || wave_any(may)) {
            float ps[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) ps[r] = (full || vis(0, r)) ? S[0][r] : 0.0f;
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int r = (t == 0 ? 4 : 0); r < 16; ++r) {
                    const bool on = full || vis(t, r);
                    ps[r & 3] += on ? S[t][r] : 0.0f;
                }
            const float sum = xsum32((ps[0] + ps[1]) + (ps[2] + ps[3]));
            const float cmu = cnt > 0 ? r16(c * (sum / (float)cnt)) : st.R;
            off = (st.R == -__builtin_inff()) ? cmu : fmaxf(cmu, st.R);
        } else {
            off = st.R;
        }
        mb = fma_to_h(m32, c, -off);
        // refine: the tile's largest entries would sit where fp16 is coarse
        // (or overflow); centre the row at its own maximum instead
        if (cnt > 0 && !(mb <= (_Float16)kTheta)) {
            off = r16(c * m32);
            mb = fma_to_h(m32, c, -off);
        }
        // the running maximum and s are known at this point, so the exponent
        // argument (the shifted tile less s) is formed directly from the fp32
        // score: X = fp16(fp32(c*S - (off + s))), an fp32 fused multiply-add
        // and a packed round-to-nearest-even convert.  The fp32 step keeps 13
        // bits more than fp16, so X equals the single rounding of the exact
        // value except in rare near-ties, where it is one fp16 step off (in
        // either direction).  Both instructions issue at a higher rate than the
        // mixed-precision FMA that would round once.
        const float top = STRICT ? (float)((_Float16)off + mb) : off + (float)mb;
        const float Rn = cnt > 0 ? fmaxf(st.R, top) : st.R;
        const _Float16 s = cnt > 0 ? (_Float16)(Rn - off) : (_Float16)0;
        const float noff = -(off + (float)s);
        pre();
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                h2 x = to_h2(__builtin_fmaf(S[t][r], c, noff), __builtin_fmaf(S[t][r + 1], c, noff));
                if (!full) {
                    if (!vis(t, r)) x.x = kHalfNegInf;
                    if (!vis(t, r + 1)) x.y = kHalfNegInf;
                }
                X[8 * t + r / 2] = x;
            }
        const _Float16 d = cnt > 0 ? (_Float16)(st.R - Rn) : (_Float16)0;
        st.R = Rn;
        return d;
    } else {
        const _Float16 ch = (_Float16)c;
        h2 mm = (h2){kHalfNegInf, kHalfNegInf};
        pre();
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                h2 x = to_h2(S[t][r], S[t][r + 1]) * (h2){ch, ch};
                if (!full) {
                    if (!vis(t, r)) x.x = kHalfNegInf;
                    if (!vis(t, r + 1)) x.y = kHalfNegInf;
                }
                X[8 * t + r / 2] = x;
                mm = hmax(mm, x);
            }
        mb = xmax32(mm.x > mm.y ? mm.x : mm.y);
    }

    const float top = STRICT ? (float)((_Float16)off + mb) : off + (float)mb;
    const float Rn = cnt > 0 ? fmaxf(st.R, top) : st.R;
    const _Float16 s = cnt > 0 ? (_Float16)(Rn - off) : (_Float16)0;
    const h2 s2 = {s, s};
#pragma unroll
    for (int i = 0; i < 8 * NT; ++i) X[i] = X[i] - s2;
    const _Float16 d = cnt > 0 ? (_Float16)(st.R - Rn) : (_Float16)0;
    st.R = Rn;
    return d;
}

// P = exp2(X) in place for the packed pairs [FIRST, LAST) of a block
// (multiples of 4).
template <int FIRST, int LAST>
__device__ __forceinline__ void exp_pairs(h2* P) {
#pragma unroll
    for (int i = FIRST; i < LAST; i += 4) hexp2_pk4(P + i);
}

// FIRST: pairs [0, FIRST) were already exponentiated by the caller.
template <int NT, bool NAIVE, int FIRST = 0>
__device__ __forceinline__ void softmax_exp(h2 (&P)[8 * NT], RowState& st, _Float16 alpha) {
    exp_pairs<FIRST, 8 * NT>(P);

    // fp16 pairwise tree sum of the lane's exponentials, then across halves
    h2 a[4 * NT];
#pragma unroll
    for (int i = 0; i < 4 * NT; ++i) a[i] = P[2 * i] + P[2 * i + 1];
#pragma unroll
    for (int w = 2 * NT; w >= 1; w >>= 1)
#pragma unroll
        for (int i = 0; i < w; ++i) a[i] = a[2 * i] + a[2 * i + 1];
    const _Float16 rsum = xsum32((_Float16)(a[0].x + a[0].y));

    if (!NAIVE)
        comp_add(st.lhi, st.llo, alpha, rsum);
    else
        st.lsum = (float)alpha * st.lsum + (float)rsum;
}

// Both steps back to back.
template <int NT, bool NAIVE, typename Vis>
__device__ __forceinline__ _Float16 softmax_block(const f16v (&S)[NT], h2 (&P)[8 * NT],
                                                  RowState& st, float c, bool full, int cnt,
                                                  Vis vis) {
    const _Float16 alpha = hexp2(softmax_tile<NT, NAIVE>(S, P, st, c, full, cnt, vis));
    softmax_exp<NT, NAIVE>(P, st, alpha);
    return alpha;
}

template <bool NAIVE>
__device__ __forceinline__ float row_sum(const RowState& st) {
    return NAIVE ? st.lsum : st.lc + ((float)st.lhi + (float)st.llo);
}

// ---------------------------------------------------------------------------
// Direct HBM -> LDS staging (buffer_load ... lds) with XOR-swizzled 16-byte
// chunks, and the matching operand reads.
//
// A tile is ROWS keys x D columns of fp16, stored row-major without padding;
// row r's 16-byte chunk c lives at chunk slot r*C + (c ^ swz(r)), C = D/8.
// K tiles use swz_k (conflict-free 16-byte reads of 16 different rows at one
// chunk); V tiles use swz_v (conflict-free transposing 8-byte reads of 4
// consecutive rows x 4 consecutive chunks).

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor (stride 0) over [base, base + bytes): reads past the
// bound return zero, which is how ragged tails are padded.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    return (i32x4){(int)(uint32_t)a, (int)(uint32_t)((a >> 32) & 0xFFFFu), (int)bytes, 0x00020000};
}

// One 16-byte-per-lane load from a buffer straight into LDS: lane l's bytes
// land at lds + 16*l, non-temporal (nt: the data is read once).  Inline
// assembly for the reason given at TileDma.
__device__ __forceinline__ void dma16_nt(i32x4 rsrc, uint32_t voff, const void* lds) {
    const uint32_t la = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(la)
                 : "memory", "m0");
}

template <int D>
__device__ __forceinline__ int swz_k(int r) {
    constexpr int C = D / 8;
    return (r / (16 / C)) % C;
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
    constexpr int C = D / 8;
    return 4 * ((r / (16 / C)) % (C / 4));
}

typedef __attribute__((address_space(3))) void lds_void;
typedef short s4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s4 lds_s4;

// The loads of keys [row0, row0 + ROWS) of one head's K or V slab into an LDS
// tile by one wave, non-temporal, with each lane's offset formed at the load
// (TileDma's layout; stride_b = bytes between consecutive keys of the slab).
// The contiguous decode stages its sub-tiles this way: measured against
// TileDma's precomputed offsets, it streams the decode workload about 4 %
// faster (the paged decode is the other way round).
template <int D, int ROWS, bool IS_V>
__device__ __forceinline__ void stage_tile_nt(i32x4 rsrc, uint32_t stride_b, int row0,
                                              _Float16* tile, int lane) {
    constexpr int C = D / 8;
    constexpr int SEGS = ROWS * C / 64;          // 1 KB segments in the tile
#pragma unroll
    for (int seg = 0; seg < SEGS; ++seg) {
        const int slot = seg * 64 + lane;
        const int row = slot / C, pos = slot % C;
        const int chunk = pos ^ (IS_V ? swz_v<D>(row) : swz_k<D>(row));
        const uint32_t off = (uint32_t)(row0 + row) * stride_b + (uint32_t)chunk * 16u;
        dma16_nt(rsrc, off, tile + seg * 512);
    }
}

// ---------------------------------------------------------------------------
// fp8 (e4m3) K tiles: ROWS rows x D one-byte columns.  Row r's 16-byte chunk c
// lives at chunk slot r*C8 + (c ^ swz_f8(r)), C8 = D/16; rows that share a
// bank window (their byte offsets are equal modulo 256) get distinct chunk
// positions, so 16 lanes reading one chunk of 16 consecutive rows touch all
// 64 banks once.
typedef int v8i __attribute__((ext_vector_type(8)));

template <int D>
__device__ __forceinline__ int swz_f8(int r) {
    constexpr int C8 = D / 16;
    return (r / (256 / D)) % C8;
}

// Staging of a ROWS-key tile straight from HBM into LDS (buffer_load ... lds,
// no staging registers), split over WAVES waves in 1 KB segments (64 lanes x
// 16 bytes; lane l's bytes land at the segment's LDS address + 16*l).
// Everything that does not change from one key block to the next is computed
// once, outside the key loop: each lane's byte offset inside a block (row,
// swizzled chunk) and each of this wave's segments' LDS byte offset inside a
// stage.  Per block the caller passes a descriptor that starts at the block's
// first key (bounded by the data's end, so rows past it read as zero) and the
// stage's LDS byte address; issuing a segment is then scalar moves and one
// load.  The loads are inline assembly on purpose: the compiler would
// otherwise wait for every such load before any later LDS read (it cannot
// tell the stages apart); the kernels order them with explicit vmcnt waits
// (and barriers where waves share a stage) before a stage is read.
// w_u is the wave index, wave-uniform.  F8: one-byte (e4m3) K tile in the fp8
// layout above.  STREAM marks the loads non-temporal (nt): for data read
// exactly once (the decode's KV cache), which streams from HBM markedly faster
// that way; tiles that other workgroups re-read through L2 (prefill K/V) keep
// the default.
template <int D, int ROWS, int WAVES, bool IS_V, bool F8 = false, bool STREAM = false>
struct TileDma {
    static constexpr int C = F8 ? D / 16 : D / 8;   // 16-byte chunks per row
    static constexpr int SEGS = ROWS * C / 64;   // 1 KB segments in the tile
    static constexpr int PER = SEGS / WAVES;
    static_assert(SEGS % WAVES == 0, "segments must split evenly over waves");
    uint32_t voff[PER];   // per lane: bytes from the block's first key
    uint32_t lds[PER];    // per wave: bytes from the stage's start

    __device__ __forceinline__ TileDma(uint32_t stride_b, uint32_t w_u, int lane) {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int seg = (int)w_u * PER + i;
            const int slot = seg * 64 + lane;
            const int row = slot / C, pos = slot % C;
            const int chunk = pos ^ (F8 ? swz_f8<D>(row) : IS_V ? swz_v<D>(row) : swz_k<D>(row));
            voff[i] = (uint32_t)row * stride_b + (uint32_t)chunk * 16u;
            lds[i] = (uint32_t)seg * 1024u;
        }
    }
    __device__ __forceinline__ void issue(i32x4 rsrc, uint32_t stage_lds) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            if constexpr (STREAM)
                asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds"
                             :
                             : "v"(voff[i]), "s"(rsrc), "s"(stage_lds + lds[i])
                             : "memory", "m0");
            else
                asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                             :
                             : "v"(voff[i]), "s"(rsrc), "s"(stage_lds + lds[i])
                             : "memory", "m0");
        }
    }
};


// S^T (32 keys x 32 query columns) from an fp8 K tile and fp8 Q registers on
// the fp8 matrix cores (v_mfma_f32_32x32x64_f8f6f4, both operands e4m3,
// fp32 accumulate).  For contraction chunk kk (64 head-dim columns) lane
// (n, g = lane / 32) supplies columns 64*kk + 32*g .. +31 of its K row (A)
// and of its query row (B); A and B use the same assignment, so the products
// pair matching columns.
template <int D>
__device__ __forceinline__ f16v qk_subtile_f8(const uint8_t* Ks, int row0, const v8i (&q8)[D / 64],
                                              int n, int hh) {
    constexpr int C8 = D / 16;
    f16v s = (f16v){};
    const int row = row0 + sigma(n);
    const uint8_t* base = Ks + row * D;
    const int sw = swz_f8<D>(row);
#pragma unroll
    for (int kk = 0; kk < D / 64; ++kk) {
        const int c0 = 4 * kk + 2 * hh;
        const u4 lo = *(const u4*)(base + 16 * ((c0) ^ sw));
        const u4 hi = *(const u4*)(base + 16 * ((c0 + 1) ^ sw));
        const v8i a = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                       (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, q8[kk], s, 0, 0, 0, 0, 0, 0);
    }
    (void)C8;
    return s;
}

// s_waitcnt immediate for "at most n vector-memory operations outstanding"
// (expcnt and lgkmcnt left at their maxima; vmcnt is split over bits 3:0
// and 15:14).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

// s_waitcnt vmcnt(0).  The builtin, unlike an asm statement, also informs the
// compiler's own wait tracking.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); }

// A operand of product kk of S^T = K Q^T for the 32-key sub-tile at row0:
// K row (row0 + sigma(n)), columns 16*kk + 8*hh .. +7.
template <int D>
__device__ __forceinline__ h8 k_operand(const _Float16* Ks, int row0, int kk, int n, int hh) {
    const int row = row0 + sigma(n);
    return *(const h8*)(Ks + row * D + 8 * ((2 * kk + hh) ^ swz_k<D>(row)));
}

template <int D>
__device__ __forceinline__ f16v qk_subtile_sw(const _Float16* Ks, int row0, const h8 (&qreg)[D / 16],
                                              int n, int hh) {
    f16v s = (f16v){};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) s = mfma_32x32x16(k_operand<D>(Ks, row0, kk, n, hh), qreg[kk], s);
    return s;
}

// O^T += V^T P^T is taken per 16-key chunk ch of a V tile and 32-column
// head-dim slice dt.  The A operand of that product (head-dim row
// 32*dt + l%32, keys 16*ch + 8*hh + 0..7) is assembled from two transposing
// LDS reads: in each 16-lane group, lane j receives element (j % 4) of what
// lane 4*e + j/4 addressed, for e = 0..3; lane 4*e + q addresses key
// (base + e), columns 4*q .. 4*q+3 of its group's 16.
template <int D>
__device__ __forceinline__ h8 v_operand_tr(const _Float16* Vs, int ch, int dt, int lane) {
    const int hh = lane >> 5;
    const int g2 = (lane >> 4) & 1;
    const int e = (lane >> 2) & 3;
    const int q = lane & 3;
    const int rowa = 16 * ch + 8 * hh + e;   // keys +0..3
    const int rowb = rowa + 4;               // keys +4..7
    const int c = 4 * dt + 2 * g2 + (q >> 1);
    const _Float16* pa = Vs + rowa * D + 8 * (c ^ swz_v<D>(rowa)) + 4 * (q & 1);
    const _Float16* pb = Vs + rowb * D + 8 * (c ^ swz_v<D>(rowb)) + 4 * (q & 1);
    const s4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)pa);
    const s4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)pb);
    const h4 ha = __builtin_bit_cast(h4, va), hb = __builtin_bit_cast(h4, vb);
    return (h8){ha[0], ha[1], ha[2], ha[3], hb[0], hb[1], hb[2], hb[3]};
}

// B operand of chunk ch: the lane's 8 probabilities of that chunk's keys.
__device__ __forceinline__ h8 p_operand(const h2* P, int ch) {
    const h2 p0 = P[4 * ch + 0], p1 = P[4 * ch + 1], p2 = P[4 * ch + 2], p3 = P[4 * ch + 3];
    return (h8){p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// O^T += V^T P^T for the chunks [ch0, ch0 + NCH) of a V tile.
template <int D, int NCH>
__device__ __forceinline__ void pv_chunks_tr(const _Float16* Vs, int ch0, const h2* P,
                                             f16v (&acc)[D / 32], int lane) {
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
        const h8 bp = p_operand(P, ch);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
            acc[dt] = mfma_32x32x16(v_operand_tr<D>(Vs, ch0 + ch, dt, lane), bp, acc[dt]);
    }
}

}  // namespace pasa
