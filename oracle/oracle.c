/*
 * CPU oracle for the PASA forward pass -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load this library. The product path (the HIP library and its Python binding)
 * never calls it, links it or shares code with it.
 *
 * What it computes.  "Online Pseudo-average Shifting Attention (PASA) for Robust
 * Low-precision LLM Inference", Abstract: PASA is a low-precision algorithm that
 * is mathematically equivalent to attention built on Flash Attention.  The oracle
 * is therefore the plain definition of softmax attention, evaluated in IEEE
 * binary64 with the classic two passes per query row (maximum, then exponentials,
 * sum and weighted value sum).  There is no blocking, no online rescaling and no
 * reduced precision anywhere.
 *
 * Definition, for batch b, query head h, query row i:
 *   g      = Hq / Hkv (query heads per key/value head), kv head = h / g
 *   V(i)   = { j : 0 <= j < Skv  and  (not causal  or  j <= i + Skv - Sq) }
 *   s_ij   = scale * sum_d q[b,i,h,d] * k[b,j,kv,d]   (+ offset[b,h,i] if given)
 *   m_i    = max_{j in V(i)} s_ij
 *   l_i    = sum_{j in V(i)} exp(s_ij - m_i)
 *   o_i    = sum_{j in V(i)} exp(s_ij - m_i) * v[b,j,kv,:] / l_i
 *   lse_i  = m_i + ln(l_i)                       (natural logarithm)
 * An empty V(i) (possible only when causal and Sq > Skv) gives o_i = 0 and
 * lse_i = -infinity.
 *
 * The causal mask is aligned to the bottom-right corner (the last query row sees
 * every key); for Sq == Skv this is the usual lower-triangular mask.
 *
 * The split combine follows the additive-partials property stated on the
 * "Block Sparse Flash Attention" topic page, FoldAttention card: softmax is
 * invariant to a common shift, so normalised partials over disjoint key ranges
 * recombine exactly once each is re-weighted by its own log-sum-exp.
 *
 * Layouts (all row-major, contiguous):
 *   q, o : [B, Sq,  Hq,  D]      k, v : [B, Skv, Hkv, D]      lse : [B, Hq, Sq]
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* One query row, two passes.  Returns lse; writes D outputs to out. */
static double attn_row(const double* qrow, const double* k, const double* v,
                       int64_t kv_stride, int n_visible, int D, double scale,
                       double offset, double* scores, double* out) {
    double m = -INFINITY;
    for (int j = 0; j < n_visible; ++j) {
        const double* krow = k + (int64_t)j * kv_stride;
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += qrow[d] * krow[d];
        double s = scale * dot + offset;
        scores[j] = s;
        if (s > m) m = s;
    }
    for (int d = 0; d < D; ++d) out[d] = 0.0;
    if (n_visible == 0) return -INFINITY;
    double l = 0.0;
    for (int j = 0; j < n_visible; ++j) {
        double p = exp(scores[j] - m);
        l += p;
        const double* vrow = v + (int64_t)j * kv_stride;
        for (int d = 0; d < D; ++d) out[d] += p * vrow[d];
    }
    for (int d = 0; d < D; ++d) out[d] /= l;
    return m + log(l);
}

static int visible_count(int i, int Sq, int Skv, int causal) {
    if (!causal) return Skv;
    long long last = (long long)i + Skv - Sq; /* last visible key index */
    if (last < 0) return 0;
    if (last >= Skv) return Skv;
    return (int)(last + 1);
}

/*
 * Full or sampled attention.
 *   rows == NULL : every row; o is [B,Sq,Hq,D] and lse is [B,Hq,Sq].
 *   rows != NULL : nrows flat row ids r = (b*Hq + h)*Sq + i; o is [nrows,D],
 *                  lse is [nrows].
 *   offset       : NULL or one additive constant per row, indexed by the flat
 *                  row id (layout [B,Hq,Sq]); used by the shift-invariance pins.
 * Each thread keeps one row of Skv scores in a heap buffer of its own.
 * Returns 0, or -1 on invalid sizes.
 */
int oracle_attn_fp64(const double* q, const double* k, const double* v,
                     int B, int Sq, int Skv, int Hq, int Hkv, int D,
                     double scale, int causal, const double* offset,
                     const int64_t* rows, int64_t nrows,
                     double* o, double* lse) {
    if (B < 0 || Sq < 0 || Skv < 0 || Hq <= 0 || Hkv <= 0 || D <= 0) return -1;
    if (Hq % Hkv != 0) return -1;
    const int g = Hq / Hkv;
    const int64_t total = rows ? nrows : (int64_t)B * Hq * Sq;
    int failed = 0;
#pragma omp parallel
    {
        double* scores = (double*)malloc(sizeof(double) * (size_t)(Skv > 0 ? Skv : 1));
        if (!scores) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (int64_t t = 0; t < total; ++t) {
                int64_t r = rows ? rows[t] : t;
                int i = (int)(r % Sq);
                int h = (int)((r / Sq) % Hq);
                int b = (int)(r / ((int64_t)Sq * Hq));
                int kvh = h / g;
                const double* qrow = q + (((int64_t)b * Sq + i) * Hq + h) * D;
                const double* kb = k + ((int64_t)b * Skv * Hkv + kvh) * D;
                const double* vb = v + ((int64_t)b * Skv * Hkv + kvh) * D;
                double* out = rows ? o + t * D : o + (((int64_t)b * Sq + i) * Hq + h) * D;
                double off = offset ? offset[r] : 0.0;
                double l = attn_row(qrow, kb, vb, (int64_t)Hkv * D,
                                    visible_count(i, Sq, Skv, causal), D, scale, off,
                                    scores, out);
                if (rows) lse[t] = l; else lse[r] = l;
            }
            free(scores);
        }
    }
    return failed ? -1 : 0;
}

/*
 * Recombine n normalised partials of one query row, each computed over a
 * disjoint key range:   M = max_s lse_s,  lse = M + ln sum_s exp(lse_s - M),
 *                       o = sum_s exp(lse_s - lse) * o_s.
 * Partials with lse_s = -infinity (empty key range) carry no weight; if all are
 * empty the result is o = 0, lse = -infinity.
 *   o_part : [rows, n, D]   lse_part : [rows, n]   o : [rows, D]   lse : [rows]
 */
void oracle_combine_fp64(const double* o_part, const double* lse_part, int64_t rows,
                         int n, int D, double* o, double* lse) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const double* ls = lse_part + r * n;
        double M = -INFINITY;
        for (int s = 0; s < n; ++s) if (ls[s] > M) M = ls[s];
        double* out = o + r * D;
        for (int d = 0; d < D; ++d) out[d] = 0.0;
        if (M == -INFINITY) { lse[r] = -INFINITY; continue; }
        double sum = 0.0;
        for (int s = 0; s < n; ++s) sum += exp(ls[s] - M);
        double L = M + log(sum);
        for (int s = 0; s < n; ++s) {
            double w = exp(ls[s] - L);
            const double* op = o_part + (r * n + s) * D;
            for (int d = 0; d < D; ++d) out[d] += w * op[d];
        }
        lse[r] = L;
    }
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
