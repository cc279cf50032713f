/*
 * attn_ref.c -- fp64 CPU oracle for the attention forward and backward passes.
 *
 * TEST INFRASTRUCTURE ONLY (the checker, never the product path); see
 * attn_ref.h for the contract and the layouts.
 *
 * Each query row is computed straight from the definition, two passes:
 *   1. scores s_j = scale * <q_i, k_j> for every visible key j, in fp64;
 *   2. m = max_j s_j, l = sum_j exp(s_j - m),
 *      o_i = sum_j exp(s_j - m) v_j / l, lse_i = m + ln l.
 * The visible set is the bottom-right aligned causal / window mask whose
 * block-level bounds are given in [FA-tiling] §3.1 (the key offset
 * seqlen_k - seqlen_q in both the causal upper bound and the window lower
 * bound); per element that is j <= i + delta and j >= i + delta - window_left.
 * The split partial restricts the keys to one range, the flash-decoding
 * partial of [FA-tiling] §5.1 and [Occupancy] "The Fix"; the merge is the
 * log-sum-exp identity those sections use to recombine the splits.
 */
#include "attn_ref.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Is key j visible to query row i (key length skb, query length sq)? */
static int visible(int i, int j, int skb, int sq, int causal, int window_left) {
    long delta = (long)skb - (long)sq;
    if (j < 0 || j >= skb) return 0;
    if (causal && (long)j > (long)i + delta) return 0;
    if (window_left >= 0 && (long)j < (long)i + delta - (long)window_left) return 0;
    return 1;
}

/* d: width of q and k rows (the score contraction); dv: width of v and o rows */
static int attn_core(const double* q, const double* k, const double* v, double* o, double* lse,
                     int B, int Hq, int Hkv, int Sq, int Sk, const int* seqlens_k, int d, int dv,
                     int causal, int window_left, double scale, int j_begin, int j_end,
                     int n_threads) {
    if (!q || !k || !v || !o) return -1;
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Sq < 0 || Sk < 0 || d <= 0 || dv <= 0) return -1;
    if (Hq % Hkv != 0) return -1;
    if (window_left < -1) return -1;
    const int G = Hq / Hkv;
    const long nrows = (long)B * Hq * Sq;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
    int bad = 0;
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(Sk > 0 ? Sk : 1));
        double* acc = (double*)malloc(sizeof(double) * (size_t)dv);
        if (!s || !acc) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (long row = 0; row < nrows; ++row) {
            if (!s || !acc) continue;
            /* row enumerates (b, hq, i) with i fastest */
            const int i = (int)(row % Sq);
            const int hq = (int)((row / Sq) % Hq);
            const int b = (int)(row / ((long)Sq * Hq));
            const int hkv = hq / G;
            int skb = seqlens_k ? seqlens_k[b] : Sk;
            if (skb > Sk) skb = Sk;
            if (skb < 0) skb = 0;
            const double* qi = q + (((long)b * Sq + i) * Hq + hq) * d;
            double* oi = o + (((long)b * Sq + i) * Hq + hq) * dv;

            /* pass 1: scores of the visible keys and their maximum */
            double m = -INFINITY;
            int nvis = 0;
            for (int j = 0; j < skb; ++j) {
                if (j < j_begin || j >= j_end || !visible(i, j, skb, Sq, causal, window_left)) {
                    s[j] = -INFINITY;
                    continue;
                }
                const double* kj = k + (((long)b * Sk + j) * Hkv + hkv) * d;
                double dot = 0.0;
                for (int c = 0; c < d; ++c) dot += qi[c] * kj[c];
                s[j] = scale * dot;
                if (s[j] > m) m = s[j];
                ++nvis;
            }
            if (nvis == 0) {
                for (int c = 0; c < dv; ++c) oi[c] = 0.0;
                if (lse) lse[((long)b * Hq + hq) * Sq + i] = -INFINITY;
                continue;
            }
            /* pass 2: normaliser and weighted sum of the value rows */
            double l = 0.0;
            for (int c = 0; c < dv; ++c) acc[c] = 0.0;
            for (int j = 0; j < skb; ++j) {
                if (s[j] == -INFINITY) continue;
                const double p = exp(s[j] - m);
                l += p;
                const double* vj = v + (((long)b * Sk + j) * Hkv + hkv) * dv;
                for (int c = 0; c < dv; ++c) acc[c] += p * vj[c];
            }
            for (int c = 0; c < dv; ++c) oi[c] = acc[c] / l;
            if (lse) lse[((long)b * Hq + hq) * Sq + i] = m + log(l);
        }
        free(s);
        free(acc);
    }
    return bad ? -1 : 0;
}

int attn_ref_f64(const double* q, const double* k, const double* v, double* o, double* lse,
                 int B, int Hq, int Hkv, int Sq, int Sk, const int* seqlens_k, int d,
                 int causal, int window_left, double scale, int n_threads) {
    return attn_core(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, seqlens_k, d, d, causal, window_left,
                     scale, 0, Sk, n_threads);
}

int attn_ref_dv_f64(const double* q, const double* k, const double* v, double* o, double* lse,
                    int B, int Hq, int Hkv, int Sq, int Sk, const int* seqlens_k, int d, int dv,
                    int causal, int window_left, double scale, int n_threads) {
    return attn_core(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, seqlens_k, d, dv, causal, window_left,
                     scale, 0, Sk, n_threads);
}

int attn_ref_partial_f64(const double* q, const double* k, const double* v, double* o,
                         double* lse, int B, int Hq, int Hkv, int Sq, int Sk,
                         const int* seqlens_k, int d, int causal, int window_left,
                         double scale, int j_begin, int j_end, int n_threads) {
    return attn_core(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, seqlens_k, d, d, causal, window_left,
                     scale, j_begin, j_end, n_threads);
}

int lse_combine_ref_f64(const double* o_part, const double* lse_part, int S, long rows, int d,
                        double* o, double* lse) {
    if (!o_part || !lse_part || !o || S < 1 || rows < 0 || d <= 0) return -1;
    for (long r = 0; r < rows; ++r) {
        double m = -INFINITY;
        for (int s = 0; s < S; ++s)
            if (lse_part[(long)s * rows + r] > m) m = lse_part[(long)s * rows + r];
        double* orow = o + r * d;
        if (m == -INFINITY) {
            for (int c = 0; c < d; ++c) orow[c] = 0.0;
            if (lse) lse[r] = -INFINITY;
            continue;
        }
        double total = 0.0;
        for (int s = 0; s < S; ++s) total += exp(lse_part[(long)s * rows + r] - m);
        const double lse_r = m + log(total);
        for (int c = 0; c < d; ++c) orow[c] = 0.0;
        for (int s = 0; s < S; ++s) {
            const double ls = lse_part[(long)s * rows + r];
            if (ls == -INFINITY) continue;
            const double w = exp(ls - lse_r);
            const double* op = o_part + ((long)s * rows + r) * d;
            for (int c = 0; c < d; ++c) orow[c] += w * op[c];
        }
        if (lse) lse[r] = lse_r;
    }
    return 0;
}

/*
 * Backward pass: the gradient of the forward definition above.
 *
 * The pages describe the backward loop structure ([FA-tiling] §3.4: one key
 * block outside, the query blocks that see it inside; §4.6: Q, dO and the dQ
 * accumulator are what the backward scheduler keeps in L2) but print no
 * gradient formulas; this is the chain rule applied to the forward definition,
 * with no tiling. For a row i with visible keys V_i, probabilities
 * p_ij = exp(s_ij - lse_i) and an output gradient g_i = dL/do_i:
 *   dp_ij = <g_i, v_j>                      (o_i = sum_j p_ij v_j)
 *   D_i   = sum_j p_ij dp_ij                (softmax Jacobian: ds = p (dp - <p, dp>))
 *   ds_ij = p_ij (dp_ij - D_i)              (gradient w.r.t. the scaled score)
 *   dq_i  = scale sum_j ds_ij k_j
 *   dk_j  = scale sum_{i, heads of the group} ds_ij q_i
 *   dv_j  = sum_{i, heads of the group} p_ij g_i
 * Pass 1 runs over query rows (scores, lse_i, D_i, dq_i); pass 2 over key rows,
 * recomputing p_ij and ds_ij from lse_i and D_i of pass 1.
 */
static int bwd_core(const double* q, const double* k, const double* v, const double* dout,
                    double* dq, double* dk, double* dv, int B, int Hq, int Hkv, int Sq, int Sk,
                    int d, int causal, int window_left, double scale, int n_threads) {
    if (!q || !k || !v || !dout || !dq || !dk || !dv) return -1;
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Sq < 0 || Sk < 0 || d <= 0) return -1;
    if (Hq % Hkv != 0 || window_left < -1) return -1;
    const int G = Hq / Hkv;
    const long nrows = (long)B * Hq * Sq;
    double* lse_row = (double*)malloc(sizeof(double) * (size_t)(nrows > 0 ? nrows : 1));
    double* d_row = (double*)malloc(sizeof(double) * (size_t)(nrows > 0 ? nrows : 1));
    if (!lse_row || !d_row) {
        free(lse_row);
        free(d_row);
        return -1;
    }
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
    int bad = 0;
    /* pass 1: per query row (b, hq, i) */
#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(Sk > 0 ? Sk : 1));
        double* dp = (double*)malloc(sizeof(double) * (size_t)(Sk > 0 ? Sk : 1));
        if (!s || !dp) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 4)
        for (long row = 0; row < nrows; ++row) {
            if (!s || !dp) continue;
            const int i = (int)(row % Sq);
            const int hq = (int)((row / Sq) % Hq);
            const int b = (int)(row / ((long)Sq * Hq));
            const int hkv = hq / G;
            const double* qi = q + (((long)b * Sq + i) * Hq + hq) * d;
            const double* gi = dout + (((long)b * Sq + i) * Hq + hq) * d;
            double* dqi = dq + (((long)b * Sq + i) * Hq + hq) * d;
            for (int c = 0; c < d; ++c) dqi[c] = 0.0;
            double m = -INFINITY;
            for (int j = 0; j < Sk; ++j) {
                if (!visible(i, j, Sk, Sq, causal, window_left)) {
                    s[j] = -INFINITY;
                    continue;
                }
                const double* kj = k + (((long)b * Sk + j) * Hkv + hkv) * d;
                double dot = 0.0;
                for (int c = 0; c < d; ++c) dot += qi[c] * kj[c];
                s[j] = scale * dot;
                if (s[j] > m) m = s[j];
            }
            if (m == -INFINITY) { /* no visible key: the row contributes nothing */
                lse_row[row] = -INFINITY;
                d_row[row] = 0.0;
                continue;
            }
            double l = 0.0;
            for (int j = 0; j < Sk; ++j)
                if (s[j] != -INFINITY) l += exp(s[j] - m);
            const double lse_i = m + log(l);
            double Di = 0.0;
            for (int j = 0; j < Sk; ++j) {
                if (s[j] == -INFINITY) continue;
                const double* vj = v + (((long)b * Sk + j) * Hkv + hkv) * d;
                double dot = 0.0;
                for (int c = 0; c < d; ++c) dot += gi[c] * vj[c];
                dp[j] = dot;
                Di += exp(s[j] - lse_i) * dot;
            }
            for (int j = 0; j < Sk; ++j) {
                if (s[j] == -INFINITY) continue;
                const double ds = exp(s[j] - lse_i) * (dp[j] - Di);
                const double* kj = k + (((long)b * Sk + j) * Hkv + hkv) * d;
                for (int c = 0; c < d; ++c) dqi[c] += scale * ds * kj[c];
            }
            lse_row[row] = lse_i;
            d_row[row] = Di;
        }
        free(s);
        free(dp);
    }
    /* pass 2: per key row (b, hkv, j), summed over the G query heads of the group */
    const long nkeys = (long)B * Hkv * Sk;
#pragma omp parallel for schedule(dynamic, 4)
    for (long key = 0; key < nkeys; ++key) {
        const int j = (int)(key % Sk);
        const int hkv = (int)((key / Sk) % Hkv);
        const int b = (int)(key / ((long)Sk * Hkv));
        const double* kj = k + (((long)b * Sk + j) * Hkv + hkv) * d;
        const double* vj = v + (((long)b * Sk + j) * Hkv + hkv) * d;
        double* dkj = dk + (((long)b * Sk + j) * Hkv + hkv) * d;
        double* dvj = dv + (((long)b * Sk + j) * Hkv + hkv) * d;
        for (int c = 0; c < d; ++c) {
            dkj[c] = 0.0;
            dvj[c] = 0.0;
        }
        for (int g = 0; g < G; ++g) {
            const int hq = hkv * G + g;
            for (int i = 0; i < Sq; ++i) {
                if (!visible(i, j, Sk, Sq, causal, window_left)) continue;
                const long row = ((long)b * Hq + hq) * Sq + i;
                const double* qi = q + (((long)b * Sq + i) * Hq + hq) * d;
                const double* gi = dout + (((long)b * Sq + i) * Hq + hq) * d;
                double sdot = 0.0, pdot = 0.0;
                for (int c = 0; c < d; ++c) {
                    sdot += qi[c] * kj[c];
                    pdot += gi[c] * vj[c];
                }
                const double p = exp(scale * sdot - lse_row[row]);
                const double ds = p * (pdot - d_row[row]);
                for (int c = 0; c < d; ++c) {
                    dkj[c] += scale * ds * qi[c];
                    dvj[c] += p * gi[c];
                }
            }
        }
    }
    free(lse_row);
    free(d_row);
    return bad ? -1 : 0;
}

int attn_bwd_ref_f64(const double* q, const double* k, const double* v, const double* dout,
                     double* dq, double* dk, double* dv, int B, int Hq, int Hkv, int Sq, int Sk,
                     int d, int causal, int window_left, double scale, int n_threads) {
    return bwd_core(q, k, v, dout, dq, dk, dv, B, Hq, Hkv, Sq, Sk, d, causal, window_left, scale,
                    n_threads);
}
