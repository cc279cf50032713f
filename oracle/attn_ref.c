/*
 * attn_ref.c -- fp64 CPU oracle for the attention forward pass.
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
