/*
 * attn_ref.h -- fp64 CPU oracle for the tiled flash-attention forward and backward passes.
 *
 * TEST INFRASTRUCTURE ONLY. This library is the checker, not the product:
 * only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load it. It shares no source, header, table or helper with the HIP
 * library under tiled_prefill_amd/csrc, and neither includes the other.
 *
 * What it computes is the plain definition of exact softmax attention with a
 * bottom-right aligned causal / sliding-window mask; it has no tiling, no
 * online rescaling and no block skipping. Citations name the page and the
 * section they follow:
 *   [FA-tiling]  "分块策略与调度" (FlashAttention tiling strategy and scheduling)
 *   [Occupancy]  "The Occupancy Awakening: Rewriting a Flash Attention Kernel
 *                for Blackwell's 188 SMs"
 *
 * Layouts (all row-major, contiguous):
 *   q, o      [B][Sq][Hq][d]
 *   k, v      [B][Sk][Hkv][d]
 *   lse       [B][Hq][Sq]       natural-log log-sum-exp of the scaled scores
 *   o_part    [S][rows][d], lse_part [S][rows]   (split partials)
 */
#ifndef ATTN_REF_H
#define ATTN_REF_H

#ifdef __cplusplus
extern "C" {
#endif

/* Exact attention, fp64.
 * Query head hq reads key/value head hq / (Hq/Hkv) (contiguous groups).
 * seqlens_k: host int[B] of per-sequence key lengths (each <= Sk), or NULL
 * for Sk everywhere. With Sk_b the key length of sequence b and
 * delta = Sk_b - Sq, key j is visible to query row i iff
 *   0 <= j < Sk_b,  and (causal => j <= i + delta),
 *   and (window_left >= 0 => j >= i + delta - window_left).
 * A row with no visible key gets o = 0 and lse = -inf.
 * n_threads <= 0 lets OpenMP choose. Returns 0, or -1 on bad arguments. */
int attn_ref_f64(const double* q, const double* k, const double* v, double* o, double* lse,
                 int B, int Hq, int Hkv, int Sq, int Sk, const int* seqlens_k, int d,
                 int causal, int window_left, double scale, int n_threads);

/* Same, with value rows of their own width: q and k rows have d elements (the
 * score contraction), v and o rows have dv -- the latent-attention verify shape
 * of [Occupancy] (one shared KV head, 576-wide keys, 512-wide values).
 * Layouts: q [B][Sq][Hq][d], k [B][Sk][Hkv][d], v [B][Sk][Hkv][dv],
 * o [B][Sq][Hq][dv]. */
int attn_ref_dv_f64(const double* q, const double* k, const double* v, double* o, double* lse,
                    int B, int Hq, int Hkv, int Sq, int Sk, const int* seqlens_k, int d, int dv,
                    int causal, int window_left, double scale, int n_threads);

/* Same, with the keys further restricted to [j_begin, j_end): the partial
 * result of one key split. o is normalised over the keys of the split and
 * lse is that split's log-sum-exp; an empty split gives o = 0, lse = -inf. */
int attn_ref_partial_f64(const double* q, const double* k, const double* v, double* o,
                         double* lse, int B, int Hq, int Hkv, int Sq, int Sk,
                         const int* seqlens_k, int d, int causal, int window_left,
                         double scale, int j_begin, int j_end, int n_threads);

/* Log-sum-exp merge of S split partials, per row r:
 *   lse[r] = log sum_s exp(lse_part[s][r])
 *   o[r]   = sum_s exp(lse_part[s][r] - lse[r]) * o_part[s][r]
 * Rows whose partials are all empty (-inf) get o = 0, lse = -inf. */
int lse_combine_ref_f64(const double* o_part, const double* lse_part, int S, long rows, int d,
                        double* o, double* lse);

/* Gradients of exact attention, fp64: given the output gradient dout (layout of
 * o), returns dq (layout of q) and dk, dv (layout of k, v) of L = <dout, o>,
 * o = attn(q, k, v) with the mask of attn_ref_f64 (fixed key length Sk). The
 * chain rule through the softmax, with no tiling; dk and dv of a KV head sum
 * over the query heads of its group. Rows with no visible key contribute
 * nothing. Returns 0, or -1 on bad arguments. */
int attn_bwd_ref_f64(const double* q, const double* k, const double* v, const double* dout,
                     double* dq, double* dk, double* dv, int B, int Hq, int Hkv, int Sq, int Sk,
                     int d, int causal, int window_left, double scale, int n_threads);

#ifdef __cplusplus
}
#endif
#endif
