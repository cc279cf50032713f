// attn_plan.h -- block ranges, split ranges and kernel parameters shared by the
// host planner and the gfx950 kernels (both sides of the product library).
//
// Citations name the page and section they follow:
//   [FA-tiling]  "分块策略与调度" (FlashAttention tiling strategy and scheduling)
//   [Occupancy]  "The Occupancy Awakening: Rewriting a Flash Attention Kernel for
//                Blackwell's 188 SMs"
//   [llama.cpp]  llama.cpp pull request 21086 review thread (blocks per SM and the
//                stream-k fixup)
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define TPA_HD __host__ __device__ __forceinline__
#else
#define TPA_HD inline
#endif

namespace tpa {

#define TPA_MAX_SPLITS 256

TPA_HD int ceil_div(int a, int b) { return (a + b - 1) / b; }
// floor division that is correct for negative numerators (b > 0)
TPA_HD int floor_div(int a, int b) { return a >= 0 ? a / b : -((-a + b - 1) / b); }
TPA_HD int imin(int a, int b) { return a < b ? a : b; }
TPA_HD int imax(int a, int b) { return a > b ? a : b; }

// Key-block range [n_min, n_max) that query block m_block must visit
// ([FA-tiling] §3.1-3.2). Rows of the block are rows [m_block*BM, (m_block+1)*BM)
// of the query rows of one (batch, grid head); with GQA packing those are the
// Sq*G packed rows and row r sits at sequence position r / G ([FA-tiling] §6.3).
// The bounds use the first and last *existing* row of the block, which is the
// tight form of the page's (m_block+1)*kBlockM upper index. Keys are aligned to
// the bottom right: delta = Skb - Sq. causal => window_right = 0; window_left
// < 0 => no lower bound. An empty range (n_max <= n_min) means no row of the
// block sees any key.
TPA_HD void n_block_range(int Sq, int Skb, int G, int pack, int causal, int window_left,
                          int BM, int BN, int m_block, int* n_min, int* n_max) {
    const int nrows = pack ? Sq * G : Sq;
    const int r0 = m_block * BM;
    const int r1 = imin((m_block + 1) * BM, nrows);  // exclusive
    const int pos_min = pack ? r0 / G : r0;
    const int pos_max = pack ? (r1 - 1) / G : r1 - 1;
    const int delta = Skb - Sq;
    int hi = ceil_div(Skb, BN);
    if (causal) hi = imin(hi, floor_div(pos_max + delta, BN) + 1);
    int lo = 0;
    if (window_left >= 0) lo = imax(0, floor_div(pos_min + delta - window_left, BN));
    *n_min = lo;
    *n_max = hi;
}

// Number of splits that batch b actually uses. Fixed-length problems use all
// num_splits. With a positive chunk (in key blocks) each sequence instead gets
// ceil(blocks / chunk) splits, at most num_splits ([FA-tiling] §5.3: the split
// count may differ per sequence in the variable-length case).
TPA_HD int splits_for(int n_blocks, int num_splits, int chunk_blocks) {
    if (chunk_blocks <= 0) return num_splits;
    if (n_blocks <= 0) return 1;
    return imin(num_splits, imax(1, ceil_div(n_blocks, chunk_blocks)));
}

// Even partition of [n_min, n_max) into `splits` pieces ([FA-tiling] §3.2 and
// §5.3): per = ceil(len / splits); split s gets [n_min + s*per, min(.. + per,
// n_max)). Trailing pieces may be empty (returned as n_max <= n_min).
TPA_HD void split_range(int n_min, int n_max, int split, int splits, int* s_min, int* s_max) {
    if (splits <= 1) {
        *s_min = n_min;
        *s_max = n_max;
        return;
    }
    const int len = imax(0, n_max - n_min);
    const int per = ceil_div(len, splits);
    const int lo = n_min + split * per;
    *s_min = lo;
    *s_max = imin(lo + per, n_max);
}

// Query-block range [m_min, m_max) whose rows see at least one key of key block
// n_block: the backward pass's inverse of n_block_range ([FA-tiling] §3.4,
// get_m_block_min_max). Row i sees key j iff j < Sk, and j <= i + delta if
// causal, and j >= i + delta - window_left if window_left >= 0 (delta = Sk - Sq).
// The first key of the block bounds the causal side, the last existing key the
// window side. An empty range (m_max <= m_min) means no row sees the block.
TPA_HD void m_block_range(int Sq, int Sk, int causal, int window_left, int BM, int BN,
                          int n_block, int* m_min, int* m_max) {
    const int k0 = n_block * BN;
    const int k1 = imin((n_block + 1) * BN, Sk) - 1;  // last existing key of the block
    const int delta = Sk - Sq;
    int lo = 0, hi = ceil_div(imax(Sq, 0), BM);
    if (k1 < k0) hi = 0;
    if (causal) lo = imax(0, floor_div(k0 - delta, BM));
    if (window_left >= 0) hi = imin(hi, imax(0, floor_div(k1 + window_left - delta, BM) + 1));
    *m_min = lo;
    *m_max = hi;
}

// Arguments of the backward kernels (passed by value).
struct BwdParams {
    const void* q;          // [B][Sq][Hq][d]
    const void* k;          // [B][Sk][Hkv][d]
    const void* v;          // [B][Sk][Hkv][d]
    const void* o;          // [B][Sq][Hq][d], forward output
    const void* dout;       // [B][Sq][Hq][d], gradient of the output
    const float* lse;       // [B][Hq][Sq], forward log-sum-exp (natural log)
    void* dq;               // [B][Sq][Hq][d]
    void* dk;               // [B][Sk][Hkv][d]
    void* dv;               // [B][Sk][Hkv][d]
    float* dq_acc;          // [B][Sq][Hq][d] fp32 accumulator (workspace)
    float* lse2;            // [B][Hq][Sq]: lse * log2(e); +inf for rows that see no key
    float* dsum;            // [B][Hq][Sq]: rowsum(dO * O)
    int B, Hq, Hkv, Sq, Sk, G;
    int causal, window_left;
    float scale;            // softmax scale
    float scale_log2;       // scale * log2(e)
    int num_n_blocks;       // key blocks per (batch, KV head)
};

// Arguments of the forward kernel (passed by value).
struct FwdParams {
    const void* q;          // [B][Sq][Hq][d]
    const void* k;          // [B][Sk][Hkv][d]
    const void* v;          // [B][Sk][Hkv][d]
    void* o;                // [B][Sq][Hq][d], dtype of q
    float* lse;             // [B][Hq][Sq] or null
    float* o_part;          // [S][B*Sq*Hq][d] fp32 split partials (num_splits > 1)
    float* lse_part;        // [S][B*Sq*Hq]
    const int* seqlens_k;   // device int[B] or null (then Sk everywhere)
    int B, Hq, Hkv, Sq, Sk, G;
    int causal, window_left;
    float scale_log2;       // scale * log2(e): scores enter exp2 pre-multiplied
    float scale;            // softmax scale (natural-log units, for lse)
    int pack;               // GQA packing: the G heads of a KV head share one tile
    int num_m_blocks;       // query blocks per (batch, grid head)
    int grid_heads;         // Hkv when packed, Hq otherwise
    int num_splits;         // grid splits (1: no split, direct output)
    int chunk_blocks;       // > 0: per-sequence split count (variable length)
    int lpt;                // reverse query-block order (heaviest causal blocks first)
    int split_major;        // grid y = split * grid_heads + head (else head * splits + split)
    int work_units;         // variable-length decode: grid (units, KV heads) over (sequence, split) units
    int* tile_counters;     // persistent kernels: one tile queue counter per XCD, zero at launch
    // Decode tiles of fixed-length problems (seqlens_k null): the key-block
    // range of the single query block and its blocks per split, computed once
    // on the host. blockIdx.y / y_div (y_div = grid_heads when split_major, else
    // num_splits) is t = umulhi(y_mul, y), (t + ((y - t) >> y_s1)) >> y_s2 with
    // the host's round-up multiplier (Granlund and Montgomery, "Division by
    // invariant integers using multiplication"): exact for every 32-bit y and
    // any y_div >= 1, with no branch and no division on the device.
    int dec_lo, dec_hi, dec_per;
    int y_div;
    unsigned int y_mul;
    int y_s1, y_s2;
};

// The multiplier and shifts above for divisor d >= 1: l = ceil(log2 d),
// mul = floor(2^32 (2^l - d) / d) + 1, s1 = min(l, 1), s2 = max(l - 1, 0).
inline void div_magic(unsigned int d, unsigned int* mul, int* s1, int* s2) {
    int l = 0;
    while (l < 32 && (1ull << l) < d) ++l;
    *mul = (unsigned int)(((1ull << 32) * ((1ull << l) - d)) / d + 1ull);
    *s1 = l < 1 ? l : 1;
    *s2 = l - 1 > 0 ? l - 1 : 0;
}

// Arguments of the log-sum-exp combine kernel. Every split writes its lse
// partial (-inf for an empty split), so the combine needs no block ranges.
struct CombineParams {
    const float* o_part;    // [S][rows][d]
    const float* lse_part;  // [S][rows]
    void* o;                // [rows][d]; rows ordered (batch, position, head) as in o
    float* lse;             // [B][Hq][Sq] or null
    int rows, num_splits, Sq, Hq;
};

}  // namespace tpa
