/*
 * attn.h -- C-ABI of the MI355X (gfx950) tiled flash-attention forward library
 * (libattn.so).
 *
 * The library computes exact softmax attention
 *     O = softmax(scale * Q K^T + mask) V,     lse = log sum_j exp(scale q.k_j)
 * as a tiled flash-attention forward pass with online softmax, block skipping
 * for causal / sliding-window masks, GQA packing and split-KV with a separate
 * log-sum-exp combine kernel, and its gradients (attn_bwd) with the
 * key-block-outer backward loop.
 *
 * Sources (page title, section):
 *   [FA-tiling]  "分块策略与调度" (FlashAttention tiling strategy and scheduling):
 *                §2 tile sizes, §3 block-range skipping, §4 tile scheduling,
 *                §5 split-K and num_splits, §6 PackGQA.
 *   [Occupancy]  "The Occupancy Awakening: Rewriting a Flash Attention Kernel for
 *                Blackwell's 188 SMs": KV-split partials and their merge.
 *   [llama.cpp]  llama.cpp pull request 21086 review thread: at least two blocks
 *                per SM, then more only while each keeps a minimum KV chunk.
 *
 * Conventions shared by every entry point
 *   Layouts (row-major, contiguous, device memory):
 *     q, o   [B][Sq][Hq][d]      element type `dtype`
 *     k, v   [B][Sk][Hkv][d]     element type `dtype`
 *     lse    [B][Hq][Sq]         fp32, natural log; may be NULL (not written)
 *   dtype: ATTN_FP32 (0) or ATTN_BF16 (1). o has q's dtype; softmax and
 *     accumulation are fp32 in both cases; bf16 outputs are rounded to nearest
 *     even.
 *   Heads: query head h reads key/value head h / (Hq / Hkv).
 *   Mask ([FA-tiling] §3.1, aligned to the bottom right, delta = Sk_b - Sq):
 *     key j is visible to query row i iff j < Sk_b, and, if causal,
 *     j <= i + delta, and, if window_left >= 0, j >= i + delta - window_left.
 *     window_left = -1 means no left bound. A row with no visible key gets
 *     o = 0 and lse = -inf.
 *   num_splits: <= 0 picks the split count with the occupancy rule
 *     ([llama.cpp]); 1 runs one pass with no combine; 2..256 forces that many
 *     key splits (splits beyond the key blocks are empty and legal).
 *   stream: a hipStream_t, or NULL for the default stream. Calls are
 *     asynchronous on the stream and never synchronise the device, except
 *     that growing the library's own workspace synchronises once.
 *   Ownership: all tensors belong to the caller; the library never frees
 *     them. Split partials (and the backward's dQ accumulator and row sums) go
 *     to a caller-owned workspace bound with attn_set_workspace, or else to a
 *     library-owned device buffer (one per device, grown on demand, released
 *     at unload). Host threads are serialised on the library's buffer by a
 *     lock, so the library is thread-safe; on the GPU, calls on one device
 *     that use it must not overlap (issue them on one stream, or order the
 *     streams, or bind one workspace per stream).
 *   Numerics: scores scale * q.k must be finite in fp32 (fp32 accumulation).
 *     Every finite bf16 value of v is handled: the bf16 prefill kernel
 *     computes P.V on fp16 operands (P and V rounded to fp16) and, when a V
 *     element of a tile lies beyond fp16's range (|v| > 65504), runs that tile
 *     again with bf16 V and P as two bf16 parts (the decode and latent kernels
 *     always take that form). Non-finite inputs give unspecified (non-finite)
 *     outputs.
 *   Errors: a negative status code; nothing is launched and the message is
 *     available from attn_last_error() (thread-local). Argument checks never
 *     touch the GPU.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_OK 0
#define ATTN_EINVAL (-1)       /* bad argument (null pointer, shape, range)   */
#define ATTN_EUNSUPPORTED (-2) /* valid but not built: d not in {64,128}, dtype */
#define ATTN_EHIP (-3)         /* a HIP runtime call or launch failed          */
#define ATTN_ENOMEM (-4)       /* the split workspace could not be allocated   */

#define ATTN_FP32 0
#define ATTN_BF16 1

#define ATTN_MAX_SPLITS 256

/* Execution plan of one call: what the host planner chose. */
typedef struct attn_plan_t {
    int pack_gqa;        /* 1: the G query heads of a KV head share a tile ([FA-tiling] §6) */
    int block_m;         /* query rows per tile (packed rows when pack_gqa)                 */
    int block_n;         /* key rows per tile                                              */
    int waves_m;         /* waves along query rows                                          */
    int waves_n;         /* waves along keys inside a tile                                  */
    int num_m_blocks;    /* query blocks per (batch, grid head)                             */
    int grid_heads;      /* Hkv when packed, Hq otherwise                                   */
    int num_splits;      /* key splits; 1 = no combine kernel                               */
    int chunk_blocks;    /* > 0: variable-length per-sequence split chunk, in key blocks    */
    int grid_x, grid_y, grid_z;  /* forward-kernel grid                                    */
    int threads;         /* threads per workgroup                                           */
    int lds_bytes;       /* LDS per workgroup                                               */
    int num_cus;         /* compute units the split rule assumed                            */
    int lpt;             /* 1: query blocks launched heaviest first ([FA-tiling] §4.4)      */
    int work_units;      /* > 0: variable-length decode grid of this many (sequence, split)
                            units per KV head (grid_x), none for a split a sequence lacks */
    long long visited_blocks;  /* key blocks all tiles visit (fixed-length problems)        */
    size_t workspace_bytes;    /* split partials needed (0 when num_splits == 1)           */
} attn_plan_t;

/* Forward attention ([FA-tiling] §1-§6; [Occupancy] for the split path).
 * q, k, v, o: device pointers in the layouts above; lse: device fp32 or NULL.
 * B >= 0, Sq >= 0, Sk >= 0 (zero sizes are a no-op or give masked rows),
 * Hq, Hkv >= 1 with Hq % Hkv == 0, d in {64, 128}, scale finite and > 0,
 * window_left >= -1, num_splits <= 256. */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int Hq, int Hkv, int Sq, int Sk, int d,
               int causal, int window_left, float scale, int num_splits,
               int dtype, void* stream);

/* attn_fwd for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc). Same arguments,
 * kernels and results as attn_fwd; its scratch (split partials, tile
 * counters) is a static device array of ATTN_NOALLOC_SCRATCH_BYTES
 * in the library, one per device, held from the library's load until the
 * process ends. The call allocates nothing and ignores attn_set_workspace. A
 * problem whose plan needs more scratch (workspace_bytes of attn_plan_fwd)
 * returns ATTN_EINVAL and launches nothing. Every call on a device shares that
 * device's array, which keeps the last call's contents: calls that can overlap
 * on one GPU (other streams, other host threads) race on it -- issue them on
 * one stream. */
#define ATTN_NOALLOC_SCRATCH_BYTES (16u << 20)
int attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int Hq, int Hkv, int Sq, int Sk, int d,
                     int causal, int window_left, float scale, int num_splits,
                     int dtype, void* stream);

/* Values of their own width: the latent-attention verify shape of [Occupancy]
 * (one KV head shared by every query head; keys 576 wide = 512 latent + 64
 * rotary, values 512 wide). q [B][Sq][Hq][d], k [B][Sk][Hkv][d],
 * v [B][Sk][Hkv][d_v], o [B][Sq][Hq][d_v] (dtype of q), lse as attn_fwd.
 * d_v == d behaves as attn_fwd; otherwise only bf16 with d = 576, d_v = 512
 * is built (ATTN_EUNSUPPORTED else). The query heads of a KV head are always
 * packed into the row dimension ([FA-tiling] §6.3); num_splits <= 0 splits as far
 * as one workgroup per CU allows (the kernel holds one per CU), with at least 64
 * keys per split (the fp32 split partials are d_v wide). Other arguments as
 * attn_fwd. */
int attn_fwd_dv(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int Hq, int Hkv, int Sq, int Sk, int d, int d_v,
                  int causal, int window_left, float scale, int num_splits,
                  int dtype, void* stream);

/* Variable key lengths ([FA-tiling] §5.3: the split count may differ per
 * sequence). k and v are padded to [B][Sk][Hkv][d]; sequence b uses its first
 * seqlens_k[b] rows (device int32[B], each clamped to [0, Sk]). The split
 * count of each sequence is ceil(its key blocks / chunk); the chunk follows the
 * occupancy rule from sum_seqlens_k (host: the sum of seqlens_k, or <= 0 if
 * unknown, then B * Sk is assumed). num_splits > 0 forces the maximum split
 * count instead. Other arguments as attn_fwd. */
int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int Hq, int Hkv, int Sq, int Sk, int d,
                      int causal, int window_left, float scale, int num_splits,
                      int dtype, const int* seqlens_k, long long sum_seqlens_k,
                      void* stream);

/* The plan attn_fwd / attn_fwd_varlen would use (varlen != 0 selects the
 * latter). num_cus <= 0 reads the current device (256 when no device is
 * present). Pure host code: never touches the GPU beyond that query. */
int attn_plan_fwd(int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal, int window_left,
                    int num_splits, int dtype, int varlen, long long sum_seqlens_k, int num_cus,
                    attn_plan_t* out);

/* attn_plan_fwd under its shorter name: the same arguments, checks and plan. */
int attn_plan(int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal, int window_left,
              int num_splits, int dtype, int varlen, long long sum_seqlens_k, int num_cus,
              attn_plan_t* out);

/* Backward pass: gradients of L = <dout, o> for o = attention(q, k, v) with the
 * mask of attn_fwd ([FA-tiling] §3.4: one workgroup per key block, looping
 * over the query blocks that see it -- get_m_block_min_max -- and the query
 * heads of its KV head; §4.6: Q, dO and an fp32 dQ accumulator are the working
 * set). Inputs: q, k, v as attn_fwd; o and lse the forward's outputs for
 * them (lse natural log, [B][Hq][Sq], -inf for rows that see no key); dout the
 * output gradient in o's layout. Outputs: dq in q's layout, dk and dv in k's
 * layout, all in `dtype` (dk, dv sum over the G query heads of a KV head).
 * Three kernels: row sums D = <dout, o>, the key-block kernel (dK, dV in
 * registers), and a query-block kernel for dQ that recomputes S and dP (no
 * atomics: the result is the same bits on every run). ATTN_BWD_ATOMIC=1
 * selects the single-pass form of the pages instead (dQ added to an fp32
 * accumulator with atomics by the key-block kernel, then scaled; its last bits
 * depend on atomic timing). Sizes and errors as attn_fwd (d in {64, 128}; no
 * num_splits). */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
               const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq,
               int Sk, int d, int causal, int window_left, float scale, int dtype, void* stream);

/* What attn_bwd would launch (host only). */
typedef struct attn_bwd_plan_t {
    int block_m;         /* query rows per inner block                                     */
    int block_n;         /* keys per workgroup                                             */
    int num_n_blocks;    /* key blocks per (batch, KV head)                                */
    int grid_x;          /* key-block tiles: num_n_blocks * Hkv * B (launch padded to 8s)   */
    int threads;         /* threads per workgroup                                          */
    int lds_bytes;       /* LDS per workgroup                                              */
    int dq_block_m;      /* query rows per workgroup of the dQ kernel (0: atomic form)     */
    long long visited_blocks;  /* (query block, key block) pairs of the key-block kernel   */
    size_t workspace_bytes;    /* lse2 + row sums (+ the fp32 dQ accumulator, atomic form) */
} attn_bwd_plan_t;
int attn_plan_bwd(int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal, int window_left,
                    int dtype, attn_bwd_plan_t* out);

/* Split workspace bytes for B*Sq*Hq rows of head dim d and num_splits splits
 * (fp32 partial outputs plus fp32 partial lse). */
size_t attn_workspace_bytes(int B, int Hq, int Sq, int d, int num_splits);

/* Log-sum-exp combine of split partials ([FA-tiling] §5.1; [Occupancy]):
 *   lse[r] = log sum_s exp(lse_part[s][r]),  o[r] = sum_s exp(lse_part[s][r] - lse[r]) o_part[s][r]
 * over rows r = (b, i, h) in o's order (B*Sq*Hq rows). o_part [S][rows][d] fp32,
 * lse_part [S][rows] fp32 (-inf marks an empty split, whose o_part is not
 * read), o in `dtype`, lse [B][Hq][Sq] fp32 or NULL. 1 <= num_splits <= 256,
 * d in {64, 128, 512} (512: the value width of attn_fwd_dv). Three kernels:
 * one parallel over splits (many splits, few rows: decode), one parallel over
 * output elements (few splits or many rows; ATTN_COMBINE_COLS=0/1 forces
 * either of these two), and for 512-wide rows one workgroup per row
 * (ATTN_COMBINE_ROWS=0 turns it off). */
int attn_lse_combine(const float* o_part, const float* lse_part, void* o, float* lse,
                       int B, int Sq, int Hq, int d, int num_splits, int dtype, void* stream);

/* Host mirrors of the planner's integer rules, for tests and tooling. */
/* Key-block range of query block m_block, then of split `split` of
 * `num_splits` ([FA-tiling] §3.2, §5.3); pack folds G heads into rows. */
int attn_n_block_range(int Sq, int Skb, int G, int pack, int causal, int window_left,
                         int block_m, int block_n, int m_block, int split, int num_splits,
                         int* n_min, int* n_max);
/* [FA-tiling] §6.2: pack iff varlen, or row efficiency without packing is
 * below 0.9 of the efficiency with packing. Returns 0 or 1. */
int attn_should_pack_gqa(int varlen, int seqlen_q, int qhead_per_khead, int block_m);
/* [FA-tiling] §5.2 split heuristic (kept as an ablation of the default rule):
 * 1 split if tiles >= 0.8 * SMs (or ceil(KV/L2) splits for a long non-causal
 * KV), 1 if there are at most 4 key blocks, else the smallest split count
 * whose wave efficiency reaches 0.85 of the best. */
int attn_num_splits_fa3(int total_mblocks, int num_sms, int num_n_blocks, int num_m_blocks,
                          long long size_one_kv_head, int is_causal_or_local, int max_splits);
/* [FA-tiling] §3.4 get_m_block_min_max: query-block range [m_min, m_max) whose
 * rows see a key of key block n_block (fixed key length Sk; empty if
 * m_max <= m_min). */
int attn_m_block_range(int Sq, int Sk, int causal, int window_left, int block_m, int block_n,
                         int n_block, int* m_min, int* m_max);
/* The plan attn_fwd_dv would use (host only). */
int attn_plan_fwd_dv(int B, int Hq, int Hkv, int Sq, int Sk, int d, int d_v, int causal,
                       int window_left, int num_splits, int dtype, int num_cus,
                       attn_plan_t* out);

/* Default split rule, a reading of [llama.cpp] for 256 CUs: 1 split when
 * tiles >= wg_per_cu * num_cus or there are fewer than 2 key blocks; else
 * min(s_occ, s_chunk), at least 1 and at most 256, with s_occ =
 * min(ceil(wg_per_cu * num_cus / tiles), n_blocks) (toward wg_per_cu
 * workgroups per CU) and s_chunk = n_blocks / ceil(min_chunk_rows / block_n)
 * (every split keeps min_chunk_rows keys). */
int attn_num_splits_occupancy(int tiles, int num_cus, int n_blocks, int block_n,
                                int min_chunk_rows, int wg_per_cu);

/* Kernel timing for measurement tools: while enabled, every launch of the
 * forward kernel, the combine kernel and the persistent kernels' counter reset
 * is bracketed by HIP events on its stream.
 * attn_profile_end synchronises those events and returns the summed
 * durations (ms) and launch counts per kind (any output pointer may be null),
 * then disables recording. */
int attn_profile_begin(int max_launches);
int attn_profile_end(double* fwd_ms, int* fwd_launches, double* combine_ms,
                       int* combine_launches, double* prep_ms, int* prep_launches);
/* Same, for every kind: ms[k], launches[k] for k < n_kinds (at most 6) with
 * kinds 0 forward, 1 combine, 2 tile counter reset, 3 backward
 * key-block kernel, 4 backward pre- and post-passes, 5 backward dQ kernel. */
int attn_profile_end_kinds(double* ms, int* launches, int n_kinds);

/* Caller-owned scratch ([Occupancy], "The Fix": the split partials live in a
 * global scratch buffer). Binds dev_ptr[0, bytes) -- device memory of the
 * device the calls run on, 256-byte aligned -- to the calling host thread:
 * later calls from this thread put their split partials, the backward's row
 * sums and tile counters there, and never allocate or
 * synchronise. A call that needs more than `bytes` (the workspace_bytes of its
 * plan: attn_plan_fwd, attn_plan_fwd_dv, attn_plan_bwd) returns ATTN_EINVAL
 * and launches nothing. dev_ptr NULL or bytes 0 unbinds (back to the
 * library's own buffer). The memory stays the caller's: keep it alive while
 * calls that use it may run, and do not give one workspace to calls that can
 * overlap on the GPU (two streams need two workspaces; then they may run
 * concurrently). Its contents need no initialisation. Errors: ATTN_EINVAL for
 * a misaligned pointer. */
int attn_set_workspace(void* dev_ptr, size_t bytes);

/* Process-wide planner switches, for tools and tests (defaults are the measured
 * best; other values select ablations). name is the switch's environment
 * variable, with or without its ATTN_ prefix, e.g. "ATTN_PREFILL_WAVES" or
 * "SPLIT_RULE"; each is read from the environment once, at the first call, and
 * afterwards changes only through attn_set_option. Not synchronised with calls
 * running on other host threads: set switches before issuing such calls.
 * ATTN_TRACE=1 prints every forward call's plan to stderr. Unknown names give
 * ATTN_EINVAL. */
int attn_set_option(const char* name, int value);
int attn_get_option(const char* name, int* value);

/* Measurement aid (not part of the attention path): reads [buf, buf + bytes)
 * of device memory once with the 16-byte non-temporal loads the decode kernel
 * streams K and V with, over `workgroups` workgroups of 256 threads (<= 0:
 * 512, the decode grid of the GQA decode workload), and writes almost nothing
 * (sink: device uint32[workgroups], written only for one improbable value).
 * The reference rate for the decode kernel's HBM bandwidth. buf 16-byte
 * aligned, bytes a multiple of 16; errors ATTN_EINVAL, ATTN_EHIP. */
int attn_stream_read(const void* buf, size_t bytes, int workgroups, void* sink, void* stream);

/* Message of the last failure on this thread ("" if none). */
const char* attn_last_error(void);

#ifdef __cplusplus
}
#endif
#endif
