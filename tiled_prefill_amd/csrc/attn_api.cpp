// attn_api.cpp -- the C-ABI of libattn.so: argument checks, the host planner
// (tile choice, GQA packing, split count, grid), the split workspace, and the
// launches of the forward and combine kernels.
//
// Citations:
//   [FA-tiling]  "分块策略与调度" (FlashAttention tiling strategy and scheduling)
//   [Occupancy]  "The Occupancy Awakening: Rewriting a Flash Attention Kernel for
//                Blackwell's 188 SMs"
//   [llama.cpp]  llama.cpp pull request 21086 review thread
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/attn.h"
#include "attn_kernels.h"
#include "attn_plan.h"

using namespace tpa;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int env_int(const char* name, int dflt) {
    const char* s = getenv(name);
    if (!s || !*s) return dflt;
    return atoi(s);
}

// ---------------------------------------------------------------------------
// process-wide switches (attn_kernels.h: Options), read from the environment
// once, then changed only by attn_set_option
// ---------------------------------------------------------------------------
struct OptionDef {
    const char* name;
    int Options::*field;
    int dflt;
};
const OptionDef kOptionDefs[] = {
    {"ATTN_GENERIC_DECODE", &Options::generic_decode, 0},
    {"ATTN_DECODE_WAVES", &Options::decode_waves, 4},
    {"ATTN_DECODE_KDMA", &Options::decode_kdma, 1},
    {"ATTN_GENERIC_PREFILL", &Options::generic_prefill, 0},
    {"ATTN_PREFILL_WAVES", &Options::prefill_waves, 0},
    {"ATTN_PREFILL_PERSIST", &Options::prefill_persist, 0},
    {"ATTN_PREFILL_SKIP", &Options::prefill_skip, 0},
    {"ATTN_VERIFY_TILE", &Options::verify_tile, 1},
    {"ATTN_F32_DMA", &Options::f32_dma, 1},
    {"ATTN_F32_WAVES", &Options::f32_waves, 4},
    {"ATTN_MIN_CHUNK", &Options::min_chunk, 256},
    {"ATTN_WG_PER_CU", &Options::wg_per_cu, 2},
    {"ATTN_SPLIT_RULE", &Options::split_rule, 0},
    {"ATTN_VARLEN_CHUNK", &Options::varlen_chunk, 1024},
    {"ATTN_VARLEN_UNITS", &Options::varlen_units, 1},
    {"ATTN_MLA_MIN_CHUNK", &Options::mla_min_chunk, 64},
    {"ATTN_MLA_WAVES", &Options::mla_waves, 8},
    {"ATTN_SPLIT_MAJOR", &Options::split_major, -1},
    {"ATTN_COMBINE_COLS", &Options::combine_cols, -1},
    {"ATTN_COMBINE_ROWS", &Options::combine_rows, 1},
    {"ATTN_COMBINE_SMALL", &Options::combine_small, 1},
    {"ATTN_BWD_BN", &Options::bwd_bn, 64},
    {"ATTN_BWD_ATOMIC", &Options::bwd_atomic, 0},
    {"ATTN_BWD_DQ_ROWS", &Options::bwd_dq_rows, 0},
    {"ATTN_BWD_DMA", &Options::bwd_dma, 2},
    {"ATTN_TRACE", &Options::trace, 0},
};
Options g_options;
std::once_flag g_options_once;

Options& mutable_options() {
    std::call_once(g_options_once, [] {
        for (const OptionDef& o : kOptionDefs) g_options.*o.field = env_int(o.name, o.dflt);
    });
    return g_options;
}

// "ATTN_X" or "X", case as declared
const OptionDef* find_option(const char* name) {
    if (!name) return nullptr;
    for (const OptionDef& o : kOptionDefs)
        if (strcmp(o.name, name) == 0 || strcmp(o.name + 5, name) == 0) return &o;
    return nullptr;
}

// ---------------------------------------------------------------------------
// split-count rules
// ---------------------------------------------------------------------------

// Default rule, a reading of the [llama.cpp] thread for 256 CUs: split toward
// wg_per_cu (2) workgroups per CU, so a CU stays busy while one workgroup waits
// at a barrier, but only as far as every split keeps at least min_chunk_rows
// keys: S = min(ceil(target / tiles), n_blocks / chunk_blocks), at least 1, at
// most 256. (Splits below the chunk cost more in partials to merge than they
// gain: fp32 decode over 256 keys, 4 splits 12.6 us vs 1 split 9.9 us; fp32
// verify, 2 x 16 heads x 17 rows over 2065 keys, 16 splits 36.5 us vs 8 35.2.)
int occupancy_rule(int tiles, int num_cus, int n_blocks, int block_n, int min_chunk_rows,
                   int wg_per_cu) {
    const int target = wg_per_cu * num_cus;
    if (tiles >= target || n_blocks < 2) return 1;
    const int min_chunk_blocks = imax(1, ceil_div(min_chunk_rows, block_n));
    const int s_occ = imin(ceil_div(target, tiles), n_blocks);
    const int s_chunk = n_blocks / min_chunk_blocks;
    return imax(1, imin(ATTN_MAX_SPLITS, imin(s_occ, s_chunk)));
}

// The other reading of the same text, as an ablation: reach the workgroup target
// even below the minimum chunk, then split further while chunks keep it.
int occupancy_first_rule(int tiles, int num_cus, int n_blocks, int block_n, int min_chunk_rows,
                         int wg_per_cu) {
    const int target = wg_per_cu * num_cus;
    if (tiles >= target || n_blocks < 2) return 1;
    const int min_chunk_blocks = imax(1, ceil_div(min_chunk_rows, block_n));
    const int s_occ = imin(ceil_div(target, tiles), n_blocks);
    const int s_chunk = n_blocks / min_chunk_blocks;
    return imax(1, imin(ATTN_MAX_SPLITS, imax(s_occ, s_chunk)));
}

// [FA-tiling] §5.2, as an ablation.
int fa3_rule(int total_mblocks, int num_sms, int num_n_blocks, int num_m_blocks,
             long long size_one_kv_head, bool is_causal_or_local, int max_splits) {
    if (total_mblocks >= 0.8f * num_sms) {
        const long long size_l2 = 50LL * 1024 * 1024;
        if (size_one_kv_head > size_l2 && num_m_blocks >= num_sms * 2 && !is_causal_or_local)
            return imin((int)((size_one_kv_head + size_l2 - 1) / size_l2), max_splits);
        return 1;
    }
    if (num_n_blocks <= 4) return 1;
    max_splits = imin(imin(max_splits, num_sms), num_n_blocks);
    float max_eff = 0.f;
    std::vector<float> eff(max_splits + 1, 0.f);
    for (int s = 1; s <= max_splits; ++s) {
        const float waves = float(total_mblocks) * s / num_sms;
        eff[s] = waves / ceilf(waves);
        if (eff[s] > max_eff) max_eff = eff[s];
    }
    for (int s = 1; s <= max_splits; ++s)
        if (eff[s] >= 0.85f * max_eff) return s;
    return 1;
}

// [Occupancy] "The Fix": NSPLIT = clamp(ceil(kv_len / 2048), 1, 32), as an ablation.
int blog_rule(int sk) { return imax(1, imin(32, ceil_div(sk, 2048))); }

// GQA packing decision ([FA-tiling] §6.2). The row efficiency of a tiling is
// the share of a query block's rows that exist: seqlen_q / (block_m *
// ceil(seqlen_q / block_m)) without packing, and the same with g * seqlen_q
// packed rows. Packing pays when the first is below nine tenths of the second.
// seqlen_q cancels from that inequality, leaving the integer comparison
//   10 * ceil(g * seqlen_q / block_m) < 9 * g * ceil(seqlen_q / block_m).
// Variable-length batches always pack.
bool should_pack(bool varlen, int seqlen_q, int g, int block_m) {
    if (varlen) return true;
    const long long blocks_packed = ((long long)seqlen_q * g + block_m - 1) / block_m;
    const long long blocks_plain = ceil_div(seqlen_q, block_m);
    return 10 * blocks_packed < 9LL * g * blocks_plain;
}

int device_cus() {
    static int cached = 0;
    if (cached > 0) return cached;
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
        cached = n;
    else
        cached = 256;  // MI355X
    return cached;
}

// ---------------------------------------------------------------------------
// planner
// ---------------------------------------------------------------------------
struct Problem {
    int B, Hq, Hkv, Sq, Sk, d, causal, window_left, num_splits, dtype, varlen;
    long long sum_seqlens_k;
    float scale;
    int dv = 0;  // value / output width; 0 means d
};

int check_problem(const Problem& p) {
    if (p.B < 0 || p.Sq < 0 || p.Sk < 0)
        return fail(ATTN_EINVAL, "negative size (B=%d Sq=%d Sk=%d)", p.B, p.Sq, p.Sk);
    if (p.Hq < 1 || p.Hkv < 1 || p.Hq % p.Hkv != 0)
        return fail(ATTN_EINVAL, "Hq=%d must be a positive multiple of Hkv=%d", p.Hq, p.Hkv);
    if (p.dtype != ATTN_FP32 && p.dtype != ATTN_BF16)
        return fail(ATTN_EUNSUPPORTED, "dtype %d is not fp32 (0) or bf16 (1)", p.dtype);
    const int dv = p.dv > 0 ? p.dv : p.d;
    if (dv != p.d) {
        if (!(p.d == 576 && dv == 512 && p.dtype == ATTN_BF16))
            return fail(ATTN_EUNSUPPORTED, "d=%d with d_v=%d is not built (bf16 576/512 only)", p.d, dv);
    } else if (p.d != 64 && p.d != 128) {
        return fail(ATTN_EUNSUPPORTED, "head dim %d is not built (64 or 128)", p.d);
    }
    if (p.window_left < -1) return fail(ATTN_EINVAL, "window_left=%d < -1", p.window_left);
    if (!(p.scale > 0.f) || !isfinite(p.scale))
        return fail(ATTN_EINVAL, "scale must be finite and > 0");
    if (p.num_splits > ATTN_MAX_SPLITS)
        return fail(ATTN_EINVAL, "num_splits=%d > %d", p.num_splits, ATTN_MAX_SPLITS);
    if (p.B > 65535) return fail(ATTN_EINVAL, "B=%d exceeds the grid limit 65535", p.B);
    const long long elems = (long long)p.B * p.Sq * p.Hq * p.d;
    const long long kv = (long long)p.B * p.Sk * p.Hkv * p.d;
    if (elems > (1LL << 40) || kv > (1LL << 40)) return fail(ATTN_EINVAL, "tensor too large");
    if ((long long)p.Sq * (p.Hq / p.Hkv) > 0x7fffffffLL / 2)
        return fail(ATTN_EINVAL, "Sq*G too large");
    return ATTN_OK;
}

struct Plan {
    attn_plan_t pub;
    const FwdVariant* var;
    size_t ctr_offset = 0;  // byte offset of the persistent kernels' tile counters
};

int make_plan(const Problem& p, int num_cus, Plan* out) {
    int rc = check_problem(p);
    if (rc) return rc;
    const int G = p.Hq / p.Hkv;
    if (num_cus <= 0) num_cus = device_cus();
    const Options& opt = options();

    // ---- tile choice ([FA-tiling] §2, retargeted to gfx950): a "decode" tile of
    // 16 rows when all query rows of a KV head (packed) fit in 16, else a
    // "prefill" tile; packing per [FA-tiling] §6.2.
    const bool decode = (G > 1) ? (p.Sq * G <= 16) : (p.Sq <= 16);
    const int dv = p.dv > 0 ? p.dv : p.d;
    const FwdVariant* var = nullptr;
    if (dv != p.d) {  // values of their own width: the latent-attention kernel
        // (ATTN_MLA_WAVES: 4 = each wave owns all output columns of its rows,
        // 8 = two waves per row block split the output columns)
        const int want_wn = opt.mla_waves == 8 ? 2 : 1;
        for (const FwdVariant* v = mla_variants(); v->launch; ++v)
            if (v->dtype == p.dtype && v->d == p.d && v->dv == dv && v->waves_n == want_wn) {
                var = v;
                break;
            }
        if (!var) return fail(ATTN_EUNSUPPORTED, "no kernel for d=%d d_v=%d", p.d, dv);
    }
    if (!var && decode && opt.generic_decode == 0) {
        const int want_waves = opt.decode_waves;  // waves per workgroup (4 or 8)
        // ATTN_DECODE_KDMA: 2 = K in registers and V through LDS in whole blocks,
        // 1 = K and V through LDS in 32-key halves, 0 = K straight into registers
        // with 16-row V tiles (ablation); a form with no variant for these waves
        // and d falls back to the next lower one
        const int want_kdma = imax(0, imin(2, opt.decode_kdma));
        for (int kd = want_kdma; kd >= 0 && !var; --kd)
            for (const FwdVariant* v = decode_variants(); v->launch; ++v)
                if (v->dtype == p.dtype && v->d == p.d && v->waves_n == want_waves && v->kdma == kd) {
                    var = v;
                    break;
                }
    }
    if (!var && !decode && opt.generic_prefill == 0) {
        // Tile rows ([FA-tiling] §2.5: smaller blocks where masking cuts tiles):
        // 256-row workgroups (8 waves) for full and causal masks, 128 rows (4
        // waves) with a sliding window, where a 256-row tile spends ~20% of its
        // work on masked corners for window 1024 (measured 599 vs 698 TFLOP/s).
        // ATTN_PREFILL_WAVES overrides (ablation).
        const int want = opt.prefill_waves > 0 ? opt.prefill_waves : (p.window_left >= 0 ? 4 : 8);
        // 1 = persistent workgroups over per-XCD tile queues
        const int want_persist = opt.prefill_persist ? 1 : 0;
        int skip = opt.prefill_skip;  // ablation: take a later match
        for (const FwdVariant* v = prefill_variants(); v->launch; ++v)
            if (v->dtype == p.dtype && v->d == p.d && v->waves_m == want &&
                (v->persistent > 0) == (want_persist > 0) && skip-- <= 0) {
                var = v;
                break;
            }
    }
    const int head_rows = G > 1 ? p.Sq * G : p.Sq;
    // fp32 with at most 32 (packed) query rows per KV head (decode, speculative
    // verify): the kernel that copies K/V into per-wave LDS stages
    // (ATTN_F32_DMA: 1 = for 17..32 rows, 2 = also for decode's 1..16 rows;
    // ATTN_F32_WAVES: waves per workgroup, 4 or 8 where d has that form)
    if (!var && p.dtype == ATTN_FP32 && head_rows <= 32 && (opt.f32_dma == 2 || (opt.f32_dma == 1 && !decode)))
        for (int pass = 0; pass < 2 && !var; ++pass)
            for (const FwdVariant* v = f32_dma_variants(); v->launch; ++v)
                if (v->d == p.d && (pass == 1 || v->waves_n == opt.f32_waves)) {
                    var = v;
                    break;
                }
    // general tile kernel: decode tiles (16 rows) for decode, 32-row tiles when a
    // KV head's query rows (packed) are at most 32, else the widest row tile
    // (ATTN_VERIFY_TILE: 0 = widest row tile, 1 = 32-row tile over 2 x 2 waves,
    // 2 = 32-row tile over 2 x 4 waves with 128-key tiles)
    const int verify_tile = opt.verify_tile;
    const int want_bm = decode ? 16 : (head_rows <= 32 && verify_tile ? 32 : 0);
    const int want_wn = want_bm == 32 ? (verify_tile == 2 ? 4 : 2) : 0;
    for (int pass = 0; pass < 2 && !var; ++pass)
        for (const FwdVariant* v = fwd_variants(); v->launch; ++v) {
            if (v->dtype != p.dtype || v->d != p.d) continue;
            const bool ok = pass == 0 ? (want_bm ? v->block_m == want_bm && (!want_wn || v->waves_n == want_wn)
                                                 : v->block_m > 32)
                                      : (decode ? v->block_m <= 16 : v->block_m > 16);
            if (ok) {
                var = v;
                break;
            }
        }
    if (!var) return fail(ATTN_EUNSUPPORTED, "no kernel variant for dtype %d d %d", p.dtype, p.d);
    const int BM = var->block_m, BN = var->block_n;
    bool pack = false;
    if (G > 1) pack = (decode || var->dv) ? true : should_pack(p.varlen != 0, p.Sq, G, BM);

    attn_plan_t& q = out->pub;
    q = attn_plan_t{};
    q.pack_gqa = pack;
    q.block_m = BM;
    q.block_n = BN;
    q.waves_m = var->waves_m;
    q.waves_n = var->waves_n;
    q.threads = 64 * var->waves_m * var->waves_n;
    q.lds_bytes = var->lds_bytes;
    q.num_cus = num_cus;
    const int rows = pack ? p.Sq * G : p.Sq;
    q.num_m_blocks = ceil_div(imax(rows, 0), BM);
    q.grid_heads = pack ? p.Hkv : p.Hq;
    q.lpt = p.causal ? 1 : 0;

    // ---- key blocks per tile (fixed-length view with Sk)
    long long visited = 0;
    int max_blocks = 0;
    for (int m = 0; m < q.num_m_blocks; ++m) {
        int lo, hi;
        n_block_range(p.Sq, p.Sk, G, pack, p.causal, p.window_left, BM, BN, m, &lo, &hi);
        const int nb = imax(0, hi - lo);
        visited += nb;
        max_blocks = imax(max_blocks, nb);
    }
    q.visited_blocks = visited * (long long)q.grid_heads * p.B;

    // ---- split count ([llama.cpp] occupancy rule; [FA-tiling] §5 ablation)
    const long long tiles = (long long)p.B * q.grid_heads * q.num_m_blocks;
    const int min_chunk = opt.min_chunk;
    const int wg_per_cu = imax(1, opt.wg_per_cu);
    const int rule = opt.split_rule;  // 0 occupancy, 1 fa3, 2 blog, 3 occupancy first
    int S = 1;
    int chunk = 0;
    if (p.num_splits >= 1) {
        S = p.num_splits;
    } else if (tiles > 0) {
        const int t = (int)(tiles > 0x7fffffff ? 0x7fffffff : tiles);
        if (rule == 1) {
            const long long kvh = (long long)p.Sk * p.d * 2 * (p.dtype == ATTN_BF16 ? 2 : 4);
            S = fa3_rule(t, num_cus, max_blocks, q.num_m_blocks, kvh,
                         p.causal || p.window_left >= 0, 128);
        } else if (rule == 2) {
            S = blog_rule(p.Sk);
        } else if (rule == 3) {
            S = occupancy_first_rule(t, num_cus, max_blocks, BN, min_chunk, wg_per_cu);
        } else if (p.varlen) {
            // per-sequence chunk: as many splits as keep >= 1024 keys each (fewer
            // partials for the combine; measured per step on 16 sequences of
            // 512..16384 keys with the work-unit grid: 512-key chunks 112.0 us,
            // 1024 108.2, 1536 109.4, 2048 112.4), but enough to reach the
            // workgroup target when the batch is short
            const long long sum = p.sum_seqlens_k > 0 ? p.sum_seqlens_k : (long long)p.B * p.Sk;
            const long long blocks = (sum + BN - 1) / BN * q.grid_heads * (long long)q.num_m_blocks;
            const long long target = (long long)wg_per_cu * num_cus;
            int cb = imax(1, ceil_div(opt.varlen_chunk, BN));
            if (blocks / cb < target) cb = (int)imax(1, (int)(blocks / target));
            chunk = cb;
            S = imax(1, imin(ATTN_MAX_SPLITS, ceil_div(imax(max_blocks, 1), cb)));
            if (S == 1) chunk = 0;
        } else if (var->dv) {
            // The latent kernel holds one workgroup per CU (136 KB of LDS): split as
            // far as one wave of workgroups allows (tiles * S <= CUs; a second,
            // partial wave costs more than the splits save: 65,536 keys, 5 query
            // blocks, 51 splits 161 us vs 64 splits 236 us) and every split keeps
            // a minimum chunk of 64 keys (the 8-wave form on 2 x 16 heads over 2065
            // keys: 64-key chunks, 25 splits, 29.7 us per call; 128-key, 16 splits,
            // 32.4 us).
            const int mc = imax(1, ceil_div(opt.mla_min_chunk, BN));
            S = imin(imax(1, num_cus / t), imax(1, max_blocks / mc));
        } else {
            S = occupancy_rule(t, num_cus, max_blocks, BN, min_chunk, wg_per_cu);
        }
    }
    S = imax(1, imin(S, ATTN_MAX_SPLITS));
    q.num_splits = S;
    q.chunk_blocks = chunk;
    if (var->grid_1d) {
        // one dimension over every tile (persistent kernels: over the resident
        // workgroups), padded to a multiple of the 8 XCDs
        const long long total = (long long)p.B * q.grid_heads * S * q.num_m_blocks;
        if (total > 0x7fffffffLL - 8) return fail(ATTN_EINVAL, "too many tiles");
        long long launch = total;
        if (var->persistent > 0) launch = std::min<long long>(total, (long long)num_cus * var->persistent);
        q.grid_x = (int)((launch + 7) / 8 * 8);
        q.grid_y = 1;
        q.grid_z = 1;
    } else if (p.varlen && chunk > 0 && S > 1 && var->kdma && opt.varlen_units) {
        // variable-length decode over (sequence, split) work units ([FA-tiling]
        // §4.5): sequence b has S_b = max(1, ceil(len_b / (BN chunk))) or fewer
        // splits, so sum_b S_b <= sum_seqlens_k / (BN chunk) + B; with no sum
        // given, B * S
        const long long per = (long long)BN * chunk;
        long long units = (long long)p.B * S;
        if (p.sum_seqlens_k > 0) units = std::min(units, p.sum_seqlens_k / per + p.B);
        q.work_units = (int)units;
        q.grid_x = (int)units;
        q.grid_y = q.grid_heads;
        q.grid_z = 1;
    } else {
        q.grid_x = q.num_m_blocks;
        q.grid_y = q.grid_heads * S;
        q.grid_z = p.B;
        if (q.grid_y > 65535) return fail(ATTN_EINVAL, "grid heads x splits = %d exceeds 65535", q.grid_y);
    }
    // workspace: split partials, then (persistent kernels) the tile counters,
    // 256-byte aligned
    size_t ws = S > 1 ? attn_workspace_bytes(p.B, p.Hq, p.Sq, dv, S) : 0;
    out->ctr_offset = (ws + 255) & ~(size_t)255;
    if (var->persistent > 0) ws = out->ctr_offset + 256;  // one tile counter per XCD
    q.workspace_bytes = ws;
    out->var = var;
    return ATTN_OK;
}

// ---------------------------------------------------------------------------
// scratch memory of a call (split partials, the backward's row sums, tile
// counters): the caller's workspace bound with attn_set_workspace if there is
// one, else the library's own buffer on the current device (grown on demand;
// host threads serialised on it by a lock)
// ---------------------------------------------------------------------------
struct Workspace {
    std::mutex mu;
    void* ptr = nullptr;
    size_t bytes = 0;
};
Workspace g_ws[64];

// The per-device workspace, at least `bytes` long (caller holds ws.mu).
int ensure_workspace(Workspace& ws, size_t bytes) {
    if (ws.bytes >= bytes) return ATTN_OK;
    if (ws.ptr) {
        (void)hipDeviceSynchronize();  // earlier calls may still use the old buffer
        (void)hipFree(ws.ptr);
        ws.ptr = nullptr;
        ws.bytes = 0;
    }
    hipError_t e = hipMalloc(&ws.ptr, bytes);
    if (e != hipSuccess) {
        ws.ptr = nullptr;
        return fail(ATTN_ENOMEM, "workspace of %zu bytes: %s", bytes, hipGetErrorString(e));
    }
    ws.bytes = bytes;
    return ATTN_OK;
}

struct UserWorkspace {
    void* ptr = nullptr;
    size_t bytes = 0;
};
thread_local UserWorkspace t_user_ws;  // per host thread

struct Scratch {
    void* ptr = nullptr;
    std::unique_lock<std::mutex> lock;  // held while the library's own buffer is in use
};

static_assert(ATTN_NOALLOC_SCRATCH_BYTES == kNoAllocScratchBytes, "header and library agree on the static scratch");

// Where a forward call's scratch comes from: the default (a bound caller
// workspace, else the library's own buffer), or attn_fwd_noalloc's static array.
enum ScratchSource { SCRATCH_DEFAULT = 0, SCRATCH_STATIC = 1 };

// Scratch of `bytes` for one call on the current device. Fails, with nothing
// launched yet, when a caller workspace is bound and too small, or when the
// static array is too small.
int get_scratch(size_t bytes, Scratch* out, int source = SCRATCH_DEFAULT) {
    if (bytes == 0) return ATTN_OK;
    if (source == SCRATCH_STATIC) {
        if (bytes > kNoAllocScratchBytes)
            return fail(ATTN_EINVAL, "this call needs %zu bytes of scratch; attn_fwd_noalloc holds %zu",
                        bytes, kNoAllocScratchBytes);
        const hipError_t e = noalloc_scratch(&out->ptr);
        if (e != hipSuccess) return fail(ATTN_EHIP, "static scratch address: %s", hipGetErrorString(e));
        return ATTN_OK;
    }
    const UserWorkspace& u = t_user_ws;
    if (u.ptr) {
        if (bytes > u.bytes)
            return fail(ATTN_EINVAL, "the workspace bound to this thread holds %zu bytes; this call needs %zu",
                        u.bytes, bytes);
        out->ptr = u.ptr;
        return ATTN_OK;
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return fail(ATTN_EHIP, "hipGetDevice failed");
    Workspace& ws = g_ws[dev];
    out->lock = std::unique_lock<std::mutex>(ws.mu);
    const int rc = ensure_workspace(ws, bytes);
    if (rc) return rc;
    out->ptr = ws.ptr;
    return ATTN_OK;
}


struct Profiler {
    std::mutex mu;
    bool on = false;
    int max_launches = 0;
    std::vector<hipEvent_t> ev;  // pairs
    std::vector<int> kind;       // 0 forward, 1 combine, 2 tile counter reset,
                                 // 3 backward key-block kernel, 4 backward pre/post
                                 // passes, 5 backward dQ kernel
    int used = 0;
} g_prof;

// Records a start event if profiling; returns the slot or -1.
int prof_start(int kind, hipStream_t s) {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    if (!g_prof.on || g_prof.used >= g_prof.max_launches) return -1;
    const int slot = g_prof.used++;
    g_prof.kind[slot] = kind;
    (void)hipEventRecord(g_prof.ev[2 * slot], s);
    return slot;
}
void prof_stop(int slot, hipStream_t s) {
    if (slot < 0) return;
    (void)hipEventRecord(g_prof.ev[2 * slot + 1], s);
}

// ATTN_TRACE=1: one line per forward call with the planner's choices
void trace_plan(const Problem& pr, const Plan& plan) {
    const attn_plan_t& q = plan.pub;
    fprintf(stderr,
            "attn: B=%d Hq=%d Hkv=%d Sq=%d Sk=%d d=%d dv=%d dtype=%d causal=%d window_left=%d varlen=%d -> "
            "tile %dx%d waves %dx%d pack=%d splits=%d chunk=%d grid=(%d,%d,%d) threads=%d lds=%d "
            "persistent=%d workspace=%zu\n",
            pr.B, pr.Hq, pr.Hkv, pr.Sq, pr.Sk, pr.d, pr.dv > 0 ? pr.dv : pr.d, pr.dtype, pr.causal,
            pr.window_left, pr.varlen, q.block_m, q.block_n, q.waves_m, q.waves_n, q.pack_gqa,
            q.num_splits, q.chunk_blocks, q.grid_x, q.grid_y, q.grid_z, q.threads, q.lds_bytes,
            plan.var->persistent, q.workspace_bytes);
}

int run_fwd(const Problem& pr, const void* q, const void* k, const void* v, void* o, float* lse,
            const int* seqlens_k, void* stream_v, int scratch_source = SCRATCH_DEFAULT) {
    // pointers are checked only where they will be read (empty tensors may be null)
    const bool has_rows = pr.B > 0 && pr.Sq > 0;
    if (has_rows && (!q || !o)) return fail(ATTN_EINVAL, "null q or o pointer");
    if (has_rows && pr.Sk > 0 && (!k || !v)) return fail(ATTN_EINVAL, "null k or v pointer");
    if (pr.varlen && pr.B > 0 && !seqlens_k) return fail(ATTN_EINVAL, "seqlens_k is null");
    Plan plan;
    int rc = make_plan(pr, 0, &plan);
    if (rc) return rc;
    if (!has_rows) return ATTN_OK;
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_v);
    const attn_plan_t& pl = plan.pub;

    FwdParams fp{};
    fp.q = q;
    fp.k = k;
    fp.v = v;
    fp.o = o;
    fp.lse = lse;
    fp.seqlens_k = seqlens_k;
    fp.B = pr.B;
    fp.Hq = pr.Hq;
    fp.Hkv = pr.Hkv;
    fp.Sq = pr.Sq;
    fp.Sk = pr.Sk;
    fp.G = pr.Hq / pr.Hkv;
    fp.causal = pr.causal ? 1 : 0;
    fp.window_left = pr.window_left;
    fp.scale = pr.scale;
    fp.scale_log2 = pr.scale * 1.4426950408889634f;
    fp.pack = pl.pack_gqa;
    fp.num_m_blocks = pl.num_m_blocks;
    fp.grid_heads = pl.grid_heads;
    fp.num_splits = pl.num_splits;
    fp.chunk_blocks = pl.chunk_blocks;
    fp.lpt = pl.lpt;
    fp.work_units = pl.work_units;
    // decode grids: the workgroups of one key range (all grid heads) are
    // dispatched together, so concurrent reads cover whole interleaved KV rows
    fp.split_major = options().split_major >= 0 ? options().split_major : (plan.var->block_m <= 16 ? 1 : 0);
    // decode tiles: block range and split share of fixed-length problems, and the
    // grid-y divisor as a multiply-high
    {
        int lo = 0, hi = 0;
        n_block_range(pr.Sq, pr.Sk, fp.G, fp.pack, fp.causal, fp.window_left, pl.block_m, pl.block_n, 0, &lo, &hi);
        fp.dec_lo = lo;
        fp.dec_hi = hi;
        fp.dec_per = pl.num_splits > 1 ? ceil_div(imax(0, hi - lo), pl.num_splits) : imax(0, hi - lo);
        fp.y_div = imax(1, fp.split_major ? pl.grid_heads : pl.num_splits);
        div_magic((unsigned int)fp.y_div, &fp.y_mul, &fp.y_s1, &fp.y_s2);
    }

    if (options().trace) trace_plan(pr, plan);
    const dim3 grid(pl.grid_x, pl.grid_y, pl.grid_z);
    if (pl.workspace_bytes == 0) {
        const int slot = prof_start(0, stream);
        hipError_t e = plan.var->launch(fp, grid, stream);
        prof_stop(slot, stream);
        if (e != hipSuccess) return fail(ATTN_EHIP, "forward launch: %s", hipGetErrorString(e));
        return ATTN_OK;
    }

    Scratch ws;
    rc = get_scratch(pl.workspace_bytes, &ws, scratch_source);
    if (rc) return rc;
    const size_t rows = (size_t)pr.B * pr.Sq * pr.Hq;
    fp.o_part = reinterpret_cast<float*>(ws.ptr);
    const int dvv = pr.dv > 0 ? pr.dv : pr.d;
    fp.lse_part = fp.o_part + (size_t)pl.num_splits * rows * dvv;
    hipError_t e;
    int slot;
    if (plan.var->persistent > 0) {
        fp.tile_counters = reinterpret_cast<int*>(static_cast<char*>(ws.ptr) + plan.ctr_offset);
        slot = prof_start(2, stream);
        e = launch_tile_counters_reset(fp.tile_counters, stream);
        prof_stop(slot, stream);
        if (e != hipSuccess) return fail(ATTN_EHIP, "tile counter reset: %s", hipGetErrorString(e));
    }

    slot = prof_start(0, stream);
    e = plan.var->launch(fp, grid, stream);
    prof_stop(slot, stream);
    if (e != hipSuccess) return fail(ATTN_EHIP, "forward launch: %s", hipGetErrorString(e));
    if (pl.num_splits == 1) return ATTN_OK;

    CombineParams cp{};
    cp.o_part = fp.o_part;
    cp.lse_part = fp.lse_part;
    cp.o = o;
    cp.lse = lse;
    cp.rows = (int)rows;
    cp.num_splits = pl.num_splits;
    cp.Sq = pr.Sq;
    cp.Hq = pr.Hq;
    slot = prof_start(1, stream);
    e = launch_combine(cp, dvv, pr.dtype == ATTN_BF16, stream);
    prof_stop(slot, stream);
    if (e != hipSuccess) return fail(ATTN_EHIP, "combine launch: %s", hipGetErrorString(e));
    return ATTN_OK;
}


// ---------------------------------------------------------------------------
// backward pass ([FA-tiling] §3.4, §4.6)
// ---------------------------------------------------------------------------
struct BwdPlan {
    attn_bwd_plan_t pub;
    const BwdVariant* var;
    size_t lse2_offset = 0, dsum_offset = 0;  // byte offsets in the workspace
};

int make_bwd_plan(const Problem& p, BwdPlan* out) {
    int rc = check_problem(p);
    if (rc) return rc;
    // key block: 64 keys (16 per wave) unless ATTN_BWD_BN asks for 128 (bf16);
    // dQ by a second kernel unless ATTN_BWD_ATOMIC=1 (fp32 atomics, ablation)
    const Options& opt = options();
    const int want_bn = opt.bwd_bn;
    const int want_atomic = opt.bwd_atomic ? 1 : 0;
    const int want_dq_rows = opt.bwd_dq_rows;  // 0: first listed
    // 2: both kernels DMA their tiles; 1: only the dQ kernel; 0: neither
    const int want_dq_dma = opt.bwd_dma;
    const BwdVariant* var = nullptr;
    for (int pass = 0; pass < 2 && !var; ++pass)
        for (const BwdVariant* v = bwd_variants(); v->launch; ++v)
            if (v->dtype == p.dtype && v->d == p.d && v->atomic_dq == want_atomic &&
                (pass == 1 || (v->block_n == want_bn && v->dq_dma <= want_dq_dma &&
                               (want_dq_rows == 0 || v->atomic_dq || v->dq_block_m == want_dq_rows)))) {
                var = v;
                break;
            }
    if (!var) return fail(ATTN_EUNSUPPORTED, "no backward kernel for dtype %d d %d", p.dtype, p.d);
    const int G = p.Hq / p.Hkv;
    attn_bwd_plan_t& q = out->pub;
    q = attn_bwd_plan_t{};
    q.block_m = var->block_m;
    q.block_n = var->block_n;
    q.threads = 256;
    q.lds_bytes = var->lds_bytes;
    q.num_n_blocks = ceil_div(imax(p.Sk, 0), var->block_n);
    const long long grid = (long long)q.num_n_blocks * p.Hkv * p.B;
    const long long dq_tiles = (long long)ceil_div(imax(p.Sq, 0), imax(1, var->dq_block_m)) * p.Hq * p.B;
    if (grid > 0x7fffffffLL - 8 || dq_tiles > 0x7fffffffLL - 8)
        return fail(ATTN_EINVAL, "too many key or query blocks");
    q.grid_x = (int)grid;
    long long visited = 0;
    for (int n = 0; n < q.num_n_blocks; ++n) {
        int lo, hi;
        m_block_range(p.Sq, p.Sk, p.causal, p.window_left, var->block_m, var->block_n, n, &lo, &hi);
        visited += imax(0, hi - lo);
    }
    q.visited_blocks = visited * G * (long long)p.Hkv * p.B;
    q.dq_block_m = var->atomic_dq ? 0 : var->dq_block_m;
    const size_t rows = (size_t)p.B * p.Sq * p.Hq;
    const size_t acc = var->atomic_dq ? rows * (size_t)p.d * sizeof(float) : 0;
    out->lse2_offset = (acc + 255) & ~(size_t)255;
    out->dsum_offset = (out->lse2_offset + rows * sizeof(float) + 255) & ~(size_t)255;
    q.workspace_bytes = rows ? out->dsum_offset + rows * sizeof(float) : 0;
    out->var = var;
    return ATTN_OK;
}

int run_bwd(const Problem& pr, const void* q, const void* k, const void* v, const void* o,
            const void* dout, const float* lse, void* dq, void* dk, void* dv, void* stream_v) {
    const bool has_rows = pr.B > 0 && pr.Sq > 0;
    const bool has_keys = pr.B > 0 && pr.Sk > 0;
    if (has_rows && (!q || !o || !dout || !lse || !dq))
        return fail(ATTN_EINVAL, "null q, o, dout, lse or dq pointer");
    if (has_keys && (!k || !v || !dk || !dv)) return fail(ATTN_EINVAL, "null k, v, dk or dv pointer");
    BwdPlan plan;
    int rc = make_bwd_plan(pr, &plan);
    if (rc) return rc;
    if (!has_rows && !has_keys) return ATTN_OK;
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_v);

    BwdParams bp{};
    bp.q = q;
    bp.k = k;
    bp.v = v;
    bp.o = o;
    bp.dout = dout;
    bp.lse = lse;
    bp.dq = dq;
    bp.dk = dk;
    bp.dv = dv;
    bp.B = pr.B;
    bp.Hq = pr.Hq;
    bp.Hkv = pr.Hkv;
    bp.Sq = pr.Sq;
    bp.Sk = pr.Sk;
    bp.G = pr.Hq / pr.Hkv;
    bp.causal = pr.causal ? 1 : 0;
    bp.window_left = pr.window_left;
    bp.scale = pr.scale;
    bp.scale_log2 = pr.scale * 1.4426950408889634f;
    bp.num_n_blocks = plan.pub.num_n_blocks;

    Scratch ws;
    if (plan.pub.workspace_bytes > 0) {
        rc = get_scratch(plan.pub.workspace_bytes, &ws);
        if (rc) return rc;
        if (plan.var->atomic_dq) bp.dq_acc = reinterpret_cast<float*>(ws.ptr);
        bp.lse2 = reinterpret_cast<float*>(static_cast<char*>(ws.ptr) + plan.lse2_offset);
        bp.dsum = reinterpret_cast<float*>(static_cast<char*>(ws.ptr) + plan.dsum_offset);
    }
    hipError_t e;
    int slot;
    if (has_rows) {
        slot = prof_start(4, stream);
        e = plan.var->launch_pre(bp, stream);
        prof_stop(slot, stream);
        if (e != hipSuccess) return fail(ATTN_EHIP, "backward pre-pass launch: %s", hipGetErrorString(e));
    }
    // two-pass form: the dQ kernel first (the bf16 form also stores the rows'
    // D = sum_j P dP there), then the key-block kernel, which reads D
    if (has_rows && !plan.var->atomic_dq) {
        slot = prof_start(5, stream);
        e = plan.var->launch_dq(bp, stream);
        prof_stop(slot, stream);
        if (e != hipSuccess) return fail(ATTN_EHIP, "backward dQ launch: %s", hipGetErrorString(e));
    }
    if (has_keys) {
        slot = prof_start(3, stream);
        e = plan.var->launch(bp, stream);
        prof_stop(slot, stream);
        if (e != hipSuccess) return fail(ATTN_EHIP, "backward launch: %s", hipGetErrorString(e));
    }
    if (has_rows && plan.var->atomic_dq) {
        slot = prof_start(4, stream);
        e = plan.var->launch_post(bp, stream);
        prof_stop(slot, stream);
        if (e != hipSuccess) return fail(ATTN_EHIP, "backward post-pass launch: %s", hipGetErrorString(e));
    }
    return ATTN_OK;
}

}  // namespace

namespace tpa {
const Options& options() { return mutable_options(); }
}  // namespace tpa

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
               int Hkv, int Sq, int Sk, int d, int causal, int window_left, float scale,
               int num_splits, int dtype, void* stream) {
    Problem p{B, Hq, Hkv, Sq, Sk, d, causal, window_left, num_splits, dtype, 0, 0, scale};
    return run_fwd(p, q, k, v, o, lse, nullptr, stream);
}

int attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int Hq, int Hkv, int Sq, int Sk, int d, int causal, int window_left,
                     float scale, int num_splits, int dtype, void* stream) {
    Problem p{B, Hq, Hkv, Sq, Sk, d, causal, window_left, num_splits, dtype, 0, 0, scale};
    return run_fwd(p, q, k, v, o, lse, nullptr, stream, SCRATCH_STATIC);
}

int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int Hq, int Hkv, int Sq, int Sk, int d, int causal, int window_left,
                      float scale, int num_splits, int dtype, const int* seqlens_k,
                      long long sum_seqlens_k, void* stream) {
    Problem p{B, Hq, Hkv, Sq, Sk, d, causal, window_left, num_splits, dtype, 1, sum_seqlens_k, scale};
    return run_fwd(p, q, k, v, o, lse, seqlens_k, stream);
}

int attn_fwd_dv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                  int Hkv, int Sq, int Sk, int d, int d_v, int causal, int window_left,
                  float scale, int num_splits, int dtype, void* stream) {
    Problem p{B, Hq, Hkv, Sq, Sk, d, causal, window_left, num_splits, dtype, 0, 0, scale};
    p.dv = d_v;
    if (d_v <= 0) return fail(ATTN_EINVAL, "d_v=%d must be positive", d_v);
    return run_fwd(p, q, k, v, o, lse, nullptr, stream);
}

int attn_plan_fwd_dv(int B, int Hq, int Hkv, int Sq, int Sk, int d, int d_v, int causal,
                       int window_left, int num_splits, int dtype, int num_cus, attn_plan_t* out) {
    if (!out) return fail(ATTN_EINVAL, "null plan pointer");
    if (d_v <= 0) return fail(ATTN_EINVAL, "d_v=%d must be positive", d_v);
    Problem p{B, Hq, Hkv, Sq, Sk, d, causal, window_left, num_splits, dtype, 0, 0, 1.0f};
    p.dv = d_v;
    Plan plan;
    int rc = make_plan(p, num_cus, &plan);
    if (rc) return rc;
    *out = plan.pub;
    return ATTN_OK;
}

int attn_plan_fwd(int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal, int window_left,
                    int num_splits, int dtype, int varlen, long long sum_seqlens_k, int num_cus,
                    attn_plan_t* out) {
    if (!out) return fail(ATTN_EINVAL, "null plan pointer");
    Problem p{B, Hq, Hkv, Sq, Sk, d, causal, window_left, num_splits, dtype, varlen ? 1 : 0,
              sum_seqlens_k, 1.0f};
    Plan plan;
    int rc = make_plan(p, num_cus, &plan);
    if (rc) return rc;
    *out = plan.pub;
    return ATTN_OK;
}

int attn_plan(int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal, int window_left,
              int num_splits, int dtype, int varlen, long long sum_seqlens_k, int num_cus,
              attn_plan_t* out) {
    return attn_plan_fwd(B, Hq, Hkv, Sq, Sk, d, causal, window_left, num_splits, dtype, varlen,
                         sum_seqlens_k, num_cus, out);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
               const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq,
               int Sk, int d, int causal, int window_left, float scale, int dtype, void* stream) {
    Problem p{B, Hq, Hkv, Sq, Sk, d, causal, window_left, 0, dtype, 0, 0, scale};
    return run_bwd(p, q, k, v, o, dout, lse, dq, dk, dv, stream);
}

int attn_plan_bwd(int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal, int window_left,
                    int dtype, attn_bwd_plan_t* out) {
    if (!out) return fail(ATTN_EINVAL, "null plan pointer");
    Problem p{B, Hq, Hkv, Sq, Sk, d, causal, window_left, 0, dtype, 0, 0, 1.0f};
    BwdPlan plan;
    int rc = make_bwd_plan(p, &plan);
    if (rc) return rc;
    *out = plan.pub;
    return ATTN_OK;
}

int attn_m_block_range(int Sq, int Sk, int causal, int window_left, int block_m, int block_n,
                         int n_block, int* m_min, int* m_max) {
    if (!m_min || !m_max) return fail(ATTN_EINVAL, "null output pointer");
    if (Sq < 0 || Sk < 0 || block_m < 1 || block_n < 1 || n_block < 0 || window_left < -1)
        return fail(ATTN_EINVAL, "bad block-range arguments");
    m_block_range(Sq, Sk, causal, window_left, block_m, block_n, n_block, m_min, m_max);
    return ATTN_OK;
}

size_t attn_workspace_bytes(int B, int Hq, int Sq, int d, int num_splits) {
    if (B <= 0 || Hq <= 0 || Sq <= 0 || d <= 0 || num_splits <= 1) return 0;
    const size_t rows = (size_t)B * Hq * Sq;
    return (size_t)num_splits * rows * ((size_t)d + 1) * sizeof(float);
}

int attn_lse_combine(const float* o_part, const float* lse_part, void* o, float* lse, int B,
                       int Sq, int Hq, int d, int num_splits, int dtype, void* stream_v) {
    if (!o_part || !lse_part || !o) return fail(ATTN_EINVAL, "null tensor pointer");
    if (B < 0 || Sq < 0 || Hq < 1) return fail(ATTN_EINVAL, "bad shape");
    if (d != 64 && d != 128 && d != 512)
        return fail(ATTN_EUNSUPPORTED, "value width %d is not built (64, 128, 512)", d);
    if (dtype != ATTN_FP32 && dtype != ATTN_BF16)
        return fail(ATTN_EUNSUPPORTED, "dtype %d", dtype);
    if (num_splits < 1 || num_splits > ATTN_MAX_SPLITS)
        return fail(ATTN_EINVAL, "num_splits=%d outside [1, 256]", num_splits);
    const long long rows = (long long)B * Sq * Hq;
    if (rows > 0x7fffffffLL) return fail(ATTN_EINVAL, "too many rows");
    if (rows == 0) return ATTN_OK;
    CombineParams cp{};
    cp.o_part = o_part;
    cp.lse_part = lse_part;
    cp.o = o;
    cp.lse = lse;
    cp.rows = (int)rows;
    cp.num_splits = num_splits;
    cp.Sq = Sq;
    cp.Hq = Hq;
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_v);
    const int slot = prof_start(1, stream);
    hipError_t e = launch_combine(cp, d, dtype == ATTN_BF16, stream);
    prof_stop(slot, stream);
    if (e != hipSuccess) return fail(ATTN_EHIP, "combine launch: %s", hipGetErrorString(e));
    return ATTN_OK;
}

int attn_n_block_range(int Sq, int Skb, int G, int pack, int causal, int window_left,
                         int block_m, int block_n, int m_block, int split, int num_splits,
                         int* n_min, int* n_max) {
    if (!n_min || !n_max) return fail(ATTN_EINVAL, "null output pointer");
    if (Sq < 1 || Skb < 0 || G < 1 || block_m < 1 || block_n < 1 || m_block < 0 ||
        num_splits < 1 || split < 0 || split >= num_splits || window_left < -1)
        return fail(ATTN_EINVAL, "bad block-range arguments");
    int lo, hi;
    n_block_range(Sq, Skb, G, pack, causal, window_left, block_m, block_n, m_block, &lo, &hi);
    split_range(lo, hi, split, num_splits, n_min, n_max);
    return ATTN_OK;
}

int attn_should_pack_gqa(int varlen, int seqlen_q, int qhead_per_khead, int block_m) {
    if (seqlen_q < 1 || qhead_per_khead < 1 || block_m < 1) return 0;
    return should_pack(varlen != 0, seqlen_q, qhead_per_khead, block_m) ? 1 : 0;
}

int attn_num_splits_fa3(int total_mblocks, int num_sms, int num_n_blocks, int num_m_blocks,
                          long long size_one_kv_head, int is_causal_or_local, int max_splits) {
    if (total_mblocks < 1 || num_sms < 1 || max_splits < 1) return 1;
    return fa3_rule(total_mblocks, num_sms, num_n_blocks, num_m_blocks, size_one_kv_head,
                    is_causal_or_local != 0, max_splits);
}

int attn_num_splits_occupancy(int tiles, int num_cus, int n_blocks, int block_n,
                                int min_chunk_rows, int wg_per_cu) {
    if (tiles < 1 || num_cus < 1 || block_n < 1 || wg_per_cu < 1) return 1;
    return occupancy_rule(tiles, num_cus, n_blocks, block_n, min_chunk_rows, wg_per_cu);
}

int attn_profile_begin(int max_launches) {
    if (max_launches < 1 || max_launches > (1 << 20)) return fail(ATTN_EINVAL, "max_launches");
    std::lock_guard<std::mutex> lk(g_prof.mu);
    for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
    g_prof.ev.assign(2 * (size_t)max_launches, nullptr);
    g_prof.kind.assign(max_launches, 0);
    for (auto& e : g_prof.ev)
        if (hipEventCreate(&e) != hipSuccess) return fail(ATTN_EHIP, "hipEventCreate");
    g_prof.max_launches = max_launches;
    g_prof.used = 0;
    g_prof.on = true;
    return ATTN_OK;
}

int attn_profile_end_kinds(double* ms, int* launches, int n_kinds) {
    std::lock_guard<std::mutex> lk(g_prof.mu);
    double t[6] = {0, 0, 0, 0, 0, 0};
    int n[6] = {0, 0, 0, 0, 0, 0};
    for (int i = 0; i < g_prof.used; ++i) {
        if (hipEventSynchronize(g_prof.ev[2 * i + 1]) != hipSuccess) continue;
        float e_ms = 0.f;
        if (hipEventElapsedTime(&e_ms, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]) == hipSuccess) {
            t[g_prof.kind[i]] += e_ms;
            n[g_prof.kind[i]] += 1;
        }
    }
    for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
    g_prof.ev.clear();
    g_prof.kind.clear();
    g_prof.on = false;
    g_prof.used = 0;
    for (int k = 0; k < n_kinds && k < 6; ++k) {
        if (ms) ms[k] = t[k];
        if (launches) launches[k] = n[k];
    }
    return ATTN_OK;
}

int attn_profile_end(double* fwd_ms, int* fwd_launches, double* combine_ms,
                       int* combine_launches, double* prep_ms, int* prep_launches) {
    double t[3];
    int n[3];
    int rc = attn_profile_end_kinds(t, n, 3);
    if (fwd_ms) *fwd_ms = t[0];
    if (fwd_launches) *fwd_launches = n[0];
    if (combine_ms) *combine_ms = t[1];
    if (combine_launches) *combine_launches = n[1];
    if (prep_ms) *prep_ms = t[2];
    if (prep_launches) *prep_launches = n[2];
    return rc;
}

int attn_set_workspace(void* dev_ptr, size_t bytes) {
    if (dev_ptr && (reinterpret_cast<uintptr_t>(dev_ptr) & 255) != 0)
        return fail(ATTN_EINVAL, "the workspace must be 256-byte aligned");
    UserWorkspace& u = t_user_ws;
    if (!dev_ptr || bytes == 0) {
        u = UserWorkspace{};
        return ATTN_OK;
    }
    u.ptr = dev_ptr;
    u.bytes = bytes;
    return ATTN_OK;
}

int attn_stream_read(const void* buf, size_t bytes, int workgroups, void* sink, void* stream) {
    if (bytes == 0) return ATTN_OK;
    if (!buf || !sink) return fail(ATTN_EINVAL, "null buffer or sink");
    if (bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(buf) & 15) != 0)
        return fail(ATTN_EINVAL, "the buffer must be 16-byte aligned and a multiple of 16 bytes long");
    if (bytes > ((size_t)1 << 40)) return fail(ATTN_EINVAL, "buffer too large");
    if (workgroups <= 0) workgroups = 512;
    if (workgroups > (1 << 20)) return fail(ATTN_EINVAL, "workgroups=%d", workgroups);
    if (bytes / (size_t)workgroups >= ((size_t)1 << 31))
        return fail(ATTN_EINVAL, "more than 2 GiB per workgroup; use more workgroups");
    const hipError_t e = launch_stream_read(buf, bytes, workgroups, sink, reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(ATTN_EHIP, "stream read launch: %s", hipGetErrorString(e));
    return ATTN_OK;
}

int attn_set_option(const char* name, int value) {
    const OptionDef* o = find_option(name);
    if (!o) return fail(ATTN_EINVAL, "unknown option %s", name ? name : "(null)");
    mutable_options().*o->field = value;
    return ATTN_OK;
}

int attn_get_option(const char* name, int* value) {
    const OptionDef* o = find_option(name);
    if (!o || !value) return fail(ATTN_EINVAL, "unknown option %s or null output", name ? name : "(null)");
    *value = mutable_options().*o->field;
    return ATTN_OK;
}

const char* attn_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
