// attn_kernels.h -- launchers of the gfx950 attention kernels (internal to the
// library; the public C-ABI is include/attn.h).
#pragma once

#include <hip/hip_runtime.h>

#include "attn_plan.h"

namespace tpa {

enum DType { DT_FP32 = 0, DT_BF16 = 1 };

// One compiled forward-kernel instantiation: element type, head dim and tile.
struct FwdVariant {
    int dtype, d;
    int block_m, block_n;   // query rows and key rows per tile
    int waves_m, waves_n;   // waves along M (rows) and along N (keys)
    int lds_bytes;
    hipError_t (*launch)(const FwdParams&, dim3 grid, hipStream_t stream);
    int grid_1d;            // 1: one-dimensional XCD-aware grid over all tiles
    int persistent;         // > 0: persistent workgroups (this many per CU) over tile queues
    int dv;                 // value / output width when it differs from d (0: equal to d)
    int kdma;               // decode kernels: 2 = K in registers, V through LDS (whole blocks);
                            // 1 = K and V through LDS in 32-key halves; 0 = K into registers, 16-row V tiles
};

// Compiled variants of the general forward kernel and of the split-KV decode
// kernel (each list null-terminated by launch == nullptr).
const FwdVariant* fwd_variants();
const FwdVariant* decode_variants();
const FwdVariant* prefill_variants();
const FwdVariant* mla_variants();   // values of their own width (d_v != d)
const FwdVariant* f32_dma_variants();  // fp32, <= 32 query rows per KV head, K/V copied into LDS

// Zeroes the per-XCD tile queue counters of a persistent kernel.
hipError_t launch_tile_counters_reset(int* counters, hipStream_t stream);

// One compiled backward instantiation: element type, head dim, key block.
struct BwdVariant {
    int dtype, d;
    int block_n;            // keys per workgroup of the key-block kernel
    int block_m;            // query rows per inner block
    int lds_bytes;
    int atomic_dq;          // 1: dQ accumulated with fp32 atomics (needs the accumulator)
    hipError_t (*launch)(const BwdParams&, hipStream_t stream);       // key-block kernel (dK, dV)
    hipError_t (*launch_pre)(const BwdParams&, hipStream_t stream);   // row sums, lse2, zero dQ acc
    hipError_t (*launch_post)(const BwdParams&, hipStream_t stream);  // atomic_dq: dQ = scale * acc
    hipError_t (*launch_dq)(const BwdParams&, hipStream_t stream);    // else: the dQ kernel
    int dq_block_m;         // query rows per workgroup of the dQ kernel
    int dq_dma;             // 1: the dQ kernel DMAs K/V tiles into LDS (bf16); 2: both kernels DMA their tiles
};
const BwdVariant* bwd_variants();  // null-terminated by launch == nullptr

// The log-sum-exp combine of split partials.
hipError_t launch_combine(const CombineParams& p, int d, int out_bf16, hipStream_t stream);

// A plain streaming read of [buf, buf + bytes) over `workgroups` workgroups
// (measurement aid, attn_tools.hip); sink is device uint32[workgroups].
hipError_t launch_stream_read(const void* buf, size_t bytes, int workgroups, void* sink, hipStream_t stream);

// The static device scratch of attn_fwd_noalloc (attn_scratch.hip): its size,
// and the address of the current device's copy (read once per device).
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
constexpr int kMaxDevices = 64;
hipError_t noalloc_scratch(void** ptr);

// Planner and launch switches. Each starts at its default, is read once per
// process from its ATTN_* environment variable (at the first use), and can be
// changed at run time with attn_set_option. Apart from `trace`, every
// non-default value selects an ablation measured against the default path.
struct Options {
    int generic_decode;   // ATTN_GENERIC_DECODE=1: general tile kernel for bf16 decode tiles
    int decode_waves;     // ATTN_DECODE_WAVES: waves per decode workgroup (4; 8)
    int decode_kdma;      // ATTN_DECODE_KDMA: 1 K through LDS in 32-key halves; 0 K into registers
    int generic_prefill;  // ATTN_GENERIC_PREFILL=1: general tile kernel for bf16 prefill
    int prefill_waves;    // ATTN_PREFILL_WAVES: 8 (256 rows) or 4 (128 rows); 0 = by mask
    int prefill_persist;  // ATTN_PREFILL_PERSIST=1: persistent workgroups over per-XCD queues
    int prefill_skip;     // ATTN_PREFILL_SKIP=n: the n-th later matching prefill variant
    int verify_tile;      // ATTN_VERIFY_TILE: 0 widest row tile, 1 32-row 2x2, 2 32-row 2x4
    int f32_dma;          // ATTN_F32_DMA: fp32 on the LDS-copy kernel for 17..32 rows per KV head (1), for 1..32 (2)
    int varlen_units;     // ATTN_VARLEN_UNITS: variable-length decode on the work-unit grid (1)
    int mla_waves;        // ATTN_MLA_WAVES: latent kernel with 4 waves (all output columns each) or 8
    int f32_waves;        // ATTN_F32_WAVES: that kernel's waves per workgroup (4; 8 where d has that form)
    int min_chunk;        // ATTN_MIN_CHUNK: minimum keys per split (256)
    int wg_per_cu;        // ATTN_WG_PER_CU: workgroup target per CU of the split rule (2)
    int split_rule;       // ATTN_SPLIT_RULE: 0 occupancy, 1 [FA-tiling] 5.2, 2 NSPLIT, 3 occupancy first
    int varlen_chunk;     // ATTN_VARLEN_CHUNK: keys per split of variable-length problems (1024)
    int mla_min_chunk;    // ATTN_MLA_MIN_CHUNK: minimum keys per split of the latent kernel (64)
    int split_major;      // ATTN_SPLIT_MAJOR: grid order of split workgroups; -1 = by tile
    int combine_cols;     // ATTN_COMBINE_COLS: -1 by split count, 0/1 force split groups / columns
    int combine_rows;     // ATTN_COMBINE_ROWS: 1 row-parallel combine for 512-wide rows
    int combine_small;    // ATTN_COMBINE_SMALL: 1 all-loads-first column combine up to 16 splits
    int bwd_bn;           // ATTN_BWD_BN: keys per backward workgroup (64; 128)
    int bwd_atomic;       // ATTN_BWD_ATOMIC=1: single-pass backward with fp32 dQ atomics
    int bwd_dq_rows;      // ATTN_BWD_DQ_ROWS: query rows per dQ workgroup (0 = first listed)
    int bwd_dma;          // ATTN_BWD_DMA: 2 both kernels DMA their tiles, 1 only dQ, 0 neither
    int trace;            // ATTN_TRACE=1: print every call's plan to stderr
};
const Options& options();

}  // namespace tpa
