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
    int needs_vt;           // > 0: reads V as fp16 V^T from the V pre-pass (FwdParams::vt),
                            // keys permuted in blocks of this many (16 or 32)
    int persistent;         // > 0: persistent workgroups (this many per CU) over tile queues
    int dv;                 // value / output width when it differs from d (0: equal to d)
    int kdma;               // decode kernels: 1 = K through LDS in 32-key halves, 0 = K into registers
};

// Compiled variants of the general forward kernel and of the split-KV decode
// kernel (each list null-terminated by launch == nullptr).
const FwdVariant* fwd_variants();
const FwdVariant* decode_variants();
const FwdVariant* prefill_variants();
const FwdVariant* mla_variants();   // values of their own width (d_v != d)

// The V pre-pass: V (bf16) -> fp16 V^T in FwdParams::vt (pitch FwdParams::skp).
hipError_t launch_v_to_f16t(const FwdParams& p, hipStream_t stream);

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

}  // namespace tpa
