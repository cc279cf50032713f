// attn_decode.hip -- gfx950 split-KV decode kernel and the log-sum-exp combine.
//
// Citations:
//   [FA-tiling]  "分块策略与调度" (FlashAttention tiling strategy and scheduling)
//   [Occupancy]  "The Occupancy Awakening: Rewriting a Flash Attention Kernel
//                for Blackwell's 188 SMs"
//
// Decode is bound by reading K and V once from HBM. All query rows of one
// (batch, KV head) -- the G packed query heads of a GQA group ([FA-tiling] §6),
// at most 16 rows -- fit one MFMA column block, so a workgroup owns one
// (batch, grid head, split) and its waves walk disjoint 64-key blocks of the
// split's key range, each with its own online-softmax state, merged in LDS at the
// end. K goes straight from global memory into the registers of the MFMA A
// operand; V is staged row-major in a per-wave LDS region and read back
// transposed with ds_read_b64_tr_b16. The loads of the next block are issued as
// soon as the registers they overwrite are consumed, so every wave keeps a full
// block of K and V in flight.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <type_traits>

#include "attn_device.h"
#include "attn_kernels.h"
#include "attn_plan.h"

namespace tpa {

// a switch read from the environment on the host (dflt when unset)
template <int D, int NW>
struct DecodeTile {
    static constexpr int KB = 64;              // keys per wave block
    static constexpr int NSLAB = D / 32;       // 32-d slabs of the QK contraction
    static constexpr int NT = KB / 16;         // 16-key sub-tiles of a block
    static constexpr int DT = D / 16;          // 16-wide d tiles of the output
    static constexpr int CPR = D / 8;          // 16-byte chunks per K/V row
    static constexpr int RPI = 64 / CPR;       // V rows per wave-wide load
    static constexpr int NVL = KB / RPI;       // V loads per lane per block
    static constexpr int ROWB = D * 2;         // bytes per V row in LDS (unpadded)
    static constexpr int V_BYTES = NW * KB * ROWB;
    static constexpr int RED_BYTES = NW * (DT * 4 * 64 + 2 * 64) * 4;
    static constexpr int LDS_BYTES = V_BYTES > RED_BYTES ? V_BYTES : RED_BYTES;
    // XOR swizzle of the 16-byte chunk of V row r in LDS: the transposed reads of
    // 8 consecutive rows x 2 chunks then hit 16 distinct 16-byte bank groups.
    static __device__ __forceinline__ int swz(int r) {
        return D == 128 ? (r & 7) << 1 : ((r >> 1) & 3) << 1;
    }
};

template <int D, int NW>
__global__ void __launch_bounds__(64 * NW, 8 / NW) attn_decode_kernel(FwdParams p) {
    using C = DecodeTile<D, NW>;
    constexpr int KB = C::KB, NSLAB = C::NSLAB, NT = C::NT, DT = C::DT;
    constexpr int CPR = C::CPR, RPI = C::RPI, NVL = C::NVL, ROWB = C::ROWB;
    __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int li = lane & 15, lg = lane >> 4;
    char* vl = smem + wave * KB * ROWB;  // this wave's V block, swizzled rows

    const int hg = p.split_major ? (int)blockIdx.y % p.grid_heads : (int)blockIdx.y / p.num_splits;
    const int split = p.split_major ? (int)blockIdx.y / p.grid_heads : (int)blockIdx.y % p.num_splits;
    const int b = blockIdx.z;
    int Skb = p.Sk;
    if (p.seqlens_k) Skb = imax(0, imin(p.seqlens_k[b], p.Sk));
    const int G = p.G;
    const int hkv = p.pack ? hg : hg / G;
    const int nrows = p.pack ? p.Sq * G : p.Sq;
    const int delta = Skb - p.Sq;

    // key blocks of this split ([FA-tiling] §3.2, §5.3)
    int n_lo, n_hi;
    n_block_range(p.Sq, Skb, G, p.pack, p.causal, p.window_left, 16, KB, 0, &n_lo, &n_hi);
    const int S_b = splits_for(imax(0, n_hi - n_lo), p.num_splits, p.chunk_blocks);
    int s_lo = 0, s_hi = 0;
    if (split < S_b) split_range(n_lo, n_hi, split, S_b, &s_lo, &s_hi);

    // this lane's query row (column li of every S^T tile)
    const int r = li;
    const bool row_ok = r < nrows;
    const int pos = row_ok ? (p.pack ? r / G : r) : 0;
    const int head = p.pack ? hkv * G + (row_ok ? r % G : 0) : hg;
    int row_lo = 0, row_hi = Skb - 1;
    int wlo = -0x7fffffff, whi = 0x7fffffff;
    if (row_ok) {
        if (p.window_left >= 0) row_lo = pos + delta - p.window_left;
        if (p.causal) row_hi = imin(row_hi, pos + delta);
        wlo = row_lo;
        whi = row_hi;
    }
    // (the 16 lanes of a group hold all of the wave's rows: wave-wide bounds)
    wlo = __builtin_amdgcn_readfirstlane(row16_imax(wlo));
    whi = __builtin_amdgcn_readfirstlane(row16_imin(whi));

    // Q^T fragments: lane (i, g) holds Q[row i][32c + 8g .. +7]
    const bf16_t* qp = reinterpret_cast<const bf16_t*>(p.q);
    const bf16_t* kp = reinterpret_cast<const bf16_t*>(p.k);
    const bf16_t* vp = reinterpret_cast<const bf16_t*>(p.v);
    u32x4 qf[NSLAB];
    {
        const bf16_t* qrow = qp + (((size_t)b * p.Sq + pos) * p.Hq + head) * D + 8 * lg;
        const bool use = row_ok && s_hi > s_lo;
#pragma unroll
        for (int c = 0; c < NSLAB; ++c) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(qrow + 32 * c);  // row 0 when !row_ok
            const u32x4 z = {0u, 0u, 0u, 0u};
            qf[c] = use ? x : z;
        }
    }

    const size_t kv_stride = (size_t)p.Hkv * D;
    const bf16_t* kbase = kp + ((size_t)b * p.Sk * p.Hkv + hkv) * D;
    const bf16_t* vbase = vp + ((size_t)b * p.Sk * p.Hkv + hkv) * D;

    u32x4 kr[NT][NSLAB];  // K fragments of the current block
    // Buffer resources over the block's rows that exist (rows at or past Skb read
    // as zeros): the loads of a block are issued without any branch.
    const uint32_t row_bytes = (uint32_t)(kv_stride * 2);
    auto block_bytes = [&](int n) { return (uint32_t)imin(KB, Skb - n * KB) * row_bytes; };
    auto load_k = [&](int n) {
        const rsrc_t rk = make_rsrc_u(kbase + (size_t)n * KB * kv_stride, block_bytes(n));
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int c = 0; c < NSLAB; ++c)
                kr[t][c] = buf_load16(rk, (16 * t + li) * row_bytes + 2 * (8 * lg + 32 * c));
    };
    // V goes from global memory straight into LDS (buffer_load ... lds): lane l of
    // load i fills bytes [16 l, 16 l + 16) of the i-th kilobyte of the region,
    // i.e. row RPI*i + l / CPR, chunk slot l % CPR, which holds the row's chunk
    // (slot ^ swz(row)).
    auto load_v = [&](int n) {
        const rsrc_t rv = make_rsrc_u(vbase + (size_t)n * KB * kv_stride, block_bytes(n));
        const int r0 = lane / CPR, slot = lane % CPR;
#pragma unroll
        for (int i = 0; i < NVL; ++i) {
            const int rr = RPI * i + r0;
            // (offset computed outside the builtin's argument list: a call there
            // makes this compiler drop the kernel's host launch stub)
            const uint32_t voff = rr * row_bytes + 16 * (slot ^ C::swz(rr));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rv, (__attribute__((address_space(3))) void*)(vl + 1024 * i), 16, voff, 0, 0, 0);
        }
    };

    f32x4 oacc[DT];
#pragma unroll
    for (int u = 0; u < DT; ++u) oacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    const float sl2 = p.scale_log2;

    // s_waitcnt encodings: vmcnt(NVL) (K landed, V's NVL DMAs may be in flight)
    // and vmcnt(0); expcnt and lgkmcnt left at their maximum
    constexpr int WAIT_K = (NVL & 15) | ((NVL >> 4) << 14) | 0x0F70;
    constexpr int NKL = NT * NSLAB;  // K loads per block
    constexpr int WAIT_KN = (NKL & 15) | ((NKL >> 4) << 14) | 0x0F70;
    int n = s_lo + wave;
    if (n < s_hi) {
        load_k(n);  // K first: QK and the softmax can run while V still streams in
        load_v(n);
    }
    for (; n < s_hi; n += NW) {
        const bool more = n + NW < s_hi;
        __builtin_amdgcn_s_waitcnt(WAIT_K);

        // S^T = K . Q^T for the 64 keys of the block
        f32x4 sacc[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < NSLAB; ++c) sacc[t] = mfma_bf16(kr[t][c], qf[c], sacc[t]);
        }
        if (more) load_k(n + NW);

        const int key0 = n * KB;
        if (!(key0 >= wlo && key0 + KB - 1 <= whi)) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int key = key0 + 16 * t + 4 * lg + e;
                    if (key < row_lo || key > row_hi) sacc[t][e] = -INFINITY;
                }
        }

        // online softmax
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) mx = vmax(mx, sacc[t][e]);
        mx = xor_max(mx);
        const float m_new = vmax(m_run, mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = fast_exp2((m_run - m_use) * sl2);
        const float neg = -m_use * sl2;
        float rs = 0.f;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float pv = fast_exp2(fmaf(sacc[t][e], sl2, neg));
                sacc[t][e] = pv;
                rs += pv;
            }
        l_run = l_run * alpha + rs;
        m_run = m_new;
#pragma unroll
        for (int u = 0; u < DT; ++u) oacc[u] *= alpha;

        // O^T += V^T . P^T with P as bf16 hi + lo parts. Outstanding loads, in
        // issue order: V(n), then K(n + NW) when there is a next block.
        if (more) __builtin_amdgcn_s_waitcnt(WAIT_KN);
        else __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
#pragma unroll
        for (int pp = 0; pp < NT / 2; ++pp) {
            const u32x2 s0 = split_bf16x2(sacc[2 * pp][0], sacc[2 * pp][1]);
            const u32x2 s1 = split_bf16x2(sacc[2 * pp][2], sacc[2 * pp][3]);
            const u32x2 s2 = split_bf16x2(sacc[2 * pp + 1][0], sacc[2 * pp + 1][1]);
            const u32x2 s3 = split_bf16x2(sacc[2 * pp + 1][2], sacc[2 * pp + 1][3]);
            const u32x4 ph = {s0[0], s1[0], s2[0], s3[0]};
            const u32x4 pl = {s0[1], s1[1], s2[1], s3[1]};
            // transposed reads of V rows 32pp + 4g + k and 32pp + 16 + 4g + k
            const int ra = 32 * pp + 4 * lg + (li >> 2), rb = ra + 16;
            const int cb = (li & 3) >> 1, hb = 8 * (li & 1);
#pragma unroll
            for (int u = 0; u < DT; ++u) {
                const int ch = 2 * u + cb;
                const u32x2 a = lds_read_tr16(reinterpret_cast<const bf16_t*>(
                    vl + ra * ROWB + 16 * (ch ^ C::swz(ra)) + hb));
                const u32x2 c = lds_read_tr16(reinterpret_cast<const bf16_t*>(
                    vl + rb * ROWB + 16 * (ch ^ C::swz(rb)) + hb));
                const u32x4 vf = {a[0], a[1], c[0], c[1]};
                oacc[u] = mfma_bf16(vf, ph, oacc[u]);
                oacc[u] = mfma_bf16(vf, pl, oacc[u]);
            }
        }
        if (more) {
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this block's LDS reads are done
            load_v(n + NW);
        }
    }
    l_run = xor_sum(l_run);

    // merge the waves' softmax states
    __syncthreads();
    float* red = reinterpret_cast<float*>(smem);
    float* red_o = red;                          // [NW][DT*4][64]
    float* red_ml = red + NW * DT * 4 * 64;      // [NW][2][64]
#pragma unroll
    for (int u = 0; u < DT; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) red_o[(wave * DT * 4 + u * 4 + e) * 64 + lane] = oacc[u][e];
    red_ml[(wave * 2 + 0) * 64 + lane] = m_run;
    red_ml[(wave * 2 + 1) * 64 + lane] = l_run;
    __syncthreads();
    if (wave != 0) return;
    float mw[NW], mstar = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        mw[w] = red_ml[(w * 2 + 0) * 64 + lane];
        mstar = vmax(mstar, mw[w]);
    }
    const float muse = mstar == -INFINITY ? 0.f : mstar;
    float l = 0.f;
#pragma unroll
    for (int u = 0; u < DT; ++u) oacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const float a = fast_exp2((mw[w] - muse) * sl2);
        l += a * red_ml[(w * 2 + 1) * 64 + lane];
#pragma unroll
        for (int u = 0; u < DT; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) oacc[u][e] += a * red_o[(w * DT * 4 + u * 4 + e) * 64 + lane];
    }

    // epilogue: the split partial (O_s normalised, lse_s) or the final O and lse
    if (!row_ok) return;
    const bool any = l > 0.f;
    const float inv = any ? 1.f / l : 0.f;
    const float lse = any ? mstar * p.scale + logf(l) : -INFINITY;
    const size_t row = ((size_t)b * p.Sq + pos) * p.Hq + head;
    if (p.num_splits > 1) {
        const size_t rows_total = (size_t)p.B * p.Sq * p.Hq;
        if (lg == 0) p.lse_part[(size_t)split * rows_total + row] = lse;
        if (any) {
            float* orow = p.o_part + ((size_t)split * rows_total + row) * D + 4 * lg;
#pragma unroll
            for (int u = 0; u < DT; ++u) *reinterpret_cast<f32x4*>(orow + 16 * u) = oacc[u] * inv;
        }
    } else {
        if (lg == 0 && p.lse) p.lse[((size_t)b * p.Hq + head) * p.Sq + pos] = lse;
        bf16_t* orow = reinterpret_cast<bf16_t*>(p.o) + row * D + 4 * lg;
#pragma unroll
        for (int u = 0; u < DT; ++u) {
            u32x2 w;
            w[0] = pack_bf16x2(oacc[u][0] * inv, oacc[u][1] * inv);
            w[1] = pack_bf16x2(oacc[u][2] * inv, oacc[u][3] * inv);
            *reinterpret_cast<u32x2*>(orow + 16 * u) = w;
        }
    }
}

// ---------------------------------------------------------------------------
// Decode with K through LDS. The kernel above loads K straight into MFMA
// operand registers, so each load instruction covers 16 key rows x 64 bytes:
// every 128-byte line is fetched by two instructions, and 64 MiB of the decode
// workload read that way take 12.7 us against 11.95 us when each instruction
// covers 4 whole rows. Here K and V both stream into LDS by buffer_load ... lds
// (4 whole rows per instruction for d = 128) in 32-key halves of each 64-key
// block, single-buffered per wave (16 KB per wave, plus a 4 KB copy of the 16
// query rows: two 4-wave workgroups fill a CU's 160 KB), each half refilled as
// soon as it has been read: K of the next half after the QK product, V after
// the PV product. The copies are untracked (explicit vmcnt waits order them)
// and non-temporal (the cache is read once). K fragments are read back with
// 16-byte LDS reads, chunk slots XOR-swizzled by row so the 16 rows of a read
// hit distinct banks. The online softmax rescales O only when a half's max
// exceeds the reference by more than 2^8 (P <= 256 as bf16 hi + lo parts).
// Fixed-length problems take their key range and split share from the host,
// so nothing is divided before the first copy.
// ---------------------------------------------------------------------------
// Work-unit grid for variable key lengths ([FA-tiling] §4.5, §5.3): sequence b
// owns S_b consecutive units, one per split (S_b its own split count), so no
// workgroup runs for a split a sequence does not have. Unit u of a KV head is
// found by a prefix sum of the S_b, 64 sequences per step across the wave's
// lanes; returns the number of units and sets the unit's sequence, split and
// that sequence's split count (wave-uniform). The host sizes the grid from the
// sum of the key lengths; should that fall short, the workgroups also take
// units u + gridDim.x, ..., so every unit runs.
__device__ __forceinline__ int decode_find_unit(const FwdParams& p, const int u, const int KB, int* b_out,
                                                int* split_out, int* sb_out) {
    const int lane = threadIdx.x & 63;
    int base = 0;
    bool found = false;
    for (int c0 = 0; c0 < p.B; c0 += 64) {
        const int bb = c0 + lane;
        int sb = 0;
        if (bb < p.B) {
            const int len = imax(0, imin(p.seqlens_k[bb], p.Sk));
            int lo, hi;
            n_block_range(p.Sq, len, p.G, p.pack, p.causal, p.window_left, 16, KB, 0, &lo, &hi);
            sb = splits_for(imax(0, hi - lo), p.num_splits, p.chunk_blocks);
        }
        int incl = sb;  // inclusive prefix sum over the lanes
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(incl, o);
            if (lane >= o) incl += y;
        }
        if (!found) {
            // sequences of this step that end at or before unit u
            const int before = __popcll(__builtin_amdgcn_ballot_w64(bb < p.B && base + incl <= u));
            if (before < imin(64, p.B - c0)) {
                const int excl = before > 0 ? __shfl(incl, before - 1) : 0;
                *b_out = __builtin_amdgcn_readfirstlane(c0 + before);
                *split_out = __builtin_amdgcn_readfirstlane(u - base - excl);
                *sb_out = __builtin_amdgcn_readfirstlane(__shfl(sb, before));
                found = true;
            }
        }
        base += __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
    }
    return base;
}

template <int D, int NW>
struct DecodeKdmaTile {
    static constexpr int KB = 64;              // keys per block (the planner's block)
    static constexpr int HB = 32;              // keys per half
    static constexpr int NSLAB = D / 32;       // 32-d slabs of the QK contraction
    static constexpr int DT = D / 16;          // 16-wide d tiles of the output
    static constexpr int CPR = D / 8;          // 16-byte chunks per row
    static constexpr int ROWB = D * 2;         // bytes per K / V row in LDS
    static constexpr int RPI = 1024 / ROWB;    // rows per wave-wide DMA
    static constexpr int NL = HB / RPI;        // DMAs per half (K or V)
    static constexpr int HALFB = HB * ROWB;    // bytes of one half tile
    static constexpr int QB = 16 * ROWB;       // the 16 (packed) query rows
    static constexpr int NQL = QB / 1024;      // DMAs for the query rows
    static constexpr int WAVEB = 2 * HALFB + QB;  // K half + V half + Q rows (80 KB per 4 waves at d = 128)
    static constexpr int RED_BYTES = NW * (DT * 4 * 64 + 2 * 64) * 4;
    static constexpr int LDS_BYTES = NW * WAVEB > RED_BYTES ? NW * WAVEB : RED_BYTES;
    static __device__ __forceinline__ int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
    static __device__ __forceinline__ int swz_v(int r) { return D == 128 ? (r & 7) << 1 : ((r >> 1) & 3) << 1; }
};

template <int D, int NW, bool UNITS>
__global__ void __launch_bounds__(64 * NW, 8 / NW) attn_decode_kdma_kernel(FwdParams p) {
    using C = DecodeKdmaTile<D, NW>;
    constexpr int KB = C::KB, HB = C::HB, NSLAB = C::NSLAB, DT = C::DT;
    constexpr int CPR = C::CPR, RPI = C::RPI, NL = C::NL, ROWB = C::ROWB;
    __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];

    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int li = lane & 15, lg = lane >> 4;
    char* kl = smem + wave * C::WAVEB;  // this wave's K half, swizzled rows
    char* vl = kl + C::HALFB;           // its V half
    char* ql = vl + C::HALFB;           // and its copy of the query rows (K's swizzle)

    // One (batch b, KV head hg, split) of work. In the work-unit grid, last_of is
    // the sequence's split count when this is its last split (that unit also
    // marks the splits the sequence does not use as empty), else 0.
    auto work = [&](const int b, const int hg, const int split, const int last_of) {
    int Skb = p.Sk;
    if (p.seqlens_k) Skb = imax(0, imin(p.seqlens_k[b], p.Sk));
    const int G = p.G;
    const int hkv = hg;  // decode tiles always pack the G heads of a KV head (checked at launch)
    const int nrows = p.pack ? p.Sq * G : p.Sq;
    const int delta = Skb - p.Sq;

    // key blocks of this split ([FA-tiling] §3.2, §5.3); a fixed-length problem
    // takes the range and the blocks per split the host computed with the same
    // functions (16-row tile, 64-key blocks)
    int s_lo = 0, s_hi = 0;
    if (!p.seqlens_k && p.chunk_blocks <= 0) {
        if (split < p.num_splits) {
            s_lo = p.dec_lo + split * p.dec_per;
            s_hi = imin(s_lo + p.dec_per, p.dec_hi);
        }
    } else {
        int n_lo, n_hi;
        n_block_range(p.Sq, Skb, G, p.pack, p.causal, p.window_left, 16, KB, 0, &n_lo, &n_hi);
        const int S_b = splits_for(imax(0, n_hi - n_lo), p.num_splits, p.chunk_blocks);
        if (split < S_b) split_range(n_lo, n_hi, split, S_b, &s_lo, &s_hi);
    }

    const size_t kv_stride = (size_t)p.Hkv * D;
    const uint32_t row_bytes = (uint32_t)(kv_stride * 2);
    const bf16_t* kbase = reinterpret_cast<const bf16_t*>(p.k) + ((size_t)b * p.Sk * p.Hkv + hkv) * D;
    const bf16_t* vbase = reinterpret_cast<const bf16_t*>(p.v) + ((size_t)b * p.Sk * p.Hkv + hkv) * D;
    // half u = 2 n + h of the key range: keys [32 u, 32 u + 32); buffer resources
    // over the rows that exist (rows at or past Skb read as zeros)
    auto half_bytes = [&](int u) { return (uint32_t)imax(0, imin(HB, Skb - u * HB)) * row_bytes; };
    // lane l of DMA i fills bytes [1024 i + 16 l, +16) of the half: row RPI i +
    // l / CPR, slot l % CPR, which holds chunk (slot ^ swz(row))
    // Issued untracked (dma16_untracked): every read of a half is preceded by
    // the explicit vmcnt wait below, and every refill by an lgkmcnt(0) wait, so
    // the V reads of one half do not also wait for the K refill issued after it.
    auto dma_half = [&](const bf16_t* base, int u, char* dst, const bool is_k) {
        const u32x4 rs = rsrc_words_u(base + (size_t)u * HB * kv_stride, half_bytes(u));
        const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds_addr(dst));
        const int r0 = lane / CPR, slot = lane % CPR;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int rr = RPI * i + r0;
            const int sw = is_k ? C::swz_k(rr) : C::swz_v(rr);
            const uint32_t off = rr * row_bytes + 16 * (slot ^ sw);
            dma16_untracked(rs, off, l0 + 1024 * i);
        }
    };

    // A wave with a block sends, in this order, the first K half, its copy of
    // the 16 query rows and the first V half, all into LDS (the waits count on
    // that order: K, Q, V). The query rows take the copy path too, so nothing
    // the compiler tracks is in flight: the first QK product waits for K and
    // Q only, while the V half still streams. Row q of the copy is packed row
    // q of this (batch, KV head); a row the tile does not own reads zeros
    // through an offset past the buffer.
    int n = s_lo + wave;
    if (n < s_hi) {
        dma_half(kbase, 2 * n, kl, true);
        const u32x4 rq = rsrc_words_u(reinterpret_cast<const bf16_t*>(p.q) + (size_t)b * p.Sq * p.Hq * D,
                                      (uint32_t)p.Sq * p.Hq * D * 2);
        const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds_addr(ql));
#pragma unroll
        for (int i = 0; i < C::NQL; ++i) {
            const int qr = RPI * i + lane / CPR, slot = lane % CPR;
            const bool own = qr < nrows;
            const int qpos = own ? (p.pack ? qr / G : qr) : 0;
            const int qhead = p.pack ? hkv * G + (own ? qr % G : 0) : hg;
            const uint32_t off = own ? (uint32_t)(((qpos * p.Hq + qhead) * D) * 2 + 16 * (slot ^ C::swz_k(qr)))
                                     : 0x80000000u;
            dma16_untracked(rq, off, l0 + 1024 * i);
        }
        dma_half(vbase, 2 * n, vl, false);
    }

    // this lane's query row (column li of every S^T tile); visible keys are
    // those with 0 <= key - lo <= span (rows that see none: lo above every key)
    const int r = li;
    const bool row_ok = r < nrows;
    const int pos = row_ok ? (p.pack ? r / G : r) : 0;
    const int head = p.pack ? hkv * G + (row_ok ? r % G : 0) : hg;
    int row_lo = 0, row_hi = Skb - 1;
    int wlo = -0x7fffffff, whi = 0x7fffffff;
    if (row_ok) {
        if (p.window_left >= 0) row_lo = pos + delta - p.window_left;
        if (p.causal) row_hi = imin(row_hi, pos + delta);
        wlo = row_lo;
        whi = row_hi;
    }
    // (the 16 lanes of a group hold all of the wave's rows: wave-wide bounds)
    wlo = __builtin_amdgcn_readfirstlane(row16_imax(wlo));
    whi = __builtin_amdgcn_readfirstlane(row16_imin(whi));
    const int row_span = row_hi < row_lo ? 0 : row_hi - row_lo;
    if (row_hi < row_lo) row_lo = 0x40000000;

    // Q^T fragments: lane (i, g) holds Q[row i][32c + 8g .. +7], read from the
    // wave's copy once K and Q have landed
    u32x4 qf[NSLAB];
    if (n < s_hi) {
        wait_vmcnt<NL>();
#pragma unroll
        for (int c = 0; c < NSLAB; ++c)
            qf[c] = *reinterpret_cast<const u32x4*>(ql + li * ROWB + 16 * ((4 * c + lg) ^ C::swz_k(li)));
    } else {
#pragma unroll
        for (int c = 0; c < NSLAB; ++c) qf[c] = u32x4{0u, 0u, 0u, 0u};
    }

    f32x4 oacc[DT];
#pragma unroll
    for (int u = 0; u < DT; ++u) oacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    const float sl2 = p.scale_log2;
    constexpr float LAZY = 8.f;

    // waits: vmcnt(NL) = the older half-group landed while the newer one (NL
    // copies) may still be in flight; vmcnt(0) = everything landed

    // halves of this wave: u = 2 n + h for its blocks n = s_lo + wave, +NW, ...
    for (; n < s_hi; n += NW) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int u = 2 * n + h;
            // the half after this one (this block's second, or the next block's first)
            const bool more = h == 0 || n + NW < s_hi;
            const int u_next = h == 0 ? u + 1 : 2 * (n + NW);

            // S^T = K . Q^T for the half's 32 keys (K half landed; V half may still stream)
            wait_vmcnt<NL>();
            f32x4 sacc[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < NSLAB; ++c) {
                    const int rr = 16 * t + li;
                    const u32x4 kf = *reinterpret_cast<const u32x4*>(kl + rr * ROWB + 16 * ((4 * c + lg) ^ C::swz_k(rr)));
                    sacc[t] = mfma_bf16(kf, qf[c], sacc[t]);
                }
            }
            if (more) {  // refill the K half once this wave's reads of it are done
                wait_lgkmcnt0();
                dma_half(kbase, u_next, kl, true);
            }

            const int key0 = u * HB;
            if (!(key0 >= wlo && key0 + HB - 1 <= whi)) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int base = key0 + 16 * t + 4 * lg - row_lo;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if ((uint32_t)(base + e) > (uint32_t)row_span) sacc[t][e] = -INFINITY;
                }
            }

            // online softmax, reference max moved lazily
            float mx = -INFINITY;
#pragma unroll
            for (int t = 0; t < 2; ++t)
                mx = vmax(vmax(vmax(vmax(mx, sacc[t][0]), sacc[t][1]), sacc[t][2]), sacc[t][3]);
            mx = xor_max(mx);
            const bool raise = m_run == -INFINITY ? mx != -INFINITY : (mx - m_run) * sl2 > LAZY;
            if (__builtin_amdgcn_ballot_w64(raise) != 0) {
                const float alpha = !raise ? 1.f : (m_run == -INFINITY ? 0.f : fast_exp2((m_run - mx) * sl2));
                if (raise) m_run = mx;
                l_run *= alpha;
#pragma unroll
                for (int w = 0; w < DT; ++w) oacc[w] *= alpha;
            }
            const float neg = m_run == -INFINITY ? 0.f : -m_run * sl2;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float pv = fast_exp2(fmaf(sacc[t][e], sl2, neg));
                    sacc[t][e] = pv;
                    l_run += pv;
                }

            // O^T += V^T . P^T with P as bf16 hi + lo parts (V half landed)
            if (more) wait_vmcnt<NL>();
            else wait_vmcnt<0>();
            const u32x2 s0 = split_bf16x2(sacc[0][0], sacc[0][1]);
            const u32x2 s1 = split_bf16x2(sacc[0][2], sacc[0][3]);
            const u32x2 s2 = split_bf16x2(sacc[1][0], sacc[1][1]);
            const u32x2 s3 = split_bf16x2(sacc[1][2], sacc[1][3]);
            const u32x4 ph = {s0[0], s1[0], s2[0], s3[0]};
            const u32x4 pl = {s0[1], s1[1], s2[1], s3[1]};
            const int ra = 4 * lg + (li >> 2), rb = ra + 16;
            const int cb = (li & 3) >> 1, hb = 8 * (li & 1);
#pragma unroll
            for (int w = 0; w < DT; ++w) {
                const int ch = 2 * w + cb;
                const u32x2 a = lds_read_tr16(reinterpret_cast<const bf16_t*>(vl + ra * ROWB + 16 * (ch ^ C::swz_v(ra)) + hb));
                const u32x2 c = lds_read_tr16(reinterpret_cast<const bf16_t*>(vl + rb * ROWB + 16 * (ch ^ C::swz_v(rb)) + hb));
                const u32x4 vf = {a[0], a[1], c[0], c[1]};
                oacc[w] = mfma_bf16(vf, ph, oacc[w]);
                oacc[w] = mfma_bf16(vf, pl, oacc[w]);
            }
            if (more) {  // refill the V half once this wave's reads of it are done
                wait_lgkmcnt0();
                dma_half(vbase, u_next, vl, false);
            }
        }
    }
    l_run = xor_sum(l_run);

    // merge the waves' softmax states: every wave merges a quarter of the d
    // tiles (DT / NW of them) from all waves and writes that part of the output
    static_assert(DT % NW == 0, "d tiles split evenly over the waves");
    constexpr int DW = DT / NW;
    __syncthreads();
    float* red = reinterpret_cast<float*>(smem);
    float* red_o = red;                          // [NW][DT*4][64]
    float* red_ml = red + NW * DT * 4 * 64;      // [NW][2][64]
#pragma unroll
    for (int w = 0; w < DT; ++w)
#pragma unroll
        for (int e = 0; e < 4; ++e) red_o[(wave * DT * 4 + w * 4 + e) * 64 + lane] = oacc[w][e];
    red_ml[(wave * 2 + 0) * 64 + lane] = m_run;
    red_ml[(wave * 2 + 1) * 64 + lane] = l_run;
    __syncthreads();
    float mw[NW], mstar = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        mw[w] = red_ml[(w * 2 + 0) * 64 + lane];
        mstar = vmax(mstar, mw[w]);
    }
    const float muse = mstar == -INFINITY ? 0.f : mstar;
    float l = 0.f;
    f32x4 om[DW];
#pragma unroll
    for (int x = 0; x < DW; ++x) om[x] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const float a = fast_exp2((mw[w] - muse) * sl2);
        l += a * red_ml[(w * 2 + 1) * 64 + lane];
#pragma unroll
        for (int x = 0; x < DW; ++x)
#pragma unroll
            for (int e = 0; e < 4; ++e) om[x][e] += a * red_o[(w * DT * 4 + (wave * DW + x) * 4 + e) * 64 + lane];
    }

    // epilogue: the split partial (O_s normalised, lse_s) or the final O and lse,
    // d tiles wave * DW .. wave * DW + DW - 1 of it
    if (!row_ok) return;
    const bool any = l > 0.f;
    const float inv = any ? 1.f / l : 0.f;
    const float lse = any ? mstar * p.scale + logf(l) : -INFINITY;
    const size_t row = ((size_t)b * p.Sq + pos) * p.Hq + head;
    if (p.num_splits > 1) {
        const size_t rows_total = (size_t)p.B * p.Sq * p.Hq;
        if (wave == 0 && lg == 0) {
            p.lse_part[(size_t)split * rows_total + row] = lse;
            if constexpr (UNITS)
                for (int s2 = last_of > 0 ? last_of : p.num_splits; s2 < p.num_splits; ++s2)
                    p.lse_part[(size_t)s2 * rows_total + row] = -INFINITY;
        }
        if (any) {
            float* orow = p.o_part + ((size_t)split * rows_total + row) * D + 4 * lg;
#pragma unroll
            for (int x = 0; x < DW; ++x) *reinterpret_cast<f32x4*>(orow + 16 * (wave * DW + x)) = om[x] * inv;
        }
    } else {
        if (wave == 0 && lg == 0 && p.lse) p.lse[((size_t)b * p.Hq + head) * p.Sq + pos] = lse;
        bf16_t* orow = reinterpret_cast<bf16_t*>(p.o) + row * D + 4 * lg;
#pragma unroll
        for (int x = 0; x < DW; ++x) {
            u32x2 wv;
            wv[0] = pack_bf16x2(om[x][0] * inv, om[x][1] * inv);
            wv[1] = pack_bf16x2(om[x][2] * inv, om[x][3] * inv);
            *reinterpret_cast<u32x2*>(orow + 16 * (wave * DW + x)) = wv;
        }
    }
    };

    if constexpr (!UNITS) {
        // (head, split) of this workgroup: blockIdx.y / y_div by the host's
        // multiplier (no branch and no integer division before the first copy)
        const unsigned int gy = blockIdx.y;
        const unsigned int ty = __umulhi(gy, p.y_mul);
        const unsigned int qy = (ty + ((gy - ty) >> p.y_s1)) >> p.y_s2;
        const int ry = (int)(gy - qy * (unsigned int)p.y_div);
        const int hg = p.split_major ? ry : (int)qy;
        const int split = p.split_major ? (int)qy : ry;
        work((int)blockIdx.z, hg, split, 0);
    } else {
        // work-unit grid (decode_find_unit)
        const int hg = blockIdx.y;
        int b = 0, split = 0, sb_u = 0;
        const int total = decode_find_unit(p, (int)blockIdx.x, KB, &b, &split, &sb_u);
        for (int u = (int)blockIdx.x; u < total; u += (int)gridDim.x) {
            if (u != (int)blockIdx.x) {
                __syncthreads();  // the previous unit's LDS reads are done
                decode_find_unit(p, u, KB, &b, &split, &sb_u);
            }
            work(b, hg, split, split == sb_u - 1 ? sb_u : 0);
        }
    }
}

// ---------------------------------------------------------------------------
// Decode with K in registers and V through LDS, in whole 64-key blocks. A wave
// sends the copies of its whole block at once: the query rows and the K block
// straight into MFMA operand registers (16-byte buffer loads; the K block is 64
// registers at d = 128), the V block into the wave's 16 KB of LDS (buffer_load
// ... lds, whole rows). Two 4-wave workgroups on a CU then hold 256 KB of K and
// V in flight, twice what the half-block pipeline above can (its K and V share
// LDS), so a split of 256 keys costs one memory round trip instead of two. A
// wave with more blocks sends the next block's copies once it has read the
// current one. P.V reads V^T with ds_read_b64_tr_b16 (P as bf16 hi + lo parts);
// the softmax, the merge of the waves and the epilogue are those of the kernel
// above.
// ---------------------------------------------------------------------------
template <int D, int NW>
struct DecodeKvTile {
    static constexpr int KB = 64;              // keys per block (the planner's block)
    static constexpr int NT = KB / 16;         // 16-key subtiles of S^T
    static constexpr int NSLAB = D / 32;       // 32-d slabs of the QK contraction
    static constexpr int DT = D / 16;          // 16-wide d tiles of the output
    static constexpr int CPR = D / 8;          // 16-byte chunks per row
    static constexpr int ROWB = D * 2;         // bytes per V row in LDS
    static constexpr int RPI = 1024 / ROWB;    // rows per wave-wide copy
    static constexpr int NL = KB / RPI;        // copies per V block
    static constexpr int WAVEB = KB * ROWB;    // one V block per wave
    static constexpr int RED_BYTES = NW * (DT * 4 * 64 + 2 * 64) * 4;
    static constexpr int LDS_BYTES = NW * WAVEB > RED_BYTES ? NW * WAVEB : RED_BYTES;
    static __device__ __forceinline__ int swz_v(int r) { return D == 128 ? (r & 7) << 1 : ((r >> 1) & 3) << 1; }
};

template <int D, int NW, bool UNITS>
__global__ void __launch_bounds__(64 * NW, 8 / NW) attn_decode_kv_kernel(FwdParams p) {
    using C = DecodeKvTile<D, NW>;
    constexpr int KB = C::KB, NT = C::NT, NSLAB = C::NSLAB, DT = C::DT;
    constexpr int CPR = C::CPR, RPI = C::RPI, NL = C::NL, ROWB = C::ROWB;
    __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];

    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int li = lane & 15, lg = lane >> 4;
    char* vl = smem + wave * C::WAVEB;  // this wave's V block, swizzled rows

    auto work = [&](const int b, const int hg, const int split, const int last_of) {
    int Skb = p.Sk;
    if (p.seqlens_k) Skb = imax(0, imin(p.seqlens_k[b], p.Sk));
    const int G = p.G;
    const int hkv = hg;  // decode tiles always pack the G heads of a KV head (checked at launch)
    const int nrows = p.pack ? p.Sq * G : p.Sq;
    const int delta = Skb - p.Sq;

    // key blocks of this split ([FA-tiling] §3.2, §5.3)
    int s_lo = 0, s_hi = 0;
    if (!p.seqlens_k && p.chunk_blocks <= 0) {
        if (split < p.num_splits) {
            s_lo = p.dec_lo + split * p.dec_per;
            s_hi = imin(s_lo + p.dec_per, p.dec_hi);
        }
    } else {
        int n_lo, n_hi;
        n_block_range(p.Sq, Skb, G, p.pack, p.causal, p.window_left, 16, KB, 0, &n_lo, &n_hi);
        const int S_b = splits_for(imax(0, n_hi - n_lo), p.num_splits, p.chunk_blocks);
        if (split < S_b) split_range(n_lo, n_hi, split, S_b, &s_lo, &s_hi);
    }

    const size_t kv_stride = (size_t)p.Hkv * D;
    const uint32_t row_bytes = (uint32_t)(kv_stride * 2);
    const bf16_t* kbase = reinterpret_cast<const bf16_t*>(p.k) + ((size_t)b * p.Sk * p.Hkv + hkv) * D;
    const bf16_t* vbase = reinterpret_cast<const bf16_t*>(p.v) + ((size_t)b * p.Sk * p.Hkv + hkv) * D;
    // rows at or past Skb lie outside the buffer resources and read as zeros
    auto block_bytes = [&](int n) { return (uint32_t)imax(0, imin(KB, Skb - n * KB)) * row_bytes; };
    // V block n: lane l of copy i fills LDS bytes [1024 i + 16 l, +16) = row
    // RPI i + l / CPR, slot l % CPR, which holds chunk (slot ^ swz_v(row))
    auto copy_v = [&](int n) {
        const u32x4 rs = rsrc_words_u(vbase + (size_t)n * KB * kv_stride, block_bytes(n));
        const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds_addr(vl));
        const int r0 = lane / CPR, slot = lane % CPR;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int rr = RPI * i + r0;
            const uint32_t off = rr * row_bytes + 16 * (slot ^ C::swz_v(rr));
            dma16_untracked(rs, off, l0 + 1024 * i);
        }
    };
    // K block n into registers: kf[t][c] = K[key 16 t + li][32 c + 8 lg .. + 7]
    u32x4 kf[NT][NSLAB];
    auto load_k = [&](int n) {
        const rsrc_t rk = make_rsrc_u(kbase + (size_t)n * KB * kv_stride, block_bytes(n));
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int c = 0; c < NSLAB; ++c) kf[t][c] = buf_load16_nt(rk, (16 * t + li) * row_bytes + 64 * c + 16 * lg);
    };

    // this lane's query row (column li of every S^T tile); visible keys are
    // those with 0 <= key - lo <= span (rows that see none: lo above every key)
    const int r = li;
    const bool row_ok = r < nrows;
    const int pos = row_ok ? (p.pack ? r / G : r) : 0;
    const int head = p.pack ? hkv * G + (row_ok ? r % G : 0) : hg;
    int row_lo = 0, row_hi = Skb - 1;
    int wlo = -0x7fffffff, whi = 0x7fffffff;
    if (row_ok) {
        if (p.window_left >= 0) row_lo = pos + delta - p.window_left;
        if (p.causal) row_hi = imin(row_hi, pos + delta);
        wlo = row_lo;
        whi = row_hi;
    }
    // (the 16 lanes of a group hold all of the wave's rows: wave-wide bounds)
    wlo = __builtin_amdgcn_readfirstlane(row16_imax(wlo));
    whi = __builtin_amdgcn_readfirstlane(row16_imin(whi));
    const int row_span = row_hi < row_lo ? 0 : row_hi - row_lo;
    if (row_hi < row_lo) row_lo = 0x40000000;

    // the first block: query rows (Q^T fragments, lane (i, g) holds Q[row i][32c
    // + 8g .. +7]; rows the tile does not own read zeros), then V, then K
    int n = s_lo + wave;
    u32x4 qf[NSLAB];
    if (n < s_hi) {
        const rsrc_t rq = make_rsrc_u(reinterpret_cast<const bf16_t*>(p.q) + (size_t)b * p.Sq * p.Hq * D,
                                      (uint32_t)p.Sq * p.Hq * D * 2);
        const uint32_t qoff = row_ok ? (uint32_t)((pos * p.Hq + head) * D) * 2 + 16 * lg : 0x80000000u;
#pragma unroll
        for (int c = 0; c < NSLAB; ++c) qf[c] = buf_load16(rq, qoff + 64 * c);
        copy_v(n);
        load_k(n);
    }

    f32x4 oacc[DT];
#pragma unroll
    for (int u = 0; u < DT; ++u) oacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    const float sl2 = p.scale_log2;
    constexpr float LAZY = 8.f;

    // blocks of this wave: n = s_lo + wave, +NW, ...
    for (; n < s_hi; n += NW) {
        // S^T = K . Q^T over the block's 64 keys (the compiler waits for K)
        f32x4 sacc[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            sacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < NSLAB; ++c) sacc[t] = mfma_bf16(kf[t][c], qf[c], sacc[t]);
        }

        const int key0 = n * KB;
        if (!(key0 >= wlo && key0 + KB - 1 <= whi)) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int base = key0 + 16 * t + 4 * lg - row_lo;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if ((uint32_t)(base + e) > (uint32_t)row_span) sacc[t][e] = -INFINITY;
            }
        }

        // online softmax, reference max moved lazily
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < NT; ++t) mx = vmax(vmax(vmax(vmax(mx, sacc[t][0]), sacc[t][1]), sacc[t][2]), sacc[t][3]);
        mx = xor_max(mx);
        const bool raise = m_run == -INFINITY ? mx != -INFINITY : (mx - m_run) * sl2 > LAZY;
        if (__builtin_amdgcn_ballot_w64(raise) != 0) {
            const float alpha = !raise ? 1.f : (m_run == -INFINITY ? 0.f : fast_exp2((m_run - mx) * sl2));
            if (raise) m_run = mx;
            l_run *= alpha;
#pragma unroll
            for (int w = 0; w < DT; ++w) oacc[w] *= alpha;
        }
        const float neg = m_run == -INFINITY ? 0.f : -m_run * sl2;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float pv = fast_exp2(fmaf(sacc[t][e], sl2, neg));
                sacc[t][e] = pv;
                l_run += pv;
            }

        // O^T += V^T . P^T with P as bf16 hi + lo parts; the V block was copied
        // before K, so it has landed (nothing else is in flight here)
        wait_vmcnt<0>();
#pragma unroll
        for (int pp = 0; pp < NT / 2; ++pp) {
            const u32x2 s0 = split_bf16x2(sacc[2 * pp][0], sacc[2 * pp][1]);
            const u32x2 s1 = split_bf16x2(sacc[2 * pp][2], sacc[2 * pp][3]);
            const u32x2 s2 = split_bf16x2(sacc[2 * pp + 1][0], sacc[2 * pp + 1][1]);
            const u32x2 s3 = split_bf16x2(sacc[2 * pp + 1][2], sacc[2 * pp + 1][3]);
            const u32x4 ph = {s0[0], s1[0], s2[0], s3[0]};
            const u32x4 pl = {s0[1], s1[1], s2[1], s3[1]};
            const int ra = 32 * pp + 4 * lg + (li >> 2), rb = ra + 16;
            const int cb = (li & 3) >> 1, hb = 8 * (li & 1);
#pragma unroll
            for (int w = 0; w < DT; ++w) {
                const int ch = 2 * w + cb;
                const u32x2 a = lds_read_tr16(reinterpret_cast<const bf16_t*>(vl + ra * ROWB + 16 * (ch ^ C::swz_v(ra)) + hb));
                const u32x2 c = lds_read_tr16(reinterpret_cast<const bf16_t*>(vl + rb * ROWB + 16 * (ch ^ C::swz_v(rb)) + hb));
                const u32x4 vf = {a[0], a[1], c[0], c[1]};
                oacc[w] = mfma_bf16(vf, ph, oacc[w]);
                oacc[w] = mfma_bf16(vf, pl, oacc[w]);
            }
        }
        if (n + NW < s_hi) {  // the next block, once this one's V reads are done
            wait_lgkmcnt0();
            copy_v(n + NW);
            load_k(n + NW);
        }
    }
    l_run = xor_sum(l_run);

    // merge the waves' softmax states: every wave merges DT / NW of the d tiles
    // from all waves and writes that part of the output
    static_assert(DT % NW == 0, "d tiles split evenly over the waves");
    constexpr int DW = DT / NW;
    __syncthreads();
    float* red = reinterpret_cast<float*>(smem);
    float* red_o = red;                          // [NW][DT*4][64]
    float* red_ml = red + NW * DT * 4 * 64;      // [NW][2][64]
#pragma unroll
    for (int w = 0; w < DT; ++w)
#pragma unroll
        for (int e = 0; e < 4; ++e) red_o[(wave * DT * 4 + w * 4 + e) * 64 + lane] = oacc[w][e];
    red_ml[(wave * 2 + 0) * 64 + lane] = m_run;
    red_ml[(wave * 2 + 1) * 64 + lane] = l_run;
    __syncthreads();
    float mw[NW], mstar = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        mw[w] = red_ml[(w * 2 + 0) * 64 + lane];
        mstar = vmax(mstar, mw[w]);
    }
    const float muse = mstar == -INFINITY ? 0.f : mstar;
    float l = 0.f;
    f32x4 om[DW];
#pragma unroll
    for (int x = 0; x < DW; ++x) om[x] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const float a = fast_exp2((mw[w] - muse) * sl2);
        l += a * red_ml[(w * 2 + 1) * 64 + lane];
#pragma unroll
        for (int x = 0; x < DW; ++x)
#pragma unroll
            for (int e = 0; e < 4; ++e) om[x][e] += a * red_o[(w * DT * 4 + (wave * DW + x) * 4 + e) * 64 + lane];
    }

    if (!row_ok) return;
    const bool any = l > 0.f;
    const float inv = any ? 1.f / l : 0.f;
    const float lse = any ? mstar * p.scale + logf(l) : -INFINITY;
    const size_t row = ((size_t)b * p.Sq + pos) * p.Hq + head;
    if (p.num_splits > 1) {
        const size_t rows_total = (size_t)p.B * p.Sq * p.Hq;
        if (wave == 0 && lg == 0) {
            p.lse_part[(size_t)split * rows_total + row] = lse;
            if constexpr (UNITS)
                for (int s2 = last_of > 0 ? last_of : p.num_splits; s2 < p.num_splits; ++s2)
                    p.lse_part[(size_t)s2 * rows_total + row] = -INFINITY;
        }
        if (any) {
            float* orow = p.o_part + ((size_t)split * rows_total + row) * D + 4 * lg;
#pragma unroll
            for (int x = 0; x < DW; ++x) *reinterpret_cast<f32x4*>(orow + 16 * (wave * DW + x)) = om[x] * inv;
        }
    } else {
        if (wave == 0 && lg == 0 && p.lse) p.lse[((size_t)b * p.Hq + head) * p.Sq + pos] = lse;
        bf16_t* orow = reinterpret_cast<bf16_t*>(p.o) + row * D + 4 * lg;
#pragma unroll
        for (int x = 0; x < DW; ++x) {
            u32x2 wv;
            wv[0] = pack_bf16x2(om[x][0] * inv, om[x][1] * inv);
            wv[1] = pack_bf16x2(om[x][2] * inv, om[x][3] * inv);
            *reinterpret_cast<u32x2*>(orow + 16 * (wave * DW + x)) = wv;
        }
    }
    };

    if constexpr (!UNITS) {
        const unsigned int gy = blockIdx.y;
        const unsigned int ty = __umulhi(gy, p.y_mul);
        const unsigned int qy = (ty + ((gy - ty) >> p.y_s1)) >> p.y_s2;
        const int ry = (int)(gy - qy * (unsigned int)p.y_div);
        work((int)blockIdx.z, p.split_major ? ry : (int)qy, p.split_major ? (int)qy : ry, 0);
    } else {
        int b = 0, split = 0, sb_u = 0;
        const int total = decode_find_unit(p, (int)blockIdx.x, KB, &b, &split, &sb_u);
        for (int u = (int)blockIdx.x; u < total; u += (int)gridDim.x) {
            if (u != (int)blockIdx.x) {
                __syncthreads();
                decode_find_unit(p, u, KB, &b, &split, &sb_u);
            }
            work(b, (int)blockIdx.y, split, split == sb_u - 1 ? sb_u : 0);
        }
    }
}

template <int D, int NW>
hipError_t launch_decode_kv(const FwdParams& p, dim3 grid, hipStream_t stream) {
    if (!p.pack && p.G > 1) return hipErrorInvalidValue;  // the kernel takes grid head = KV head
    if (p.work_units) {
        if (!p.seqlens_k || p.chunk_blocks <= 0 || p.num_splits <= 1) return hipErrorInvalidValue;
        hipLaunchKernelGGL((attn_decode_kv_kernel<D, NW, true>), grid, dim3(64 * NW), 0, stream, p);
    } else {
        hipLaunchKernelGGL((attn_decode_kv_kernel<D, NW, false>), grid, dim3(64 * NW), 0, stream, p);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Log-sum-exp combine of split partials ([FA-tiling] §5.1; [Occupancy] "The
// Fix"): per output row, lse = M + ln sum_s exp(lse_s - M) with M = max_s lse_s,
// O = sum_s exp(lse_s - lse) O_s. A workgroup owns one row and a 32-wide slice
// of d: lane c4 = tid % 8 owns a float4 column, split group sg = tid / 8 owns
// splits sg, sg + 32, .... Every load is issued first; each thread merges its
// splits in registers, then the (max, sum, weighted O) states are merged across
// the 8 split groups of a wave with DPP / lane swaps and across the 4 waves with
// one LDS exchange. Empty splits (lse_s = -inf) carry zero weight and their O_s
// is never used; a row whose splits are all empty gets O = 0, lse = -inf.
// ---------------------------------------------------------------------------
struct LseState {
    float m, l;
    f32x4 acc;
};
// merge of two partial states (both may be empty: m = -inf)
__device__ __forceinline__ LseState lse_merge(const LseState& a, const LseState& b) {
    const float m = vmax(a.m, b.m);
    const float wa = a.m == -INFINITY ? 0.f : __expf(a.m - m);
    const float wb = b.m == -INFINITY ? 0.f : __expf(b.m - m);
    return LseState{m, a.l * wa + b.l * wb, a.acc * wa + b.acc * wb};
}
template <int CTRL>
__device__ __forceinline__ LseState lse_dpp(const LseState& x) {
    LseState y;
    y.m = dpp<CTRL>(x.m);
    y.l = dpp<CTRL>(x.l);
#pragma unroll
    for (int e = 0; e < 4; ++e) y.acc[e] = dpp<CTRL>(x.acc[e]);
    return y;
}
__device__ __forceinline__ float swap16(float x) {  // value of lane l ^ 16
    auto r = __builtin_amdgcn_permlane16_swap(f2u(x), f2u(x), false, false);
    return (__lane_id() & 16) ? u2f(r[0]) : u2f(r[1]);
}
__device__ __forceinline__ float swap32(float x) {  // value of lane l ^ 32
    auto r = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
    return (__lane_id() & 32) ? u2f(r[0]) : u2f(r[1]);
}
__device__ __forceinline__ LseState lse_swap(const LseState& x, bool by32) {
    LseState y;
    y.m = by32 ? swap32(x.m) : swap16(x.m);
    y.l = by32 ? swap32(x.l) : swap16(x.l);
#pragma unroll
    for (int e = 0; e < 4; ++e) y.acc[e] = by32 ? swap32(x.acc[e]) : swap16(x.acc[e]);
    return y;
}

template <bool OUT_BF16, int MAXI>
__global__ void __launch_bounds__(256) lse_combine_kernel(CombineParams p, int D) {
    constexpr int SG = 32;                   // split groups (MAXI splits per thread: S <= SG * MAXI)
    __shared__ float red_m[4][8], red_l[4][8];
    __shared__ f32x4 red_a[4][8];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int row = blockIdx.x;
    const int d0 = 32 * blockIdx.y;
    const int c4 = tid & 7, sg = tid >> 3;
    const int S = p.num_splits;
    const size_t rows = (size_t)p.rows;

    // every load issued before any is used; a split index past S is clamped to
    // S - 1 (the load stays inside the workspace) and its lse forced to -inf
    // (a guarded load became a branch and a wait per split)
    f32x4 ov[MAXI];
    float ls[MAXI];
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
        const int s = sg + SG * i;
        const int sc = s < S ? s : S - 1;
        ls[i] = p.lse_part[(size_t)sc * rows + row];
        ov[i] = *reinterpret_cast<const f32x4*>(p.o_part + ((size_t)sc * rows + row) * D + d0 + 4 * c4);
    }
#pragma unroll
    for (int i = 0; i < MAXI; ++i)
        if (sg + SG * i >= S) ls[i] = -INFINITY;
    // this thread's splits (no branch around the sum, so the O_s loads are not
    // sunk behind the max; an empty split contributes by select, never 0 * O_s)
    LseState st{-INFINITY, 0.f, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int i = 0; i < MAXI; ++i) st.m = vmax(st.m, ls[i]);
    const float mref = st.m == -INFINITY ? 0.f : st.m;
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
        const bool live = ls[i] != -INFINITY;
        const float w = live ? __expf(ls[i] - mref) : 0.f;
        st.l += w;
        const f32x4 t = st.acc + w * ov[i];
        st.acc = live ? t : st.acc;
    }
    // merge the 8 split groups of the wave (lanes c4 + 8k): partner l ^ 8 is
    // row_mirror(half_mirror(.)), then the lane-bit swaps for l ^ 16 and l ^ 32
    st = lse_merge(st, lse_dpp<DPP_MIRROR>(lse_dpp<DPP_HALF_MIRROR>(st)));
    st = lse_merge(st, lse_swap(st, false));
    st = lse_merge(st, lse_swap(st, true));
    if (lane < 8) {
        red_m[wave][lane] = st.m;
        red_l[wave][lane] = st.l;
        red_a[wave][lane] = st.acc;
    }
    __syncthreads();
    if (tid >= 8) return;
    LseState t{red_m[0][tid], red_l[0][tid], red_a[0][tid]};
#pragma unroll
    for (int w = 1; w < 4; ++w) t = lse_merge(t, LseState{red_m[w][tid], red_l[w][tid], red_a[w][tid]});
    const bool any = t.m != -INFINITY && t.l > 0.f;
    const float inv = any ? 1.f / t.l : 0.f;
    const f32x4 o = t.acc * inv;
    if constexpr (OUT_BF16) {
        u32x2 w;
        w[0] = pack_bf16x2(o[0], o[1]);
        w[1] = pack_bf16x2(o[2], o[3]);
        *reinterpret_cast<u32x2*>(reinterpret_cast<bf16_t*>(p.o) + (size_t)row * D + d0 + 4 * tid) = w;
    } else {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.o) + (size_t)row * D + d0 + 4 * tid) = o;
    }
    if (tid == 0 && blockIdx.y == 0 && p.lse) {
        const int h = row % p.Hq;
        const int pos = (row / p.Hq) % p.Sq;
        const int bb = row / (p.Hq * p.Sq);
        p.lse[((size_t)bb * p.Hq + h) * p.Sq + pos] = any ? t.m + logf(t.l) : -INFINITY;
    }
}

// Column-parallel combine, for few splits and many output elements: one thread
// per (row, 4 columns) merges every split of its columns itself -- a pass over
// the row's lse_s for M, then sum_s exp(lse_s - M) (O_s, 1) -- so no partial
// state crosses lanes. Consecutive threads read consecutive 16-byte column
// chunks of a partial row.
template <bool OUT_BF16>
__global__ void __launch_bounds__(256) lse_combine_cols_kernel(CombineParams p, int D) {
    const int cpr = D / 4;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long long)p.rows * cpr) return;
    const int row = (int)(idx / cpr), c4 = (int)(idx % cpr);
    const size_t rows = (size_t)p.rows;
    const int S = p.num_splits;
    float m = -INFINITY;
    for (int s = 0; s < S; ++s) m = vmax(m, p.lse_part[(size_t)s * rows + row]);
    float l = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (m != -INFINITY) {
        int s = 0;
        for (; s + 4 <= S; s += 4) {  // four partials in flight
            float ls[4];
            f32x4 ov[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                ls[j] = p.lse_part[(size_t)(s + j) * rows + row];
                ov[j] = *reinterpret_cast<const f32x4*>(p.o_part + ((size_t)(s + j) * rows + row) * D + 4 * c4);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float w = ls[j] == -INFINITY ? 0.f : __expf(ls[j] - m);
                l += w;
                if (w != 0.f) acc += w * ov[j];
            }
        }
        for (; s < S; ++s) {
            const float ls = p.lse_part[(size_t)s * rows + row];
            if (ls == -INFINITY) continue;
            const float w = __expf(ls - m);
            l += w;
            acc += w * *reinterpret_cast<const f32x4*>(p.o_part + ((size_t)s * rows + row) * D + 4 * c4);
        }
    }
    const bool any = m != -INFINITY && l > 0.f;
    const float inv = any ? 1.f / l : 0.f;
    const f32x4 o = acc * inv;
    if constexpr (OUT_BF16) {
        u32x2 w;
        w[0] = pack_bf16x2(o[0], o[1]);
        w[1] = pack_bf16x2(o[2], o[3]);
        *reinterpret_cast<u32x2*>(reinterpret_cast<bf16_t*>(p.o) + (size_t)row * D + 4 * c4) = w;
    } else {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.o) + (size_t)row * D + 4 * c4) = o;
    }
    if (c4 == 0 && p.lse) {
        const int h = row % p.Hq;
        const int pos = (row / p.Hq) % p.Sq;
        const int bb = row / (p.Hq * p.Sq);
        p.lse[((size_t)bb * p.Hq + h) * p.Sq + pos] = any ? m + logf(l) : -INFINITY;
    }
}

// The same for at most SMAX splits: every lse_s and O_s load of the thread is
// issued before any is used (one memory round trip instead of a max pass and
// then groups of partials); split indices past S are clamped to S - 1 and
// their weight forced to zero, so every load stays inside the workspace.
template <bool OUT_BF16, int SMAX>
__global__ void __launch_bounds__(256) lse_combine_cols_small_kernel(CombineParams p, int D) {
    const int cpr = D / 4;
    const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (long long)p.rows * cpr) return;
    const int row = (int)(idx / cpr), c4 = (int)(idx % cpr);
    const size_t rows = (size_t)p.rows;
    const int S = p.num_splits;
    float ls[SMAX];
    f32x4 ov[SMAX];
#pragma unroll
    for (int j = 0; j < SMAX; ++j) {
        const int s = j < S ? j : S - 1;
        ls[j] = p.lse_part[(size_t)s * rows + row];
        ov[j] = *reinterpret_cast<const f32x4*>(p.o_part + ((size_t)s * rows + row) * D + 4 * c4);
    }
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < SMAX; ++j) {
        if (j >= S) ls[j] = -INFINITY;
        m = vmax(m, ls[j]);
    }
    float l = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    // no branch around the sum (the O_s loads stay ahead of the max); an empty
    // split (lse_s = -inf) may hold no O_s at all: select, never 0 * O_s
    const float mref = m == -INFINITY ? 0.f : m;
#pragma unroll
    for (int j = 0; j < SMAX; ++j) {
        const bool live = ls[j] != -INFINITY;
        const float w = live ? __expf(ls[j] - mref) : 0.f;
        l += w;
        const f32x4 t = acc + w * ov[j];
        acc = live ? t : acc;
    }
    const bool any = m != -INFINITY && l > 0.f;
    const float inv = any ? 1.f / l : 0.f;
    const f32x4 o = acc * inv;
    if constexpr (OUT_BF16) {
        u32x2 w;
        w[0] = pack_bf16x2(o[0], o[1]);
        w[1] = pack_bf16x2(o[2], o[3]);
        *reinterpret_cast<u32x2*>(reinterpret_cast<bf16_t*>(p.o) + (size_t)row * D + 4 * c4) = w;
    } else {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.o) + (size_t)row * D + 4 * c4) = o;
    }
    if (c4 == 0 && p.lse) {
        const int h = row % p.Hq;
        const int pos = (row / p.Hq) % p.Sq;
        const int bb = row / (p.Hq * p.Sq);
        p.lse[((size_t)bb * p.Hq + h) * p.Sq + pos] = any ? m + logf(l) : -INFINITY;
    }
}

// Row-parallel combine for wide rows (the 512-wide values of the latent path):
// one 512-thread workgroup per output row; thread (c4 = tid % C4, sq = tid / C4)
// merges splits sq, sq + SQ, ... of its 4 columns online, eight partials in
// flight, and the SQ partial states of each column quad are merged through LDS.
// A row is read once by one workgroup, with every load of a thread issued in
// batches instead of one dependent round per split.
template <bool OUT_BF16, int D>
__global__ void __launch_bounds__(512) lse_combine_rows_kernel(CombineParams p) {
    constexpr int C4 = D / 4, SQ = 512 / C4;
    static_assert(512 % C4 == 0, "column quads must divide the workgroup");
    __shared__ float red_m[SQ][C4], red_l[SQ][C4];
    __shared__ f32x4 red_a[SQ][C4];
    const int row = blockIdx.x, tid = threadIdx.x;
    const int c4 = tid % C4, sq = tid / C4;
    const size_t rows = (size_t)p.rows;
    const int S = p.num_splits;
    LseState st{-INFINITY, 0.f, f32x4{0.f, 0.f, 0.f, 0.f}};
    for (int s0 = sq; s0 < S; s0 += 8 * SQ) {
        float ls[8];
        f32x4 ov[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {  // all eight loads first (indices past S clamped, then masked)
            const int s = s0 + j * SQ;
            const int sc = s < S ? s : S - 1;
            ls[j] = p.lse_part[(size_t)sc * rows + row];
            ov[j] = *reinterpret_cast<const f32x4*>(p.o_part + ((size_t)sc * rows + row) * D + 4 * c4);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (s0 + j * SQ < S && ls[j] != -INFINITY) st = lse_merge(st, LseState{ls[j], 1.f, ov[j]});
    }
    red_m[sq][c4] = st.m;
    red_l[sq][c4] = st.l;
    red_a[sq][c4] = st.acc;
    __syncthreads();
    if (sq != 0) return;
#pragma unroll
    for (int g = 1; g < SQ; ++g) st = lse_merge(st, LseState{red_m[g][c4], red_l[g][c4], red_a[g][c4]});
    const bool any = st.m != -INFINITY && st.l > 0.f;
    const f32x4 o = st.acc * (any ? 1.f / st.l : 0.f);
    if constexpr (OUT_BF16) {
        u32x2 w;
        w[0] = pack_bf16x2(o[0], o[1]);
        w[1] = pack_bf16x2(o[2], o[3]);
        *reinterpret_cast<u32x2*>(reinterpret_cast<bf16_t*>(p.o) + (size_t)row * D + 4 * c4) = w;
    } else {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.o) + (size_t)row * D + 4 * c4) = o;
    }
    if (c4 == 0 && p.lse) {
        const int h = row % p.Hq;
        const int pos = (row / p.Hq) % p.Sq;
        const int bb = row / (p.Hq * p.Sq);
        p.lse[((size_t)bb * p.Hq + h) * p.Sq + pos] = any ? st.m + logf(st.l) : -INFINITY;
    }
}

template <int D, int NW>
hipError_t launch_decode(const FwdParams& p, dim3 grid, hipStream_t stream) {
    hipLaunchKernelGGL((attn_decode_kernel<D, NW>), grid, dim3(64 * NW), 0, stream, p);
    return hipGetLastError();
}

template <int D, int NW>
hipError_t launch_decode_kdma(const FwdParams& p, dim3 grid, hipStream_t stream) {
    if (!p.pack && p.G > 1) return hipErrorInvalidValue;  // the kernel takes grid head = KV head
    if (p.work_units) {  // grid (units, KV heads, 1) over variable key lengths
        if (!p.seqlens_k || p.chunk_blocks <= 0 || p.num_splits <= 1) return hipErrorInvalidValue;
        hipLaunchKernelGGL((attn_decode_kdma_kernel<D, NW, true>), grid, dim3(64 * NW), 0, stream, p);
    } else {
        hipLaunchKernelGGL((attn_decode_kdma_kernel<D, NW, false>), grid, dim3(64 * NW), 0, stream, p);
    }
    return hipGetLastError();
}

const FwdVariant* decode_variants() {
    static const FwdVariant v[] = {
        // K in registers, V through LDS, whole 64-key blocks (attn_decode_kv_kernel)
        {DT_BF16, 128, 16, 64, 1, 4, DecodeKvTile<128, 4>::LDS_BYTES, &launch_decode_kv<128, 4>, 0, 0, 0, 2},
        {DT_BF16, 64, 16, 64, 1, 4, DecodeKvTile<64, 4>::LDS_BYTES, &launch_decode_kv<64, 4>, 0, 0, 0, 2},
        // K through LDS in 32-key halves (see attn_decode_kdma_kernel)
        {DT_BF16, 128, 16, 64, 1, 4, DecodeKdmaTile<128, 4>::LDS_BYTES, &launch_decode_kdma<128, 4>, 0, 0, 0, 1},
        {DT_BF16, 64, 16, 64, 1, 4, DecodeKdmaTile<64, 4>::LDS_BYTES, &launch_decode_kdma<64, 4>, 0, 0, 0, 1},
        {DT_BF16, 128, 16, 64, 1, 4, DecodeTile<128, 4>::LDS_BYTES, &launch_decode<128, 4>, 0},
        {DT_BF16, 64, 16, 64, 1, 4, DecodeTile<64, 4>::LDS_BYTES, &launch_decode<64, 4>, 0},
        // 8 waves (512 keys per workgroup at one block per wave), one workgroup per CU
        // (K through LDS: 8 x 20 KB, the whole 160 KB; d = 128 only, where the
        // merge splits the 8 d tiles one per wave)
        {DT_BF16, 128, 16, 64, 1, 8, DecodeKdmaTile<128, 8>::LDS_BYTES, &launch_decode_kdma<128, 8>, 0, 0, 0, 1},
        {DT_BF16, 128, 16, 64, 1, 8, DecodeTile<128, 8>::LDS_BYTES, &launch_decode<128, 8>, 0},
        {DT_BF16, 64, 16, 64, 1, 8, DecodeTile<64, 8>::LDS_BYTES, &launch_decode<64, 8>, 0},
        {0, 0, 0, 0, 0, 0, 0, nullptr, 0},
    };
    return v;
}

// Kernel choice: the split-group kernel parallelises over splits (decode: many
// splits, few rows); the column kernel over output elements.
bool combine_by_columns(int rows, int d, int num_splits) {
    const int force = options().combine_cols;
    if (force >= 0) return force != 0;
    (void)rows;
    (void)d;
    // measured: columns win at <= 16 splits (latent verify, 4 splits x 544 rows:
    // 6.4 vs 32.8 us); split groups at 52..128 splits (varlen decode 16.2 vs 42.2)
    return num_splits <= 16;
}

hipError_t launch_combine(const CombineParams& p, int d, int out_bf16, hipStream_t stream) {
    // 512-wide rows (latent values): one workgroup per row (measured on the latent
    // verify shape, 16 splits x 544 rows: the column kernel took 11.1 us; on the
    // 65,536-key prefix, 51 splits x 272 rows: 24 us with either other kernel)
    if (d == 512 && options().combine_rows != 0) {
        if (out_bf16) hipLaunchKernelGGL((lse_combine_rows_kernel<true, 512>), dim3(p.rows), dim3(512), 0, stream, p);
        else hipLaunchKernelGGL((lse_combine_rows_kernel<false, 512>), dim3(p.rows), dim3(512), 0, stream, p);
        return hipGetLastError();
    }
    if (combine_by_columns(p.rows, d, p.num_splits)) {
        const long long n = (long long)p.rows * (d / 4);
        dim3 grid((unsigned)((n + 255) / 256)), block(256);
        // every partial of a thread in flight at once for up to 8 / 16 splits
        // (ATTN_COMBINE_SMALL=0: the looped form for any count)
        const int small = options().combine_small;
        if (small && p.num_splits <= 8) {
            if (out_bf16) hipLaunchKernelGGL((lse_combine_cols_small_kernel<true, 8>), grid, block, 0, stream, p, d);
            else hipLaunchKernelGGL((lse_combine_cols_small_kernel<false, 8>), grid, block, 0, stream, p, d);
        } else if (small && p.num_splits <= 16) {
            if (out_bf16) hipLaunchKernelGGL((lse_combine_cols_small_kernel<true, 16>), grid, block, 0, stream, p, d);
            else hipLaunchKernelGGL((lse_combine_cols_small_kernel<false, 16>), grid, block, 0, stream, p, d);
        } else {
            if (out_bf16) hipLaunchKernelGGL((lse_combine_cols_kernel<true>), grid, block, 0, stream, p, d);
            else hipLaunchKernelGGL((lse_combine_cols_kernel<false>), grid, block, 0, stream, p, d);
        }
        return hipGetLastError();
    }
    dim3 grid(p.rows, d / 32), block(256);
    // splits per thread: the smallest of 1, 2, 4, 8 that covers S over 32 split groups
    const int per = (p.num_splits + 31) / 32;
    auto go = [&](auto maxi) {
        constexpr int M = decltype(maxi)::value;
        if (out_bf16) hipLaunchKernelGGL((lse_combine_kernel<true, M>), grid, block, 0, stream, p, d);
        else hipLaunchKernelGGL((lse_combine_kernel<false, M>), grid, block, 0, stream, p, d);
    };
    static_assert(TPA_MAX_SPLITS <= 32 * 8, "split groups x splits per thread");
    if (per <= 1) go(std::integral_constant<int, 1>{});
    else if (per <= 2) go(std::integral_constant<int, 2>{});
    else if (per <= 4) go(std::integral_constant<int, 4>{});
    else go(std::integral_constant<int, 8>{});
    return hipGetLastError();
}

}  // namespace tpa
