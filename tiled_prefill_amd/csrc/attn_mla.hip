// attn_mla.hip -- gfx950 forward kernel for values of their own width (bf16):
// the latent-attention verify shape of [Occupancy] -- one KV head shared by
// every query head, 576-wide keys (512 latent + 64 rotary) and 512-wide values.
//
// Citations:
//   [Occupancy]  "The Occupancy Awakening: Rewriting a Flash Attention Kernel
//                for Blackwell's 188 SMs" (the MLA verify workload, Dl 512, Dr 64)
//   [FA-tiling]  "分块策略与调度" (FlashAttention tiling strategy and scheduling):
//                §2 tile sizes (small blocks for a large V head dim), §3 block
//                ranges, §5 split-KV, §6 PackGQA
//
// All G = Hq / Hkv query heads of a KV head are packed into the row dimension
// ([FA-tiling] §6.3: packed row r is query position r / G, head hkv G + r % G),
// so every K/V tile is read once for all of them. One workgroup: 64 packed rows
// in 4 blocks of 16, 32-key tiles, double-buffered in LDS (K 36 KB by DMA, V 32
// KB through registers; 136 KB, one workgroup per CU). Two forms: 4 waves, one
// per row block, each holding the 576-wide Q^T fragments (72 registers) and all
// 512 output columns (128 accumulators), one wave per SIMD; or 8 waves, the two
// waves of a row block each computing the block's scores and half of its output
// columns (64 accumulators, no AGPRs), two waves per SIMD to hide each other's
// LDS and memory latency -- the QK product runs twice, and the kernel still wins
// (the latency, not the matrix core, bounds it). S^T = K Q^T on 16x16x32 bf16 MFMA, online softmax with a lazy
// reference max, O^T += V^T P^T on 16x16x32 bf16 MFMA with V as stored and P
// as two bf16 parts (P ~= hi + lo to about 16 bits: one bf16 rounding of P
// would cost up to 2^-9 per term, and fp16 operands would not hold V beyond
// 65504), row sums of hi + lo on the matrix core. The kernel is bound by its
// per-tile latency, not the matrix core, so the second P.V product is cheap
// here. Split-KV partials ([FA-tiling] §5) go to the combine kernel with rows
// of DV values.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_device.h"
#include "attn_kernels.h"
#include "attn_plan.h"

namespace tpa {

template <int DK, int DV, int SV = 1>
struct MlaTile {
    // SV = 1: 4 waves, each owning 16 packed rows and all DV output columns;
    // SV = 2: 8 waves, wave w owning rows 16 (w % 4) .. +15 and half w / 4 of the
    // output columns (the QK product is computed by both waves of a row block)
    static constexpr int SV_ = SV, RWV = 4, NWV = RWV * SV, MW = 16, BM = RWV * MW, BN = 32, NTHR = 64 * NWV;
    static constexpr int NSLAB = DK / 32;  // QK contraction slabs
    static constexpr int NT = BN / 16;     // 16-key sub-tiles
    static constexpr int DT = DV / 16;     // 16-wide output d tiles
    static constexpr int KCPR = DK / 8;    // 16-byte chunks per K row
    static constexpr int VCPR = DV / 8;    // 16-byte chunks per V row
    static constexpr int KROWB = 2 * DK, VROWB = 2 * DV;
    static constexpr int KTILEB = BN * KROWB, VTILEB = BN * VROWB, STAGEB = KTILEB + VTILEB;
    static constexpr int LDS_BYTES = 2 * STAGEB;
    static constexpr int KDMA = KTILEB / 1024;        // wave-wide K DMAs per tile
    static constexpr int KDMA_PER_WAVE = (KDMA + NWV - 1) / NWV;
    static constexpr int VCH = BN * VCPR / NTHR;      // V chunks per thread per tile
    static constexpr int DTW = DT / SV;               // output d tiles per wave
    static_assert(DK % 32 == 0 && DV % (16 * SV) == 0 && KTILEB % 1024 == 0, "tile shape");
    static_assert(BN * VCPR % NTHR == 0, "V tile must split evenly over the threads");
    // LDS chunk swizzles. K rows are 72 chunks: the XOR touches only the low 3
    // bits of the chunk index (the row stays whole); with rows an odd multiple of
    // 128 bytes, rows r and r + 1 sit in opposite halves of the 64 banks, so the
    // 16 rows of a quarter-wave read hit 16 distinct 16-byte bank groups. V rows
    // are 1024 bytes: the 4 rows x 2 chunks of a transposed read are spread by
    // XORing chunk pairs with the row.
    static __device__ __forceinline__ int kslot(int c, int r) { return (c & ~7) | ((c & 7) ^ ((r >> 1) & 7)); }
    static __device__ __forceinline__ int vslot(int c, int r) { return c ^ ((r & 7) << 1); }
};

template <int DK, int DV, int SV>
__global__ void __launch_bounds__(256 * SV, 1) attn_mla_kernel(FwdParams p) {
    using C = MlaTile<DK, DV, SV>;
    constexpr int BN = C::BN, BM = C::BM, NT = C::NT, NSLAB = C::NSLAB, DTW = C::DTW;
    constexpr int KROWB = C::KROWB, VROWB = C::VROWB, KTILEB = C::KTILEB, STAGEB = C::STAGEB;
    __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rw = wave % C::RWV, vh = wave / C::RWV;  // row block, output-column part
    const int li = lane & 15, lg = lane >> 4;

    // ---- tile coordinates: XCD-aware one-dimensional grid, heaviest query block first
    const int M = p.num_m_blocks, S = p.num_splits;
    const int total = p.B * p.grid_heads * S * M;
    const int per_xcd = (total + NUM_XCD - 1) / NUM_XCD;
    const int t = ((int)blockIdx.x % NUM_XCD) * per_xcd + (int)blockIdx.x / NUM_XCD;
    if (t >= total) return;
    int rest = t / M;
    const int m_rev = t % M;
    const int m_block = p.lpt ? M - 1 - m_rev : m_rev;
    const int split = rest % S;
    rest /= S;
    const int hg = rest % p.grid_heads;
    const int b = rest / p.grid_heads;

    int Skb = p.Sk;
    if (p.seqlens_k) Skb = imax(0, imin(p.seqlens_k[b], p.Sk));
    const int G = p.G;
    const int hkv = p.pack ? hg : hg / G;
    const int nrows = p.pack ? p.Sq * G : p.Sq;
    const int delta = Skb - p.Sq;

    int n_lo, n_hi;
    n_block_range(p.Sq, Skb, G, p.pack, p.causal, p.window_left, BM, BN, m_block, &n_lo, &n_hi);
    const int S_b = splits_for(imax(0, n_hi - n_lo), S, p.chunk_blocks);
    int s_lo = 0, s_hi = 0;
    if (split < S_b) split_range(n_lo, n_hi, split, S_b, &s_lo, &s_hi);
    const bool has_work = s_hi > s_lo;

    // ---- this lane's query row (query column li of the wave's 16) and its keys
    const int r = m_block * BM + rw * 16 + li;
    const bool row_ok = r < nrows;
    const int row_pos = row_ok ? (p.pack ? r / G : r) : 0;
    const int row_head = p.pack ? hkv * G + (row_ok ? r % G : 0) : hg;
    int row_lo = 0, row_hi = Skb - 1;
    int wlo = -0x7fffffff, whi = 0x7fffffff;
    if (row_ok) {
        if (p.window_left >= 0) row_lo = row_pos + delta - p.window_left;
        if (p.causal) row_hi = imin(row_hi, row_pos + delta);
        wlo = row_lo;
        whi = row_hi;
    }
    // (the 16 lanes of a group hold all of the wave's rows: wave-wide bounds)
    wlo = __builtin_amdgcn_readfirstlane(row16_imax(wlo));
    whi = __builtin_amdgcn_readfirstlane(row16_imin(whi));

    // ---- Q^T fragments: lane (i, g) holds Q[row i][32 s + 8 g .. +7]
    u32x4 qf[NSLAB];
    {
        const bf16_t* qrow = reinterpret_cast<const bf16_t*>(p.q) + (((size_t)b * p.Sq + row_pos) * p.Hq + row_head) * DK + 8 * lg;
        const bool use = row_ok && has_work;
#pragma unroll
        for (int s2 = 0; s2 < NSLAB; ++s2) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(qrow + 32 * s2);
            const u32x4 z = {0u, 0u, 0u, 0u};
            qf[s2] = use ? x : z;
        }
    }

    f32x4 oacc[DTW], lacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < DTW; ++u) oacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY;
    const u32x4 ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};  // bf16 1.0
    const float sl2 = p.scale_log2;
    constexpr float LAZY = 8.f;  // lazy reference max: O is rescaled only when the max moves by > 2^8

    // ---- K/V tiles
    const size_t k_stride = (size_t)p.Hkv * DK, v_stride = (size_t)p.Hkv * DV;
    const uint32_t k_row_bytes = (uint32_t)(k_stride * 2), v_row_bytes = (uint32_t)(v_stride * 2);
    const bf16_t* kbase = reinterpret_cast<const bf16_t*>(p.k) + ((size_t)b * p.Sk * p.Hkv + hkv) * DK;
    const bf16_t* vbase = reinterpret_cast<const bf16_t*>(p.v) + ((size_t)b * p.Sk * p.Hkv + hkv) * DV;
    auto tile_rows = [&](int n) { return (uint32_t)imin(BN, Skb - n * BN); };
    // K DMA i fills LDS bytes [1024 i, 1024 i + 1024): flat chunk f = 64 i + lane is
    // row f / KCPR, slot f % KCPR, which holds the row's chunk kslot(slot, row)
    // (issued untracked: the compiler's tracking cannot tell the stages apart and
    // waited for the next tile's copy before the current tile's P.V reads; the
    // vmcnt(0) wait before the tile's barrier orders the copy before its reads)
    auto load_k = [&](int n, int stage) {
        const u32x4 rk = rsrc_words_u(kbase + (size_t)n * BN * k_stride, tile_rows(n) * k_row_bytes);
        const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds_addr(smem + stage * STAGEB));
#pragma unroll
        for (int j = 0; j < C::KDMA_PER_WAVE; ++j) {
            const int i = wave + C::NWV * j;
            if (C::KDMA % C::NWV != 0 && i >= C::KDMA) break;
            const int f = 64 * i + lane;
            const int rr = f / C::KCPR, slot = f % C::KCPR;
            const uint32_t voff = rr * k_row_bytes + 16 * C::kslot(slot, rr);
            dma16_untracked_cached(rk, voff, l0 + 1024 * i);
        }
    };
    u32x4 vst[C::VCH];
    auto load_v = [&](int n) {
        const rsrc_t rv = make_rsrc(vbase + (size_t)n * BN * v_stride, tile_rows(n) * v_row_bytes);
#pragma unroll
        for (int j = 0; j < C::VCH; ++j) {
            const int id = tid + C::NTHR * j;
            vst[j] = buf_load16(rv, (id / C::VCPR) * v_row_bytes + 16 * (id % C::VCPR));
        }
    };
    auto store_v = [&](int stage) {
        char* dst = smem + stage * STAGEB + KTILEB;
#pragma unroll
        for (int j = 0; j < C::VCH; ++j) {
            const int id = tid + C::NTHR * j;
            const int rr = id / C::VCPR, ch = id % C::VCPR;
            *reinterpret_cast<u32x4*>(dst + rr * VROWB + 16 * C::vslot(ch, rr)) = vst[j];
        }
    };

    if (has_work) {
        load_k(s_hi - 1, 0);
        load_v(s_hi - 1);
        store_v(0);
        wait_vmcnt<0>();  // the K copies have landed
    }
    __syncthreads();

    int stage = 0;
    for (int n = s_hi - 1; n >= s_lo; --n) {
        const bool more = n > s_lo;
        if (more) {  // prefetch the next (lower) tile into the other stage
            load_k(n - 1, stage ^ 1);
            load_v(n - 1);
        }
        const char* kt = smem + stage * STAGEB;
        const char* vt = kt + KTILEB;

        // S^T = K . Q^T. The fragment of slab s2 is logical chunk 4 s2 + g of row
        // 16 tt + i; its slot is 8 (s2 / 2) + ((4 (s2 % 2) + g) ^ ((i / 2) % 8)), so
        // every address is one of two per-lane bases plus a constant offset.
        f32x4 sacc[NT];
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) sacc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
        const char* kb0 = kt + li * KROWB + 16 * C::kslot(lg, li);
        const char* kb1 = kt + li * KROWB + 16 * C::kslot(4 + lg, li);
#pragma unroll
        for (int s2 = 0; s2 < NSLAB; ++s2)
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                const u32x4 kf = *reinterpret_cast<const u32x4*>((s2 & 1 ? kb1 : kb0) + 128 * (s2 >> 1) + 16 * KROWB * tt);
                sacc[tt] = mfma_bf16(kf, qf[s2], sacc[tt]);
            }

        // mask (only tiles that cut a row's visible interval); element (tt, e) is
        // key n BN + 16 tt + 4 g + e
        const int key0 = n * BN;
        if (!(key0 >= wlo && key0 + BN - 1 <= whi)) {
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int key = key0 + 16 * tt + 4 * lg + e;
                    if (key < row_lo || key > row_hi) sacc[tt][e] = -INFINITY;
                }
        }
        // online softmax, lazy reference max
        float mx = -INFINITY;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
            mx = vmax(vmax(vmax(vmax(mx, sacc[tt][0]), sacc[tt][1]), sacc[tt][2]), sacc[tt][3]);
        mx = xor_max(mx);
        const bool raise = m_run == -INFINITY ? mx != -INFINITY : (mx - m_run) * sl2 > LAZY;
        if (raise) {
            const float alpha = m_run == -INFINITY ? 0.f : fast_exp2((m_run - mx) * sl2);
            m_run = mx;
            lacc *= alpha;
#pragma unroll
            for (int u = 0; u < DTW; ++u) oacc[u] *= alpha;
        }
        const float neg = m_run == -INFINITY ? 0.f : -m_run * sl2;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int e = 0; e < 4; ++e) sacc[tt][e] = fast_exp2(fmaf(sacc[tt][e], sl2, neg));

        // O^T += V^T . P^T (bf16, P as hi + lo): one 32-key step; lane group g
        // supplies keys 4 g .. 4 g + 3 and 16 + 4 g .. 16 + 4 g + 3
        u32x4 ph, plo;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const u32x2 hl = split_bf16x2(sacc[w >> 1][2 * (w & 1)], sacc[w >> 1][2 * (w & 1) + 1]);
            ph[w] = hl[0];
            plo[w] = hl[1];
        }
        lacc = mfma_bf16(ones, ph, lacc);
        lacc = mfma_bf16(ones, plo, lacc);
        const int ra = 4 * lg + (li >> 2), rb = ra + 16;
        const int cb = (li & 3) >> 1, hb = 8 * (li & 1);
#pragma unroll
        for (int u = 0; u < DTW; ++u) {
            const int ch = 2 * (vh * DTW + u) + cb;
            const u32x2 a = lds_read_tr16(reinterpret_cast<const bf16_t*>(vt + ra * VROWB + 16 * C::vslot(ch, ra) + hb));
            const u32x2 c = lds_read_tr16(reinterpret_cast<const bf16_t*>(vt + rb * VROWB + 16 * C::vslot(ch, rb) + hb));
            const u32x4 vf = {a[0], a[1], c[0], c[1]};
            oacc[u] = mfma_bf16(vf, ph, oacc[u]);
            oacc[u] = mfma_bf16(vf, plo, oacc[u]);
        }

        if (more) {
            store_v(stage ^ 1);
            wait_vmcnt<0>();  // this wave's K copies landed
        }
        __syncthreads();
        stage ^= 1;
    }

    // ---- epilogue: lane (i, g) holds O^T[16 u + 4 g + 0..3][row i]
    if (!row_ok) return;
    const float l = lacc[0];
    const bool any = l > 0.f;
    const float inv = any ? 1.f / l : 0.f;
    const float lse = any ? m_run * p.scale + logf(l) : -INFINITY;
    const size_t row = ((size_t)b * p.Sq + row_pos) * p.Hq + row_head;
    const int c0 = 16 * DTW * vh;  // this wave's first output column
    if (S > 1) {
        const size_t rows_total = (size_t)p.B * p.Sq * p.Hq;
        if (lg == 0 && vh == 0) p.lse_part[(size_t)split * rows_total + row] = lse;
        if (any) {
            float* orow = p.o_part + ((size_t)split * rows_total + row) * DV + c0 + 4 * lg;
#pragma unroll
            for (int u = 0; u < DTW; ++u) *reinterpret_cast<f32x4*>(orow + 16 * u) = oacc[u] * inv;
        }
    } else {
        if (lg == 0 && vh == 0 && p.lse) p.lse[((size_t)b * p.Hq + row_head) * p.Sq + row_pos] = lse;
        bf16_t* orow = reinterpret_cast<bf16_t*>(p.o) + row * DV + c0 + 4 * lg;
#pragma unroll
        for (int u = 0; u < DTW; ++u) {
            u32x2 w;
            w[0] = pack_bf16x2(oacc[u][0] * inv, oacc[u][1] * inv);
            w[1] = pack_bf16x2(oacc[u][2] * inv, oacc[u][3] * inv);
            *reinterpret_cast<u32x2*>(orow + 16 * u) = w;
        }
    }
}

template <int DK, int DV, int SV>
hipError_t launch_mla(const FwdParams& p, dim3 grid, hipStream_t stream) {
    hipLaunchKernelGGL((attn_mla_kernel<DK, DV, SV>), grid, dim3(256 * SV), 0, stream, p);
    return hipGetLastError();
}

const FwdVariant* mla_variants() {
    static const FwdVariant v[] = {
        // d = 576, d_v = 512 (latent attention); block_n 32, 4 waves x 16 packed rows
        {DT_BF16, 576, 64, 32, 4, 1, MlaTile<576, 512>::LDS_BYTES, &launch_mla<576, 512, 1>, 1, 0, 512},
        // the same rows over 8 waves, each pair of waves splitting the 512 output columns
        {DT_BF16, 576, 64, 32, 4, 2, MlaTile<576, 512, 2>::LDS_BYTES, &launch_mla<576, 512, 2>, 1, 0, 512},
        {0, 0, 0, 0, 0, 0, 0, nullptr, 0},
    };
    return v;
}

}  // namespace tpa
