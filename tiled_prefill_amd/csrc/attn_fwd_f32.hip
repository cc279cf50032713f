// attn_fwd_f32.hip -- gfx950 (MI355X) forward kernel for fp32 inputs with few
// query rows per KV head (speculative verify, decode).
//
// Citations:
//   [FA-tiling]  "分块策略与调度" (FlashAttention tiling strategy and scheduling):
//                §3 block ranges, §5 split-KV, §6 PackGQA
//   [Occupancy]  "The Occupancy Awakening: Rewriting a Flash Attention Kernel
//                for Blackwell's 188 SMs" (the verify workload: 17 query rows
//                per head over a 2065-key prefix)
//
// One workgroup of NW waves (4 or 8) owns up to 32 (packed) query rows of one
// (batch, grid head, split). Its key range is cut into 16-key blocks and the
// waves take them in turn (wave w: blocks w, w + NW, ...), each wave with its
// own online-softmax state for all 32 rows and its own LDS stage: K and V of a
// block stream straight into LDS by buffer_load ... lds (two or four whole rows
// per instruction, no registers), and the stage is refilled in two parts -- K
// with the wave's next block once the QK product has read it, V once P.V has --
// so the next block's copy overlaps the current block's softmax and P.V, and no
// workgroup barrier stands in the loop. The states are merged through LDS at
// the end. Four waves take 80 KB of LDS at d = 128, so two workgroups fit a CU.
//
// Products on the fp32 16x16x4 MFMA, transposed so that the query rows sit on
// the N axis:
//   S^T[key][row] = K . Q^T   A: lane (i, g) reads K[key i][its d], 16-byte LDS
//                             reads serving four MFMAs; B: Q^T in registers
//                             (lane group g owns d in [g D/4, (g+1) D/4))
//   O^T[d][row] += V^T . P^T  A: lane (i, g) reads V[key 4g + r][16u + i] (one
//                             float per MFMA, from the row-major V tile);
//                             B: the S^T accumulators after the softmax
// LDS rows are XOR-swizzled by 16-byte chunk so that both reads are free of bank
// conflicts: chunk c of key row r sits in slot c ^ (r & 15) (K: 16 rows at one
// chunk), slot c ^ (4 ((r >> 2) & 3)) (V: 4 rows at 16 consecutive floats).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_device.h"
#include "attn_kernels.h"
#include "attn_plan.h"

namespace tpa {

template <int D, int NW_ = 4>
struct F32DmaTile {
    static constexpr int NW = NW_, NTHR = 64 * NW;
    static constexpr int BM = 32, NQ = 2;      // query rows per workgroup, 16-row column blocks
    static constexpr int KB = 16;              // keys per block (one wave's unit of work)
    static constexpr int ROWB = 4 * D;         // bytes per K / V row
    static constexpr int CPR = D / 4;          // 16-byte chunks per row
    static constexpr int RPI = 1024 / ROWB;    // rows per wave-wide copy
    static constexpr int NL = KB / RPI;        // copies per block (K or V)
    static constexpr int BLKB = KB * ROWB;     // bytes of one K (or V) block
    static constexpr int STAGEB = 2 * BLKB;    // K + V
    static constexpr int WAVEB = STAGEB;
    static constexpr int QB = BM * ROWB;       // the workgroup's query rows
    static constexpr int NQL = QB / 1024 / NW; // query-row copies per wave
    static constexpr int DL = D / 4, QV = DL / 4;  // d per lane group, 16-byte vectors of it
    static constexpr int DT = D / 16;          // 16-wide d tiles of O^T
    static constexpr int RED_BYTES = NW * (DT * NQ * 4 + 2 * NQ) * 64 * 4;
    static constexpr int MAIN_BYTES = NW * WAVEB + QB;
    static constexpr int LDS_BYTES = MAIN_BYTES > RED_BYTES ? MAIN_BYTES : RED_BYTES;
    static_assert(CPR >= 16 && KB % RPI == 0 && QB % (1024 * NW) == 0, "tile shape");
    static_assert(DT % NW == 0, "d tiles split evenly over the waves in the merge");
    static __host__ __device__ __forceinline__ int swz_k(int r) { return r & 15; }
    static __host__ __device__ __forceinline__ int swz_v(int r) { return ((r >> 2) & 3) << 2; }
};

template <int D, int NW_>
__global__ void __launch_bounds__(64 * NW_, NW_ == 4 ? 2 : 1) attn_fwd_f32_dma_kernel(FwdParams p) {
    using C = F32DmaTile<D, NW_>;
    constexpr int BM = C::BM, NQ = C::NQ, KB = C::KB, ROWB = C::ROWB, CPR = C::CPR, RPI = C::RPI;
    constexpr int NL = C::NL, QV = C::QV, DT = C::DT, NW = C::NW;
    __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];

    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int li = lane & 15, lg = lane >> 4;
    char* wbuf = smem + wave * C::WAVEB;     // this wave's stage (K then V)
    char* qs = smem + NW * C::WAVEB;         // the workgroup's query rows (K's swizzle)

    // ---- tile: (query block, grid head x split, batch); heaviest query block first
    const int m_block = p.lpt ? p.num_m_blocks - 1 - (int)blockIdx.x : (int)blockIdx.x;
    const int hg = (int)blockIdx.y / p.num_splits;
    const int split = (int)blockIdx.y % p.num_splits;
    const int b = blockIdx.z;
    int Skb = p.Sk;
    if (p.seqlens_k) Skb = imax(0, imin(p.seqlens_k[b], p.Sk));
    const int G = p.G;
    const int hkv = p.pack ? hg : hg / G;
    const int nrows = p.pack ? p.Sq * G : p.Sq;
    const int delta = Skb - p.Sq;

    // key blocks of this tile and split ([FA-tiling] §3.2, §5.3), in 16-key units
    int n_lo, n_hi;
    n_block_range(p.Sq, Skb, G, p.pack, p.causal, p.window_left, BM, KB, m_block, &n_lo, &n_hi);
    const int S_b = splits_for(imax(0, n_hi - n_lo), p.num_splits, p.chunk_blocks);
    int s_lo = 0, s_hi = 0;
    if (split < S_b) split_range(n_lo, n_hi, split, S_b, &s_lo, &s_hi);

    // ---- copies into LDS (untracked; ordered by explicit waits below)
    const size_t kv_stride = (size_t)p.Hkv * D;
    const uint32_t row_bytes = (uint32_t)(kv_stride * 4);
    const float* kbase = reinterpret_cast<const float*>(p.k) + ((size_t)b * p.Sk * p.Hkv + hkv) * D;
    const float* vbase = reinterpret_cast<const float*>(p.v) + ((size_t)b * p.Sk * p.Hkv + hkv) * D;
    // copy i of a block fills LDS bytes [1024 i + 16 l, +16) for lane l: key row
    // RPI i + l / CPR, slot l % CPR, which holds chunk slot ^ swz(row); rows at
    // or past Skb lie outside the buffer resource and read as zeros
    auto copy_part = [&](int n, const bool is_v) {
        const uint32_t valid = (uint32_t)imax(0, imin(KB, Skb - n * KB));
        const u32x4 rs = rsrc_words_u((is_v ? vbase : kbase) + (size_t)n * KB * kv_stride, valid * row_bytes);
        const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds_addr(wbuf + (is_v ? C::BLKB : 0)));
        const int r0 = lane / CPR, slot = lane % CPR;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
            const int rr = RPI * i + r0;
            const int sw = is_v ? C::swz_v(rr) : C::swz_k(rr);
            dma16_untracked(rs, rr * row_bytes + 16 * (slot ^ sw), l0 + 1024 * i);
        }
    };
    auto copy_block = [&](int n) {
        copy_part(n, false);
        copy_part(n, true);
    };

    // this wave's blocks: n = s_lo + wave + NW j
    int n = s_lo + wave;
    const bool first = n < s_hi;
    if (first) copy_block(n);
    // the query rows: wave w copies rows [BM w / NW, BM (w + 1) / NW); row r of the
    // tile is packed row m_block BM + r; rows the tile does not own read zeros
    {
        const u32x4 rq = rsrc_words_u(reinterpret_cast<const float*>(p.q) + (size_t)b * p.Sq * p.Hq * D,
                                      (uint32_t)p.Sq * p.Hq * D * 4);
        const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds_addr(qs));
#pragma unroll
        for (int i = 0; i < C::NQL; ++i) {
            const int ci = wave * C::NQL + i;             // copy index within the query tile
            const int qr = RPI * ci + lane / CPR, slot = lane % CPR;
            const int r = m_block * BM + qr;
            const bool own = r < nrows;
            const int qpos = own ? (p.pack ? r / G : r) : 0;
            const int qhead = p.pack ? hkv * G + (own ? r % G : 0) : hg;
            const uint32_t off = own ? (uint32_t)((qpos * p.Hq + qhead) * D) * 4 + 16 * (slot ^ C::swz_k(qr))
                                     : 0x80000000u;
            dma16_untracked(rq, off, l0 + 1024 * ci);
        }
    }

    // ---- this lane's query rows and their visible key intervals
    int row_pos[NQ], row_head[NQ], row_lo[NQ], row_span[NQ];
    bool row_ok[NQ];
    int wlo = -0x7fffffff, whi = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int r = m_block * BM + 16 * q + li;
        const bool ok = r < nrows;
        const int pos = ok ? (p.pack ? r / G : r) : 0;
        int lo = 0, hi = Skb - 1;
        if (ok) {
            if (p.window_left >= 0) lo = pos + delta - p.window_left;
            if (p.causal) hi = imin(hi, pos + delta);
            wlo = imax(wlo, lo);
            whi = imin(whi, hi);
        }
        row_pos[q] = pos;
        row_head[q] = p.pack ? hkv * G + (ok ? r % G : 0) : hg;
        row_ok[q] = ok;
        // visible iff 0 <= key - lo <= span (rows that see no key: lo above every key)
        row_span[q] = hi < lo ? 0 : hi - lo;
        row_lo[q] = hi < lo ? 0x40000000 : lo;
    }
    // (the 16 lanes of a group hold all of the wave's rows: wave-wide bounds)
    wlo = __builtin_amdgcn_readfirstlane(row16_imax(wlo));
    whi = __builtin_amdgcn_readfirstlane(row16_imin(whi));

    // the query rows have landed (and block n, copied before them) in every wave
    wait_vmcnt<0>();
    __syncthreads();
    // Q^T fragments: lane (i, g) holds Q[row 16 q + i][g D/4 + 4 c .. + 3]
    f32x4 qf[NQ][QV];
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
        for (int c = 0; c < QV; ++c) {
            const int rr = 16 * q + li, ch = lg * QV + c;
            qf[q][c] = *reinterpret_cast<const f32x4*>(qs + rr * ROWB + 16 * (ch ^ C::swz_k(rr)));
        }

    f32x4 oacc[DT][NQ];
    float m_run[NQ], l_run[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        m_run[q] = -INFINITY;
        l_run[q] = 0.f;
#pragma unroll
        for (int u = 0; u < DT; ++u) oacc[u][q] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const float sl2 = p.scale_log2;
    constexpr float LAZY = 8.f;  // the reference max moves only when a score exceeds it by 2^8

    for (; n < s_hi; n += NW) {
        const bool next = n + NW < s_hi;  // the wave has a further block
        wait_vmcnt<NL>();                 // this block's K (its V may still stream)
        const char* kt = wbuf;
        const char* vt = kt + C::BLKB;

        // S^T = K . Q^T over this block's 16 keys
        f32x4 sacc[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) sacc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < QV; ++c) {
            const int ch = lg * QV + c;
            const f32x4 kv = *reinterpret_cast<const f32x4*>(kt + li * ROWB + 16 * (ch ^ C::swz_k(li)));
#pragma unroll
            for (int q = 0; q < NQ; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e) sacc[q] = mfma_f32(kv[e], qf[q][c][e], sacc[q]);
        }
        if (next) {  // refill K with the wave's next block once read
            wait_lgkmcnt0();
            copy_part(n + NW, false);
        }

        // mask the keys a row cannot see (only blocks that cut a row's interval)
        const int key0 = n * KB;
        if (!(key0 >= wlo && key0 + KB - 1 <= whi)) {
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const int base = key0 + 4 * lg - row_lo[q];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if ((uint32_t)(base + e) > (uint32_t)row_span[q]) sacc[q][e] = -INFINITY;
            }
        }

        // online softmax in fp32 with a lazily moved reference max
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            float mx = vmax(vmax(sacc[q][0], sacc[q][1]), vmax(sacc[q][2], sacc[q][3]));
            mx = xor_max(mx);
            const bool raise = m_run[q] == -INFINITY ? mx != -INFINITY : (mx - m_run[q]) * sl2 > LAZY;
            if (__builtin_amdgcn_ballot_w64(raise) != 0) {
                const float alpha = !raise ? 1.f : (m_run[q] == -INFINITY ? 0.f : fast_exp2((m_run[q] - mx) * sl2));
                if (raise) m_run[q] = mx;
                l_run[q] *= alpha;
#pragma unroll
                for (int u = 0; u < DT; ++u) oacc[u][q] *= alpha;
            }
            const float neg = m_run[q] == -INFINITY ? 0.f : -m_run[q] * sl2;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float pv = fast_exp2(fmaf(sacc[q][e], sl2, neg));
                sacc[q][e] = pv;
                l_run[q] += pv;
            }
        }

        // O^T += V^T . P^T: MFMA e contracts keys 4 g + e over the lane groups g
        if (next) wait_vmcnt<NL>();  // this block's V (behind it only the next K, if any)
        else wait_vmcnt<0>();
#pragma unroll
        for (int u = 0; u < DT; ++u) {
            float vf[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int kr = 4 * lg + e, col = 16 * u + li;
                vf[e] = *reinterpret_cast<const float*>(vt + kr * ROWB + 16 * ((col >> 2) ^ C::swz_v(kr)) +
                                                        4 * (col & 3));
            }
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int q = 0; q < NQ; ++q) oacc[u][q] = mfma_f32(vf[e], sacc[q][e], oacc[u][q]);
        }

        if (next) {  // refill V with the next block once read
            wait_lgkmcnt0();
            copy_part(n + NW, true);
        }
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) l_run[q] = xor_sum(l_run[q]);

    // ---- merge the waves' states; wave w merges and writes the d tiles
    // [w DT / NW, (w + 1) DT / NW) of every row
    constexpr int DW = DT / NW, OV = DT * 4;
    __syncthreads();
    float* red_o = reinterpret_cast<float*>(smem);     // [NW][NQ][OV][64]
    float* red_ml = red_o + NW * NQ * OV * 64;          // [NW][NQ][2][64]
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
#pragma unroll
        for (int u = 0; u < DT; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) red_o[((wave * NQ + q) * OV + 4 * u + e) * 64 + lane] = oacc[u][q][e];
        red_ml[((wave * NQ + q) * 2 + 0) * 64 + lane] = m_run[q];
        red_ml[((wave * NQ + q) * 2 + 1) * 64 + lane] = l_run[q];
    }
    __syncthreads();
    const bool split_out = p.num_splits > 1;
    const size_t rows_total = (size_t)p.B * p.Sq * p.Hq;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        float mw[NW], mstar = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            mw[w] = red_ml[((w * NQ + q) * 2 + 0) * 64 + lane];
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
            l += a * red_ml[((w * NQ + q) * 2 + 1) * 64 + lane];
#pragma unroll
            for (int x = 0; x < DW; ++x)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    om[x][e] += a * red_o[((w * NQ + q) * OV + 4 * (wave * DW + x) + e) * 64 + lane];
        }
        if (!row_ok[q]) continue;
        const bool any = l > 0.f;
        const float inv = any ? 1.f / l : 0.f;
        const float lse = any ? mstar * p.scale + logf(l) : -INFINITY;
        const size_t row = ((size_t)b * p.Sq + row_pos[q]) * p.Hq + row_head[q];
        if (split_out) {
            if (wave == 0 && lg == 0) p.lse_part[(size_t)split * rows_total + row] = lse;
            if (any) {
                float* orow = p.o_part + ((size_t)split * rows_total + row) * D + 4 * lg;
#pragma unroll
                for (int x = 0; x < DW; ++x) *reinterpret_cast<f32x4*>(orow + 16 * (wave * DW + x)) = om[x] * inv;
            }
        } else {
            if (wave == 0 && lg == 0 && p.lse) p.lse[((size_t)b * p.Hq + row_head[q]) * p.Sq + row_pos[q]] = lse;
            float* orow = reinterpret_cast<float*>(p.o) + row * D + 4 * lg;
#pragma unroll
            for (int x = 0; x < DW; ++x) *reinterpret_cast<f32x4*>(orow + 16 * (wave * DW + x)) = om[x] * inv;
        }
    }
}

template <int D, int NW>
hipError_t launch_fwd_f32_dma(const FwdParams& p, dim3 grid, hipStream_t stream) {
    hipLaunchKernelGGL((attn_fwd_f32_dma_kernel<D, NW>), grid, dim3(64 * NW), 0, stream, p);
    return hipGetLastError();
}

const FwdVariant* f32_dma_variants() {
    static const FwdVariant v[] = {
        // 32 query rows, 16-key blocks taken by the waves in turn, one LDS stage per
        // wave: 4 waves (two workgroups per CU fit), or 8 (one per CU, d = 128)
        {DT_FP32, 128, 32, 16, 1, 4, F32DmaTile<128, 4>::LDS_BYTES, &launch_fwd_f32_dma<128, 4>, 0},
        {DT_FP32, 64, 32, 16, 1, 4, F32DmaTile<64, 4>::LDS_BYTES, &launch_fwd_f32_dma<64, 4>, 0},
        {DT_FP32, 128, 32, 16, 1, 8, F32DmaTile<128, 8>::LDS_BYTES, &launch_fwd_f32_dma<128, 8>, 0},
        {0, 0, 0, 0, 0, 0, 0, nullptr, 0},
    };
    return v;
}

}  // namespace tpa
