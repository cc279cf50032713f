// attn_prefill.hip -- gfx950 flash-attention forward for many query rows (bf16).
//
// Citations:
//   [FA-tiling]  "分块策略与调度" (FlashAttention tiling strategy and scheduling)
//
// One workgroup of NWV waves owns BM = NWV * MW query rows of one (batch, query
// head[, split]) and walks its key-block range ([FA-tiling] §3) from the first
// block to the last, so the query blocks of a head, which run together on one
// XCD, move over its K/V tiles in step and share them in L2. Per 64-key tile:
//   * K (bf16) streams from global memory straight into LDS (buffer_load ...
//     lds), V is loaded into registers, converted to fp16 and written to LDS;
//     both double-buffered, so tile n+1 loads while tile n computes, with one
//     workgroup barrier per tile;
//   * S^T = K Q^T on 16x16x32 bf16 MFMA (Q^T stays in registers);
//   * online softmax in fp32 (row max over the 4 lanes of a query column with
//     v_permlane16/32_swap) with a lazily moved reference max: O is rescaled
//     only when a score exceeds the reference by more than 2^8, which after the
//     first tile of a row almost never happens; the row sums of P come from an
//     extra MFMA with an all-ones operand instead of VALU adds. Once every row
//     of a wave has a reference, tiles skip the row max: P is formed against
//     the reference and its row sums, which bound every element, detect an fp16
//     overflow, after which the tile runs again with the exact max;
//   * O^T += V^T P^T on 16x16x32 fp16 MFMA: P is rounded to fp16 (11 significant
//     bits: one bf16 rounding of P would cost up to 2^-9 per term) and V^T comes
//     from ds_read_b64_tr_b16 of the row-major fp16 tile.
// LDS rows are XOR-swizzled by 16-byte chunk so both the K fragment reads (16
// rows, one chunk) and the V transpose reads (8 rows, two chunks) are
// bank-conflict free.
//
// Grid: one dimension over all tiles. Workgroups are dealt round-robin to the 8
// XCDs, so tile t is placed on XCD (t / per_xcd): the query blocks of one head
// share one XCD's L2 (HBM fetch 1.9x the algorithmic bytes on the causal
// 8192-position prefill; 4.6x when the keys were walked downward). Within a
// head the query blocks run heaviest first ([FA-tiling] §4.4).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_device.h"
#include "attn_kernels.h"
#include "attn_plan.h"

namespace tpa {


template <int D, int NWV, int MW>
struct PrefillTile {
    static constexpr int BN = 64;              // keys per tile
    static constexpr int BM = NWV * MW;        // query rows per workgroup
    static constexpr int NTHR = 64 * NWV;
    static constexpr int NQ = MW / 16;         // 16-row column blocks per wave
    static constexpr int NT = BN / 16;         // 16-key sub-tiles
    static constexpr int NSLAB = D / 32;       // QK contraction slabs
    static constexpr int DT = D / 16;          // output d tiles
    static constexpr int CPR = D / 8;          // 16-byte chunks per row
    static constexpr int ROWB = 2 * D;         // bytes per K / V row in LDS
    static constexpr int TILEB = BN * ROWB;    // bytes of one K (or V) tile
    static constexpr int STAGEB = 2 * TILEB;   // K + V
    static constexpr int LDS_BYTES = 2 * STAGEB;
    static constexpr int QBYTES = BM * ROWB;   // the workgroup's Q rows (attn_prefill_kernel)
    static constexpr int KROWS_PER_DMA = 1024 / ROWB;              // rows per wave-wide DMA
    static constexpr int KDMA = BN / KROWS_PER_DMA;                // DMA instructions per tile
    static constexpr int KDMA_PER_WAVE = (KDMA + NWV - 1) / NWV;
    static constexpr int VCH = BN * CPR / NTHR;                    // V chunks per thread
    static_assert(BN * CPR % NTHR == 0, "V tile must split evenly over the threads");
    static_assert(MW % 16 == 0, "rows per wave");
    // chunk swizzles (see header comment)
    static __host__ __device__ __forceinline__ int swz_k(int r) {
        return D == 128 ? (r & 15) : ((r >> 1) & 7);
    }
    static __host__ __device__ __forceinline__ int swz_v(int r) {
        return D == 128 ? (r & 7) << 1 : ((r >> 1) & 3) << 1;
    }
};

template <int D, int NWV, int MW, int PRI, int PERSIST = 0>
__global__ void __launch_bounds__(64 * NWV, MW > 32 ? 1 : 8 / NWV) attn_prefill_kernel(FwdParams p) {
    constexpr bool PRIO = PRI != 0;
    using C = PrefillTile<D, NWV, MW>;
    constexpr int BN = C::BN, BM = C::BM, NT = C::NT, NSLAB = C::NSLAB, DT = C::DT;
    constexpr int CPR = C::CPR, ROWB = C::ROWB, TILEB = C::TILEB, STAGEB = C::STAGEB;
    __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;

    // ---- tiles: t in [0, total) ordered (batch, head, split, query block heaviest
    // first); XCD x owns the section [x per_xcd, (x + 1) per_xcd)
    const int M = p.num_m_blocks, S = p.num_splits;
    const int total = p.B * p.grid_heads * S * M;
    const int per_xcd = (total + NUM_XCD - 1) / NUM_XCD;
    // run_tile(t, vbf16, nq, q0) computes tile t for the 16-row column blocks q0
    // .. q0 + nq - 1 of every wave's MW rows. The fast form (vbf16 false, all
    // C::NQ blocks at once) converts V to fp16; when its O accumulators come out
    // non-finite -- a V element beyond fp16's range (|v| > 65504) became +-inf
    // -- it writes nothing and returns true, and the tile runs again in the
    // bf16 form (vbf16 true): V kept in bf16 and P split into bf16 hi + lo parts,
    // exact for any finite bf16 V, one column block at a time so that it needs
    // fewer registers than the fast form and the kernel none beyond them.
    __shared__ int s_bad;
    auto run_tile = [&](const int t, auto vbf16, auto nqc, const int q0) -> bool {
    constexpr bool VB = decltype(vbf16)::value;
    constexpr int NQ = decltype(nqc)::value;
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

    // ---- this lane's query rows and their visible key intervals
    int row_pos[NQ], row_head[NQ], row_lo[NQ], row_hi[NQ];
    bool row_ok[NQ];
    int wlo = -0x7fffffff, whi = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int r = m_block * BM + wave * MW + 16 * (q0 + q) + li;
        const bool ok = r < nrows;
        const int pos = ok ? (p.pack ? r / G : r) : 0;
        const int head = p.pack ? hkv * G + (ok ? r % G : 0) : hg;
        int lo = 0, hi = Skb - 1;
        if (ok) {
            if (p.window_left >= 0) lo = pos + delta - p.window_left;
            if (p.causal) hi = imin(hi, pos + delta);
            wlo = imax(wlo, lo);
            whi = imin(whi, hi);
        }
        row_pos[q] = pos;
        row_head[q] = head;
        row_lo[q] = lo;
        row_hi[q] = hi;
        row_ok[q] = ok;
    }
    // The 16 lanes of a lane group hold all of the wave's rows, so these
    // reductions give wave-wide values: [wlo, whi], the keys every row sees
    // (a tile inside it needs no mask), and [ulo, uhi], the keys some row
    // sees (a tile outside it is skipped by the whole wave).
    int ulo = 0x7fffffff, uhi = -1;
#pragma unroll
    for (int q = 0; q < NQ; ++q)
        if (row_ok[q] && row_hi[q] >= row_lo[q]) {
            ulo = imin(ulo, row_lo[q]);
            uhi = imax(uhi, row_hi[q]);
        }
    wlo = __builtin_amdgcn_readfirstlane(row16_imax(wlo));
    whi = __builtin_amdgcn_readfirstlane(row16_imin(whi));
    ulo = __builtin_amdgcn_readfirstlane(row16_imin(ulo));
    uhi = __builtin_amdgcn_readfirstlane(row16_imax(uhi));
    int row_span[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const bool none = row_hi[q] < row_lo[q];
        row_span[q] = none ? 0 : row_hi[q] - row_lo[q];
        if (none) row_lo[q] = 0x40000000;
    }

    // ---- Q^T fragments: lane (i, g) holds Q[row i][32c + 8g .. +7]
    const bf16_t* qp = reinterpret_cast<const bf16_t*>(p.q);
    u32x4 qreg[NQ][NSLAB];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const bf16_t* qrow = qp + (((size_t)b * p.Sq + row_pos[q]) * p.Hq + row_head[q]) * D + 8 * lg;
        const bool use = row_ok[q] && has_work;
#pragma unroll
        for (int c = 0; c < NSLAB; ++c) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(qrow + 32 * c);
            const u32x4 z = {0u, 0u, 0u, 0u};
            qreg[q][c] = use ? x : z;
        }
    }
    auto q_frag = [&](const int q, const int c) { return qreg[q][c]; };

    // O^T accumulators, and the row sums of P computed on the matrix core: an
    // all-ones A operand turns a PV-shaped MFMA into sum_j P[j][i] for every lane
    // of query column i, which also keeps l consistent with the fp16-rounded P.
    f32x4 oacc[DT][NQ];
    // m_run: the reference max of each row; negm = -m_run * scale * log2(e), the
    // exponent offset of P, kept beside it (0 while the row has no reference) so
    // a steady tile does not recompute it
    float m_run[NQ], l_run[NQ], negm[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        m_run[q] = -INFINITY;
        negm[q] = 0.f;
        l_run[q] = 0.f;
#pragma unroll
        for (int u = 0; u < DT; ++u) oacc[u][q] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const u32x4 ones = {0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u};  // fp16 1.0
    const float sl2 = p.scale_log2;
    // Lazy max: when the exact row max is taken, the reference max of a row moves
    // only if a new score exceeds it by more than 2^LAZY (log2 units), so the O
    // rescale (and its exponential) is skipped on most tiles.
    constexpr float LAZY = 8.f;
    // Once every row of the wave has a finite reference max ("steady"), a tile
    // skips the row max altogether: P = exp2(S - m_ref) is formed directly and
    // its fp16 row sums (the matrix-core sums above, which l needs anyway) bound
    // every element, since P >= 0. A sum at most P_MAX means no element overflowed
    // fp16; otherwise (a score that jumped far above the reference, or an inf)
    // the tile is recomputed from the K tile still in LDS with the exact max.
    constexpr float P_MAX = 65504.f;

    // ---- K/V tile loads
    const size_t kv_stride = (size_t)p.Hkv * D;
    const uint32_t row_bytes = (uint32_t)(kv_stride * 2);
    const bf16_t* kbase = reinterpret_cast<const bf16_t*>(p.k) + ((size_t)b * p.Sk * p.Hkv + hkv) * D;
    const bf16_t* vbase = reinterpret_cast<const bf16_t*>(p.v) + ((size_t)b * p.Sk * p.Hkv + hkv) * D;
    auto tile_bytes = [&](int n) { return (uint32_t)imin(BN, Skb - n * BN) * row_bytes; };
    // K: wave-wide DMAs into the stage's K tile; lane l of DMA i fills 16 bytes
    // at 1024 i + 16 l, i.e. row KROWS_PER_DMA*i + l / CPR, slot l % CPR, which
    // holds the row's chunk (slot ^ swz_k(row)).
    // The copies are issued untracked (dma16_untracked_cached): the compiler's own
    // tracking cannot tell the two stages apart and put a wait for the next
    // tile's copy in front of the first K read of the current tile, exposing the
    // copy's whole latency on every tile (the same kernel with no K copies at all
    // ran 10% faster). The one vmcnt(0) wait before the tile's barrier orders
    // the copy before its reads.
    auto load_k = [&](int n, int stage) {
        const u32x4 rk = rsrc_words_u(kbase + (size_t)n * BN * kv_stride, tile_bytes(n));
        const uint32_t l0 = __builtin_amdgcn_readfirstlane(lds_addr(smem + stage * STAGEB));
#pragma unroll
        for (int j = 0; j < C::KDMA_PER_WAVE; ++j) {
            const int i = wave * C::KDMA_PER_WAVE + j;
            if (C::KDMA % NWV == 0 || i < C::KDMA) {
                const int rr = C::KROWS_PER_DMA * i + lane / CPR;
                const int slot = lane % CPR;
                const uint32_t voff = rr * row_bytes + 16 * (slot ^ C::swz_k(rr));
                dma16_untracked_cached(rk, voff, l0 + 1024 * i);
            }
        }
    };
    // V: each thread loads C::VCH chunks (row id / CPR, chunk id % CPR) into registers
    u32x4 vst[C::VCH];
    auto load_v = [&](int n) {
        const rsrc_t rv = make_rsrc(vbase + (size_t)n * BN * kv_stride, tile_bytes(n));
#pragma unroll
        for (int j = 0; j < C::VCH; ++j) {
            const int id = tid + C::NTHR * j;
            vst[j] = buf_load16(rv, (id / CPR) * row_bytes + 16 * (id % CPR));
        }
    };
    auto store_v = [&](int stage) {
        char* dst = smem + stage * STAGEB + TILEB;
#pragma unroll
        for (int j = 0; j < C::VCH; ++j) {
            const int id = tid + C::NTHR * j;
            const int rr = id / CPR, ch = id % CPR;
            u32x4 h = vst[j];
            if constexpr (!VB) {
#pragma unroll
                for (int e = 0; e < 4; ++e) h[e] = bf16x2_to_f16x2(vst[j][e]);
            }
            *reinterpret_cast<u32x4*>(dst + rr * ROWB + 16 * (ch ^ C::swz_v(rr))) = h;
        }
    };

    if (has_work) {
        load_k(s_lo, 0);
        load_v(s_lo);
        store_v(0);
        wait_vmcnt<0>();  // the K copies have landed
    }
    if (!VB && tid == 0) s_bad = 0;
    __syncthreads();

    f32x4 sacc[NT][NQ];
    // S^T = K . Q^T for the tile at kt (raised wave priority while feeding the
    // matrix core, so the partner wave on the SIMD runs its VALU work in the
    // gaps), then -inf on the elements a row cannot see
    auto scores = [&](const char* kt, const int key0) {
        if (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int q = 0; q < NQ; ++q) sacc[tt][q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NSLAB; ++c) {
            u32x4 qf[NQ];
#pragma unroll
            for (int q = 0; q < NQ; ++q) qf[q] = q_frag(q, c);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                const int rr = 16 * tt + li;
                const u32x4 kf = *reinterpret_cast<const u32x4*>(kt + rr * ROWB + 16 * ((4 * c + lg) ^ C::swz_k(rr)));
#pragma unroll
                for (int q = 0; q < NQ; ++q) sacc[tt][q] = mfma_bf16(kf, qf[q], sacc[tt][q]);
            }
        }
        if (PRIO) __builtin_amdgcn_s_setprio(0);
        if (!(key0 >= wlo && key0 + BN - 1 <= whi)) {
            // key visible iff 0 <= key - lo <= span (one unsigned compare; rows
            // with no visible key carry lo far above every key and span 0)
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    const int base = key0 + 16 * tt + 4 * lg - row_lo[q];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if ((uint32_t)(base + e) > (uint32_t)row_span[q]) sacc[tt][q][e] = -INFINITY;
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    // exact row max of the tile; moves the reference max (and rescales O and l)
    // of the rows whose max exceeds it by more than 2^LAZY
    auto exact_max = [&]() {
        bool raise[NQ];
        bool any_raise = false;
        float mxs[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            float mx = -INFINITY;
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
                mx = vmax(vmax(vmax(vmax(mx, sacc[tt][q][0]), sacc[tt][q][1]), sacc[tt][q][2]), sacc[tt][q][3]);
            mx = xor_max(mx);
            mxs[q] = mx;
            raise[q] = m_run[q] == -INFINITY ? mx != -INFINITY : (mx - m_run[q]) * sl2 > LAZY;
            any_raise |= raise[q];
        }
        if (__builtin_amdgcn_ballot_w64(any_raise) != 0) {  // rare after the first tile
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                if (!raise[q]) continue;
                const float alpha = m_run[q] == -INFINITY ? 0.f : fast_exp2((m_run[q] - mxs[q]) * sl2);
                m_run[q] = mxs[q];
                negm[q] = -mxs[q] * sl2;
                l_run[q] *= alpha;
#pragma unroll
                for (int u = 0; u < DT; ++u) oacc[u][q] *= alpha;
            }
        }
    };
    // P = exp2(S * scale * log2e - m_ref) as fp16 pairs, and the tile's row sums
    // (bf16 form: P stays fp32 in sacc and the row sums are VALU adds; P.V splits
    // it into bf16 hi and lo parts, P ~= hi + lo to about 16 bits)
    u32x4 pf[NT / 2][NQ];
    f32x4 tsum[NQ];
    auto exps = [&]() {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const float neg = negm[q];
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                for (int e = 0; e < 4; ++e) sacc[tt][q][e] = fast_exp2(fmaf(sacc[tt][q][e], sl2, neg));
        }
        if constexpr (!VB) {
#pragma unroll
            for (int pp = 0; pp < NT / 2; ++pp)
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    pf[pp][q][0] = pack_f16x2(sacc[2 * pp][q][0], sacc[2 * pp][q][1]);
                    pf[pp][q][1] = pack_f16x2(sacc[2 * pp][q][2], sacc[2 * pp][q][3]);
                    pf[pp][q][2] = pack_f16x2(sacc[2 * pp + 1][q][0], sacc[2 * pp + 1][q][1]);
                    pf[pp][q][3] = pack_f16x2(sacc[2 * pp + 1][q][2], sacc[2 * pp + 1][q][3]);
                }
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                tsum[q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int pp = 0; pp < NT / 2; ++pp) tsum[q] = mfma_f16(ones, pf[pp][q], tsum[q]);
            }
        } else {
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                float ssum = 0.f;
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) ssum += (sacc[tt][q][0] + sacc[tt][q][1]) + (sacc[tt][q][2] + sacc[tt][q][3]);
                tsum[q][0] = xor_sum(ssum);
            }
        }
    };

    bool steady = false;  // every row of the wave has a finite reference max
    bool redo = false;    // this tile runs again with the exact max
    int stage = 0;
    for (int n = s_lo; n < s_hi;) {
        const bool more = n + 1 < s_hi;
        if (more && !redo) {  // prefetch the next (higher) tile into the other stage
            load_k(n + 1, stage ^ 1);
            if constexpr (!VB) load_v(n + 1);
        }
        const char* kt = smem + stage * STAGEB;
        const char* vt = kt + TILEB;
        const int key0 = n * BN;

        // a tile no row of the wave can see is skipped by the wave (the copies and the
        // barrier still run)
        if (key0 <= uhi && key0 + BN - 1 >= ulo) {
            // online softmax: exact max until steady, then the bounded fast form; a
            // steady tile whose row sums show an fp16 overflow runs again, exactly.
            // (The bf16 form always takes the exact max.)
            scores(kt, key0);
            if (VB || !steady || redo) exact_max();
            exps();
            if (!VB && steady && !redo) {
                bool bad = false;
#pragma unroll
                for (int q = 0; q < NQ; ++q) bad |= !(tsum[q][0] <= P_MAX);
                if (__builtin_amdgcn_ballot_w64(bad) != 0) {
                    redo = true;
                    continue;
                }
            }
            redo = false;
            if (!VB && !steady) {
                bool open = false;
#pragma unroll
                for (int q = 0; q < NQ; ++q) open |= m_run[q] == -INFINITY;
                steady = __builtin_amdgcn_ballot_w64(open) == 0;
            }
#pragma unroll
            for (int q = 0; q < NQ; ++q) l_run[q] += tsum[q][0];

            // O^T += V^T . P^T (fp16)
            if (PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int pp = 0; pp < NT / 2; ++pp) {
                const int ra = 32 * pp + 4 * lg + (li >> 2), rb = ra + 16;
                const int cb = (li & 3) >> 1, hb = 8 * (li & 1);
                auto v_frag = [&](const int u) {
                    const int ch = 2 * u + cb;
                    const u32x2 a = lds_read_tr16(reinterpret_cast<const bf16_t*>(vt + ra * ROWB + 16 * (ch ^ C::swz_v(ra)) + hb));
                    const u32x2 c = lds_read_tr16(reinterpret_cast<const bf16_t*>(vt + rb * ROWB + 16 * (ch ^ C::swz_v(rb)) + hb));
                    return u32x4{a[0], a[1], c[0], c[1]};
                };
                if constexpr (!VB) {
#pragma unroll
                    for (int u = 0; u < DT; ++u) {
                        const u32x4 vf = v_frag(u);
#pragma unroll
                        for (int q = 0; q < NQ; ++q) oacc[u][q] = mfma_f16(vf, pf[pp][q], oacc[u][q]);
                    }
                } else {
                    // bf16 form: P of this key half as hi + lo parts
                    u32x4 ph[NQ], plo[NQ];
#pragma unroll
                    for (int q = 0; q < NQ; ++q)
#pragma unroll
                        for (int w = 0; w < 4; ++w) {
                            const f32x4& src = sacc[2 * pp + (w >> 1)][q];
                            const u32x2 hl = split_bf16x2(src[2 * (w & 1)], src[2 * (w & 1) + 1]);
                            ph[q][w] = hl[0];
                            plo[q][w] = hl[1];
                        }
#pragma unroll
                    for (int u = 0; u < DT; ++u) {
                        const u32x4 vf = v_frag(u);
#pragma unroll
                        for (int q = 0; q < NQ; ++q) {
                            oacc[u][q] = mfma_bf16(vf, ph[q], oacc[u][q]);
                            oacc[u][q] = mfma_bf16(vf, plo[q], oacc[u][q]);
                        }
                    }
                }
            }

            if (PRIO) __builtin_amdgcn_s_setprio(0);
        }
        if (more) {
            // (the bf16 form, which runs only when a V element is beyond fp16's
            // range, loads V here rather than ahead, so its registers are not
            // live across the tile and the kernel needs no more of them)
            if constexpr (VB) load_v(n + 1);
            store_v(stage ^ 1);
            wait_vmcnt<0>();  // this wave's K copies landed
        }
        __syncthreads();
        stage ^= 1;
        ++n;
    }

    // ---- epilogue. fp16 form: finite inputs give finite accumulators unless a V
    // element overflowed fp16 (then inf, or NaN where it met P = 0); the whole
    // workgroup then runs the tile again in the bf16 form.
    if constexpr (!VB) {
        float chk = 0.f;
#pragma unroll
        for (int u = 0; u < DT; ++u)
#pragma unroll
            for (int q = 0; q < NQ; ++q) chk += (oacc[u][q][0] + oacc[u][q][1]) + (oacc[u][q][2] + oacc[u][q][3]);
        if (__builtin_amdgcn_ballot_w64(!(__builtin_fabsf(chk) <= 3.0e38f)) != 0 && lane == 0) s_bad = 1;
        __syncthreads();
        if (s_bad) return true;
    }
    const bool split_out = S > 1;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        if (!row_ok[q]) continue;
        const float l = l_run[q];
        const bool any = l > 0.f;
        const float inv = any ? 1.f / l : 0.f;
        const float lse = any ? m_run[q] * p.scale + logf(l) : -INFINITY;
        const size_t row = ((size_t)b * p.Sq + row_pos[q]) * p.Hq + row_head[q];
        if (split_out) {
            const size_t rows_total = (size_t)p.B * p.Sq * p.Hq;
            if (lg == 0) p.lse_part[(size_t)split * rows_total + row] = lse;
            if (any) {
                float* orow = p.o_part + ((size_t)split * rows_total + row) * D + 4 * lg;
#pragma unroll
                for (int u = 0; u < DT; ++u) *reinterpret_cast<f32x4*>(orow + 16 * u) = oacc[u][q] * inv;
            }
        } else {
            if (lg == 0 && p.lse) p.lse[((size_t)b * p.Hq + row_head[q]) * p.Sq + row_pos[q]] = lse;
            bf16_t* orow = reinterpret_cast<bf16_t*>(p.o) + row * D + 4 * lg;
#pragma unroll
            for (int u = 0; u < DT; ++u) {
                u32x2 w;
                w[0] = pack_bf16x2(oacc[u][q][0] * inv, oacc[u][q][1] * inv);
                w[1] = pack_bf16x2(oacc[u][q][2] * inv, oacc[u][q][3] * inv);
                *reinterpret_cast<u32x2*>(orow + 16 * u) = w;
            }
        }
    }
    return false;
    };
    auto run = [&](const int t) {
        if (run_tile(t, std::false_type{}, std::integral_constant<int, C::NQ>{}, 0))
            for (int q0 = 0; q0 < C::NQ; ++q0) run_tile(t, std::true_type{}, std::integral_constant<int, 1>{}, q0);
    };

    if constexpr (PERSIST == 0) {
        // one tile per workgroup; workgroups are dealt round-robin to the 8 XCDs,
        // so tile t of section blockIdx % 8 lands on that XCD
        const int t = ((int)blockIdx.x % NUM_XCD) * per_xcd + (int)blockIdx.x / NUM_XCD;
        if (t < total) run(t);
    } else {
        // persistent: each workgroup pops tiles from its own XCD's queue (an
        // atomic counter per section, zeroed before the launch), then from the
        // other queues once its own is empty; every workgroup leaves when all
        // eight are exhausted. (Measured slower than the dealt grid above on the
        // causal and windowed prefills: the dispatcher already balances these
        // tiles, and each pop adds an atomic's latency; popping during a tile
        // instead breaks the heaviest-first balance.)
        __shared__ int s_next;
        const int xcd = __builtin_amdgcn_s_getreg((3 << 11) | 20) & (NUM_XCD - 1);  // HW_REG_XCC_ID
        int qi = 0;  // queues tried so far (thread 0)
        while (true) {
            if (tid == 0) {
                int next = -1;
                for (; qi < NUM_XCD; ++qi) {
                    const int x = (xcd + qi) & (NUM_XCD - 1);
                    const int size = imin(per_xcd, total - x * per_xcd);
                    if (size <= 0) continue;
                    const int i = atomicAdd(p.tile_counters + x, 1);
                    if (i < size) {
                        next = x * per_xcd + i;
                        break;
                    }
                }
                s_next = next;
            }
            __syncthreads();
            const int t = s_next;
            __syncthreads();  // all waves have read s_next before thread 0 overwrites it
            if (t < 0) break;
            run(t);
        }
    }
}


__global__ void tile_counters_reset_kernel(int* c, int n) {
    if ((int)threadIdx.x < n) c[threadIdx.x] = 0;
}
hipError_t launch_tile_counters_reset(int* counters, hipStream_t stream) {
    hipLaunchKernelGGL(tile_counters_reset_kernel, dim3(1), dim3(64), 0, stream, counters, NUM_XCD);
    return hipGetLastError();
}

template <int D, int NWV, int MW, int PRI = 1, int PERSIST = 0>
hipError_t launch_prefill(const FwdParams& p, dim3 grid, hipStream_t stream) {
    // grid: one dimension over every tile (persistent: over the resident
    // workgroups), padded to a multiple of the XCD count
    hipLaunchKernelGGL((attn_prefill_kernel<D, NWV, MW, PRI, PERSIST>), grid, dim3(64 * NWV), 0, stream, p);
    return hipGetLastError();
}

const FwdVariant* prefill_variants() {
    static const FwdVariant v[] = {
        // one 8-wave workgroup per CU: K/V tiles shared by 256 rows
        {DT_BF16, 128, 256, 64, 8, 1, PrefillTile<128, 8, 32>::LDS_BYTES, &launch_prefill<128, 8, 32, 0>, 1},
        // ablation: raised wave priority around the MFMA phases (measured slower)
        {DT_BF16, 128, 256, 64, 8, 1, PrefillTile<128, 8, 32>::LDS_BYTES, &launch_prefill<128, 8, 32, 1>, 1},
        {DT_BF16, 64, 256, 64, 8, 1, PrefillTile<64, 8, 32>::LDS_BYTES, &launch_prefill<64, 8, 32, 0>, 1},
        // two 4-wave workgroups per CU (independent barriers): the default with a
        // sliding window, an ablation otherwise
        {DT_BF16, 128, 128, 64, 4, 1, PrefillTile<128, 4, 32>::LDS_BYTES, &launch_prefill<128, 4, 32, 0>, 1},
        {DT_BF16, 64, 128, 64, 4, 1, PrefillTile<64, 4, 32>::LDS_BYTES, &launch_prefill<64, 4, 32, 0>, 1},
        // persistent workgroups with per-XCD tile queues
        {DT_BF16, 128, 256, 64, 8, 1, PrefillTile<128, 8, 32>::LDS_BYTES, &launch_prefill<128, 8, 32, 0, 1>, 1, 1},
        {DT_BF16, 128, 128, 64, 4, 1, PrefillTile<128, 4, 32>::LDS_BYTES, &launch_prefill<128, 4, 32, 0, 1>, 1, 2},
        {DT_BF16, 64, 256, 64, 8, 1, PrefillTile<64, 8, 32>::LDS_BYTES, &launch_prefill<64, 8, 32, 0, 1>, 1, 1},
        {DT_BF16, 64, 128, 64, 4, 1, PrefillTile<64, 4, 32>::LDS_BYTES, &launch_prefill<64, 4, 32, 0, 1>, 1, 2},
        {0, 0, 0, 0, 0, 0, 0, nullptr, 0},
    };
    return v;
}

}  // namespace tpa
