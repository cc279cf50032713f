// attn_prefill.hip -- gfx950 flash-attention forward for many query rows (bf16).
//
// Citations:
//   [FA-tiling]  "分块策略与调度" (FlashAttention tiling strategy and scheduling)
//
// One workgroup of NWV waves owns BM = NWV * MW query rows of one (batch, query
// head[, split]) and walks its key-block range ([FA-tiling] §3) from the last
// block to the first. Per 64-key tile:
//   * K (bf16) streams from global memory straight into LDS (buffer_load ...
//     lds), V is loaded into registers, converted to fp16 and written to LDS;
//     both double-buffered, so tile n-1 loads while tile n computes, with one
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
// share one XCD's L2 and its K/V are fetched from HBM about once. Within a head
// the query blocks run heaviest first ([FA-tiling] §4.4).
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
    constexpr int BN = C::BN, BM = C::BM, NQ = C::NQ, NT = C::NT, NSLAB = C::NSLAB, DT = C::DT;
    constexpr int CPR = C::CPR, ROWB = C::ROWB, TILEB = C::TILEB, STAGEB = C::STAGEB;
    __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;

    // ---- tiles: t in [0, total) ordered (batch, head, split, query block heaviest
    // first); XCD x owns the section [x per_xcd, (x + 1) per_xcd)
    const int M = p.num_m_blocks, S = p.num_splits;
    const int total = p.B * p.grid_heads * S * M;
    const int per_xcd = (total + NUM_XCD - 1) / NUM_XCD;
    auto run_tile = [&](const int t) {
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
        const int r = m_block * BM + wave * MW + 16 * q + li;
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
    wlo = row16_imax(wlo);
    whi = row16_imin(whi);
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
    float m_run[NQ], l_run[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        m_run[q] = -INFINITY;
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
    auto load_k = [&](int n, int stage) {
        const rsrc_t rk = make_rsrc(kbase + (size_t)n * BN * kv_stride, tile_bytes(n));
        char* dst = smem + stage * STAGEB;
#pragma unroll
        for (int j = 0; j < C::KDMA_PER_WAVE; ++j) {
            const int i = wave * C::KDMA_PER_WAVE + j;
            if (C::KDMA % NWV == 0 || i < C::KDMA) {
                const int rr = C::KROWS_PER_DMA * i + lane / CPR;
                const int slot = lane % CPR;
                const uint32_t voff = rr * row_bytes + 16 * (slot ^ C::swz_k(rr));
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rk, (__attribute__((address_space(3))) void*)(dst + 1024 * i), 16, voff, 0, 0, 0);
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
            u32x4 h;
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] = bf16x2_to_f16x2(vst[j][e]);
            *reinterpret_cast<u32x4*>(dst + rr * ROWB + 16 * (ch ^ C::swz_v(rr))) = h;
        }
    };

    if (has_work) {
        load_k(s_hi - 1, 0);
        load_v(s_hi - 1);
        store_v(0);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the K DMA has landed
    }
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
                l_run[q] *= alpha;
#pragma unroll
                for (int u = 0; u < DT; ++u) oacc[u][q] *= alpha;
            }
        }
    };
    // P = exp2(S * scale * log2e - m_ref) as fp16 pairs, and the tile's row sums
    u32x4 pf[NT / 2][NQ];
    f32x4 tsum[NQ];
    auto exps = [&]() {
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const float neg = m_run[q] == -INFINITY ? 0.f : -m_run[q] * sl2;
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                for (int e = 0; e < 4; ++e) sacc[tt][q][e] = fast_exp2(fmaf(sacc[tt][q][e], sl2, neg));
        }
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
    };

    bool steady = false;  // every row of the wave has a finite reference max
    bool redo = false;    // this tile runs again with the exact max
    int stage = 0;
    for (int n = s_hi - 1; n >= s_lo;) {
        const bool more = n > s_lo;
        if (more && !redo) {  // prefetch the next (lower) tile into the other stage
            load_k(n - 1, stage ^ 1);
            load_v(n - 1);
        }
        const char* kt = smem + stage * STAGEB;
        const char* vt = kt + TILEB;
        const int key0 = n * BN;

        // online softmax: exact max until steady, then the bounded fast form; a
        // steady tile whose row sums show an fp16 overflow runs again, exactly
        scores(kt, key0);
        if (!steady || redo) exact_max();
        exps();
        if (steady && !redo) {
            bool bad = false;
#pragma unroll
            for (int q = 0; q < NQ; ++q) bad |= !(tsum[q][0] <= P_MAX);
            if (__builtin_amdgcn_ballot_w64(bad) != 0) {
                redo = true;
                continue;
            }
        }
        redo = false;
        if (!steady) {
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
#pragma unroll
            for (int u = 0; u < DT; ++u) {
                const int ch = 2 * u + cb;
                const u32x2 a = lds_read_tr16(reinterpret_cast<const bf16_t*>(vt + ra * ROWB + 16 * (ch ^ C::swz_v(ra)) + hb));
                const u32x2 c = lds_read_tr16(reinterpret_cast<const bf16_t*>(vt + rb * ROWB + 16 * (ch ^ C::swz_v(rb)) + hb));
                const u32x4 vf = {a[0], a[1], c[0], c[1]};
#pragma unroll
                for (int q = 0; q < NQ; ++q) oacc[u][q] = mfma_f16(vf, pf[pp][q], oacc[u][q]);
            }
        }

        if (PRIO) __builtin_amdgcn_s_setprio(0);
        if (more) {
            store_v(stage ^ 1);
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's K DMAs landed
        }
        __syncthreads();
        stage ^= 1;
        --n;
    }

    // ---- epilogue
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
    };

    if constexpr (PERSIST == 0) {
        // one tile per workgroup; workgroups are dealt round-robin to the 8 XCDs,
        // so tile t of section blockIdx % 8 lands on that XCD
        const int t = ((int)blockIdx.x % NUM_XCD) * per_xcd + (int)blockIdx.x / NUM_XCD;
        if (t < total) run_tile(t);
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
            run_tile(t);
        }
    }
}


// ---------------------------------------------------------------------------
// Software-pipelined variant: within every wave, the QK MFMAs of tile n-1 are
// issued before the softmax of tile n (two score buffers), so the matrix core
// works on the next tile while the VALU exponentiates the current one; the
// exponentials of the second key half overlap the first half's PV MFMAs.
// K runs one tile ahead of V: K tiles j and j-1 and V tiles j and j-1 occupy
// the two K and two V buffers, still one workgroup barrier per tile.
// ---------------------------------------------------------------------------
template <int D, int NWV, int MW>
__global__ void __launch_bounds__(64 * NWV, MW > 32 ? 1 : 8 / NWV) attn_prefill_pipe_kernel(FwdParams p) {
    using C = PrefillTile<D, NWV, MW>;
    constexpr int BN = C::BN, BM = C::BM, NQ = C::NQ, NT = C::NT, NSLAB = C::NSLAB, DT = C::DT;
    constexpr int CPR = C::CPR, ROWB = C::ROWB, TILEB = C::TILEB;
    // LDS: K buffers 0,1 then V buffers 0,1
    __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;

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

    int row_pos[NQ], row_head[NQ], row_lo[NQ], row_hi[NQ];
    bool row_ok[NQ];
    int wlo = -0x7fffffff, whi = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int r = m_block * BM + wave * MW + 16 * q + li;
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
    wlo = row16_imax(wlo);
    whi = row16_imin(whi);

    const bf16_t* qp = reinterpret_cast<const bf16_t*>(p.q);
    u32x4 qf[NQ][NSLAB];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const bf16_t* qrow = qp + (((size_t)b * p.Sq + row_pos[q]) * p.Hq + row_head[q]) * D + 8 * lg;
        const bool use = row_ok[q] && has_work;
#pragma unroll
        for (int c = 0; c < NSLAB; ++c) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(qrow + 32 * c);
            const u32x4 z = {0u, 0u, 0u, 0u};
            qf[q][c] = use ? x : z;
        }
    }

    f32x4 oacc[DT][NQ], lacc[NQ];
    float m_run[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        m_run[q] = -INFINITY;
        lacc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < DT; ++u) oacc[u][q] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const u32x4 ones = {0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u};  // fp16 1.0
    const float sl2 = p.scale_log2;
    constexpr float LAZY = 8.f;

    const size_t kv_stride = (size_t)p.Hkv * D;
    const uint32_t row_bytes = (uint32_t)(kv_stride * 2);
    const bf16_t* kbase = reinterpret_cast<const bf16_t*>(p.k) + ((size_t)b * p.Sk * p.Hkv + hkv) * D;
    const bf16_t* vbase = reinterpret_cast<const bf16_t*>(p.v) + ((size_t)b * p.Sk * p.Hkv + hkv) * D;
    auto tile_bytes = [&](int n) { return (uint32_t)imin(BN, Skb - n * BN) * row_bytes; };
    auto kbuf = [&](int n) { return smem + (n & 1) * TILEB; };
    auto vbuf = [&](int n) { return smem + 2 * TILEB + (n & 1) * TILEB; };
    auto load_k = [&](int n) {
        const rsrc_t rk = make_rsrc(kbase + (size_t)n * BN * kv_stride, tile_bytes(n));
        char* dst = kbuf(n);
#pragma unroll
        for (int j = 0; j < C::KDMA_PER_WAVE; ++j) {
            const int i = wave * C::KDMA_PER_WAVE + j;
            if (C::KDMA % NWV == 0 || i < C::KDMA) {
                const int rr = C::KROWS_PER_DMA * i + lane / CPR;
                const int slot = lane % CPR;
                const uint32_t voff = rr * row_bytes + 16 * (slot ^ C::swz_k(rr));
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rk, (__attribute__((address_space(3))) void*)(dst + 1024 * i), 16, voff, 0, 0, 0);
            }
        }
    };
    u32x4 vst[C::VCH];
    auto load_v = [&](int n) {
        const rsrc_t rv = make_rsrc(vbase + (size_t)n * BN * kv_stride, tile_bytes(n));
#pragma unroll
        for (int j = 0; j < C::VCH; ++j) {
            const int id = tid + C::NTHR * j;
            vst[j] = buf_load16(rv, (id / CPR) * row_bytes + 16 * (id % CPR));
        }
    };
    auto store_v = [&](int n) {
        char* dst = vbuf(n);
#pragma unroll
        for (int j = 0; j < C::VCH; ++j) {
            const int id = tid + C::NTHR * j;
            const int rr = id / CPR, ch = id % CPR;
            u32x4 h;
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] = bf16x2_to_f16x2(vst[j][e]);
            *reinterpret_cast<u32x4*>(dst + rr * ROWB + 16 * (ch ^ C::swz_v(rr))) = h;
        }
    };
    auto qk = [&](int n, f32x4 (&sacc)[NT][NQ]) {
        const char* kt = kbuf(n);
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int q = 0; q < NQ; ++q) sacc[tt][q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NSLAB; ++c) {
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) {
                const int rr = 16 * tt + li;
                const u32x4 kf = *reinterpret_cast<const u32x4*>(kt + rr * ROWB + 16 * ((4 * c + lg) ^ C::swz_k(rr)));
#pragma unroll
                for (int q = 0; q < NQ; ++q) sacc[tt][q] = mfma_bf16(kf, qf[q][c], sacc[tt][q]);
            }
        }
    };

    f32x4 sa[NT][NQ], sb[NT][NQ];

    // softmax bookkeeping for the scores of tile n held in sa: optional element
    // mask, row max, lazy rescale of O (rare, branchy, before the main block)
    auto prologue_softmax = [&](int n, bool masked, float (&neg)[NQ]) {
        if (masked) {
            const int key0 = n * BN;
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                for (int q = 0; q < NQ; ++q)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int key = key0 + 16 * tt + 4 * lg + e;
                        if (key < row_lo[q] || key > row_hi[q]) sa[tt][q][e] = -INFINITY;
                    }
        }
        bool raise[NQ];
        bool any_raise = false;
        float mxs[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            float mx = -INFINITY;
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
                mx = vmax(vmax(vmax(vmax(mx, sa[tt][q][0]), sa[tt][q][1]), sa[tt][q][2]), sa[tt][q][3]);
            mx = xor_max(mx);
            mxs[q] = mx;
            raise[q] = m_run[q] == -INFINITY ? mx != -INFINITY : (mx - m_run[q]) * sl2 > LAZY;
            any_raise |= raise[q];
        }
        if (__builtin_amdgcn_ballot_w64(any_raise) != 0) {
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                if (!raise[q]) continue;
                const float alpha = m_run[q] == -INFINITY ? 0.f : fast_exp2((m_run[q] - mxs[q]) * sl2);
                m_run[q] = mxs[q];
                lacc[q] *= alpha;
#pragma unroll
                for (int u = 0; u < DT; ++u) oacc[u][q] *= alpha;
            }
        }
#pragma unroll
        for (int q = 0; q < NQ; ++q) neg[q] = m_run[q] == -INFINITY ? 0.f : -m_run[q] * sl2;
    };
    // exponentials of one 32-key half of sa, packed to fp16 B operands
    auto exp_half = [&](int pp, const float (&neg)[NQ], u32x4 (&pf)[NQ]) {
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int tt = 2 * pp + h;
                const float p0 = fast_exp2(fmaf(sa[tt][q][0], sl2, neg[q]));
                const float p1 = fast_exp2(fmaf(sa[tt][q][1], sl2, neg[q]));
                const float p2 = fast_exp2(fmaf(sa[tt][q][2], sl2, neg[q]));
                const float p3 = fast_exp2(fmaf(sa[tt][q][3], sl2, neg[q]));
                pf[q][2 * h] = pack_f16x2(p0, p1);
                pf[q][2 * h + 1] = pack_f16x2(p2, p3);
            }
    };
    auto pv_half = [&](int n, int pp, const u32x4 (&pf)[NQ]) {
        const char* vt = vbuf(n);
        const int ra = 32 * pp + 4 * lg + (li >> 2), rb = ra + 16;
        const int cb = (li & 3) >> 1, hb = 8 * (li & 1);
#pragma unroll
        for (int q = 0; q < NQ; ++q) lacc[q] = mfma_f16(ones, pf[q], lacc[q]);
#pragma unroll
        for (int u = 0; u < DT; ++u) {
            const int ch = 2 * u + cb;
            const u32x2 a = lds_read_tr16(reinterpret_cast<const bf16_t*>(vt + ra * ROWB + 16 * (ch ^ C::swz_v(ra)) + hb));
            const u32x2 c = lds_read_tr16(reinterpret_cast<const bf16_t*>(vt + rb * ROWB + 16 * (ch ^ C::swz_v(rb)) + hb));
            const u32x4 vf = {a[0], a[1], c[0], c[1]};
#pragma unroll
            for (int q = 0; q < NQ; ++q) oacc[u][q] = mfma_f16(vf, pf[q], oacc[u][q]);
        }
    };
    auto needs_mask = [&](int n) {
        const int key0 = n * BN;
        return !(key0 >= wlo && key0 + BN - 1 <= whi);
    };

    int n = s_hi - 1;
    if (has_work) {
        load_k(n);
        load_v(n);
        if (n - 1 >= s_lo) load_k(n - 1);
        store_v(n);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    }
    __syncthreads();
    if (has_work) qk(n, sa);
    __syncthreads();  // every wave has read K(n) before its buffer is reused

    // steady state: tiles n > s_lo (each has a next tile n - 1)
    for (; n > s_lo; --n) {
        float neg[NQ];
        prologue_softmax(n, needs_mask(n), neg);
        if (n - 2 >= s_lo) load_k(n - 2);
        load_v(n - 1);
        // one straight-line block: QK(n-1) | exp(n, first half) | PV(n) | exp(n, second half)
        u32x4 pf0[NQ], pf1[NQ];
        qk(n - 1, sb);
        exp_half(0, neg, pf0);
        pv_half(n, 0, pf0);
        exp_half(1, neg, pf1);
        pv_half(n, 1, pf1);
        store_v(n - 1);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's K DMA landed
        __syncthreads();
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int q = 0; q < NQ; ++q) sa[tt][q] = sb[tt][q];
    }
    // last tile (no next)
    if (has_work) {
        float neg[NQ];
        prologue_softmax(n, needs_mask(n), neg);
        u32x4 pf0[NQ], pf1[NQ];
        exp_half(0, neg, pf0);
        pv_half(n, 0, pf0);
        exp_half(1, neg, pf1);
        pv_half(n, 1, pf1);
    }

    const bool split_out = S > 1;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        if (!row_ok[q]) continue;
        const float l = lacc[q][0];
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
}

// ===========================================================================
// 32x32x16 MFMA variant with V pre-converted to fp16 and transposed.
//
// A pre-pass writes V once per call as fp16 V^T per (batch, KV head), so the main
// loop streams both operands into LDS by DMA (no register staging, no per-tile
// conversion: the 16-row kernel above converts every V tile again for every query
// block that visits it) and reads both with 16-byte LDS reads. Each wave owns 32
// query rows; lane l holds query l % 32 of every 32x32 accumulator, so a row max
// needs one cross-lane step (v_permlane32_swap), and a 32x32x16 MFMA takes less
// of the issue slots the softmax needs than two 16x16x32 MFMAs.
// Measured on the causal 8192 x 32-head prefill: about 13% fewer cycles than
// attn_prefill_kernel, but the clock settles near 2.1 GHz instead of 2.4 (with
// random operands the 32x32x16 bf16 MFMA alone sustains 1.9 PFLOP/s against
// 2.14 for 16x16x32), and the pre-pass costs ~26 us, so it is not the default.
//
// vt layout: vt[((b * Hkv + h) * D + d) * skp + pos], skp = Sk rounded up to 64.
// Within each block of BLK keys (BLK = 16 for the 32x32x16 kernel; a 16x16x32 PV
// would take 32), position 8 g + e (lane group g, element e = 0..7) holds key
// (BLK / 2) (e / 4) + 4 g + e % 4: the order in which lane group g of the S^T
// accumulators holds the block's keys, so P^T goes from the accumulators into
// the PV MFMA's B operand without moving between lanes. Keys at or past the
// sequence's length are zero.
template <int D, int BLK>
__global__ void __launch_bounds__(256) v_to_f16t_kernel(const bf16_t* __restrict__ v, _Float16* __restrict__ vt,
                                                        const int* seqlens_k, int Sk, int Hkv, int skp) {
    constexpr int KB = 64, CPR = D / 8, PITCH = D + 2;  // LDS row pitch in halves (bank spread)
    __shared__ _Float16 t[KB * PITCH];
    const int key0 = blockIdx.x * KB, h = blockIdx.y, b = blockIdx.z;
    int Skb = Sk;
    if (seqlens_k) Skb = imax(0, imin(seqlens_k[b], Sk));
    const int tid = threadIdx.x;
    // load 64 key rows (16-byte chunks), convert to fp16, store row-major
#pragma unroll
    for (int j = 0; j < KB * CPR / 256; ++j) {
        const int id = tid + 256 * j;
        const int kr = id / CPR, c = id % CPR;
        const int key = key0 + kr;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (key < Skb) x = *reinterpret_cast<const u32x4*>(v + (((size_t)b * Sk + key) * Hkv + h) * D + 8 * c);
        uint32_t* dst = reinterpret_cast<uint32_t*>(t + kr * PITCH + 8 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f16x2 hv;
            hv[0] = (_Float16)__uint_as_float(x[e] << 16);
            hv[1] = (_Float16)__uint_as_float(x[e] & 0xffff0000u);
            dst[e] = __builtin_bit_cast(uint32_t, hv);
        }
    }
    __syncthreads();
    // write V^T rows: 8 lanes per d row, each 8 positions (16 bytes)
    _Float16* out = vt + ((size_t)b * Hkv + h) * D * (size_t)skp + key0;
#pragma unroll
    for (int j = 0; j < D * 8 / 256; ++j) {
        const int id = tid + 256 * j;
        const int d = id / 8, c = id % 8;
        f16x8 w;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int pos = 8 * c + e;                      // position within the 64-key tile
            const int pe = pos & (BLK - 1), g = pe >> 3, ee = pe & 7;
            const int kr = (pos & ~(BLK - 1)) + (BLK / 2) * (ee >> 2) + 4 * g + (ee & 3);
            w[e] = t[kr * PITCH + d];
        }
        *reinterpret_cast<f16x8*>(out + (size_t)d * skp + 8 * c) = w;
    }
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32_bf16(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32_f16(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

template <int D, int NWV>
struct M32Tile {
    static constexpr int BN = 64;               // keys per tile
    static constexpr int BM = 32 * NWV;         // query rows per workgroup
    static constexpr int NTHR = 64 * NWV;
    static constexpr int KSTEP = D / 16;        // QK contraction steps
    static constexpr int DB = D / 32;           // 32-wide d blocks of O^T
    static constexpr int KCPR = D / 8;          // 16-byte chunks per K row
    static constexpr int KROWB = 2 * D;         // bytes per K row in LDS
    static constexpr int VROWB = 2 * BN;        // bytes per V^T row in LDS
    static constexpr int KTILEB = BN * KROWB, VTILEB = D * VROWB;
    static constexpr int KDMA = KTILEB / 1024, VDMA = VTILEB / 1024;  // wave-wide DMAs per tile
    static constexpr int KROWS_PER_DMA = 1024 / KROWB, VROWS_PER_DMA = 1024 / VROWB;
    static constexpr int LDS_BYTES = 2 * (KTILEB + VTILEB);
    static_assert(KDMA % NWV == 0 && VDMA % NWV == 0, "DMAs must split evenly over the waves");
    // 16-byte chunk swizzles: the 16 lanes of a quarter-wave read 16 different
    // rows at one logical chunk and hit 16 different bank groups
    static __host__ __device__ __forceinline__ int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
    static __host__ __device__ __forceinline__ int swz_v(int r) { return (r >> 1) & 7; }
};

template <int D, int NWV>
__global__ void __launch_bounds__(64 * NWV, 8 / NWV) attn_prefill_m32_kernel(FwdParams p) {
    using C = M32Tile<D, NWV>;
    constexpr int BN = C::BN, BM = C::BM, KSTEP = C::KSTEP, DB = C::DB;
    constexpr int KROWB = C::KROWB, VROWB = C::VROWB;
    __shared__ __attribute__((aligned(16))) char k_lds0[C::KTILEB];
    __shared__ __attribute__((aligned(16))) char k_lds1[C::KTILEB];
    __shared__ __attribute__((aligned(16))) char v_lds0[C::VTILEB];
    __shared__ __attribute__((aligned(16))) char v_lds1[C::VTILEB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lq = lane & 31, lg = lane >> 5;

    // ---- tile coordinates: XCD-aware placement, heaviest query block first
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

    // ---- this lane's query row and its visible key interval
    const int r = m_block * BM + wave * 32 + lq;
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
    wlo = row16_imax(wlo);
    whi = row16_imin(whi);
    wlo = imax(wlo, __shfl_xor(wlo, 16));
    whi = imin(whi, __shfl_xor(whi, 16));

    // ---- Q^T fragments: lane (q, g) holds Q[row q][16 s + 8 g .. +7]
    u32x4 qf[KSTEP];
    {
        const bf16_t* qrow = reinterpret_cast<const bf16_t*>(p.q) + (((size_t)b * p.Sq + row_pos) * p.Hq + row_head) * D + 8 * lg;
        const bool use = row_ok && has_work;
#pragma unroll
        for (int s2 = 0; s2 < KSTEP; ++s2) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(qrow + 16 * s2);
            const u32x4 z = {0u, 0u, 0u, 0u};
            qf[s2] = use ? x : z;
        }
    }

    // row sums of P: each lane adds its fp16 P values (v_dot2 with (1, 1), so l is
    // the sum of exactly the P that enters the PV MFMA); lanes q and q + 32 hold
    // the two halves of a row's keys and are added at the end
    f32x16 oacc[DB];
    float lsum = 0.f;
#pragma unroll
    for (int u = 0; u < DB; ++u)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[u][e] = 0.f;
    float m_run = -INFINITY;
    const f16x2 one2 = {(_Float16)1.f, (_Float16)1.f};
    const float sl2 = p.scale_log2;
    constexpr float LAZY = 8.f;  // lazy reference max (see attn_prefill_kernel)

    // ---- K / V^T tile DMAs (each wave issues KDMA/NWV + VDMA/NWV of them)
    const size_t kv_stride = (size_t)p.Hkv * D;
    const uint32_t k_row_bytes = (uint32_t)(kv_stride * 2);
    const bf16_t* kbase = reinterpret_cast<const bf16_t*>(p.k) + ((size_t)b * p.Sk * p.Hkv + hkv) * D;
    const _Float16* vthead = reinterpret_cast<const _Float16*>(p.vt) + ((size_t)b * p.Hkv + hkv) * D * (size_t)p.skp;
    const uint32_t vt_row_bytes = (uint32_t)p.skp * 2;
    auto load_tile = [&](int n, char* kdst, char* vdst) {
        const rsrc_t rk = make_rsrc(kbase + (size_t)n * BN * kv_stride, (uint32_t)imin(BN, Skb - n * BN) * k_row_bytes);
#pragma unroll
        for (int j = 0; j < C::KDMA / NWV; ++j) {
            const int i = wave + NWV * j;
            const int rr = C::KROWS_PER_DMA * i + lane / C::KCPR;
            const int slot = lane % C::KCPR;
            const uint32_t voff = rr * k_row_bytes + 16 * (slot ^ C::swz_k(rr));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rk, (__attribute__((address_space(3))) void*)(kdst + 1024 * i), 16, voff, 0, 0, 0);
        }
        const rsrc_t rv = make_rsrc(vthead + (size_t)n * BN, (uint32_t)(D - 1) * vt_row_bytes + 2 * BN);
#pragma unroll
        for (int j = 0; j < C::VDMA / NWV; ++j) {
            const int i = wave + NWV * j;
            const int d = C::VROWS_PER_DMA * i + lane / 8;
            const int slot = lane % 8;
            const uint32_t voff = d * vt_row_bytes + 16 * (slot ^ C::swz_v(d));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rv, (__attribute__((address_space(3))) void*)(vdst + 1024 * i), 16, voff, 0, 0, 0);
        }
    };

    auto tile = [&](auto stage_c, int n) {
        constexpr int ST = decltype(stage_c)::value;
        const char* kt = ST ? k_lds1 : k_lds0;
        const char* vt = ST ? v_lds1 : v_lds0;
        const bool more = n > s_lo;
        if (more) load_tile(n - 1, ST ? k_lds0 : k_lds1, ST ? v_lds0 : v_lds1);

        // S^T = K . Q^T: two 32-key blocks
        f32x16 sacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int e = 0; e < 16; ++e) sacc[kb][e] = 0.f;
            const int rr = 32 * kb + lq;
#pragma unroll
            for (int s2 = 0; s2 < KSTEP; ++s2) {
                const u32x4 kf = *reinterpret_cast<const u32x4*>(kt + rr * KROWB + 16 * ((2 * s2 + lg) ^ C::swz_k(rr)));
                sacc[kb] = mfma32_bf16(kf, qf[s2], sacc[kb]);
            }
        }

        // mask (tiles that cut a row's visible interval only); element (kb, e)
        // is key key0 + 32 kb + 8 (e / 4) + 4 g + e % 4
        const int key0 = n * BN;
        if (!(key0 >= wlo && key0 + BN - 1 <= whi)) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int key = key0 + 32 * kb + 8 * (e >> 2) + 4 * lg + (e & 3);
                    if (key < row_lo || key > row_hi) sacc[kb][e] = -INFINITY;
                }
        }
        // online softmax with a lazily moved reference max
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; e += 2) mx = vmax(vmax(mx, sacc[kb][e]), sacc[kb][e + 1]);
        mx = max32(mx);
        const bool raise = m_run == -INFINITY ? mx != -INFINITY : (mx - m_run) * sl2 > LAZY;
        if (raise) {
            const float alpha = m_run == -INFINITY ? 0.f : fast_exp2((m_run - mx) * sl2);
            m_run = mx;
            lsum *= alpha;
#pragma unroll
            for (int u = 0; u < DB; ++u) oacc[u] *= alpha;
        }
        const float neg = m_run == -INFINITY ? 0.f : -m_run * sl2;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) sacc[kb][e] = fast_exp2(fmaf(sacc[kb][e], sl2, neg));

        // O^T += V^T . P^T, four 16-key steps; step t takes accumulator groups
        // j0 = 2 (t % 2), j0 + 1 of block t / 2 (see the vt layout above)
#pragma unroll
        for (int t2 = 0; t2 < 4; ++t2) {
            const int kb = t2 >> 1, j0 = 2 * (t2 & 1);
            u32x4 pf;
            pf[0] = pack_f16x2(sacc[kb][4 * j0 + 0], sacc[kb][4 * j0 + 1]);
            pf[1] = pack_f16x2(sacc[kb][4 * j0 + 2], sacc[kb][4 * j0 + 3]);
            pf[2] = pack_f16x2(sacc[kb][4 * j0 + 4], sacc[kb][4 * j0 + 5]);
            pf[3] = pack_f16x2(sacc[kb][4 * j0 + 6], sacc[kb][4 * j0 + 7]);
            {
                const f16x8 ph = __builtin_bit_cast(f16x8, pf);  // whole-vector cast: an element cast miscompiles
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const f16x2 pair = {ph[2 * w], ph[2 * w + 1]};
                    lsum = __builtin_amdgcn_fdot2(pair, one2, lsum, false);
                }
            }
#pragma unroll
            for (int u = 0; u < DB; ++u) {
                const int rv = 32 * u + lq;
                const u32x4 vf = *reinterpret_cast<const u32x4*>(vt + rv * VROWB + 16 * ((2 * t2 + lg) ^ C::swz_v(rv)));
                oacc[u] = mfma32_f16(vf, pf, oacc[u]);
            }
        }

        if (more) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's DMAs landed
        __syncthreads();
    };

    if (has_work) {
        load_tile(s_hi - 1, k_lds0, v_lds0);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    }
    __syncthreads();
    for (int n = s_hi - 1; n >= s_lo; n -= 2) {
        tile(std::integral_constant<int, 0>{}, n);
        if (n - 1 >= s_lo) tile(std::integral_constant<int, 1>{}, n - 1);
    }

    // ---- epilogue: lane (q, g) holds O^T[32 u + 8 j + 4 g + 0..3][q]
    const float l = lsum + __shfl_xor(lsum, 32);
    if (!row_ok) return;
    const bool any = l > 0.f;
    const float inv = any ? 1.f / l : 0.f;
    const float lse = any ? m_run * p.scale + logf(l) : -INFINITY;
    const size_t row = ((size_t)b * p.Sq + row_pos) * p.Hq + row_head;
    if (S > 1) {
        const size_t rows_total = (size_t)p.B * p.Sq * p.Hq;
        if (lg == 0) p.lse_part[(size_t)split * rows_total + row] = lse;
        if (any) {
            float* orow = p.o_part + ((size_t)split * rows_total + row) * D + 4 * lg;
#pragma unroll
            for (int u = 0; u < DB; ++u)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    f32x4 w = {oacc[u][4 * j] * inv, oacc[u][4 * j + 1] * inv, oacc[u][4 * j + 2] * inv,
                               oacc[u][4 * j + 3] * inv};
                    *reinterpret_cast<f32x4*>(orow + 32 * u + 8 * j) = w;
                }
        }
    } else {
        if (lg == 0 && p.lse) p.lse[((size_t)b * p.Hq + row_head) * p.Sq + row_pos] = lse;
        bf16_t* orow = reinterpret_cast<bf16_t*>(p.o) + row * D + 4 * lg;
#pragma unroll
        for (int u = 0; u < DB; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                u32x2 w;
                w[0] = pack_bf16x2(oacc[u][4 * j] * inv, oacc[u][4 * j + 1] * inv);
                w[1] = pack_bf16x2(oacc[u][4 * j + 2] * inv, oacc[u][4 * j + 3] * inv);
                *reinterpret_cast<u32x2*>(orow + 32 * u + 8 * j) = w;
            }
    }
}

template <int D, int NWV>
hipError_t launch_prefill_m32(const FwdParams& p, dim3 grid, hipStream_t stream) {
    hipLaunchKernelGGL((attn_prefill_m32_kernel<D, NWV>), grid, dim3(64 * NWV), 0, stream, p);
    return hipGetLastError();
}

__global__ void tile_counters_reset_kernel(int* c, int n) {
    if ((int)threadIdx.x < n) c[threadIdx.x] = 0;
}
hipError_t launch_tile_counters_reset(int* counters, hipStream_t stream) {
    hipLaunchKernelGGL(tile_counters_reset_kernel, dim3(1), dim3(64), 0, stream, counters, NUM_XCD);
    return hipGetLastError();
}

hipError_t launch_v_to_f16t(const FwdParams& p, hipStream_t stream) {
    const dim3 grid(p.skp / 64, p.Hkv, p.B);
    const bf16_t* v = reinterpret_cast<const bf16_t*>(p.v);
    _Float16* vt = reinterpret_cast<_Float16*>(const_cast<void*>(p.vt));
    if (p.skp <= 0 || p.B <= 0 || p.Hkv <= 0) return hipSuccess;
    const int key = p.d_head * 1000 + p.vt_blk;
    switch (key) {
        case 64016: hipLaunchKernelGGL((v_to_f16t_kernel<64, 16>), grid, dim3(256), 0, stream, v, vt, p.seqlens_k, p.Sk, p.Hkv, p.skp); break;
        case 128016: hipLaunchKernelGGL((v_to_f16t_kernel<128, 16>), grid, dim3(256), 0, stream, v, vt, p.seqlens_k, p.Sk, p.Hkv, p.skp); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int D, int NWV, int MW>
hipError_t launch_prefill_pipe(const FwdParams& p, dim3 grid, hipStream_t stream) {
    hipLaunchKernelGGL((attn_prefill_pipe_kernel<D, NWV, MW>), grid, dim3(64 * NWV), 0, stream, p);
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
        // ablations: raised wave priority around the MFMA phases (measured slower),
        // and the software-pipelined loop (QK of tile n-1 overlaps softmax of n;
        // measured slower: both waves of a SIMD then compete in every phase)
        {DT_BF16, 128, 256, 64, 8, 1, PrefillTile<128, 8, 32>::LDS_BYTES, &launch_prefill<128, 8, 32, 1>, 1},
        {DT_BF16, 128, 256, 64, 8, 1, PrefillTile<128, 8, 32>::LDS_BYTES, &launch_prefill_pipe<128, 8, 32>, 1},
        {DT_BF16, 64, 256, 64, 8, 1, PrefillTile<64, 8, 32>::LDS_BYTES, &launch_prefill<64, 8, 32, 0>, 1},
        // two 4-wave workgroups per CU (independent barriers), kept as an ablation
        {DT_BF16, 128, 128, 64, 4, 1, PrefillTile<128, 4, 32>::LDS_BYTES, &launch_prefill<128, 4, 32, 0>, 1},
        {DT_BF16, 64, 128, 64, 4, 1, PrefillTile<64, 4, 32>::LDS_BYTES, &launch_prefill<64, 4, 32, 0>, 1},
        // persistent workgroups with per-XCD tile queues
        {DT_BF16, 128, 256, 64, 8, 1, PrefillTile<128, 8, 32>::LDS_BYTES, &launch_prefill<128, 8, 32, 0, 1>, 1, 0, 1},
        {DT_BF16, 128, 128, 64, 4, 1, PrefillTile<128, 4, 32>::LDS_BYTES, &launch_prefill<128, 4, 32, 0, 1>, 1, 0, 2},
        {DT_BF16, 64, 256, 64, 8, 1, PrefillTile<64, 8, 32>::LDS_BYTES, &launch_prefill<64, 8, 32, 0, 1>, 1, 0, 1},
        {DT_BF16, 64, 128, 64, 4, 1, PrefillTile<64, 4, 32>::LDS_BYTES, &launch_prefill<64, 4, 32, 0, 1>, 1, 0, 2},
        // 32x32x16 MFMA kernel on fp16 V^T from the V pre-pass
        {DT_BF16, 128, 256, 64, 8, 1, M32Tile<128, 8>::LDS_BYTES, &launch_prefill_m32<128, 8>, 1, 16},
        {DT_BF16, 128, 128, 64, 4, 1, M32Tile<128, 4>::LDS_BYTES, &launch_prefill_m32<128, 4>, 1, 16},
        {DT_BF16, 64, 256, 64, 8, 1, M32Tile<64, 8>::LDS_BYTES, &launch_prefill_m32<64, 8>, 1, 16},
        {DT_BF16, 64, 128, 64, 4, 1, M32Tile<64, 4>::LDS_BYTES, &launch_prefill_m32<64, 4>, 1, 16},
        {0, 0, 0, 0, 0, 0, 0, nullptr, 0},
    };
    return v;
}

}  // namespace tpa
