// attn_fwd.hip -- gfx950 (MI355X) flash-attention forward kernels.
//
// KA  attn_fwd_kernel     one workgroup per (query block, grid head x split,
//                         batch): skips key blocks outside the causal / window
//                         range, runs S = K Q^T on MFMA, the online softmax in
//                         fp32, and O += V^T P^T on MFMA; writes O and lse, or
//                         the split partial (O_s, lse_s).
// (the log-sum-exp combine of split partials lives in attn_decode.hip)
//
// Citations:
//   [FA-tiling]  "分块策略与调度" (FlashAttention tiling strategy and scheduling)
//   [Occupancy]  "The Occupancy Awakening: Rewriting a Flash Attention Kernel
//                for Blackwell's 188 SMs"
//
// Layout of the matrix-core work (wave64, 16x16 MFMA tiles). Every product is
// computed transposed, with the query rows on the MFMA N axis:
//   S^T[key][query] = K . Q^T      A = K tile (LDS), B = Q^T (registers)
//   O^T[d][query]  += V^T . P^T    A = V^T tile (LDS, stored transposed),
//                                  B = P^T (the S^T accumulators, in place)
// so lane (i = lane % 16, g = lane / 16) owns query column i and, of every
// 16x16 accumulator, the four rows 4g..4g+3. The softmax statistics of a query
// row then live in the four lanes i, i+16, i+32, i+48: the row max needs two
// cross-lane steps, the rescale of O is a per-lane scalar, and P feeds the
// second product without leaving registers. The reduction index of each MFMA
// (d for the first product, key for the second) is assigned to (g, element)
// the same way on the A and B side, which is all an MFMA contraction needs.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_device.h"
#include "attn_kernels.h"
#include "attn_plan.h"

namespace tpa {

// ---------------------------------------------------------------------------
// KA: forward kernel.
//   T      element type (float or bf16_t)
//   D      head dim
//   BM,BN  query rows / key rows per tile
//   WM,WN  waves along rows and along keys (WN > 1 splits each key tile
//          between waves and merges their partial softmax states at the end)
// ---------------------------------------------------------------------------
template <class T, int D, int BM, int BN, int WM, int WN>
struct FwdTile {
    static constexpr bool BF = std::is_same<T, bf16_t>::value;
    static constexpr int NW = WM * WN, NTHR = 64 * NW;
    static constexpr int MW = BM / WM, NQ = MW / 16;  // rows per wave, 16-row column blocks
    static constexpr int NK = BN / WN, NT = NK / 16;  // keys per wave, 16-key sub-tiles
    static constexpr int ESZ = sizeof(T);
    static constexpr int DL = D / 4;                  // d elements owned by one lane group
    static constexpr int CE = 16 / ESZ;               // elements per 16-byte chunk
    static constexpr int KST = D + CE;                // K tile row stride (elements)
    // V^T tile row stride (elements): padded for bf16; for fp32 unpadded, with
    // the 16-byte key slot of row d XOR-swizzled by vswz(d) instead
    static constexpr int VST = BF ? BN + CE : BN;
    static constexpr int CPR = D / CE;                // 16-byte chunks per row
    static constexpr int ITEMS = (BN / 4) * CPR / NTHR;  // (4 rows x chunk) items per thread
    static constexpr int K_BYTES = BN * KST * ESZ;
    static constexpr int V_BYTES = D * VST * ESZ;
    static constexpr int TILE_BYTES = K_BYTES + V_BYTES;
    // split-key merge area: O^T accumulators + (m, l) of every wave
    static constexpr int RED_BYTES = WN > 1 ? NW * NQ * (D / 16) * 4 * 64 * 4 + NW * NQ * 64 * 8 : 0;
    static constexpr int LDS_BYTES = TILE_BYTES > RED_BYTES ? TILE_BYTES : RED_BYTES;
    static_assert(MW % 16 == 0, "rows per wave must be a multiple of 16");
    static_assert(NK % (BF ? 32 : 16) == 0, "keys per wave must fill the PV contraction");
    static_assert(ITEMS >= 1 && (BN / 4) * CPR % NTHR == 0, "tile load must divide evenly");
    // fp32 V^T: slot of keys 4j..4j+3 in row d is j ^ vswz(d). The tile store
    // writes rows d = 4c + e for 16 consecutive c (one key slot j) per 16 lanes,
    // the P.V read rows d = 16u + i for 16 consecutive i: both see 16 distinct
    // slots, i.e. distinct LDS banks (a row of 64 keys spans the 64 banks once).
    // (masked to the row's BN / 4 slots when a row has fewer than 16)
    static constexpr int VSLOTS = BN / 4 < 16 ? BN / 4 : 16;
    static __device__ __forceinline__ int vswz(int d) { return (d ^ (d >> 4)) & (VSLOTS - 1); }
};

template <class T, int D, int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(64 * WM * WN)
attn_fwd_kernel(FwdParams p) {
    using C = FwdTile<T, D, BM, BN, WM, WN>;
    constexpr bool BF = C::BF;
    constexpr int NQ = C::NQ, NT = C::NT, NK = C::NK, DL = C::DL, CE = C::CE;
    constexpr int KST = C::KST, VST = C::VST, CPR = C::CPR, ITEMS = C::ITEMS;

    __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];
    T* Ks = reinterpret_cast<T*>(smem);
    T* Vt = reinterpret_cast<T*>(smem + C::K_BYTES);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave % WM, wn = wave / WM;
    const int li = lane & 15, lg = lane >> 4;

    // ---- tile coordinates ([FA-tiling] §4.2 grid; §4.4 heaviest-first order)
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

    // ---- key-block range of this tile and of this split ([FA-tiling] §3.2, §5.3)
    int n_lo, n_hi;
    n_block_range(p.Sq, Skb, G, p.pack, p.causal, p.window_left, BM, BN, m_block, &n_lo, &n_hi);
    const int S_b = splits_for(imax(0, n_hi - n_lo), p.num_splits, p.chunk_blocks);
    int s_lo = 0, s_hi = 0;
    if (split < S_b) split_range(n_lo, n_hi, split, S_b, &s_lo, &s_hi);
    const bool has_work = s_hi > s_lo;

    // ---- this lane's query rows: visible key interval [row_lo, row_hi]
    int row_pos[NQ], row_head[NQ], row_lo[NQ], row_hi[NQ];
    bool row_ok[NQ];
    int wlo = -0x7fffffff, whi = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int r = m_block * BM + wm * C::MW + 16 * q + li;
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
    // bounds over the whole wave: a key slice inside [wlo, whi] needs no mask
    wlo = row16_imax(wlo);  // lane groups g hold the same rows
    whi = row16_imin(whi);

    // ---- Q^T fragments: lane group g holds d in [g*DL, (g+1)*DL) of its row
    constexpr int QV = DL * (int)sizeof(T) / 16;  // 16-byte vectors per lane per row
    // every load unconditional (a row the tile does not own points at row 0 of
    // the batch, which exists, and is zeroed by a select afterwards): a load
    // inside the condition compiled to a branch per load and a wait
    u32x4 qf[NQ][QV];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const T* qrow = reinterpret_cast<const T*>(p.q) +
                        (((size_t)b * p.Sq + row_pos[q]) * p.Hq + row_head[q]) * D + lg * DL;
        const bool use = row_ok[q] && has_work;
#pragma unroll
        for (int c = 0; c < QV; ++c) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(qrow + c * CE);
            const u32x4 z = {0u, 0u, 0u, 0u};
            qf[q][c] = use ? x : z;
        }
    }

    // ---- running softmax state and output accumulators
    f32x4 oacc[D / 16][NQ];
    float m_run[NQ], l_run[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        m_run[q] = -INFINITY;
        l_run[q] = 0.f;
#pragma unroll
        for (int u = 0; u < D / 16; ++u) oacc[u][q] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const float sl2 = p.scale_log2;

    // ---- K/V tile staging: thread item = (group of 4 key rows, 16-byte chunk)
    const T* kbase = reinterpret_cast<const T*>(p.k) + ((size_t)b * p.Sk * p.Hkv + hkv) * D;
    const T* vbase = reinterpret_cast<const T*>(p.v) + ((size_t)b * p.Sk * p.Hkv + hkv) * D;
    const size_t kv_stride = (size_t)p.Hkv * D;
    u32x4 kst[ITEMS][4], vst[ITEMS][4];

    // buffer loads over the tile's rows that exist: rows at or past Skb read as
    // zeros, with no branch per load
    const uint32_t row_bytes = (uint32_t)(kv_stride * C::ESZ);
    auto load_tile = [&](int n) {
        const uint32_t valid = (uint32_t)imax(0, imin(BN, Skb - n * BN));
        const rsrc_t rk = make_rsrc_u(kbase + (size_t)n * BN * kv_stride, valid * row_bytes);
        const rsrc_t rv = make_rsrc_u(vbase + (size_t)n * BN * kv_stride, valid * row_bytes);
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const int item = tid + it * C::NTHR;
            const int c = item % CPR, rg = item / CPR;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t off = (uint32_t)(4 * rg + r) * row_bytes + 16 * c;
                // decode and verify tiles (one query block per head) read each
                // K/V row once: non-temporal; prefill tiles share them in L2
                if constexpr (BM <= 32) {
                    kst[it][r] = buf_load16_nt(rk, off);
                    vst[it][r] = buf_load16_nt(rv, off);
                } else {
                    kst[it][r] = buf_load16(rk, off);
                    vst[it][r] = buf_load16(rv, off);
                }
            }
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const int item = tid + it * C::NTHR;
            const int c = item % CPR, rg = item / CPR;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                *reinterpret_cast<u32x4*>(Ks + (4 * rg + r) * KST + c * CE) = kst[it][r];
            if constexpr (BF) {
                // chunk c holds d = 8c..8c+7 of rows 4rg..4rg+3; write V^T[d][4rg..4rg+3]
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int w = e >> 1;
                    uint32_t a0 = vst[it][0][w], a1 = vst[it][1][w];
                    uint32_t a2 = vst[it][2][w], a3 = vst[it][3][w];
                    u32x2 pr;
                    if (e & 1) {
                        pr[0] = (a0 >> 16) | (a1 & 0xffff0000u);
                        pr[1] = (a2 >> 16) | (a3 & 0xffff0000u);
                    } else {
                        pr[0] = (a0 & 0xffffu) | (a1 << 16);
                        pr[1] = (a2 & 0xffffu) | (a3 << 16);
                    }
                    *reinterpret_cast<u32x2*>(Vt + (8 * c + e) * VST + 4 * rg) = pr;
                }
            } else {
                // chunk c holds d = 4c..4c+3 of rows 4rg..4rg+3
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    u32x4 col = {vst[it][0][e], vst[it][1][e], vst[it][2][e], vst[it][3][e]};
                    const int d = 4 * c + e;
                    *reinterpret_cast<u32x4*>(Vt + d * VST + 4 * (rg ^ C::vswz(d))) = col;
                }
            }
        }
    };

    // ---- main loop over this split's key blocks, last block first so that a
    // masked diagonal block is met before the full ones ([FA-tiling] §3.1)
    if (s_hi > s_lo) load_tile(s_hi - 1);
    for (int n = s_hi - 1; n >= s_lo; --n) {
        __syncthreads();
        store_tile();
        __syncthreads();
        if (n > s_lo) load_tile(n - 1);

        const int kw0 = wn * NK;  // first key of this wave's slice within the tile
        // S^T = K . Q^T
        f32x4 sacc[NT][NQ];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int q = 0; q < NQ; ++q) sacc[t][q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < QV; ++c) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const u32x4 kf = *reinterpret_cast<const u32x4*>(
                    Ks + (kw0 + 16 * t + li) * KST + lg * DL + c * CE);
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    if constexpr (BF) {
                        sacc[t][q] = mfma_bf16(kf, qf[q][c], sacc[t][q]);
                    } else {
                        // whole-vector casts: a bit_cast of one vector element is
                        // not reliable with this compiler
                        const f32x4 kv = __builtin_bit_cast(f32x4, kf);
                        const f32x4 qv = __builtin_bit_cast(f32x4, qf[q][c]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) sacc[t][q] = mfma_f32(kv[e], qv[e], sacc[t][q]);
                    }
                }
            }
        }

        // element mask, only where the slice is not inside every row's interval
        const int key0 = n * BN + kw0;
        const bool full = key0 >= wlo && key0 + NK - 1 <= whi;
        if (!full) {
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int q = 0; q < NQ; ++q)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int key = key0 + 16 * t + 4 * lg + r;
                        if (key < row_lo[q] || key > row_hi[q]) sacc[t][q][r] = -INFINITY;
                    }
        }

        // online softmax (fp32): running sum l and O against a reference max m
        // that moves lazily, only when the tile's row max exceeds it by more than
        // 2^LAZY (log2 units): P <= 2^LAZY then, and the rescale of O (a read,
        // multiply and write of every accumulator) runs on few tiles. l and O
        // share the reference, so O / l and lse = m * scale + ln l are exact.
        constexpr float LAZY = 8.f;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            float mx = -INFINITY;
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) mx = vmax(mx, sacc[t][q][r]);
            mx = xor_max(mx);
            const bool raise = m_run[q] == -INFINITY ? mx != -INFINITY : (mx - m_run[q]) * sl2 > LAZY;
            if (__builtin_amdgcn_ballot_w64(raise) != 0) {
                const float alpha = !raise ? 1.f : (m_run[q] == -INFINITY ? 0.f : fast_exp2((m_run[q] - mx) * sl2));
                if (raise) m_run[q] = mx;
                l_run[q] *= alpha;
#pragma unroll
                for (int u = 0; u < D / 16; ++u) oacc[u][q] *= alpha;
            }
            const float neg = m_run[q] == -INFINITY ? 0.f : -m_run[q] * sl2;
            float rs = 0.f;
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float pv = fast_exp2(fmaf(sacc[t][q][r], sl2, neg));
                    sacc[t][q][r] = pv;
                    rs += pv;
                }
            l_run[q] += rs;
        }

        // O^T += V^T . P^T. On the bf16 path P enters the MFMA as two bf16
        // parts, P = P_hi + P_lo (P_lo = bf16(P - P_hi)), so that P carries about
        // 16 significant bits: rounding P to one bf16 alone costs up to 2^-9 of
        // every term and breaks a 1e-2 relative error bar on rows with few keys.
        if constexpr (BF) {
#pragma unroll
            for (int pp = 0; pp < NT / 2; ++pp) {
                u32x4 pf_hi[NQ], pf_lo[NQ];
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        const float a = sacc[2 * pp + (h >> 1)][q][2 * (h & 1)];
                        const float c = sacc[2 * pp + (h >> 1)][q][2 * (h & 1) + 1];
                        const uint32_t hi = pack_bf16x2(a, c);
                        pf_hi[q][h] = hi;
                        pf_lo[q][h] = pack_bf16x2(a - __uint_as_float(hi << 16),
                                                  c - __uint_as_float(hi & 0xffff0000u));
                    }
                }
#pragma unroll
                for (int u = 0; u < D / 16; ++u) {
                    const T* vrow = Vt + (16 * u + li) * VST + kw0 + 32 * pp + 4 * lg;
                    const u32x2 lo = *reinterpret_cast<const u32x2*>(vrow);
                    const u32x2 hi = *reinterpret_cast<const u32x2*>(vrow + 16);
                    const u32x4 vf = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
                    for (int q = 0; q < NQ; ++q) {
                        oacc[u][q] = mfma_bf16(vf, pf_hi[q], oacc[u][q]);
                        oacc[u][q] = mfma_bf16(vf, pf_lo[q], oacc[u][q]);
                    }
                }
            }
        } else {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
#pragma unroll
                for (int u = 0; u < D / 16; ++u) {
                    const int d = 16 * u + li;
                    const f32x4 vf = *reinterpret_cast<const f32x4*>(
                        Vt + d * VST + 4 * (((kw0 + 16 * t + 4 * lg) >> 2) ^ C::vswz(d)));
#pragma unroll
                    for (int r = 0; r < 4; ++r)
#pragma unroll
                        for (int q = 0; q < NQ; ++q)
                            oacc[u][q] = mfma_f32(vf[r], sacc[t][q][r], oacc[u][q]);
                }
            }
        }
    }

    // ---- row sums across the four lane groups
#pragma unroll
    for (int q = 0; q < NQ; ++q) l_run[q] = xor_sum(l_run[q]);

    // ---- merge the key-split waves (log-sum-exp merge inside the workgroup)
    if constexpr (WN > 1) {
        __syncthreads();
        float* red = reinterpret_cast<float*>(smem);
        constexpr int OV = (D / 16) * 4;  // O^T values per lane per column block
        float* red_o = red;                                  // [NW][NQ][OV][64]
        float* red_ml = red + C::NW * NQ * OV * 64;          // [NW][NQ][2][64]
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
#pragma unroll
            for (int u = 0; u < D / 16; ++u)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    red_o[((wave * NQ + q) * OV + u * 4 + r) * 64 + lane] = oacc[u][q][r];
            red_ml[((wave * NQ + q) * 2 + 0) * 64 + lane] = m_run[q];
            red_ml[((wave * NQ + q) * 2 + 1) * 64 + lane] = l_run[q];
        }
        __syncthreads();
        if (wn != 0) return;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            float mw[WN], lw[WN];
            float mstar = -INFINITY;
#pragma unroll
            for (int w = 0; w < WN; ++w) {
                const int ww = w * WM + wm;
                mw[w] = red_ml[((ww * NQ + q) * 2 + 0) * 64 + lane];
                lw[w] = red_ml[((ww * NQ + q) * 2 + 1) * 64 + lane];
                mstar = vmax(mstar, mw[w]);
            }
            const float muse = mstar == -INFINITY ? 0.f : mstar;
            float l = 0.f;
#pragma unroll
            for (int u = 0; u < D / 16; ++u) oacc[u][q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w = 0; w < WN; ++w) {
                const int ww = w * WM + wm;
                const float a = fast_exp2((mw[w] - muse) * sl2);
                l += a * lw[w];
#pragma unroll
                for (int u = 0; u < D / 16; ++u)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        oacc[u][q][r] += a * red_o[((ww * NQ + q) * OV + u * 4 + r) * 64 + lane];
            }
            m_run[q] = mstar;
            l_run[q] = l;
        }
    }

    // ---- epilogue: normalise; write O and lse, or the split partial
    const bool split_out = p.num_splits > 1;
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
                for (int u = 0; u < D / 16; ++u) {
                    f32x4 v = oacc[u][q] * inv;
                    *reinterpret_cast<f32x4*>(orow + 16 * u) = v;
                }
            }
        } else {
            if (lg == 0 && p.lse)
                p.lse[((size_t)b * p.Hq + row_head[q]) * p.Sq + row_pos[q]] = lse;
            if constexpr (BF) {
                bf16_t* orow = reinterpret_cast<bf16_t*>(p.o) + row * D + 4 * lg;
#pragma unroll
                for (int u = 0; u < D / 16; ++u) {
                    u32x2 w;
                    w[0] = pack_bf16x2(oacc[u][q][0] * inv, oacc[u][q][1] * inv);
                    w[1] = pack_bf16x2(oacc[u][q][2] * inv, oacc[u][q][3] * inv);
                    *reinterpret_cast<u32x2*>(orow + 16 * u) = w;
                }
            } else {
                float* orow = reinterpret_cast<float*>(p.o) + row * D + 4 * lg;
#pragma unroll
                for (int u = 0; u < D / 16; ++u)
                    *reinterpret_cast<f32x4*>(orow + 16 * u) = oacc[u][q] * inv;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// launchers and the variant table
// ---------------------------------------------------------------------------
template <class T, int D, int BM, int BN, int WM, int WN>
hipError_t launch_fwd(const FwdParams& p, dim3 grid, hipStream_t stream) {
    hipLaunchKernelGGL((attn_fwd_kernel<T, D, BM, BN, WM, WN>), grid, dim3(64 * WM * WN), 0, stream, p);
    return hipGetLastError();
}

#define TPA_VARIANT(T, DT, D, BM, BN, WM, WN) \
    {DT, D, BM, BN, WM, WN, FwdTile<T, D, BM, BN, WM, WN>::LDS_BYTES, &launch_fwd<T, D, BM, BN, WM, WN>, 0}

// Tile table for gfx950: 64-wide waves, 160 KB LDS per CU. "Decode" tiles
// (16 rows, keys split across 4 waves) serve a handful of (packed) query rows;
// "prefill" tiles give each of 4 waves its own 16..32 rows.
static const FwdVariant kVariants[] = {
    // bf16 prefill: 128 rows (4 waves x 32), 64-key tiles
    TPA_VARIANT(bf16_t, DT_BF16, 128, 128, 64, 4, 1),
    TPA_VARIANT(bf16_t, DT_BF16, 64, 128, 128, 4, 1),
    // bf16 decode: 16 rows, 128-key tiles split over 4 waves
    TPA_VARIANT(bf16_t, DT_BF16, 128, 16, 128, 1, 4),
    TPA_VARIANT(bf16_t, DT_BF16, 64, 16, 128, 1, 4),
    // fp32 prefill: 64 rows (4 waves x 16), 32-key tiles
    TPA_VARIANT(float, DT_FP32, 128, 64, 32, 4, 1),
    TPA_VARIANT(float, DT_FP32, 64, 64, 64, 4, 1),
    // fp32 "verify" tiles for 17..32 rows: 2 waves x 16 rows, keys split over 2 waves
    // (a 64-row tile would leave half its waves on padding rows)
    TPA_VARIANT(float, DT_FP32, 128, 32, 64, 2, 2),
    TPA_VARIANT(float, DT_FP32, 64, 32, 64, 2, 2),
    // the same rows with 128-key tiles over 4 key waves (8 waves, two per SIMD)
    TPA_VARIANT(float, DT_FP32, 128, 32, 128, 2, 4),
    TPA_VARIANT(float, DT_FP32, 64, 32, 128, 2, 4),
    // fp32 decode: 16 rows, 64-key tiles split over 4 waves
    TPA_VARIANT(float, DT_FP32, 128, 16, 64, 1, 4),
    TPA_VARIANT(float, DT_FP32, 64, 16, 64, 1, 4),
    {0, 0, 0, 0, 0, 0, 0, nullptr, 0},
};

const FwdVariant* fwd_variants() { return kVariants; }

}  // namespace tpa
