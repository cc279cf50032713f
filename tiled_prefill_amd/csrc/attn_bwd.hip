// attn_bwd.hip -- gfx950 (MI355X) flash-attention backward kernels.
//
//   bwd_pre_kernel      per query row: the row sum D = <dO, O>, lse2 = lse *
//                       log2(e) (+inf where the row sees no key), and (atomic
//                       form) zero for the row's fp32 dQ accumulator.
//   attn_bwd_kernel     one workgroup per (key block, KV head, batch): key blocks
//                       outside, the query blocks that see them inside
//                       ([FA-tiling] §3.4, get_m_block_min_max). Its K and V rows
//                       stay in registers, and so do the dK and dV accumulators
//                       of those rows, summed over the G query heads of the
//                       group; each query block recomputes S and P from lse,
//                       then dV += P^T dO and dK += dS^T Q on MFMA.
//   attn_bwd_dq_kernel  one workgroup per (query block, query head, batch),
//                       looping over the key blocks that query block sees:
//                       recomputes S and dP and forms dQ = dS K on MFMA.
//   attn_bwd_dkdv_dma_kernel, attn_bwd_dq_dma_kernel
//                       the bf16 forms of the two kernels above (the default):
//                       their tiles (Q, dO, lse2, D; or K, V) are DMA'd into
//                       double-buffered LDS one block ahead, work proceeds in
//                       32-row / 32-key halves, and both run on XCD-aware
//                       one-dimensional grids so that the blocks of a head share
//                       one XCD's L2.
//   (atomic form)       the pages' single pass ([FA-tiling] §4.6: Q, dO and an
//                       fp32 dQ accumulator are the backward's working set):
//                       attn_bwd_kernel<.., ATOMIC> also forms dQ = dS K per
//                       (query block, key block) pair and adds it to the
//                       accumulator with fp32 atomics; bwd_post_kernel scales it.
//                       On this GPU those atomics cost about three times all of
//                       the matrix work (6.6 ms vs 2.2 ms without them on the
//                       causal 8192 x 32-head workload), so the default recomputes
//                       S and dP in the dQ kernel instead (40% more matrix work,
//                       no atomics, the same bits on every run).
//
// The pages print no gradient formulas; the kernels implement the chain rule
// through the softmax: dP = dO V^T, D_i = sum_j P_ij dP_ij = <dO_i, O_i>,
// dS = P (dP - D), dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO.
//
// Citations:
//   [FA-tiling]  "分块策略与调度" (FlashAttention tiling strategy and scheduling)
//
// Matrix-core layout of attn_bwd_kernel (wave64, 16x16 MFMA tiles; lane =
// 16 lg + li). Each wave owns NKW keys of the workgroup's key block. Per query
// block of BM = 64 rows:
//   S  [q][key]  = Q . K^T     A = Q rows (LDS), B = K rows (registers)
//   dP [q][key]  = dO . V^T    A = dO rows (LDS), B = V rows (registers)
// so lane (li, lg) holds key li and query rows 4 lg .. 4 lg + 3 of every 16x16
// block, which is the B-operand layout of the two products that contract over
// query rows:
//   dV^T [d][key] += dO^T . P    A = dO columns (LDS transpose reads), B = P
//   dK^T [d][key] += Q^T . dS    A = Q columns, B = dS
// In the atomic form dS^T then goes to LDS, and after a barrier each wave
// computes 16 rows of
//   dQ [q][d] = dS . K           A = dS (transpose reads of dS^T), B = K columns
// For fp32 the same products run on the 16x16x4 fp32 MFMA with per-lane LDS
// reads in place of the transpose reads.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_device.h"
#include "attn_kernels.h"
#include "attn_plan.h"

namespace tpa {

template <class T, int D, int NKW, bool ATOMIC = false>
struct BwdTile {
    static constexpr bool BF = std::is_same<T, bf16_t>::value;
    static constexpr int NW = 4, NTHR = 64 * NW;
    static constexpr int BM = 16 * NW;          // query rows per block (16 per wave in dQ)
    static constexpr int BN = NW * NKW;         // keys per workgroup
    static constexpr int NT = NKW / 16;         // 16-key blocks per wave
    static constexpr int NQB = BM / 16;         // 16-row query blocks
    static constexpr int ESZ = sizeof(T);
    static constexpr int CE = 16 / ESZ;         // elements per 16-byte chunk
    static constexpr int QST = D + CE;          // row pitch of the Q, dO and K tiles (elements)
    static constexpr int SST = BM + CE;         // row pitch of the dS^T tile (elements)
    static constexpr int CPR = D / CE;          // 16-byte chunks per row
    static constexpr int QITEMS = BM * CPR / NTHR;
    static constexpr int KITEMS = BN * CPR / NTHR;
    static constexpr int DL = D / 4;            // fp32: d elements of one lane group
    static constexpr int KC = BF ? D / 32 : DL / 4;  // register chunks per key row
    static constexpr int Q_BYTES = BM * QST * ESZ;
    // the K tile and the dS^T tile are needed only when dQ is accumulated here
    static constexpr int K_BYTES = ATOMIC ? BN * QST * ESZ : 0;
    // (bf16: dS^T as hi and lo tiles, one after the other)
    static constexpr int S_BYTES = ATOMIC ? (BF ? 2 : 1) * BN * SST * ESZ : 0;
    static constexpr int LDS_BYTES = 2 * Q_BYTES + K_BYTES + S_BYTES + 2 * BM * 4;
    static_assert(NKW % 16 == 0 && (!BF || BN % 32 == 0), "key slice must fill the MFMA");
    static_assert(QITEMS >= 1 && BM * CPR % NTHR == 0, "Q tile load must divide evenly");
    static_assert(KITEMS >= 1 && BN * CPR % NTHR == 0, "K tile load must divide evenly");
    // element offset of register chunk c of lane group lg within a row
    static __device__ __forceinline__ int chunk_off(int c, int lg) {
        return BF ? 32 * c + 8 * lg : lg * DL + 4 * c;
    }
};

// ---------------------------------------------------------------------------
// pre-pass: D = <dO, O> per row (WITH_D), lse in log2 units, zero dQ accumulator
// ---------------------------------------------------------------------------
template <class T, int D, bool WITH_D = true>
__global__ void __launch_bounds__(256) bwd_pre_kernel(BwdParams p) {
    constexpr int CE = 16 / (int)sizeof(T);
    constexpr int TPR = D / CE;  // threads per row (8, 16 or 32; divides 64)
    constexpr int RPB = 256 / TPR;
    const long long rows = (long long)p.B * p.Sq * p.Hq;
    const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
    const int c = threadIdx.x % TPR;
    float dot = 0.f;
    if (WITH_D && row < rows) {
        const u32x4 ov = *reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(p.o) + row * D + c * CE);
        const u32x4 gv = *reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(p.dout) + row * D + c * CE);
        if constexpr (std::is_same<T, bf16_t>::value) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dot += __uint_as_float(ov[e] << 16) * __uint_as_float(gv[e] << 16);
                dot += __uint_as_float(ov[e] & 0xffff0000u) * __uint_as_float(gv[e] & 0xffff0000u);
            }
        } else {
            const f32x4 of = __builtin_bit_cast(f32x4, ov), gf = __builtin_bit_cast(f32x4, gv);
#pragma unroll
            for (int e = 0; e < 4; ++e) dot += of[e] * gf[e];
        }
        if (p.dq_acc) {
            float* acc = p.dq_acc + row * D + c * CE;
#pragma unroll
            for (int e = 0; e < CE; e += 4) *reinterpret_cast<f32x4*>(acc + e) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
#pragma unroll
    for (int off = TPR / 2; off >= 1; off >>= 1) dot += __shfl_xor(dot, off, 64);
    if (row < rows && c == 0) {
        const int h = (int)(row % p.Hq);
        const int i = (int)((row / p.Hq) % p.Sq);
        const int b = (int)(row / ((long long)p.Hq * p.Sq));
        const size_t idx = ((size_t)b * p.Hq + h) * p.Sq + i;
        const float l = p.lse[idx];
        if (WITH_D) p.dsum[idx] = dot;
        p.lse2[idx] = l == -INFINITY ? INFINITY : l * 1.4426950408889634f;
    }
}

// ---------------------------------------------------------------------------
// post-pass: dQ = scale * accumulator
// ---------------------------------------------------------------------------
template <class T>
__global__ void __launch_bounds__(256) bwd_post_kernel(BwdParams p, long long n4) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    const f32x4 a = *reinterpret_cast<const f32x4*>(p.dq_acc + 4 * i) * p.scale;
    if constexpr (std::is_same<T, bf16_t>::value) {
        u32x2 w = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
        *reinterpret_cast<u32x2*>(reinterpret_cast<bf16_t*>(p.dq) + 4 * i) = w;
    } else {
        *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.dq) + 4 * i) = a;
    }
}

// ---------------------------------------------------------------------------
// main kernel
// ---------------------------------------------------------------------------
template <class T, int D, int NKW, int OCC, bool ATOMIC>
__global__ void __launch_bounds__(256, OCC) attn_bwd_kernel(BwdParams p) {
    using C = BwdTile<T, D, NKW, ATOMIC>;
    constexpr bool BF = C::BF;
    constexpr int BM = C::BM, BN = C::BN, NT = C::NT, NQB = C::NQB, CE = C::CE;
    constexpr int QST = C::QST, SST = C::SST, CPR = C::CPR, KC = C::KC;

    __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];
    T* Qs = reinterpret_cast<T*>(smem);
    T* dOs = reinterpret_cast<T*>(smem + C::Q_BYTES);
    T* Ks = reinterpret_cast<T*>(smem + 2 * C::Q_BYTES);
    T* dSt = reinterpret_cast<T*>(smem + 2 * C::Q_BYTES + C::K_BYTES);
    float* ls2 = reinterpret_cast<float*>(smem + 2 * C::Q_BYTES + C::K_BYTES + C::S_BYTES);
    float* lds_dsum = ls2 + BM;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;

    // ---- work unit: key block nb of KV head hkv in batch b. Key blocks run
    // slowest, so the heaviest causal blocks (lowest nb) of every head go
    // first; consecutive workgroups take consecutive heads, which deals a head
    // to the same XCD (workgroup i runs on XCD i % 8) when Hkv % 8 == 0.
    const int bid = blockIdx.x;
    const int hkv = bid % p.Hkv;
    const int b = (bid / p.Hkv) % p.B;
    const int nb = bid / (p.Hkv * p.B);
    const int G = p.G, Sq = p.Sq, Sk = p.Sk;
    const int delta = Sk - Sq;
    const int key0 = nb * BN;
    const int kw0 = wave * NKW;  // this wave's keys within the block

    int m_lo, m_hi;
    m_block_range(Sq, Sk, p.causal, p.window_left, BM, BN, nb, &m_lo, &m_hi);
    const int nm = imax(0, m_hi - m_lo);
    const int total = G * nm;

    const T* qg = reinterpret_cast<const T*>(p.q);
    const T* dog = reinterpret_cast<const T*>(p.dout);
    const size_t kv_stride = (size_t)p.Hkv * D;
    const T* kbase = reinterpret_cast<const T*>(p.k) + ((size_t)b * Sk * p.Hkv + hkv) * D;
    const T* vbase = reinterpret_cast<const T*>(p.v) + ((size_t)b * Sk * p.Hkv + hkv) * D;

    // ---- K and V rows of this wave as MFMA B fragments, K tile in LDS for dQ
    u32x4 kf[NT][KC], vf[NT][KC];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int key = key0 + kw0 + 16 * t + li;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            u32x4 z = {0u, 0u, 0u, 0u};
            kf[t][c] = z;
            vf[t][c] = z;
            if (key < Sk && total > 0) {
                kf[t][c] = *reinterpret_cast<const u32x4*>(kbase + key * kv_stride + C::chunk_off(c, lg));
                vf[t][c] = *reinterpret_cast<const u32x4*>(vbase + key * kv_stride + C::chunk_off(c, lg));
            }
        }
    }
    if (ATOMIC && total > 0) {
#pragma unroll
        for (int it = 0; it < C::KITEMS; ++it) {
            const int item = tid + it * C::NTHR;
            const int r = item / CPR, c = item % CPR;
            const int key = key0 + r;
            u32x4 val = {0u, 0u, 0u, 0u};
            if (key < Sk) val = *reinterpret_cast<const u32x4*>(kbase + key * kv_stride + c * CE);
            *reinterpret_cast<u32x4*>(Ks + r * QST + c * CE) = val;
        }
    }

    f32x4 dvT[D / 16][NT], dkT[D / 16][NT];
#pragma unroll
    for (int u = 0; u < D / 16; ++u)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            dvT[u][t] = f32x4{0.f, 0.f, 0.f, 0.f};
            dkT[u][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

    // ---- staging of one query block (rows m*BM.. of head hq) through registers
    u32x4 qpre[C::QITEMS], dopre[C::QITEMS];
    float lpre = INFINITY, dpre = 0.f;
    auto load_block = [&](int it) {
        const int g = it / nm, m = m_lo + it % nm;
        const int hq = hkv * G + g;
#pragma unroll
        for (int i = 0; i < C::QITEMS; ++i) {
            const int item = tid + i * C::NTHR;
            const int r = item / CPR, c = item % CPR;
            const int pos = m * BM + r;
            u32x4 z = {0u, 0u, 0u, 0u};
            qpre[i] = z;
            dopre[i] = z;
            if (pos < Sq) {
                const size_t off = (((size_t)b * Sq + pos) * p.Hq + hq) * D + c * CE;
                qpre[i] = *reinterpret_cast<const u32x4*>(qg + off);
                dopre[i] = *reinterpret_cast<const u32x4*>(dog + off);
            }
        }
        if (tid < BM) {
            const int pos = m * BM + tid;
            lpre = INFINITY;
            dpre = 0.f;
            if (pos < Sq) {
                const size_t idx = ((size_t)b * p.Hq + hq) * Sq + pos;
                lpre = p.lse2[idx];
                dpre = p.dsum[idx];
            }
        }
    };
    auto store_block = [&]() {
#pragma unroll
        for (int i = 0; i < C::QITEMS; ++i) {
            const int item = tid + i * C::NTHR;
            const int r = item / CPR, c = item % CPR;
            *reinterpret_cast<u32x4*>(Qs + r * QST + c * CE) = qpre[i];
            *reinterpret_cast<u32x4*>(dOs + r * QST + c * CE) = dopre[i];
        }
        if (tid < BM) {
            ls2[tid] = lpre;
            lds_dsum[tid] = dpre;
        }
    };

    const float sl2 = p.scale_log2;
    if (total > 0) load_block(0);
    for (int it = 0; it < total; ++it) {
        const int g = it / nm, m = m_lo + it % nm;
        const int hq = hkv * G + g;
        __syncthreads();  // every wave is done with the previous block's tiles
        store_block();
        __syncthreads();
        if (it + 1 < total) load_block(it + 1);

        // S = Q K^T and dP = dO V^T
        f32x4 sacc[NQB][NT], pacc[NQB][NT];
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                sacc[qb][t] = f32x4{0.f, 0.f, 0.f, 0.f};
                pacc[qb][t] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
        for (int c = 0; c < KC; ++c) {
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) {
                const u32x4 qa = *reinterpret_cast<const u32x4*>(Qs + (16 * qb + li) * QST + C::chunk_off(c, lg));
                const u32x4 da = *reinterpret_cast<const u32x4*>(dOs + (16 * qb + li) * QST + C::chunk_off(c, lg));
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    if constexpr (BF) {
                        sacc[qb][t] = mfma_bf16(qa, kf[t][c], sacc[qb][t]);
                        pacc[qb][t] = mfma_bf16(da, vf[t][c], pacc[qb][t]);
                    } else {
                        const f32x4 qv = __builtin_bit_cast(f32x4, qa), dv = __builtin_bit_cast(f32x4, da);
                        const f32x4 kv = __builtin_bit_cast(f32x4, kf[t][c]);
                        const f32x4 vv = __builtin_bit_cast(f32x4, vf[t][c]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            sacc[qb][t] = mfma_f32(qv[e], kv[e], sacc[qb][t]);
                            pacc[qb][t] = mfma_f32(dv[e], vv[e], pacc[qb][t]);
                        }
                    }
                }
            }
        }

        // P = exp2(S scale log2e - lse2) on visible pairs; dS = P (dP - D)
        const int kk0 = key0 + kw0;  // first key of this wave's slice
        const int row0 = m * BM;
        const int row1 = imin(row0 + BM, Sq) - 1;
        // the slice is visible to every existing row of the block: no element mask
        const bool full = kk0 + NKW <= Sk && (!p.causal || kk0 + NKW - 1 <= row0 + delta) &&
                          (p.window_left < 0 || kk0 >= row1 + delta - p.window_left);
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            const f32x4 lv = *reinterpret_cast<const f32x4*>(ls2 + 16 * qb + 4 * lg);
            const f32x4 dsv = *reinterpret_cast<const f32x4*>(lds_dsum + 16 * qb + 4 * lg);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const int key = kk0 + 16 * t + li;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float pv = fast_exp2(fmaf(sacc[qb][t][r], sl2, -lv[r]));
                    if (!full) {
                        const int pos = row0 + 16 * qb + 4 * lg + r;
                        const bool vis = key < Sk && (!p.causal || key <= pos + delta) &&
                                         (p.window_left < 0 || key >= pos + delta - p.window_left);
                        pv = vis ? pv : 0.f;
                    }
                    sacc[qb][t][r] = pv;
                    pacc[qb][t][r] = pv * (pacc[qb][t][r] - dsv[r]);
                }
            }
        }

        // dV^T += dO^T P and dK^T += Q^T dS (contraction over the query rows)
        if constexpr (BF) {
#pragma unroll
            for (int pp = 0; pp < BM / 32; ++pp) {
                u32x4 pb[NT], sb[NT], pbl[NT], sbl[NT];  // P and dS as bf16 hi + lo
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    split_bf16x8(sacc[2 * pp][t], sacc[2 * pp + 1][t], pb[t], pbl[t]);
                    split_bf16x8(pacc[2 * pp][t], pacc[2 * pp + 1][t], sb[t], sbl[t]);
                }
                const int ra = (32 * pp + 4 * lg + (li >> 2)) * QST + 4 * (li & 3);
                const int rb = ra + 16 * QST;
#pragma unroll
                for (int u = 0; u < D / 16; ++u) {
                    const u32x2 d0 = lds_read_tr16(dOs + ra + 16 * u);
                    const u32x2 d1 = lds_read_tr16(dOs + rb + 16 * u);
                    const u32x2 q0 = lds_read_tr16(Qs + ra + 16 * u);
                    const u32x2 q1 = lds_read_tr16(Qs + rb + 16 * u);
                    const u32x4 da = {d0[0], d0[1], d1[0], d1[1]};
                    const u32x4 qa = {q0[0], q0[1], q1[0], q1[1]};
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        dvT[u][t] = mfma_bf16(da, pb[t], dvT[u][t]);
                        dvT[u][t] = mfma_bf16(da, pbl[t], dvT[u][t]);
                        dkT[u][t] = mfma_bf16(qa, sb[t], dkT[u][t]);
                        dkT[u][t] = mfma_bf16(qa, sbl[t], dkT[u][t]);
                    }
                }
            }
        } else {
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * qb + 4 * lg + r;
#pragma unroll
                    for (int u = 0; u < D / 16; ++u) {
                        const float da = dOs[row * QST + 16 * u + li];
                        const float qa = Qs[row * QST + 16 * u + li];
#pragma unroll
                        for (int t = 0; t < NT; ++t) {
                            dvT[u][t] = mfma_f32(da, sacc[qb][t][r], dvT[u][t]);
                            dkT[u][t] = mfma_f32(qa, pacc[qb][t][r], dkT[u][t]);
                        }
                    }
                }
        }

        if constexpr (ATOMIC) {
        // dS^T -> LDS: key row kw0 + 16 t + li, query rows 16 qb + 4 lg .. +3
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                T* dst = dSt + (kw0 + 16 * t + li) * SST + 16 * qb + 4 * lg;
                if constexpr (BF) {
                    const u32x2 w0 = split_bf16x2(pacc[qb][t][0], pacc[qb][t][1]);
                    const u32x2 w1 = split_bf16x2(pacc[qb][t][2], pacc[qb][t][3]);
                    *reinterpret_cast<u32x2*>(dst) = u32x2{w0[0], w1[0]};
                    *reinterpret_cast<u32x2*>(dst + BN * SST) = u32x2{w0[1], w1[1]};  // lo parts
                } else {
                    *reinterpret_cast<f32x4*>(dst) = pacc[qb][t];
                }
            }
        __syncthreads();

        // dQ rows 16 wave .. +15 of this block: dQ = dS K over the block's keys
        f32x4 dqa[D / 16];
#pragma unroll
        for (int u = 0; u < D / 16; ++u) dqa[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (BF) {
#pragma unroll
            for (int kk = 0; kk < BN / 32; ++kk) {
                const int ka = (32 * kk + 8 * lg + (li >> 2));
                const u32x2 a0 = lds_read_tr16(dSt + ka * SST + 16 * wave + 4 * (li & 3));
                const u32x2 a1 = lds_read_tr16(dSt + (ka + 4) * SST + 16 * wave + 4 * (li & 3));
                const u32x4 sa = {a0[0], a0[1], a1[0], a1[1]};
                const u32x2 c0 = lds_read_tr16(dSt + BN * SST + ka * SST + 16 * wave + 4 * (li & 3));
                const u32x2 c1 = lds_read_tr16(dSt + BN * SST + (ka + 4) * SST + 16 * wave + 4 * (li & 3));
                const u32x4 sl = {c0[0], c0[1], c1[0], c1[1]};
#pragma unroll
                for (int u = 0; u < D / 16; ++u) {
                    const u32x2 b0 = lds_read_tr16(Ks + ka * QST + 16 * u + 4 * (li & 3));
                    const u32x2 b1 = lds_read_tr16(Ks + (ka + 4) * QST + 16 * u + 4 * (li & 3));
                    const u32x4 kb = {b0[0], b0[1], b1[0], b1[1]};
                    dqa[u] = mfma_bf16(sa, kb, dqa[u]);
                    dqa[u] = mfma_bf16(sl, kb, dqa[u]);
                }
            }
        } else {
#pragma unroll 4
            for (int kk = 0; kk < BN / 4; ++kk) {
                const float sa = dSt[(4 * kk + lg) * SST + 16 * wave + li];
#pragma unroll
                for (int u = 0; u < D / 16; ++u)
                    dqa[u] = mfma_f32(sa, Ks[(4 * kk + lg) * QST + 16 * u + li], dqa[u]);
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int pos = row0 + 16 * wave + 4 * lg + r;
            if (pos < Sq) {
                float* dst = p.dq_acc + (((size_t)b * Sq + pos) * p.Hq + hq) * D + li;
#pragma unroll
                for (int u = 0; u < D / 16; ++u) unsafeAtomicAdd(dst + 16 * u, dqa[u][r]);
            }
        }
            }
    }

    // ---- dK = scale (dK^T)^T, dV: lane holds d = 16u + 4lg .. +3 of key kw0 + 16t + li
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int key = key0 + kw0 + 16 * t + li;
        if (key >= Sk) continue;
        const size_t off = (((size_t)b * Sk + key) * p.Hkv + hkv) * D + 4 * lg;
#pragma unroll
        for (int u = 0; u < D / 16; ++u) {
            const f32x4 kv = dkT[u][t] * p.scale;
            const f32x4 vv = dvT[u][t];
            if constexpr (BF) {
                *reinterpret_cast<u32x2*>(reinterpret_cast<bf16_t*>(p.dk) + off + 16 * u) =
                    u32x2{pack_bf16x2(kv[0], kv[1]), pack_bf16x2(kv[2], kv[3])};
                *reinterpret_cast<u32x2*>(reinterpret_cast<bf16_t*>(p.dv) + off + 16 * u) =
                    u32x2{pack_bf16x2(vv[0], vv[1]), pack_bf16x2(vv[2], vv[3])};
            } else {
                *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.dk) + off + 16 * u) = kv;
                *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.dv) + off + 16 * u) = vv;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// dQ kernel: one workgroup per (query block, query head, batch), looping over
// the key blocks the query block sees (the forward's n_block_range, [FA-tiling]
// §3.2). With the query rows on the MFMA N axis (lane li = query row):
//   S^T  [key][q] = K . Q^T      A = K rows (LDS), B = Q (registers)
//   dP^T [key][q] = V . dO^T     A = V rows (LDS), B = dO (registers)
//   dS^T = P^T (dP^T - D),  P^T = exp2(S^T scale log2e - lse2)
//   dQ^T [d][q]  += K^T . dS^T   A = K^T tile (LDS, stored transposed),
//                                B = dS^T (the accumulators, in place)
// Each wave owns NQW 16-row blocks of the query block.
// ---------------------------------------------------------------------------
template <class T, int D, int NQW>
struct BwdDqTile {
    static constexpr bool BF = std::is_same<T, bf16_t>::value;
    static constexpr int NW = 4, NTHR = 64 * NW;
    static constexpr int MW = 16 * NQW;         // query rows per wave
    static constexpr int BM = NW * MW;          // query rows per workgroup
    static constexpr int BN = 64;               // keys per tile
    static constexpr int NT = BN / 16;
    static constexpr int ESZ = sizeof(T);
    static constexpr int CE = 16 / ESZ;
    static constexpr int KST = D + CE;          // K, V tile row pitch (elements)
    static constexpr int TST = BN + CE;         // K^T tile row pitch (elements)
    static constexpr int CPR = D / CE;
    static constexpr int GROUPS = (BN / 4) * CPR;                   // (4 rows x chunk) items
    static constexpr int ITEMS = (GROUPS + NTHR - 1) / NTHR;
    static constexpr int DL = D / 4;
    static constexpr int QV = DL / CE;          // 16-byte chunks per lane per row
    static constexpr int K_BYTES = BN * KST * ESZ;
    static constexpr int KT_BYTES = D * TST * ESZ;
    static constexpr int LDS_BYTES = 2 * K_BYTES + KT_BYTES;
};

template <class T, int D, int NQW, int OCC>
__global__ void __launch_bounds__(256, OCC) attn_bwd_dq_kernel(BwdParams p) {
    using C = BwdDqTile<T, D, NQW>;
    constexpr bool BF = C::BF;
    constexpr int BM = C::BM, BN = C::BN, NT = C::NT, CE = C::CE, DL = C::DL, QV = C::QV;
    constexpr int KST = C::KST, TST = C::TST, CPR = C::CPR, ITEMS = C::ITEMS;

    __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];
    T* Ks = reinterpret_cast<T*>(smem);
    T* Vs = reinterpret_cast<T*>(smem + C::K_BYTES);
    T* KT = reinterpret_cast<T*>(smem + 2 * C::K_BYTES);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int num_m = ceil_div(p.Sq, BM);
    // heaviest causal query blocks (the last ones) first ([FA-tiling] §4.4)
    const int m_block = p.causal ? num_m - 1 - (int)blockIdx.x : (int)blockIdx.x;
    const int hq = blockIdx.y, b = blockIdx.z;
    const int hkv = hq / p.G;
    const int Sq = p.Sq, Sk = p.Sk, delta = Sk - Sq;

    int n_lo, n_hi;
    n_block_range(Sq, Sk, 1, 0, p.causal, p.window_left, BM, BN, m_block, &n_lo, &n_hi);

    // this lane's query rows and their visible key interval [row_lo, row_hi]
    int row_pos[NQW], row_lo[NQW], row_hi[NQW];
    float l2[NQW], dsum[NQW];
    int wlo = -0x7fffffff, whi = 0x7fffffff;
#pragma unroll
    for (int qq = 0; qq < NQW; ++qq) {
        const int pos = m_block * BM + wave * C::MW + 16 * qq + li;
        row_pos[qq] = pos;
        int lo = 0, hi = Sk - 1;
        l2[qq] = INFINITY;
        dsum[qq] = 0.f;
        if (pos < Sq) {
            if (p.window_left >= 0) lo = pos + delta - p.window_left;
            if (p.causal) hi = imin(hi, pos + delta);
            wlo = imax(wlo, lo);
            whi = imin(whi, hi);
            const size_t idx = ((size_t)b * p.Hq + hq) * Sq + pos;
            l2[qq] = p.lse2[idx];
            dsum[qq] = p.dsum[idx];
        }
        row_lo[qq] = lo;
        row_hi[qq] = hi;
    }
    wlo = row16_imax(wlo);
    whi = row16_imin(whi);

    // Q and dO fragments: lane group lg holds d in [lg DL, (lg + 1) DL) of its row
    u32x4 qf[NQW][QV], gf[NQW][QV];
    const bool has_work = n_hi > n_lo;
#pragma unroll
    for (int qq = 0; qq < NQW; ++qq) {
        const size_t off = (((size_t)b * Sq + row_pos[qq]) * p.Hq + hq) * D + lg * DL;
#pragma unroll
        for (int c = 0; c < QV; ++c) {
            u32x4 z = {0u, 0u, 0u, 0u};
            qf[qq][c] = z;
            gf[qq][c] = z;
            if (row_pos[qq] < Sq && has_work) {
                qf[qq][c] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(p.q) + off + c * CE);
                gf[qq][c] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(p.dout) + off + c * CE);
            }
        }
    }

    f32x4 dqT[D / 16][NQW];
#pragma unroll
    for (int u = 0; u < D / 16; ++u)
#pragma unroll
        for (int qq = 0; qq < NQW; ++qq) dqT[u][qq] = f32x4{0.f, 0.f, 0.f, 0.f};
    const float sl2 = p.scale_log2;

    // K/V tile staging through registers: item = (4 key rows, 16-byte chunk)
    const T* kbase = reinterpret_cast<const T*>(p.k) + ((size_t)b * Sk * p.Hkv + hkv) * D;
    const T* vbase = reinterpret_cast<const T*>(p.v) + ((size_t)b * Sk * p.Hkv + hkv) * D;
    const size_t kv_stride = (size_t)p.Hkv * D;
    u32x4 kst[ITEMS][4], vst[ITEMS][4];
    auto load_tile = [&](int n) {
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const int item = tid + it * C::NTHR;
            const int c = item % CPR, rg = item / CPR;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = n * BN + 4 * rg + r;
                u32x4 z = {0u, 0u, 0u, 0u};
                kst[it][r] = z;
                vst[it][r] = z;
                if (item < C::GROUPS && key < Sk) {
                    kst[it][r] = *reinterpret_cast<const u32x4*>(kbase + key * kv_stride + c * CE);
                    vst[it][r] = *reinterpret_cast<const u32x4*>(vbase + key * kv_stride + c * CE);
                }
            }
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int it = 0; it < ITEMS; ++it) {
            const int item = tid + it * C::NTHR;
            if (item >= C::GROUPS) continue;
            const int c = item % CPR, rg = item / CPR;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                *reinterpret_cast<u32x4*>(Ks + (4 * rg + r) * KST + c * CE) = kst[it][r];
                *reinterpret_cast<u32x4*>(Vs + (4 * rg + r) * KST + c * CE) = vst[it][r];
            }
            if constexpr (BF) {
                // chunk c holds d = 8c..8c+7 of keys 4rg..4rg+3: write K^T[d][4rg..4rg+3]
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int w = e >> 1;
                    const uint32_t a0 = kst[it][0][w], a1 = kst[it][1][w];
                    const uint32_t a2 = kst[it][2][w], a3 = kst[it][3][w];
                    u32x2 pr;
                    if (e & 1) {
                        pr[0] = (a0 >> 16) | (a1 & 0xffff0000u);
                        pr[1] = (a2 >> 16) | (a3 & 0xffff0000u);
                    } else {
                        pr[0] = (a0 & 0xffffu) | (a1 << 16);
                        pr[1] = (a2 & 0xffffu) | (a3 << 16);
                    }
                    *reinterpret_cast<u32x2*>(KT + (8 * c + e) * TST + 4 * rg) = pr;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const u32x4 col = {kst[it][0][e], kst[it][1][e], kst[it][2][e], kst[it][3][e]};
                    *reinterpret_cast<u32x4*>(KT + (4 * c + e) * TST + 4 * rg) = col;
                }
            }
        }
    };

    if (has_work) load_tile(n_hi - 1);
    for (int n = n_hi - 1; n >= n_lo; --n) {
        __syncthreads();
        store_tile();
        __syncthreads();
        if (n > n_lo) load_tile(n - 1);

        // S^T = K Q^T and dP^T = V dO^T
        f32x4 sacc[NT][NQW], pacc[NT][NQW];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int qq = 0; qq < NQW; ++qq) {
                sacc[t][qq] = f32x4{0.f, 0.f, 0.f, 0.f};
                pacc[t][qq] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
        for (int c = 0; c < QV; ++c) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const u32x4 kf = *reinterpret_cast<const u32x4*>(Ks + (16 * t + li) * KST + lg * DL + c * CE);
                const u32x4 vf = *reinterpret_cast<const u32x4*>(Vs + (16 * t + li) * KST + lg * DL + c * CE);
#pragma unroll
                for (int qq = 0; qq < NQW; ++qq) {
                    if constexpr (BF) {
                        sacc[t][qq] = mfma_bf16(kf, qf[qq][c], sacc[t][qq]);
                        pacc[t][qq] = mfma_bf16(vf, gf[qq][c], pacc[t][qq]);
                    } else {
                        const f32x4 kv = __builtin_bit_cast(f32x4, kf), vv = __builtin_bit_cast(f32x4, vf);
                        const f32x4 qv = __builtin_bit_cast(f32x4, qf[qq][c]);
                        const f32x4 gv = __builtin_bit_cast(f32x4, gf[qq][c]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            sacc[t][qq] = mfma_f32(kv[e], qv[e], sacc[t][qq]);
                            pacc[t][qq] = mfma_f32(vv[e], gv[e], pacc[t][qq]);
                        }
                    }
                }
            }
        }

        // P^T and dS^T; element mask only where the tile is not inside every row's interval
        const int key0 = n * BN;
        const bool full = key0 >= wlo && key0 + BN - 1 <= whi;
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int qq = 0; qq < NQW; ++qq)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float pv = fast_exp2(fmaf(sacc[t][qq][r], sl2, -l2[qq]));
                    if (!full) {
                        const int key = key0 + 16 * t + 4 * lg + r;
                        pv = (key < row_lo[qq] || key > row_hi[qq]) ? 0.f : pv;
                    }
                    pacc[t][qq][r] = pv * (pacc[t][qq][r] - dsum[qq]);
                }

        // dQ^T += K^T dS^T
        if constexpr (BF) {
#pragma unroll
            for (int pp = 0; pp < NT / 2; ++pp) {
                u32x4 sb[NQW], sbl[NQW];  // dS as bf16 hi + lo
#pragma unroll
                for (int qq = 0; qq < NQW; ++qq)
                    split_bf16x8(pacc[2 * pp][qq], pacc[2 * pp + 1][qq], sb[qq], sbl[qq]);
#pragma unroll
                for (int u = 0; u < D / 16; ++u) {
                    const T* krow = KT + (16 * u + li) * TST + 32 * pp + 4 * lg;
                    const u32x2 lo = *reinterpret_cast<const u32x2*>(krow);
                    const u32x2 hi = *reinterpret_cast<const u32x2*>(krow + 16);
                    const u32x4 ka = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
                    for (int qq = 0; qq < NQW; ++qq) {
                        dqT[u][qq] = mfma_bf16(ka, sb[qq], dqT[u][qq]);
                        dqT[u][qq] = mfma_bf16(ka, sbl[qq], dqT[u][qq]);
                    }
                }
            }
        } else {
#pragma unroll
            for (int t = 0; t < NT; ++t)
#pragma unroll
                for (int u = 0; u < D / 16; ++u) {
                    const f32x4 ka = *reinterpret_cast<const f32x4*>(KT + (16 * u + li) * TST + 16 * t + 4 * lg);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
#pragma unroll
                        for (int qq = 0; qq < NQW; ++qq)
                            dqT[u][qq] = mfma_f32(ka[r], pacc[t][qq][r], dqT[u][qq]);
                }
        }
    }

    // dQ = scale (dQ^T)^T: lane holds d = 16u + 4lg .. +3 of row 16qq + li
#pragma unroll
    for (int qq = 0; qq < NQW; ++qq) {
        if (row_pos[qq] >= Sq) continue;
        const size_t off = (((size_t)b * Sq + row_pos[qq]) * p.Hq + hq) * D + 4 * lg;
#pragma unroll
        for (int u = 0; u < D / 16; ++u) {
            const f32x4 v = dqT[u][qq] * p.scale;
            if constexpr (BF) {
                *reinterpret_cast<u32x2*>(reinterpret_cast<bf16_t*>(p.dq) + off + 16 * u) =
                    u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            } else {
                *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.dq) + off + 16 * u) = v;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// dQ kernel, bf16: the same products with K and V tiles DMA'd straight into
// double-buffered LDS (buffer_load ... lds), so a whole tile of work hides each
// tile's load and no registers stage it. Each 16-byte chunk c of LDS row r sits
// in slot c ^ swz(r); the S^T / dP^T operands are 16-byte row reads, and K^T
// for dQ^T comes from the same K tile by transpose reads (ds_read_b64_tr_b16),
// whose 8-byte pieces never straddle a chunk.
// ---------------------------------------------------------------------------
template <int D, int NQW>
struct BwdDqDmaTile {
    static constexpr int NW = 4, NTHR = 64 * NW;
    static constexpr int MW = 16 * NQW, BM = NW * MW, BN = 64, NT = BN / 16;
    static constexpr int CPR = D / 8;             // 16-byte chunks per row
    static constexpr int ROWB = 2 * D;            // bytes per K / V row in LDS
    static constexpr int TILEB = BN * ROWB;
    static constexpr int STAGEB = 2 * TILEB;      // K + V
    static constexpr int LDS_BYTES = 2 * STAGEB;
    static constexpr int KROWS = 1024 / ROWB;     // rows per wave-wide DMA
    static constexpr int KDMA = BN / KROWS;       // DMAs per tile
    static constexpr int KDMA_PER_WAVE = KDMA / NW;
    static constexpr int DL = D / 4, QV = DL / 8;
    static_assert(KDMA % NW == 0, "tile DMAs must split evenly over the waves");
    // XOR swizzle of the 16-byte chunk slots of row r: 16 consecutive rows read
    // at one chunk (16-byte row reads) hit distinct banks, and so do the two
    // chunks of 4 consecutive rows that one 16-lane transpose read touches
    static __host__ __device__ __forceinline__ int swz(int r) {
        return D == 128 ? (((r & 7) << 1) | ((r >> 3) & 1)) : ((((r >> 1) & 3) << 1) | ((r >> 3) & 1));
    }
};

template <int D, int NQW, int OCC>
__global__ void __launch_bounds__(256, OCC) attn_bwd_dq_dma_kernel(BwdParams p) {
    using C = BwdDqDmaTile<D, NQW>;
    constexpr int BM = C::BM, BN = C::BN, NT = C::NT, DL = C::DL, QV = C::QV;
    constexpr int CPR = C::CPR, ROWB = C::ROWB, TILEB = C::TILEB, STAGEB = C::STAGEB;
    __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    // XCD-aware one-dimensional grid: tile t = (batch, head, query block), query
    // blocks fastest and heaviest first; XCD x (workgroup i runs on XCD i % 8)
    // owns tiles [x per_xcd, (x + 1) per_xcd), so the query blocks of a head run
    // together on one XCD and share its 4 MB L2 for the head's K and V
    const int num_m = ceil_div(p.Sq, BM);
    const int total = num_m * p.Hq * p.B;
    const int per_xcd = (total + NUM_XCD - 1) / NUM_XCD;
    const int t = ((int)blockIdx.x % NUM_XCD) * per_xcd + (int)blockIdx.x / NUM_XCD;
    if (t >= total) return;
    const int m_rev = t % num_m;
    const int m_block = p.causal ? num_m - 1 - m_rev : m_rev;
    const int hq = (t / num_m) % p.Hq, b = t / (num_m * p.Hq);
    const int hkv = hq / p.G;
    const int Sq = p.Sq, Sk = p.Sk, delta = Sk - Sq;

    int n_lo, n_hi;
    n_block_range(Sq, Sk, 1, 0, p.causal, p.window_left, BM, BN, m_block, &n_lo, &n_hi);
    const bool has_work = n_hi > n_lo;

    int row_pos[NQW], row_lo[NQW], row_hi[NQW];
    float l2[NQW], dsum[NQW];
    int wlo = -0x7fffffff, whi = 0x7fffffff;
#pragma unroll
    for (int qq = 0; qq < NQW; ++qq) {
        const int pos = m_block * BM + wave * C::MW + 16 * qq + li;
        row_pos[qq] = pos;
        int lo = 0, hi = Sk - 1;
        l2[qq] = INFINITY;
        dsum[qq] = 0.f;
        if (pos < Sq) {
            if (p.window_left >= 0) lo = pos + delta - p.window_left;
            if (p.causal) hi = imin(hi, pos + delta);
            wlo = imax(wlo, lo);
            whi = imin(whi, hi);
            const size_t idx = ((size_t)b * p.Hq + hq) * Sq + pos;
            l2[qq] = p.lse2[idx];
        }
        row_lo[qq] = lo;
        row_hi[qq] = hi;
    }
    wlo = row16_imax(wlo);
    whi = row16_imin(whi);

    u32x4 qf[NQW][QV], gf[NQW][QV];
#pragma unroll
    for (int qq = 0; qq < NQW; ++qq) {
        const size_t off = (((size_t)b * Sq + row_pos[qq]) * p.Hq + hq) * D + lg * DL;
#pragma unroll
        for (int c = 0; c < QV; ++c) {
            u32x4 z = {0u, 0u, 0u, 0u};
            qf[qq][c] = z;
            gf[qq][c] = z;
            if (row_pos[qq] < Sq && has_work) {
                qf[qq][c] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16_t*>(p.q) + off + 8 * c);
                gf[qq][c] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16_t*>(p.dout) + off + 8 * c);
            }
        }
    }

    f32x4 dqT[D / 16][NQW];
#pragma unroll
    for (int u = 0; u < D / 16; ++u)
#pragma unroll
        for (int qq = 0; qq < NQW; ++qq) dqT[u][qq] = f32x4{0.f, 0.f, 0.f, 0.f};
    const float sl2 = p.scale_log2;

    const size_t kv_stride = (size_t)p.Hkv * D;
    const uint32_t row_bytes = (uint32_t)(kv_stride * 2);
    const bf16_t* kbase = reinterpret_cast<const bf16_t*>(p.k) + ((size_t)b * Sk * p.Hkv + hkv) * D;
    const bf16_t* vbase = reinterpret_cast<const bf16_t*>(p.v) + ((size_t)b * Sk * p.Hkv + hkv) * D;
    // lane l of DMA i fills 16 bytes at 1024 i + 16 l: row KROWS i + l / CPR, slot
    // l % CPR, which holds the row's chunk slot ^ swz(row); rows at or beyond Sk
    // lie past the buffer resource and read as zeros
    auto load_kv = [&](int n, int stage) {
        const uint32_t bytes = (uint32_t)imin(BN, Sk - n * BN) * row_bytes;
        const rsrc_t rk = make_rsrc(kbase + (size_t)n * BN * kv_stride, bytes);
        const rsrc_t rv = make_rsrc(vbase + (size_t)n * BN * kv_stride, bytes);
        char* dk = smem + stage * STAGEB;
        char* dv = dk + TILEB;
#pragma unroll
        for (int j = 0; j < C::KDMA_PER_WAVE; ++j) {
            const int i = wave * C::KDMA_PER_WAVE + j;
            const int rr = C::KROWS * i + lane / CPR;
            const uint32_t voff = rr * row_bytes + 16 * ((lane % CPR) ^ C::swz(rr));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rk, (__attribute__((address_space(3))) void*)(dk + 1024 * i), 16, voff, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rv, (__attribute__((address_space(3))) void*)(dv + 1024 * i), 16, voff, 0, 0, 0);
        }
    };

    // Two sweeps over the key blocks, in ascending order (the query blocks of a
    // head, which run together on one XCD, then walk the head's K and V tiles
    // roughly in step and share them in L2). The first forms the row sums
    // D_i = sum_j P_ij dP_ij of the exact softmax -- <dO_i, O_i> of the forward
    // output would carry O's bf16 rounding, which dS = P (dP - D) turns into a
    // relative error of several percent in dQ and dK of rows with few keys --
    // and stores them for the key-block kernel, which runs after this one; the
    // second forms dS and dQ.
    float dacc[NQW];
#pragma unroll
    for (int qq = 0; qq < NQW; ++qq) dacc[qq] = 0.f;
    auto sweep = [&](auto pass) {
    constexpr bool ROWSUM = decltype(pass)::value;
    if (has_work) {
        load_kv(n_lo, 0);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the tile has landed
    }
    __syncthreads();

    int stage = 0;
    for (int n = n_lo; n < n_hi; ++n) {
        if (n + 1 < n_hi) load_kv(n + 1, stage ^ 1);
        const char* kt = smem + stage * STAGEB;
        const char* vt = kt + TILEB;

        // per 32-key half of the tile: S^T = K Q^T and dP^T = V dO^T (lane group lg
        // contracts d in [lg DL, (lg+1) DL)), then P^T, dS^T and dQ^T += K^T dS^T
        const int key0 = n * BN;
        // every row of the wave sees the whole tile (wave-uniform, so the masked
        // path below is one scalar branch per half tile, not a divergent branch
        // per element)
        const bool full = __builtin_amdgcn_ballot_w64(!(key0 >= wlo && key0 + BN - 1 <= whi)) == 0;
#pragma unroll
        for (int pp = 0; pp < NT / 2; ++pp) {
            f32x4 sacc[2][NQW], pacc[2][NQW];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int qq = 0; qq < NQW; ++qq) {
                    sacc[h][qq] = f32x4{0.f, 0.f, 0.f, 0.f};
                    pacc[h][qq] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
            for (int c = 0; c < QV; ++c) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int row = 16 * (2 * pp + h) + li;
                    const int off = row * ROWB + 16 * ((lg * QV + c) ^ C::swz(row));
                    const u32x4 kf = *reinterpret_cast<const u32x4*>(kt + off);
                    const u32x4 vf = *reinterpret_cast<const u32x4*>(vt + off);
#pragma unroll
                    for (int qq = 0; qq < NQW; ++qq) {
                        sacc[h][qq] = mfma_bf16(kf, qf[qq][c], sacc[h][qq]);
                        pacc[h][qq] = mfma_bf16(vf, gf[qq][c], pacc[h][qq]);
                    }
                }
            }
            if (!full) {  // -inf on the scores a row cannot see (P = 0 there)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int qq = 0; qq < NQW; ++qq)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int key = key0 + 16 * (2 * pp + h) + 4 * lg + r;
                            if ((key < row_lo[qq]) | (key > row_hi[qq])) sacc[h][qq][r] = -INFINITY;
                        }
            }
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int qq = 0; qq < NQW; ++qq)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float pv = fast_exp2(fmaf(sacc[h][qq][r], sl2, -l2[qq]));
                        if constexpr (ROWSUM) dacc[qq] += pv * pacc[h][qq][r];
                        else pacc[h][qq][r] = pv * (pacc[h][qq][r] - dsum[qq]);
                    }
            if constexpr (ROWSUM) continue;
            // K^T by transpose reads of the K tile; source lane s of a 16-lane
            // group addresses key row k0 + s / 4, columns 16u + 4 (s % 4)
            u32x4 sb[NQW], sbl[NQW];  // dS as bf16 hi + lo
#pragma unroll
            for (int qq = 0; qq < NQW; ++qq) split_bf16x8(pacc[0][qq], pacc[1][qq], sb[qq], sbl[qq]);
            const int r0 = 32 * pp + 4 * lg + (li >> 2), r1 = r0 + 16;
#pragma unroll
            for (int u = 0; u < D / 16; ++u) {
                const int ch = 2 * u + ((li & 3) >> 1);
                const int o0 = r0 * ROWB + 16 * (ch ^ C::swz(r0)) + 8 * (li & 1);
                const int o1 = r1 * ROWB + 16 * (ch ^ C::swz(r1)) + 8 * (li & 1);
                const u32x2 lo = lds_read_tr16(reinterpret_cast<const bf16_t*>(kt + o0));
                const u32x2 hi = lds_read_tr16(reinterpret_cast<const bf16_t*>(kt + o1));
                const u32x4 ka = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
                for (int qq = 0; qq < NQW; ++qq) {
                    dqT[u][qq] = mfma_bf16(ka, sb[qq], dqT[u][qq]);
                    dqT[u][qq] = mfma_bf16(ka, sbl[qq], dqT[u][qq]);
                }
            }
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the next tile has landed
        __syncthreads();
        stage ^= 1;
    }
    };
    sweep(std::true_type{});
#pragma unroll
    for (int qq = 0; qq < NQW; ++qq) {
        dsum[qq] = xor_sum(dacc[qq]);  // the four lane groups hold disjoint keys of the row
        if (lg == 0 && row_pos[qq] < Sq) p.dsum[((size_t)b * p.Hq + hq) * Sq + row_pos[qq]] = dsum[qq];
    }
    sweep(std::false_type{});

#pragma unroll
    for (int qq = 0; qq < NQW; ++qq) {
        if (row_pos[qq] >= Sq) continue;
        const size_t off = (((size_t)b * Sq + row_pos[qq]) * p.Hq + hq) * D + 4 * lg;
#pragma unroll
        for (int u = 0; u < D / 16; ++u) {
            const f32x4 v = dqT[u][qq] * p.scale;
            *reinterpret_cast<u32x2*>(reinterpret_cast<bf16_t*>(p.dq) + off + 16 * u) =
                u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        }
    }
}

// ---------------------------------------------------------------------------
// Key-block kernel, bf16, with the query-block tiles (Q, dO, and the rows'
// lse2 and D) DMA'd into double-buffered LDS one block ahead. Q and dO serve
// both as 16-byte row reads (the A operands of S and dP) and, by transpose
// reads, as the column operands of dV^T and dK^T; chunk c of LDS row r sits in
// slot c ^ swz(r). Query rows past Sq read as zeros (their Q and dO rows are 0,
// so they add nothing whatever their P).
// ---------------------------------------------------------------------------
template <int D, int NKW_ = 16>
struct BwdKvDmaTile {
    static constexpr int NW = 4, NTHR = 64 * NW, NKW = NKW_;
    static constexpr int NT = NKW / 16;           // 16-key blocks per wave
    static constexpr int BM = 64, BN = NW * NKW;
    static constexpr int NQB = BM / 16;
    static constexpr int CPR = D / 8, ROWB = 2 * D;
    static constexpr int TILEB = BM * ROWB;
    static constexpr int STAGEB = 2 * TILEB + 2 * BM * 4;   // Q, dO, lse2, D
    static constexpr int LDS_BYTES = 2 * STAGEB;
    static constexpr int KROWS = 1024 / ROWB, KDMA = BM / KROWS, KDMA_PER_WAVE = KDMA / NW;
    static constexpr int KC = D / 32;
    static_assert(KDMA % NW == 0, "tile DMAs must split evenly over the waves");
    // XOR swizzle of the 16-byte chunk slots of row r: 16 consecutive rows read
    // at one chunk (16-byte row reads) hit distinct banks, and so do the two
    // chunks of 4 consecutive rows that one 16-lane transpose read touches
    static __host__ __device__ __forceinline__ int swz(int r) {
        return D == 128 ? (((r & 7) << 1) | ((r >> 3) & 1)) : ((((r >> 1) & 3) << 1) | ((r >> 3) & 1));
    }
};

template <int D, int NKW_, int OCC>
__global__ void __launch_bounds__(256, OCC) attn_bwd_dkdv_dma_kernel(BwdParams p) {
    using C = BwdKvDmaTile<D, NKW_>;
    constexpr int BM = C::BM, BN = C::BN, KC = C::KC, NKW = C::NKW, NT = C::NT;
    constexpr int CPR = C::CPR, ROWB = C::ROWB, TILEB = C::TILEB, STAGEB = C::STAGEB;
    __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    // XCD-aware one-dimensional grid: tile t = (batch, KV head, key block), key
    // blocks fastest (heaviest causal blocks first); XCD x owns tiles
    // [x per_xcd, (x + 1) per_xcd), so the key blocks of a head run together on
    // one XCD and share its L2 for the head's Q and dO ([FA-tiling] §4.6: Q and dO
    // are what the backward keeps in L2)
    const int tiles = p.num_n_blocks * p.Hkv * p.B;
    const int per_xcd = (tiles + NUM_XCD - 1) / NUM_XCD;
    const int tile = ((int)blockIdx.x % NUM_XCD) * per_xcd + (int)blockIdx.x / NUM_XCD;
    if (tile >= tiles) return;
    const int nb = tile % p.num_n_blocks;
    const int hkv = (tile / p.num_n_blocks) % p.Hkv;
    const int b = tile / (p.num_n_blocks * p.Hkv);
    const int G = p.G, Sq = p.Sq, Sk = p.Sk;
    const int delta = Sk - Sq;
    const int key0 = nb * BN;
    const int kw0 = wave * NKW;

    int m_lo, m_hi;
    m_block_range(Sq, Sk, p.causal, p.window_left, BM, BN, nb, &m_lo, &m_hi);
    const int nm = imax(0, m_hi - m_lo);
    const int total = G * nm;

    // this wave's K and V rows as MFMA B fragments: key kw0 + 16t + li, d = (D/4) lg + 8c..
    const size_t kv_stride = (size_t)p.Hkv * D;
    const bf16_t* kbase = reinterpret_cast<const bf16_t*>(p.k) + ((size_t)b * Sk * p.Hkv + hkv) * D;
    const bf16_t* vbase = reinterpret_cast<const bf16_t*>(p.v) + ((size_t)b * Sk * p.Hkv + hkv) * D;
    u32x4 kf[NT][KC], vf[NT][KC];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int key = key0 + kw0 + 16 * t + li;
#pragma unroll
        for (int c = 0; c < KC; ++c) {
            u32x4 z = {0u, 0u, 0u, 0u};
            kf[t][c] = z;
            vf[t][c] = z;
            if (key < Sk && total > 0) {
                kf[t][c] = *reinterpret_cast<const u32x4*>(kbase + key * kv_stride + (D / 4) * lg + 8 * c);
                vf[t][c] = *reinterpret_cast<const u32x4*>(vbase + key * kv_stride + (D / 4) * lg + 8 * c);
            }
        }
    }
    f32x4 dvT[D / 16][NT], dkT[D / 16][NT];
#pragma unroll
    for (int u = 0; u < D / 16; ++u)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            dvT[u][t] = f32x4{0.f, 0.f, 0.f, 0.f};
            dkT[u][t] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

    const uint32_t row_bytes = (uint32_t)((size_t)p.Hq * D * 2);
    // DMA of query block it into stage st: Q and dO rows (KDMA_PER_WAVE per wave
    // each), then lse2 and D (one 4-byte-per-lane DMA each, waves 0 and 1).
    // Issued untracked: the compiler's own tracking cannot tell the two stages
    // apart and waited for the next block's copies early in every block; the one
    // vmcnt(0) wait before the block's barrier orders them before their reads.
    auto load_block = [&](int it, int st) {
        const int g = it / nm, m = m_lo + it % nm;
        const int hq = hkv * G + g;
        const int valid = imin(BM, Sq - m * BM);
        const size_t row0 = ((size_t)b * Sq + m * BM) * p.Hq + hq;
        const u32x4 rq = rsrc_words_u(reinterpret_cast<const bf16_t*>(p.q) + row0 * D, (uint32_t)valid * row_bytes);
        const u32x4 rg = rsrc_words_u(reinterpret_cast<const bf16_t*>(p.dout) + row0 * D, (uint32_t)valid * row_bytes);
        const uint32_t lq = __builtin_amdgcn_readfirstlane(lds_addr(smem + st * STAGEB));
        const uint32_t lg_ = lq + TILEB;
#pragma unroll
        for (int j = 0; j < C::KDMA_PER_WAVE; ++j) {
            const int i = wave * C::KDMA_PER_WAVE + j;
            const int rr = C::KROWS * i + lane / CPR;
            const uint32_t voff = rr * row_bytes + 16 * ((lane % CPR) ^ C::swz(rr));
            dma16_untracked_cached(rq, voff, lq + 1024 * i);
            dma16_untracked_cached(rg, voff, lg_ + 1024 * i);
        }
        if (wave < 2) {
            const float* src = (wave == 0 ? p.lse2 : p.dsum) + ((size_t)b * p.Hq + hq) * Sq + m * BM;
            const u32x4 rl = rsrc_words_u(src, (uint32_t)valid * 4);
            dma4_untracked_cached(rl, 4 * lane, lg_ + TILEB + wave * BM * 4);
        }
    };

    if (total > 0) {
        load_block(0, 0);
        wait_vmcnt<0>();
    }
    // (the compiler's own record: the K and V register loads above have landed,
    // so it places no wait for them inside the loop, where the hardware count
    // would include the next block's copies)
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();

    const float sl2 = p.scale_log2;
    int st = 0;
    for (int it = 0; it < total; ++it) {
        const int m = m_lo + it % nm;
        if (it + 1 < total) load_block(it + 1, st ^ 1);
        const char* qt = smem + st * STAGEB;
        const char* gt = qt + TILEB;
        const float* ls2 = reinterpret_cast<const float*>(gt + TILEB);
        const float* lds_dsum = ls2 + BM;

        // per 32-row half of the query block: S = Q K^T and dP = dO V^T (contraction
        // slot (lg, e) of step c = d (D/4) lg + 8c + e), P and dS (lane holds key kw0 + 16t + li,
        // query rows 16 qb + 4 lg .. +3), then dV^T += dO^T P and dK^T += Q^T dS
        // with dO and Q read as columns (transpose reads)
        const int kk0 = key0 + kw0;
        const int row0 = m * BM;
        const int row1 = imin(row0 + BM, Sq) - 1;
        // every (row, key) pair of the wave's block is visible (wave-uniform, so the
        // masked path below is one scalar branch per half block)
        const bool full = __builtin_amdgcn_readfirstlane(
                              (kk0 + NKW <= Sk) & (!p.causal | (kk0 + NKW - 1 <= row0 + delta)) &
                              ((p.window_left < 0) | (kk0 >= row1 + delta - p.window_left))) != 0;
#pragma unroll
        for (int pp = 0; pp < BM / 32; ++pp) {
            f32x4 sacc[2][NT], pacc[2][NT];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    sacc[h][t] = f32x4{0.f, 0.f, 0.f, 0.f};
                    pacc[h][t] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
            for (int c = 0; c < KC; ++c)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int row = 16 * (2 * pp + h) + li;
                    const int off = row * ROWB + 16 * ((KC * lg + c) ^ C::swz(row));
                    const u32x4 qa = *reinterpret_cast<const u32x4*>(qt + off);
                    const u32x4 ga = *reinterpret_cast<const u32x4*>(gt + off);
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        sacc[h][t] = mfma_bf16(qa, kf[t][c], sacc[h][t]);
                        pacc[h][t] = mfma_bf16(ga, vf[t][c], pacc[h][t]);
                    }
                }
            if (!full) {  // -inf on the pairs that are not visible (P = 0 there)
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int t = 0; t < NT; ++t) {
                        const int key = kk0 + 16 * t + li;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int pos = row0 + 16 * (2 * pp + h) + 4 * lg + r;
                            const bool vis = (key < Sk) & (!p.causal | (key <= pos + delta)) &
                                             ((p.window_left < 0) | (key >= pos + delta - p.window_left));
                            if (!vis) sacc[h][t][r] = -INFINITY;
                        }
                    }
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int qb = 2 * pp + h;
                const f32x4 lv = *reinterpret_cast<const f32x4*>(ls2 + 16 * qb + 4 * lg);
                const f32x4 dsv = *reinterpret_cast<const f32x4*>(lds_dsum + 16 * qb + 4 * lg);
#pragma unroll
                for (int t = 0; t < NT; ++t) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float pv = fast_exp2(fmaf(sacc[h][t][r], sl2, -lv[r]));
                        sacc[h][t][r] = pv;
                        pacc[h][t][r] = pv * (pacc[h][t][r] - dsv[r]);
                    }
                }
            }
            u32x4 pb[NT], sb[NT], pbl[NT], sbl[NT];  // P and dS as bf16 hi + lo
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                split_bf16x8(sacc[0][t], sacc[1][t], pb[t], pbl[t]);
                split_bf16x8(pacc[0][t], pacc[1][t], sb[t], sbl[t]);
            }
            const int r0 = 32 * pp + 4 * lg + (li >> 2), r1 = r0 + 16;
#pragma unroll
            for (int u = 0; u < D / 16; ++u) {
                const int ch = 2 * u + ((li & 3) >> 1);
                const int o0 = r0 * ROWB + 16 * (ch ^ C::swz(r0)) + 8 * (li & 1);
                const int o1 = r1 * ROWB + 16 * (ch ^ C::swz(r1)) + 8 * (li & 1);
                const u32x2 d0 = lds_read_tr16(reinterpret_cast<const bf16_t*>(gt + o0));
                const u32x2 d1 = lds_read_tr16(reinterpret_cast<const bf16_t*>(gt + o1));
                const u32x2 q0 = lds_read_tr16(reinterpret_cast<const bf16_t*>(qt + o0));
                const u32x2 q1 = lds_read_tr16(reinterpret_cast<const bf16_t*>(qt + o1));
                const u32x4 da = {d0[0], d0[1], d1[0], d1[1]};
                const u32x4 qa = {q0[0], q0[1], q1[0], q1[1]};
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    dvT[u][t] = mfma_bf16(da, pb[t], dvT[u][t]);
                    dvT[u][t] = mfma_bf16(da, pbl[t], dvT[u][t]);
                    dkT[u][t] = mfma_bf16(qa, sb[t], dkT[u][t]);
                    dkT[u][t] = mfma_bf16(qa, sbl[t], dkT[u][t]);
                }
            }
        }
        wait_vmcnt<0>();  // the next block has landed
        __syncthreads();
        st ^= 1;
    }

    // dK = scale (dK^T)^T, dV: lane holds d = 16u + 4lg .. +3 of key kw0 + 16t + li
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int key = key0 + kw0 + 16 * t + li;
        if (key >= Sk) continue;
        const size_t off = (((size_t)b * Sk + key) * p.Hkv + hkv) * D + 4 * lg;
#pragma unroll
        for (int u = 0; u < D / 16; ++u) {
            const f32x4 kv = dkT[u][t] * p.scale;
            const f32x4 vv = dvT[u][t];
            *reinterpret_cast<u32x2*>(reinterpret_cast<bf16_t*>(p.dk) + off + 16 * u) =
                u32x2{pack_bf16x2(kv[0], kv[1]), pack_bf16x2(kv[2], kv[3])};
            *reinterpret_cast<u32x2*>(reinterpret_cast<bf16_t*>(p.dv) + off + 16 * u) =
                u32x2{pack_bf16x2(vv[0], vv[1]), pack_bf16x2(vv[2], vv[3])};
        }
    }
}

// ---------------------------------------------------------------------------
// launchers and the variant table
// ---------------------------------------------------------------------------
template <class T, int D, bool WITH_D = true>
hipError_t launch_bwd_pre(const BwdParams& p, hipStream_t stream) {
    constexpr int TPR = D / (16 / (int)sizeof(T));
    const long long rows = (long long)p.B * p.Sq * p.Hq;
    const long long blocks = (rows + 256 / TPR - 1) / (256 / TPR);
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((bwd_pre_kernel<T, D, WITH_D>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <class T, int D>
hipError_t launch_bwd_post(const BwdParams& p, hipStream_t stream) {
    const long long n4 = (long long)p.B * p.Sq * p.Hq * D / 4;
    const long long blocks = (n4 + 255) / 256;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((bwd_post_kernel<T>), dim3((unsigned)blocks), dim3(256), 0, stream, p, n4);
    return hipGetLastError();
}

template <class T, int D, int NKW, int OCC, bool ATOMIC>
hipError_t launch_bwd(const BwdParams& p, hipStream_t stream) {
    const long long grid = (long long)p.num_n_blocks * p.Hkv * p.B;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((attn_bwd_kernel<T, D, NKW, OCC, ATOMIC>), dim3((unsigned)grid), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <int D, int NKW, int OCC>
hipError_t launch_bwd_dkdv_dma(const BwdParams& p, hipStream_t stream) {
    const long long tiles = (long long)p.num_n_blocks * p.Hkv * p.B;
    if (tiles == 0) return hipSuccess;
    const long long grid = (tiles + NUM_XCD - 1) / NUM_XCD * NUM_XCD;
    hipLaunchKernelGGL((attn_bwd_dkdv_dma_kernel<D, NKW, OCC>), dim3((unsigned)grid), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <int D, int NQW, int OCC>
hipError_t launch_bwd_dq_dma(const BwdParams& p, hipStream_t stream) {
    const long long tiles = (long long)ceil_div(p.Sq, BwdDqDmaTile<D, NQW>::BM) * p.Hq * p.B;
    if (tiles == 0) return hipSuccess;
    const long long grid = (tiles + NUM_XCD - 1) / NUM_XCD * NUM_XCD;
    hipLaunchKernelGGL((attn_bwd_dq_dma_kernel<D, NQW, OCC>), dim3((unsigned)grid), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <class T, int D, int NQW, int OCC>
hipError_t launch_bwd_dq(const BwdParams& p, hipStream_t stream) {
    const int num_m = ceil_div(p.Sq, BwdDqTile<T, D, NQW>::BM);
    if (num_m == 0 || p.B == 0) return hipSuccess;
    hipLaunchKernelGGL((attn_bwd_dq_kernel<T, D, NQW, OCC>), dim3(num_m, p.Hq, p.B), dim3(256), 0, stream, p);
    return hipGetLastError();
}

// dQ by fp32 atomics from the key-block kernel (ATOMIC, one pass) or by a
// second, query-block-outer kernel (two passes, no atomics, deterministic).
#define TPA_BWD_ATOMIC(T, DT, D, NKW, OCC)                                                       \
    {DT, D, BwdTile<T, D, NKW, true>::BN, BwdTile<T, D, NKW, true>::BM,                          \
     BwdTile<T, D, NKW, true>::LDS_BYTES, 1, &launch_bwd<T, D, NKW, OCC, true>,                  \
     &launch_bwd_pre<T, D>, &launch_bwd_post<T, D>, nullptr, 0, 0}
#define TPA_BWD_TWO_PASS(T, DT, D, NKW, OCC, NQW, QOCC)                                          \
    {DT, D, BwdTile<T, D, NKW>::BN, BwdTile<T, D, NKW>::BM, BwdTile<T, D, NKW>::LDS_BYTES, 0,    \
     &launch_bwd<T, D, NKW, OCC, false>, &launch_bwd_pre<T, D>, nullptr,                        \
     &launch_bwd_dq<T, D, NQW, QOCC>, BwdDqTile<T, D, NQW>::BM, 0}

#define TPA_BWD_TWO_PASS_DMA(D, NKW, OCC, NQW, QOCC)                                                  \
    {DT_BF16, D, BwdTile<bf16_t, D, NKW>::BN, BwdTile<bf16_t, D, NKW>::BM,                          \
     BwdTile<bf16_t, D, NKW>::LDS_BYTES, 0, &launch_bwd<bf16_t, D, NKW, OCC, false>,               \
     &launch_bwd_pre<bf16_t, D, false>, nullptr, &launch_bwd_dq_dma<D, NQW, QOCC>, BwdDqDmaTile<D, NQW>::BM, 1}
// both kernels on DMA'd tiles
#define TPA_BWD_DMA(D, NKW, OCC, NQW, QOCC)                                                          \
    {DT_BF16, D, BwdKvDmaTile<D, NKW>::BN, BwdKvDmaTile<D, NKW>::BM,                               \
     BwdKvDmaTile<D, NKW>::LDS_BYTES, 0, &launch_bwd_dkdv_dma<D, NKW, OCC>,                       \
     &launch_bwd_pre<bf16_t, D, false>, nullptr,                                                  \
     &launch_bwd_dq_dma<D, NQW, QOCC>, BwdDqDmaTile<D, NQW>::BM, 2}

static const BwdVariant kBwdVariants[] = {
    // two passes (default): both kernels on DMA'd tiles; 64-key blocks for dK/dV,
    // 128-row blocks for dQ (32 rows per wave, two workgroups per CU)
    TPA_BWD_DMA(128, 16, 2, 2, 2),
    TPA_BWD_DMA(64, 16, 2, 2, 2),
    TPA_BWD_DMA(128, 16, 2, 1, 2),  // 64-row dQ blocks (16 rows per wave)
    TPA_BWD_DMA(64, 16, 2, 1, 2),
    TPA_BWD_DMA(128, 32, 1, 2, 2),  // 128-key blocks (32 keys per wave)
    TPA_BWD_DMA(64, 32, 1, 2, 2),
    // dK/dV with register-staged query tiles
    TPA_BWD_TWO_PASS_DMA(128, 16, 2, 1, 2),
    TPA_BWD_TWO_PASS_DMA(64, 16, 2, 1, 2),
    TPA_BWD_TWO_PASS_DMA(128, 16, 2, 2, 2),  // 128-row dQ blocks
    TPA_BWD_TWO_PASS_DMA(64, 16, 2, 2, 2),
    // fp32: register-staged tiles (D from the fp32 forward output)
    TPA_BWD_TWO_PASS(float, DT_FP32, 128, 16, 1, 1, 1),
    TPA_BWD_TWO_PASS(float, DT_FP32, 64, 16, 1, 1, 2),
    // dQ by atomics (ablation)
    TPA_BWD_ATOMIC(bf16_t, DT_BF16, 128, 16, 2),
    TPA_BWD_ATOMIC(bf16_t, DT_BF16, 64, 16, 2),
    TPA_BWD_ATOMIC(bf16_t, DT_BF16, 128, 32, 1),
    TPA_BWD_ATOMIC(bf16_t, DT_BF16, 64, 32, 1),
    TPA_BWD_ATOMIC(float, DT_FP32, 128, 16, 1),
    TPA_BWD_ATOMIC(float, DT_FP32, 64, 16, 1),
    {0, 0, 0, 0, 0, 0, nullptr, nullptr, nullptr, nullptr, 0, 0},
};

const BwdVariant* bwd_variants() { return kBwdVariants; }

}  // namespace tpa
