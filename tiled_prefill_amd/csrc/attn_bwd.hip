// attn_bwd.hip -- gfx950 (MI355X) flash-attention backward kernels.
//
//   bwd_pre_kernel   per query row: the row sum D = <dO, O>, lse2 = lse * log2(e)
//                    (+inf where the row sees no key), and zero for the row's
//                    fp32 dQ accumulator.
//   attn_bwd_kernel  one workgroup per (key block, KV head, batch): key blocks
//                    outside, the query blocks that see them inside
//                    ([FA-tiling] §3.4, get_m_block_min_max). Its K and V rows
//                    stay in registers, and so do the dK and dV accumulators of
//                    those rows, summed over the G query heads of the group;
//                    each query block recomputes S and P from lse, then
//                    dV += P^T dO, dK += dS^T Q and dQ += dS K on MFMA, the last
//                    added to the fp32 dQ accumulator with atomics ([FA-tiling]
//                    §4.6 names Q, dO and that accumulator as the backward's
//                    working set).
//   bwd_post_kernel  dQ = scale * accumulator, in the output dtype.
//
// The pages print no gradient formulas; the kernels implement the chain rule
// through the softmax: dP = dO V^T, D_i = sum_j P_ij dP_ij = <dO_i, O_i>,
// dS = P (dP - D), dQ = scale dS K, dK = scale dS^T Q, dV = P^T dO.
//
// Citations:
//   [FA-tiling]  "分块策略与调度" (FlashAttention tiling strategy and scheduling)
//
// Matrix-core layout (wave64, 16x16 MFMA tiles; lane = 16 lg + li). Each wave
// owns NKW keys of the workgroup's key block. Per query block of BM = 64 rows:
//   S  [q][key]  = Q . K^T     A = Q rows (LDS), B = K rows (registers)
//   dP [q][key]  = dO . V^T    A = dO rows (LDS), B = V rows (registers)
// so lane (li, lg) holds key li and query rows 4 lg .. 4 lg + 3 of every 16x16
// block, which is the B-operand layout of the two products that contract over
// query rows:
//   dV^T [d][key] += dO^T . P    A = dO columns (LDS transpose reads), B = P
//   dK^T [d][key] += Q^T . dS    A = Q columns, B = dS
// dS^T goes to LDS, and after a barrier each wave computes 16 rows of
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

template <class T, int D, int NKW>
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
    static constexpr int K_BYTES = BN * QST * ESZ;
    static constexpr int S_BYTES = BN * SST * ESZ;
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
// pre-pass: D = <dO, O> per row, lse in log2 units, zero dQ accumulator
// ---------------------------------------------------------------------------
template <class T, int D>
__global__ void __launch_bounds__(256) bwd_pre_kernel(BwdParams p) {
    constexpr int CE = 16 / (int)sizeof(T);
    constexpr int TPR = D / CE;  // threads per row (8, 16 or 32; divides 64)
    constexpr int RPB = 256 / TPR;
    const long long rows = (long long)p.B * p.Sq * p.Hq;
    const long long row = (long long)blockIdx.x * RPB + threadIdx.x / TPR;
    const int c = threadIdx.x % TPR;
    float dot = 0.f;
    if (row < rows) {
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
        float* acc = p.dq_acc + row * D + c * CE;
#pragma unroll
        for (int e = 0; e < CE; e += 4) *reinterpret_cast<f32x4*>(acc + e) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int off = TPR / 2; off >= 1; off >>= 1) dot += __shfl_xor(dot, off, 64);
    if (row < rows && c == 0) {
        const int h = (int)(row % p.Hq);
        const int i = (int)((row / p.Hq) % p.Sq);
        const int b = (int)(row / ((long long)p.Hq * p.Sq));
        const size_t idx = ((size_t)b * p.Hq + h) * p.Sq + i;
        const float l = p.lse[idx];
        p.dsum[idx] = dot;
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
template <class T, int D, int NKW, int OCC>
__global__ void __launch_bounds__(256, OCC) attn_bwd_kernel(BwdParams p) {
    using C = BwdTile<T, D, NKW>;
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
    if (total > 0) {
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
                u32x4 pb[NT], sb[NT];
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    pb[t] = u32x4{pack_bf16x2(sacc[2 * pp][t][0], sacc[2 * pp][t][1]),
                                  pack_bf16x2(sacc[2 * pp][t][2], sacc[2 * pp][t][3]),
                                  pack_bf16x2(sacc[2 * pp + 1][t][0], sacc[2 * pp + 1][t][1]),
                                  pack_bf16x2(sacc[2 * pp + 1][t][2], sacc[2 * pp + 1][t][3])};
                    sb[t] = u32x4{pack_bf16x2(pacc[2 * pp][t][0], pacc[2 * pp][t][1]),
                                  pack_bf16x2(pacc[2 * pp][t][2], pacc[2 * pp][t][3]),
                                  pack_bf16x2(pacc[2 * pp + 1][t][0], pacc[2 * pp + 1][t][1]),
                                  pack_bf16x2(pacc[2 * pp + 1][t][2], pacc[2 * pp + 1][t][3])};
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
                        dkT[u][t] = mfma_bf16(qa, sb[t], dkT[u][t]);
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

        // dS^T -> LDS: key row kw0 + 16 t + li, query rows 16 qb + 4 lg .. +3
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                T* dst = dSt + (kw0 + 16 * t + li) * SST + 16 * qb + 4 * lg;
                if constexpr (BF) {
                    *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(pacc[qb][t][0], pacc[qb][t][1]),
                                                           pack_bf16x2(pacc[qb][t][2], pacc[qb][t][3])};
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
#pragma unroll
                for (int u = 0; u < D / 16; ++u) {
                    const u32x2 b0 = lds_read_tr16(Ks + ka * QST + 16 * u + 4 * (li & 3));
                    const u32x2 b1 = lds_read_tr16(Ks + (ka + 4) * QST + 16 * u + 4 * (li & 3));
                    const u32x4 kb = {b0[0], b0[1], b1[0], b1[1]};
                    dqa[u] = mfma_bf16(sa, kb, dqa[u]);
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

    // ---- dK = scale dK^T^T, dV: lane holds d = 16u + 4lg .. +3 of key kw0 + 16t + li
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
// launchers and the variant table
// ---------------------------------------------------------------------------
template <class T, int D>
hipError_t launch_bwd_pre(const BwdParams& p, hipStream_t stream) {
    constexpr int TPR = D / (16 / (int)sizeof(T));
    const long long rows = (long long)p.B * p.Sq * p.Hq;
    const long long blocks = (rows + 256 / TPR - 1) / (256 / TPR);
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, stream, p);
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

template <class T, int D, int NKW, int OCC>
hipError_t launch_bwd(const BwdParams& p, hipStream_t stream) {
    const long long grid = (long long)p.num_n_blocks * p.Hkv * p.B;
    if (grid == 0) return hipSuccess;
    hipLaunchKernelGGL((attn_bwd_kernel<T, D, NKW, OCC>), dim3((unsigned)grid), dim3(256), 0, stream, p);
    return hipGetLastError();
}

#define TPA_BWD_VARIANT(T, DT, D, NKW, OCC)                                                   \
    {DT, D, BwdTile<T, D, NKW>::BN, BwdTile<T, D, NKW>::BM, BwdTile<T, D, NKW>::LDS_BYTES, \
     &launch_bwd<T, D, NKW, OCC>, &launch_bwd_pre<T, D>, &launch_bwd_post<T, D>}

// bf16: 64-key blocks (16 keys per wave), two workgroups per CU; fp32: 64-key
// blocks, one workgroup per CU (its tiles take 117 KB of LDS).
static const BwdVariant kBwdVariants[] = {
    TPA_BWD_VARIANT(bf16_t, DT_BF16, 128, 16, 2),
    TPA_BWD_VARIANT(bf16_t, DT_BF16, 64, 16, 2),
    TPA_BWD_VARIANT(bf16_t, DT_BF16, 128, 32, 1),
    TPA_BWD_VARIANT(bf16_t, DT_BF16, 64, 32, 1),
    TPA_BWD_VARIANT(float, DT_FP32, 128, 16, 1),
    TPA_BWD_VARIANT(float, DT_FP32, 64, 16, 1),
    {0, 0, 0, 0, 0, nullptr, nullptr, nullptr},
};

const BwdVariant* bwd_variants() { return kBwdVariants; }

}  // namespace tpa
