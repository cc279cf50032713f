// attn_device.h -- gfx950 device helpers shared by the attention kernels:
// MFMA wrappers, bf16 conversion, cross-lane reductions, the LDS transpose read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

typedef uint16_t bf16_t;  // bf16 storage (raw bits)

// D[16x16] += A[16x32] . B[32x16], bf16 inputs, fp32 accumulate. Lane l supplies
// A[l % 16][k(l / 16, e)] and B[k(l / 16, e)][l % 16] for its 8 elements e, and
// holds D[4 (l / 16) + r][l % 16] for r = 0..3.
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// fp32 16x16x4: lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16].
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// fp32 -> bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2 v;
    v[0] = (__bf16)lo;
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

// A pair of values as two bf16 parts, x ~= hi + lo: returns {hi pair, lo pair}.
__device__ __forceinline__ u32x2 split_bf16x2(float a, float b) {
    const uint32_t hi = pack_bf16x2(a, b);
    const uint32_t lo = pack_bf16x2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
    return u32x2{hi, lo};
}

// Eight fp32 values (a[0..3], then b[0..3]) as bf16 hi and lo parts, x ~= hi + lo
// to about 16 significant bits, each packed in pairs in that order: the B operand
// of a 16x16x32 bf16 MFMA twice over (one product with hi, one with lo).
__device__ __forceinline__ void split_bf16x8(f32x4 a, f32x4 b, u32x4& hi, u32x4& lo) {
    const u32x2 w0 = split_bf16x2(a[0], a[1]), w1 = split_bf16x2(a[2], a[3]);
    const u32x2 w2 = split_bf16x2(b[0], b[1]), w3 = split_bf16x2(b[2], b[3]);
    hi = u32x4{w0[0], w1[0], w2[0], w3[0]};
    lo = u32x4{w0[1], w1[1], w2[1], w3[1]};
}

// Cross-lane moves without the LDS crossbar. v_permlane16_swap(v, v) returns a
// pair whose elements are {v[l], v[l ^ 16]} in some order for every lane l (and
// v_permlane32_swap likewise for l ^ 32), so combining the pair reduces over
// that lane bit. DPP quad_perm / row_half_mirror / row_mirror pair lanes inside
// quads, half-rows and rows of 16.
__device__ __forceinline__ uint32_t f2u(float x) { return __float_as_uint(x); }

// NaN-propagating maximum. fmaxf must quiet signalling NaNs, so the compiler puts
// a canonicalising v_max_f32 x, x in front of every operand it cannot prove
// canonical (MFMA results, lane moves); this form needs none, and a chain
// max(max(m, a), b) folds into one v_maximum3_f32.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float u2f(uint32_t x) { return __uint_as_float(x); }
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return u2f((uint32_t)__builtin_amdgcn_mov_dpp((int)f2u(x), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp(int x) {
    return __builtin_amdgcn_mov_dpp(x, CTRL, 0xf, 0xf, false);
}
constexpr int DPP_QUAD_1032 = 0xB1, DPP_QUAD_2301 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140;

__device__ __forceinline__ float max16(float x) {  // max over lanes l, l ^ 16
    auto r = __builtin_amdgcn_permlane16_swap(f2u(x), f2u(x), false, false);
    return vmax(u2f(r[0]), u2f(r[1]));
}
__device__ __forceinline__ float max32(float x) {  // max over lanes l, l ^ 32
    auto r = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
    return vmax(u2f(r[0]), u2f(r[1]));
}
__device__ __forceinline__ float sum16(float x) {
    auto r = __builtin_amdgcn_permlane16_swap(f2u(x), f2u(x), false, false);
    return u2f(r[0]) + u2f(r[1]);
}
__device__ __forceinline__ float sum32(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(f2u(x), f2u(x), false, false);
    return u2f(r[0]) + u2f(r[1]);
}

// Reductions over the four lanes i, i+16, i+32, i+48 that share a query column.
__device__ __forceinline__ float xor_max(float x) { return max32(max16(x)); }
__device__ __forceinline__ float xor_sum(float x) { return sum32(sum16(x)); }

// Reductions over the 16 lanes of a row (lanes with equal l / 16).
__device__ __forceinline__ float row16_max(float x) {
    x = vmax(x, dpp<DPP_QUAD_1032>(x));
    x = vmax(x, dpp<DPP_QUAD_2301>(x));
    x = vmax(x, dpp<DPP_HALF_MIRROR>(x));
    return vmax(x, dpp<DPP_MIRROR>(x));
}
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp<DPP_QUAD_1032>(x);
    x += dpp<DPP_QUAD_2301>(x);
    x += dpp<DPP_HALF_MIRROR>(x);
    return x + dpp<DPP_MIRROR>(x);
}
__device__ __forceinline__ int row16_imax(int x) {
    x = max(x, dpp<DPP_QUAD_1032>(x));
    x = max(x, dpp<DPP_QUAD_2301>(x));
    x = max(x, dpp<DPP_HALF_MIRROR>(x));
    return max(x, dpp<DPP_MIRROR>(x));
}
__device__ __forceinline__ int row16_imin(int x) {
    x = min(x, dpp<DPP_QUAD_1032>(x));
    x = min(x, dpp<DPP_QUAD_2301>(x));
    x = min(x, dpp<DPP_HALF_MIRROR>(x));
    return min(x, dpp<DPP_MIRROR>(x));
}
// Whole-wave (64 lane) reductions.
__device__ __forceinline__ float wave_max(float x) { return xor_max(row16_max(x)); }
__device__ __forceinline__ float wave_sum(float x) { return xor_sum(row16_sum(x)); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Raw buffer resource over [base, base + bytes): a buffer load whose offset is at
// or beyond `bytes` returns zeros instead of touching memory, so ragged tiles
// need no branches. base must be uniform across the wave.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// The same for a base and size the caller knows to be wave-uniform but the
// compiler may hold in VGPRs (e.g. after v_med3 / v_min): read from the first
// lane, so buffer instructions get scalar operands instead of a waterfall loop.
__device__ __forceinline__ rsrc_t make_rsrc_u(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return make_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo),
                     __builtin_amdgcn_readfirstlane(bytes));
}
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}
// The same with the non-temporal hint (cache policy bit 1: nt), for data read once.
__device__ __forceinline__ u32x4 buf_load16_nt(rsrc_t r, uint32_t byte_off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 2));
}

// The same resource as four raw words (base, stride 0, size in bytes, the
// format word make_rsrc uses), read from the first lane, for buffer
// instructions issued by inline asm.
__device__ __forceinline__ u32x4 rsrc_words_u(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    u32x4 w;
    w[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
    w[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) & 0xffffu;
    w[2] = __builtin_amdgcn_readfirstlane(bytes);
    w[3] = 0x00020000u;
    return w;
}

// Global -> LDS copy of 16 bytes per lane (buffer_load_dwordx4 ... lds): lane l
// reads the buffer at byte voff and writes LDS bytes [lds + 16 l, +16); lds is
// the wave-uniform LDS byte address. Issued from inline asm, so the compiler
// does not track it. The compiler's own tracking of such copies is coarse: a
// `ds_read_b64_tr_b16` (whose memory operand carries no alias information)
// waits for every copy in flight, including one that fills a different buffer,
// which serialises a prefetch with the reads of the buffer in use. Callers of
// this form order everything themselves: an explicit s_waitcnt vmcnt before
// the first LDS read of what a copy fills (vmcnt retires in issue order,
// counting these copies with every other vector memory load), and an
// lgkmcnt(0) wait before a copy overwrites LDS that reads may still use. The
// compiler's own waits for its tracked loads stay correct (they only grow
// stricter when these copies are in flight too). The copies carry the
// non-temporal hint (nt): decode streams K and V once, and without the hint
// they displace lines that are read again soon. The LDS address goes in M0
// (an operand the compiler sets); the s_nop covers the wait states between a
// VALU write of an SGPR operand (v_readfirstlane) or of M0 and a vector memory
// instruction that reads it.
__device__ __forceinline__ void dma16_untracked(u32x4 rs, uint32_t voff, uint32_t lds) {
    asm volatile(
        "s_nop 4\n\t"
        "buffer_load_dwordx4 %0, %1, 0 offen nt lds"
        :
        : "v"(voff), "s"(rs), "{m0}"(lds)
        : "memory");
}
// The same copy without the non-temporal hint, for tiles that other workgroups
// read again soon from L2 (the prefill's K tiles are shared by a head's query
// blocks).
__device__ __forceinline__ void dma16_untracked_cached(u32x4 rs, uint32_t voff, uint32_t lds) {
    asm volatile(
        "s_nop 4\n\t"
        "buffer_load_dwordx4 %0, %1, 0 offen lds"
        :
        : "v"(voff), "s"(rs), "{m0}"(lds)
        : "memory");
}
// 4 bytes per lane (buffer_load_dword ... lds): lane l writes LDS bytes
// [lds + 4 l, +4).
__device__ __forceinline__ void dma4_untracked_cached(u32x4 rs, uint32_t voff, uint32_t lds) {
    asm volatile(
        "s_nop 4\n\t"
        "buffer_load_dword %0, %1, 0 offen lds"
        :
        : "v"(voff), "s"(rs), "{m0}"(lds)
        : "memory");
}
// s_waitcnt written as a compiler memory barrier (no load or store moves across
// it), for the copies above that the compiler does not track
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt field");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkmcnt0() { asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory"); }
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// LDS transpose read (ds_read_b64_tr_b16). Within each 16-lane group, lane s
// supplies an 8-byte address; lane n receives element k = 0..3 from source lane
// 4k + n/4, element n % 4. With source lane s pointing at row k0 + s/4, columns
// c0 + 4 (s % 4) .. +3 of a row-major 16-bit matrix, lane n receives
// M[k0 + k][c0 + n] for k = 0..3.
__device__ __forceinline__ u32x2 lds_read_tr16(const bf16_t* p) {
    i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
    return __builtin_bit_cast(u32x2, r);
}

// ---- fp16 operands (the P.V product of the bf16 prefill kernels) ----------
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
// fp32 pair -> fp16 pair, round to nearest even (v_cvt_pk_f16_f32)
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    f16x2 v;
    v[0] = (_Float16)lo;
    v[1] = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, v);
}
// two bf16 (one 32-bit word) -> two fp16, exact for |x| <= 65504
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
    return pack_f16x2(__uint_as_float(w << 16), __uint_as_float(w & 0xffff0000u));
}

// Workgroups of a one-dimensional grid are dealt round-robin to the 8 XCDs of
// an MI355X (workgroup i runs on XCD i % 8).
constexpr int NUM_XCD = 8;

}  // namespace tpa
