// gemv_impl.h - fused quantized GEMV for decode: y = W x for 1..8 fp32 columns
// (device code and launch templates; instantiated per column count).
//
// What is computed follows dequantize_mul_mat_vec ("dmmv", named with its
// tuning block in the "llama_cpp 0.12.1 -> 0.12.2" ggml-cuda.cu diff) and the
// ggml_cuda_op_mul_mat driver (a row range times a column count): each output
// is the dot product of one dequantized weight row with one activation column,
// reduced across lanes (the diff's warp_reduce_sum).  That kernel's body is not
// on the page; this one is designed for gfx950.
//
// Work split.  A workgroup of WPG waves owns a group of consecutive rows.  K
// is walked in chunks of pairs of blocks: a pair of Q4_0 / Q4_1 / Q8_0 /
// Q5_0 / Q5_1 blocks is 36 / 40 / 68 / 44 / 48 bytes, a whole number of
// dwords, so with an even block count
// per row every pair starts on 4 bytes and comes straight into registers with
// dword-aligned 16-byte loads (plain loads: streaming hints measured slower on
// this chip).  For rows of more than 32 pairs a wave owns RWV rows and lane p
// takes pair p of each 64-pair (4096-weight) chunk; shorter rows (one column
// only) cut the wave into 2, 4 or 8 segments of 32, 16 or 8 lanes, one row
// each, so a row of 2048 or 768 weights does not leave most lanes idle.
//
// Activations are the expensive side: every row needs all of x.  The chunk of
// x (4096 x NC floats) is copied once per workgroup into LDS and read from
// there by all of its rows; its global loads are issued before the weight
// loads so the copy never waits behind HBM.  In LDS each run of 64 floats is
// followed by 4 floats of padding, so the 16-byte reads of lanes p = 0..15 (at
// float offset 68p + 4t) fall in distinct banks.  A workgroup takes a range
// of consecutive row groups (of one or several problems of a grouped or
// expert-indexed launch) and restages x only when a step enters a new problem
// or window.
//
// Arithmetic, exact per term (every term is the exact weight times x):
//  * Q4_0: the nibble becomes the exact fp16 number q - 8 by placing it in
//    the mantissa of an fp16 with a byte permute (0x64XX is 1024 + XX) and
//    removing the bias with one packed fp16 add; v_fma_mix_f32 multiplies that
//    fp16 by the fp32 activation into an fp32 accumulator with one rounding.
//    The block's sum is scaled by d once (d * (q - 8) is the exact weight).
//  * Q8_0: the signed byte converts to fp32 exactly with a byte-select
//    convert and is multiplied by x in one FMA; the block's sum is scaled by d.
//  * Q4_1: the exact fp32 weight d*q + m is rebuilt per element (one FMA,
//    exact because d*q is exact) and multiplied into the accumulator.
//  * Q5_0 / Q5_1: as Q4_0 / Q4_1 with 5-bit codes, bit 4 of each taken from
//    the block's qh word (q - 16 is exact in fp16 as well).
// Reduction: a 64-lane DPP butterfly per (row, column); lane 0 writes y.
#pragma once

#include "gemv.h"
#include "qk_common.h"
#include "qk_internal.h"

#include <type_traits>

namespace qk {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
// 16 activation bytes at a 4-byte aligned address (one dwordx4 load).
typedef float f32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

template <int FMT> struct Pair;
template <> struct Pair<QK_Q4_0> { static constexpr int kDwords = 9; };
template <> struct Pair<QK_Q4_1> { static constexpr int kDwords = 10; };
template <> struct Pair<QK_Q8_0> { static constexpr int kDwords = 17; };
template <> struct Pair<QK_Q5_0> { static constexpr int kDwords = 11; };
template <> struct Pair<QK_Q5_1> { static constexpr int kDwords = 12; };

// Formats whose weight is d*q + m (rebuilt exactly in fp32 per element).
template <int FMT> constexpr bool kHasM = FMT == QK_Q4_1 || FMT == QK_Q5_1;
// Formats whose block sum is scaled by d once (codes exact as small numbers).
template <int FMT> constexpr bool kNibbleOffset = FMT == QK_Q4_0 || FMT == QK_Q5_0;

// acc + (fp16 in the low / high half of h) * x, fused, one rounding.
__device__ __forceinline__ float fma_mix_lo(uint32_t h, float x, float acc) {
    float r;
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(x), "v"(acc));
    return r;
}
__device__ __forceinline__ float fma_mix_hi(uint32_t h, float x, float acc) {
    float r;
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
        : "=v"(r) : "v"(h), "v"(x), "v"(acc));
    return r;
}

// Bytes 0,1 (lo) or 2,3 (hi) of src become the low mantissa bytes of two fp16
// numbers with high byte 0x64: value 1024 + byte.
__device__ __forceinline__ uint32_t bytes_to_f16_lo(uint32_t src) {
    return __builtin_amdgcn_perm(0x64646464u, src, 0x04010400u);  // [b0, 64, b1, 64]
}
__device__ __forceinline__ uint32_t bytes_to_f16_hi(uint32_t src) {
    return __builtin_amdgcn_perm(0x64646464u, src, 0x04030402u);  // [b2, 64, b3, 64]
}

__device__ __forceinline__ uint32_t pk_add_f16(uint32_t a, float b) {
    const half2_t r = __builtin_bit_cast(half2_t, a) + half2_t{(_Float16)b, (_Float16)b};
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ uint32_t pk_fma_f16(uint32_t a, float s, float t) {
    const half2_t r = __builtin_elementwise_fma(__builtin_bit_cast(half2_t, a),
                                                half2_t{(_Float16)s, (_Float16)s},
                                                half2_t{(_Float16)t, (_Float16)t});
    return __builtin_bit_cast(uint32_t, r);
}

// 32-bit word starting 2 bytes into (lo, hi).
__device__ __forceinline__ uint32_t shift2(uint32_t lo, uint32_t hi) {
    return __builtin_amdgcn_alignbyte(hi, lo, 2);
}

// ---------------------------------------------------------------------------
// One pair (two consecutive blocks) of a row in registers.
// ---------------------------------------------------------------------------

// FAST: the pair starts on a 4-byte boundary and both blocks exist.
template <int FMT>
__device__ __forceinline__ void load_pair_fast(const uint8_t *__restrict__ p,
                                               uint32_t (&v)[Pair<FMT>::kDwords]) {
    constexpr int N = Pair<FMT>::kDwords;
#pragma unroll
    for (int i = 0; i + 4 <= N; i += 4) {
        const u32x4_a4 t = *reinterpret_cast<const u32x4_a4 *>(p + 4 * i);
        v[i] = t.x; v[i + 1] = t.y; v[i + 2] = t.z; v[i + 3] = t.w;
    }
#pragma unroll
    for (int i = N & ~3; i < N; ++i)
        v[i] = *reinterpret_cast<const uint32_t *>(p + 4 * i);
}

// Generic: 2-byte aligned; if only the first block exists (odd block count,
// last pair) the second block reads as d = m = 0 and codes 0, i.e. weights 0.
template <int FMT>
__device__ __forceinline__ void load_pair_generic(const uint8_t *__restrict__ p, bool second,
                                                  uint32_t (&v)[Pair<FMT>::kDwords]) {
    constexpr int N = Pair<FMT>::kDwords;
    constexpr int BS = Format<FMT>::kBytes;
    const uint16_t *h = reinterpret_cast<const uint16_t *>(p);
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const uint32_t a = (4 * i < BS || second) ? (uint32_t)h[2 * i] : 0u;
        const uint32_t b = (4 * i + 2 < BS || second) ? (uint32_t)h[2 * i + 1] : 0u;
        v[i] = a | (b << 16);
    }
}

// Generic, whole dwords: a pair that starts 2 bytes past a dword boundary
// (rows of an odd block count, or a 2-byte aligned matrix) is read as the
// ND + 1 dwords from the boundary below it and shifted into place.  Reads
// from 2 bytes before p (inside p's own dword) to kPairReach bytes after it;
// if only the first block exists the second block's words are junk, which
// the caller ignores.
template <int FMT> constexpr int kPairReach = 4 * (Pair<FMT>::kDwords + 1);

template <int FMT>
__device__ __forceinline__ void load_pair_shift(const uint8_t *__restrict__ p,
                                                uint32_t (&v)[Pair<FMT>::kDwords]) {
    constexpr int N = Pair<FMT>::kDwords + 1;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    const uint8_t *base = reinterpret_cast<const uint8_t *>(a & ~uintptr_t(3));
    const uint32_t sh = (uint32_t)(a & 3);
    uint32_t d[N];
#pragma unroll
    for (int i = 0; i + 4 <= N; i += 4) {
        const u32x4_a4 t = *reinterpret_cast<const u32x4_a4 *>(base + 4 * i);
        d[i] = t.x; d[i + 1] = t.y; d[i + 2] = t.z; d[i + 3] = t.w;
    }
#pragma unroll
    for (int i = N & ~3; i < N; ++i) d[i] = *reinterpret_cast<const uint32_t *>(base + 4 * i);
#pragma unroll
    for (int i = 0; i < N - 1; ++i) v[i] = __builtin_amdgcn_alignbyte(d[i + 1], d[i], sh);
}

// fp16 bits of d (and m) of block b of the pair.  Block 1 starts at byte 18
// (Q4_0), 20 (Q4_1), 34 (Q8_0), 22 (Q5_0) or 24 (Q5_1).
template <int FMT>
__device__ __forceinline__ uint32_t pair_d(const uint32_t (&v)[Pair<FMT>::kDwords], int b) {
    if constexpr (FMT == QK_Q4_0) return b == 0 ? (v[0] & 0xFFFFu) : (v[4] >> 16);
    if constexpr (FMT == QK_Q4_1) return b == 0 ? (v[0] & 0xFFFFu) : (v[5] & 0xFFFFu);
    if constexpr (FMT == QK_Q5_0) return b == 0 ? (v[0] & 0xFFFFu) : (v[5] >> 16);
    if constexpr (FMT == QK_Q5_1) return b == 0 ? (v[0] & 0xFFFFu) : (v[6] & 0xFFFFu);
    return b == 0 ? (v[0] & 0xFFFFu) : (v[8] >> 16);
}
template <int FMT>
__device__ __forceinline__ uint32_t pair_m(const uint32_t (&v)[Pair<FMT>::kDwords], int b) {
    static_assert(kHasM<FMT>, "d*q + m formats");
    if constexpr (FMT == QK_Q4_1) return b == 0 ? (v[0] >> 16) : (v[5] >> 16);
    return b == 0 ? (v[0] >> 16) : (v[6] >> 16);
}

// Quant word i of block b (Q4 / Q5: i < 4, bytes 4i..4i+3 of qs; Q8: i < 8).
template <int FMT>
__device__ __forceinline__ uint32_t pair_qs(const uint32_t (&v)[Pair<FMT>::kDwords], int b, int i) {
    if constexpr (FMT == QK_Q4_0) return b == 0 ? shift2(v[i], v[i + 1]) : v[5 + i];
    if constexpr (FMT == QK_Q4_1) return b == 0 ? v[1 + i] : v[6 + i];
    if constexpr (FMT == QK_Q5_0) return b == 0 ? shift2(v[1 + i], v[2 + i]) : v[7 + i];
    if constexpr (FMT == QK_Q5_1) return b == 0 ? v[2 + i] : v[8 + i];
    return b == 0 ? shift2(v[i], v[i + 1]) : v[9 + i];
}

// Q5: the qh word of block b (bit t = bit 4 of code t).
template <int FMT>
__device__ __forceinline__ uint32_t pair_qh(const uint32_t (&v)[Pair<FMT>::kDwords], int b) {
    if constexpr (FMT == QK_Q5_0) return b == 0 ? shift2(v[0], v[1]) : v[6];
    else return b == 0 ? v[1] : v[7];
}

// The codes of quant word i of block b as bytes: lo = elements 4i..4i+3,
// hi = elements 16+4i..16+4i+3 (Q4: 0..15; Q5: 0..31 with bit 4 from qh).
template <int FMT>
__device__ __forceinline__ void pair_codes(const uint32_t (&v)[Pair<FMT>::kDwords], int b, int i,
                                           uint32_t &lo, uint32_t &hi) {
    const uint32_t qw = pair_qs<FMT>(v, b, i);
    lo = qw & 0x0F0F0F0Fu;
    hi = (qw >> 4) & 0x0F0F0F0Fu;
    if constexpr (FMT == QK_Q5_0 || FMT == QK_Q5_1) {
        const uint32_t qh = pair_qh<FMT>(v, b);
        lo |= q5_high4((qh >> (4 * i)) & 0xFu);
        hi |= q5_high4((qh >> (16 + 4 * i)) & 0xFu);
    }
}

// ---------------------------------------------------------------------------
// Per-group products.  A group is quant word i of block b: Q4 elements
// 4i..4i+3 (low nibbles) and 16+4i..16+4i+3 (high nibbles); Q8 elements
// 4i..4i+3 (i < 8).  xa / xb are the matching activations.
// ---------------------------------------------------------------------------

// Q4_0 group: sum over the 8 elements of (q - 8) * x, added to s.  Each
// fp16 pair is masked straight out of the quant word into the mantissas of
// 0x6400 6400 (one and-or): the low nibbles of bytes 0 and 2 (elements 0
// and 2) and, from the word shifted by a byte, of bytes 1 and 3 give
// 1024 + c, and c - 8 after subtracting 1032; the high nibbles are taken in
// place (1024 + 16c), and (1024 + 16c) / 16 - 72 = c - 8 is one fused,
// exact operation.
__device__ __forceinline__ float group_q4_0(uint32_t qw, const float4 &xa, const float4 &xb, float s) {
    // (v_bitop3 with truth table 0xEA is (a & b) | c: one instruction)
    auto mask_or = [](uint32_t a, uint32_t m) { return __builtin_amdgcn_bitop3_b32(a, m, 0x64006400u, 0xEA); };
    const uint32_t qs = qw >> 8;
    const uint32_t l02 = pk_add_f16(mask_or(qw, 0x000F000Fu), -1032.0f);
    const uint32_t l13 = pk_add_f16(mask_or(qs, 0x000F000Fu), -1032.0f);
    const uint32_t h02 = pk_fma_f16(mask_or(qw, 0x00F000F0u), 0.0625f, -72.0f);
    const uint32_t h13 = pk_fma_f16(mask_or(qs, 0x00F000F0u), 0.0625f, -72.0f);
    s = fma_mix_lo(l02, xa.x, s);
    s = fma_mix_lo(l13, xa.y, s);
    s = fma_mix_hi(l02, xa.z, s);
    s = fma_mix_hi(l13, xa.w, s);
    s = fma_mix_lo(h02, xb.x, s);
    s = fma_mix_lo(h13, xb.y, s);
    s = fma_mix_hi(h02, xb.z, s);
    s = fma_mix_hi(h13, xb.w, s);
    return s;
}

// Q8_0 group: sum over 4 elements of q * x, added to s.  A signed byte
// converts to fp32 exactly in one instruction (byte-select SDWA), and the
// product q * x is rounded once inside the FMA.
__device__ __forceinline__ float group_q8_0(uint32_t qw, const float4 &xa, float s) {
    s = __builtin_fmaf((float)(int8_t)(qw), xa.x, s);
    s = __builtin_fmaf((float)(int8_t)(qw >> 8), xa.y, s);
    s = __builtin_fmaf((float)(int8_t)(qw >> 16), xa.z, s);
    s = __builtin_fmaf((float)(int8_t)(qw >> 24), xa.w, s);
    return s;
}

// Q8_0 group of block 0 of a pair: its quant word straddles two dwords
// (bytes 2, 3 of lo and 0, 1 of hi), which byte selects read directly.
__device__ __forceinline__ float group_q8_0_split(uint32_t lo, uint32_t hi, const float4 &xa, float s) {
    s = __builtin_fmaf((float)(int8_t)(lo >> 16), xa.x, s);
    s = __builtin_fmaf((float)(int8_t)(lo >> 24), xa.y, s);
    s = __builtin_fmaf((float)(int8_t)(hi), xa.z, s);
    s = __builtin_fmaf((float)(int8_t)(hi >> 8), xa.w, s);
    return s;
}

// Q5_0 group: sum over the 8 elements of (q - 16) * x, added to s; lo / hi
// hold the 5-bit codes of elements 4i..4i+3 and 16+4i..16+4i+3 as bytes
// (1024 + q - 1040 = q - 16, exact in fp16).
__device__ __forceinline__ float group_q5_0(uint32_t lo, uint32_t hi, const float4 &xa, const float4 &xb,
                                            float s) {
    const uint32_t l01 = pk_add_f16(bytes_to_f16_lo(lo), -1040.0f);
    const uint32_t l23 = pk_add_f16(bytes_to_f16_hi(lo), -1040.0f);
    const uint32_t h01 = pk_add_f16(bytes_to_f16_lo(hi), -1040.0f);
    const uint32_t h23 = pk_add_f16(bytes_to_f16_hi(hi), -1040.0f);
    s = fma_mix_lo(l01, xa.x, s);
    s = fma_mix_hi(l01, xa.y, s);
    s = fma_mix_lo(l23, xa.z, s);
    s = fma_mix_hi(l23, xa.w, s);
    s = fma_mix_lo(h01, xb.x, s);
    s = fma_mix_hi(h01, xb.y, s);
    s = fma_mix_lo(h23, xb.z, s);
    s = fma_mix_hi(h23, xb.w, s);
    return s;
}

// Q4_1 group: exact weights d*q + m times x, added to acc.
__device__ __forceinline__ float group_q4_1(uint32_t qw, float d, float mm, const float4 &xa,
                                            const float4 &xb, float a) {
    const uint32_t lo = qw & 0x0F0F0F0Fu;
    const uint32_t hi = (qw >> 4) & 0x0F0F0F0Fu;
    a = __builtin_fmaf(wval(d, ubyte_f<0>(lo), mm), xa.x, a);
    a = __builtin_fmaf(wval(d, ubyte_f<1>(lo), mm), xa.y, a);
    a = __builtin_fmaf(wval(d, ubyte_f<2>(lo), mm), xa.z, a);
    a = __builtin_fmaf(wval(d, ubyte_f<3>(lo), mm), xa.w, a);
    a = __builtin_fmaf(wval(d, ubyte_f<0>(hi), mm), xb.x, a);
    a = __builtin_fmaf(wval(d, ubyte_f<1>(hi), mm), xb.y, a);
    a = __builtin_fmaf(wval(d, ubyte_f<2>(hi), mm), xb.z, a);
    a = __builtin_fmaf(wval(d, ubyte_f<3>(hi), mm), xb.w, a);
    return a;
}

// float4 of x (column j) at window-relative element e (e % 4 == 0) from LDS;
// column pitch xp floats.
__device__ __forceinline__ float4 x_lds(const float *xs, int xp, int j, int e) {
    return *reinterpret_cast<const float4 *>(xs + j * xp + e + (e >> 6) * 4);
}

// Split of the launch's `total` row groups over the grid: workgroup b takes
// per groups, plus one more if b < rem (computed on the host; no division on
// the device).
struct GemvSplit {
    int total;
    int per;
    int rem;
    int gpi;  // row groups per problem (expert-indexed launches)
};

// Dot products of one wave's RWV rows with this lane's pair, added to acc.
template <int FMT, int NC, int RWV, bool FAST>
__device__ __forceinline__ void pair_dot(const uint32_t (&v)[RWV][Pair<FMT>::kDwords], int nrows,
                                         bool second, const float *xs, int xp, int el,
                                         float (&acc)[RWV][NC]) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        if (!FAST && b == 1 && !second) break;
        if constexpr (kHasM<FMT>) {
            // d and m converted to fp32 once per block and held opaque, so each
            // weight is one fp32 FMA (left to itself the compiler folded the
            // conversions into a mixed-precision FMA per weight, a slower
            // instruction); the code words are opaque too, so each nibble
            // converts with one byte-select convert instead of a field extract
            // and a convert.  The weights are the same exact fp32 values.
            float dd[RWV], mv[RWV];
#pragma unroll
            for (int r = 0; r < RWV; ++r) {
                dd[r] = h2f(pair_d<FMT>(v[r], b));
                mv[r] = h2f(pair_m<FMT>(v[r], b));
                asm volatile("" : "+v"(dd[r]), "+v"(mv[r]));
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float4 xa[NC], xb[NC];
#pragma unroll
                for (int j = 0; j < NC; ++j) {
                    xa[j] = x_lds(xs, xp, j, el + 32 * b + 4 * i);
                    xb[j] = x_lds(xs, xp, j, el + 32 * b + 16 + 4 * i);
                }
#pragma unroll
                for (int r = 0; r < RWV; ++r) {
                    if (FAST || r < nrows) {  // fast path: rows clamped, stores guarded
                        const float d = dd[r];
                        const float mm = mv[r];
                        uint32_t lo, hi;
                        pair_codes<FMT>(v[r], b, i, lo, hi);
                        asm volatile("" : "+v"(lo), "+v"(hi));
                        const float w0 = wval(d, ubyte_f<0>(lo), mm), w1 = wval(d, ubyte_f<1>(lo), mm);
                        const float w2 = wval(d, ubyte_f<2>(lo), mm), w3 = wval(d, ubyte_f<3>(lo), mm);
                        const float w4 = wval(d, ubyte_f<0>(hi), mm), w5 = wval(d, ubyte_f<1>(hi), mm);
                        const float w6 = wval(d, ubyte_f<2>(hi), mm), w7 = wval(d, ubyte_f<3>(hi), mm);
#pragma unroll
                        for (int j = 0; j < NC; ++j) {
                            float a = acc[r][j];
                            a = __builtin_fmaf(w0, xa[j].x, a);
                            a = __builtin_fmaf(w1, xa[j].y, a);
                            a = __builtin_fmaf(w2, xa[j].z, a);
                            a = __builtin_fmaf(w3, xa[j].w, a);
                            a = __builtin_fmaf(w4, xb[j].x, a);
                            a = __builtin_fmaf(w5, xb[j].y, a);
                            a = __builtin_fmaf(w6, xb[j].z, a);
                            a = __builtin_fmaf(w7, xb[j].w, a);
                            acc[r][j] = a;
                        }
                    }
                }
                // keep the next group's LDS reads from being hoisted above
                // this one (bounds the live activations)
                if constexpr (NC >= 2) asm volatile("" ::: "memory");
            }
        } else {
            float s[RWV][NC];
#pragma unroll
            for (int r = 0; r < RWV; ++r)
#pragma unroll
                for (int j = 0; j < NC; ++j) s[r][j] = 0.0f;
            constexpr int NGRP = (FMT == QK_Q8_0) ? 8 : 4;
#pragma unroll
            for (int i = 0; i < NGRP; ++i) {
                float4 xa[NC], xb[NC];
#pragma unroll
                for (int j = 0; j < NC; ++j) {
                    xa[j] = x_lds(xs, xp, j, el + 32 * b + 4 * i);
                    if (kNibbleOffset<FMT>) xb[j] = x_lds(xs, xp, j, el + 32 * b + 16 + 4 * i);
                }
#pragma unroll
                for (int r = 0; r < RWV; ++r) {
                    if (FAST || r < nrows) {  // fast path: rows clamped, stores guarded
                        uint32_t lo = 0, hi = 0;
                        if constexpr (FMT == QK_Q5_0) pair_codes<FMT>(v[r], b, i, lo, hi);
#pragma unroll
                        for (int j = 0; j < NC; ++j) {
                            if constexpr (FMT == QK_Q4_0) {
                                s[r][j] = group_q4_0(pair_qs<FMT>(v[r], b, i), xa[j], xb[j], s[r][j]);
                            } else if constexpr (FMT == QK_Q5_0) {
                                s[r][j] = group_q5_0(lo, hi, xa[j], xb[j], s[r][j]);
                            } else if (b == 0) {
                                s[r][j] = group_q8_0_split(v[r][i], v[r][i + 1], xa[j], s[r][j]);
                            } else {
                                s[r][j] = group_q8_0(v[r][9 + i], xa[j], s[r][j]);
                            }
                        }
                    }
                }
                if constexpr (NC >= 3) asm volatile("" ::: "memory");
            }
#pragma unroll
            for (int r = 0; r < RWV; ++r) {
                if (FAST || r < nrows) {
                    const float d = h2f(pair_d<FMT>(v[r], b));
#pragma unroll
                    for (int j = 0; j < NC; ++j) acc[r][j] = __builtin_fmaf(d, s[r][j], acc[r][j]);
                }
            }
        }
    }
}

// The activation window staged in LDS: 4096 weights per column, each run of
// 64 floats followed by 4 floats of padding.
constexpr int kGvWindow = kGvChunkElems;
constexpr int kGvPitch = kGvWindow + kGvWindow / 16;

// 8-bit activations in LDS, per column: the codes of pair p of the window at
// byte 80p (64 bytes and 16 of padding, so the 16-byte reads of eight lanes
// cover all 32 banks), then 8 bytes per block: (scale, sum of the codes).
constexpr int kX8PairPitch = 80;
constexpr int kX8ScaleOff = kGvChunkPairs * kX8PairPitch;
constexpr int kX8ColBytes = kX8ScaleOff + 8 * 2 * kGvChunkPairs;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Quantize one block of 32 activations (v) to 8-bit codes with a power-of-two
// scale d = 2^e, e the smallest integer >= -126 with 127 * 2^e >= max|x|, and
// q = x / d rounded half to even (exact decisions: the division by a power of
// two rounds nothing).  Writes the 32 codes to `codes` (16-byte aligned LDS)
// and (d, sum of the codes) to `scale`.  An all-zero block has d = 0; a block
// holding an infinite or NaN value has d = NaN (its codes are then
// meaningless), so every product that uses it is NaN.
__device__ __forceinline__ void x8_block(const f32x4_t (&v)[8], uint8_t *codes, uint8_t *scale) {
    float amax = 0.0f;
    bool finite = true;  // (|x| <= FLT_MAX is false for infinities and NaN)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        amax = fmaxf(fmaxf(fmaxf(amax, fabsf(v[i].x)), fmaxf(fabsf(v[i].y), fabsf(v[i].z))), fabsf(v[i].w));
        finite = finite && fabsf(v[i].x) <= 3.40282347e38f && fabsf(v[i].y) <= 3.40282347e38f &&
                 fabsf(v[i].z) <= 3.40282347e38f && fabsf(v[i].w) <= 3.40282347e38f;
    }
    if (!finite) amax = 0.0f;  // keeps the scale computation below in range
    int ex;
    const float mant = frexpf(amax, &ex);  // amax = mant * 2^ex, mant in [0.5, 1)
    // 127 * 2^(ex-7) >= amax  <=>  mant <= 127/128
    const int e = max(ex - 7 + (mant > 0.9921875f ? 1 : 0), -126);
    const float inv = ldexpf(1.0f, -e);  // exact: 2^-e (e <= 121 here, so inv >= 2^-121)
    // x * 2^-e is exact with |.| <= 127; adding 1.5 * 2^23 rounds it to an
    // integer half to even (one ulp is 1 there), and the low byte of the
    // sum's bits is that integer in two's complement
    constexpr float kMagic = 12582912.0f;
    auto code = [&](float x) -> uint32_t { return __builtin_bit_cast(uint32_t, x * inv + kMagic); };
    uint32_t wd[8];
    int qsum = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t lo = __builtin_amdgcn_perm(code(v[i].y), code(v[i].x), 0x0c0c0400u);  // [q0, q1, 0, 0]
        const uint32_t hi = __builtin_amdgcn_perm(code(v[i].w), code(v[i].z), 0x04000c0cu);  // [0, 0, q2, q3]
        wd[i] = lo | hi;
        qsum = __builtin_amdgcn_sdot4((int)wd[i], 0x01010101, qsum, false);
    }
    *reinterpret_cast<u32x4_t *>(codes) = u32x4_t{wd[0], wd[1], wd[2], wd[3]};
    *reinterpret_cast<u32x4_t *>(codes + 16) = u32x4_t{wd[4], wd[5], wd[6], wd[7]};
    const float d = !finite ? __builtin_nanf("") : (amax == 0.0f ? 0.0f : ldexpf(1.0f, e));
    *reinterpret_cast<u32x2_t *>(scale) = u32x2_t{__builtin_bit_cast(uint32_t, d), (uint32_t)qsum};
}

// Integer-dot products of one wave's RWV rows with this lane's pair (pair pw
// of the window) against 8-bit activations, added to acc: per block and
// column, eight 4-way int8 dot products (exact), then one scaled add,
// d_w * d_x * I (Q4_0 / Q5_0: codes taken as q - 8 / q - 16 through the code
// sum), and for Q4_1 / Q5_1 also m_w * d_x * (sum of the activation codes).
template <int FMT, int NC, int RWV, bool FAST>
__device__ __forceinline__ void pair_dot_x8(const uint32_t (&v)[RWV][Pair<FMT>::kDwords], int nrows,
                                            bool second, const uint8_t *xq, int pw,
                                            float (&acc)[RWV][NC]) {
    constexpr int NW = FMT == QK_Q8_0 ? 8 : 4;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        if (!FAST && b == 1 && !second) break;
        uint32_t wq[RWV][8];
        float dw[RWV], mw[RWV];
#pragma unroll
        for (int r = 0; r < RWV; ++r) {
            dw[r] = h2f(pair_d<FMT>(v[r], b));
            if constexpr (kHasM<FMT>) mw[r] = h2f(pair_m<FMT>(v[r], b));
            else mw[r] = 0.0f;
#pragma unroll
            for (int i = 0; i < NW; ++i) {
                if constexpr (FMT == QK_Q8_0) {
                    wq[r][i] = pair_qs<FMT>(v[r], b, i);
                } else {
                    // elements 4i..4i+3 and 16+4i..16+4i+3
                    pair_codes<FMT>(v[r], b, i, wq[r][i], wq[r][4 + i]);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            const uint8_t *c = xq + j * kX8ColBytes + kX8PairPitch * pw + 32 * b;
            const u32x4_t c0 = *reinterpret_cast<const u32x4_t *>(c);
            const u32x4_t c1 = *reinterpret_cast<const u32x4_t *>(c + 16);
            const u32x2_t sc = *reinterpret_cast<const u32x2_t *>(xq + j * kX8ColBytes + kX8ScaleOff +
                                                                  8 * (2 * pw + b));
            const uint32_t xc[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
            const float dx = __builtin_bit_cast(float, sc.x);
            const int qs = (int)sc.y;
#pragma unroll
            for (int r = 0; r < RWV; ++r) {
                if (FAST || r < nrows) {  // fast path: rows clamped, stores guarded
                    int isum = 0;
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        isum = __builtin_amdgcn_sdot4((int)wq[r][i], (int)xc[i], isum, false);
                    if constexpr (FMT == QK_Q4_0) isum -= 8 * qs;
                    if constexpr (FMT == QK_Q5_0) isum -= 16 * qs;
                    acc[r][j] += (float)isum * (dw[r] * dx);
                    if constexpr (kHasM<FMT>) acc[r][j] += (float)qs * (mw[r] * dx);
                }
            }
            if constexpr (NC >= 3) asm volatile("" ::: "memory");
        }
    }
}

// Lane split of a grouped one-column launch whose problems need different
// splits (each problem then uses the split its own launch would use, so the
// outputs are bitwise those of separate launches).
constexpr int kSubMixed = -1;

// Where a launch's problems come from.
enum GemvSource {
    kSrcOne = 0,     // one problem, passed in its own argument
    kSrcTable = 1,   // a table of up to kGvMaxItems problems
    kSrcExpert = 2,  // expert-indexed problems, ids read on the device
};
template <int SRC> struct GemvSrc;
template <> struct GemvSrc<kSrcOne> { using Args = GemvItem; };
template <> struct GemvSrc<kSrcTable> { using Args = GemvArgs; };
template <> struct GemvSrc<kSrcExpert> { using Args = GemvExpert; };

// Sum over aligned segments of LPR lanes (8, 16, 32 or 64) with DPP.  The
// sum ends in every lane of a segment of 8 or 16 (and of the wave for 64),
// and in the last lane of each 32-lane half for 32 (seg_store_lane).
template <int LPR>
__device__ __forceinline__ float seg_sum(float v) {
    if constexpr (LPR == 64) {
        return wave_sum(v);
    } else {
        v += dpp<0xB1>(v);                                 // quad_perm [1,0,3,2]
        v += dpp<0x4E>(v);                                 // quad_perm [2,3,0,1]
        v += dpp<0x141>(v);                                // row_half_mirror: 8 lanes
        if constexpr (LPR >= 16) v += dpp<0x140>(v);       // row_mirror: 16 lanes
        if constexpr (LPR == 32) v += dpp<0x142, 0xA>(v);  // row_bcast:15 into rows 1, 3
        return v;
    }
}
__host__ __device__ constexpr int seg_store_lane(int lpr) { return lpr == 32 ? 31 : 0; }

// FAST: for every problem, w 4-byte aligned and an even number of blocks per
// row (activations need only their 4-byte alignment: they are read with
// 16-byte loads at any 4-byte boundary).
//
// Lanes and rows.  A wave owns RPW = RWV << SUB rows of its row group: the
// wave is cut into 2^SUB segments of LPR = 64 >> SUB lanes and segment q
// takes RWV rows (SUB > 0 only with RWV = 1, for short rows: a row of 2048
// weights fills half a wave).  A step covers LPR pairs of each row, lane l
// taking pair l % LPR.
//
// The launch's row groups (WPG * RPW rows each, the problems numbered one
// after another) are split into gridDim.x contiguous ranges, one per
// workgroup.  A workgroup walks its range as a sequence of steps (row group,
// chunk of LPR pairs).  Each step's weights were requested during the
// previous step (two register sets used in turn).  The activations are
// staged into LDS in windows of 4096 weights, only when the problem or the
// window changes.
// SRC: where the problems come from (GemvSource).  kSrcOne has fixed
// offsets and no indexed reads of a table before the first weight load;
// kSrcExpert reads each problem's expert id from device memory when a step
// enters the problem (an id outside the stack reads expert 0 and stores NaN).
template <int FMT, int NC, int RWV, int WPG, bool FAST, int SRC, int SUB, bool X8>
__global__ __launch_bounds__(64 * WPG) __attribute__((amdgpu_waves_per_eu(NC == 1 || (NC == 2 && FMT != QK_Q8_0) ? 4 : (NC == 2 ? 2 : 1)))) void gemv_kernel(const typename GemvSrc<SRC>::Args args, const GemvSplit split) {
    static_assert(SUB == 0 || RWV == 1, "several rows per wave only with one row per segment");
    static_assert(SRC != kSrcExpert || NC == 1, "expert-indexed problems have one column");
    static_assert(SUB != kSubMixed || (SRC == kSrcTable && NC == 1 && !X8),
                  "per-problem lane split: grouped one-column launches");
    constexpr int BS = Format<FMT>::kBytes;
    constexpr int ND = Pair<FMT>::kDwords;
    constexpr int NT = 64 * WPG;                // lanes per workgroup
    constexpr int XW = kGvWindow;               // weights per activation window
    constexpr int XP = kGvPitch;                // LDS floats per staged column
    static_assert(SUB == kSubMixed || XW / (64 * (64 >> SUB)) == (1 << SUB), "steps per activation window");
    extern __shared__ __attribute__((aligned(16))) float xs[];
    uint8_t *const xq = reinterpret_cast<uint8_t *>(xs);  // 8-bit activations (X8)

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    // Lane geometry for a lane split `sub` (2^sub row segments per wave):
    // constants when the launch has one split, per problem otherwise.
    struct Geo {
        int sub;  // log2 of the row segments per wave (= log2 of the steps per window)
        int lpr;  // lanes per row segment = pairs per step
        int rpw;  // rows per wave
        int rg;   // rows per group
        int seg;  // row segment of this lane
        int sl;   // lane within the segment
    };
    auto geo = [&](int sub) __attribute__((always_inline)) {
        Geo g;
        g.sub = sub;
        g.lpr = 64 >> sub;
        g.rpw = RWV << sub;
        g.rg = WPG * g.rpw;
        g.seg = lane >> (6 - sub);
        g.sl = lane & (g.lpr - 1);
        return g;
    };
    // log2 of the steps per window of a fixed split, opaque to the optimiser:
    // with the constant folded in, its schedule of the LDS reads of the
    // eight-column Q4_1 kernel no longer fits in registers
    int cpw_log = SUB == kSubMixed ? 0 : SUB;
    asm volatile("" : "+s"(cpw_log));
    const int b = blockIdx.x;
    const int gbeg = b * split.per + min(b, split.rem);
    const int gend = gbeg + split.per + (b < split.rem ? 1 : 0);
    // The launcher never starts more workgroups than row groups (per >= 1),
    // so no range is empty.  Expert-indexed launches state it rather than
    // test it, so their argument loads are not split around a branch (one
    // round trip before the id load; measured faster there, slower for the
    // grouped table).
    if constexpr (SRC == kSrcExpert) __builtin_assume(gbeg < gend);
    else if (gbeg >= gend) return;  // whole workgroup, before any barrier

    auto gbase = [&](int i) -> int {
        if constexpr (SRC == kSrcOne) return i == 0 ? 0 : split.total;
        else if constexpr (SRC == kSrcTable) return args.gbase[i];
        else return i * split.gpi;
    };
    auto item = [&](int i) -> const GemvItem * {
        if constexpr (SRC == kSrcOne) return &args;
        else if constexpr (SRC == kSrcTable) return &args.item[i];
        else return nullptr;  // expert problems are formed in enter()
    };
    // lane split of problem i
    auto sub_of = [&](int i) -> int {
        if constexpr (SUB == kSubMixed) return args.sub[i];
        else return SUB;
    };
    auto chunks = [](int nb, int sub) { return (((nb + 1) >> 1) + (64 >> sub) - 1) >> (6 - sub); };

    // Step position (uniform across the workgroup): row group g of problem
    // mi, chunk c, with the problem's descriptor held in registers.  It is
    // formed only when a step enters a new problem.
    struct Pos {
        int g, mi, c;
        int gb0, gb1;   // the problem's first row group and one past its last
        int nchunks;    // steps per row group
        int e;          // expert id (expert-indexed problems); it.w is the stack
        int sub;        // the problem's lane split
        GemvItem it;
    };
    auto geo_of = [&](const Pos &q) __attribute__((always_inline)) {
        if constexpr (SUB == kSubMixed) return geo(q.sub);
        else return geo(SUB);
    };
    // (field by field: a whole-struct copy out of the argument segment is
    // lowered through scratch memory)
    auto enter = [&](Pos &q, int i) __attribute__((always_inline)) {
        q.mi = i;
        if constexpr (SRC == kSrcExpert) {
            const int t = i / args.n_used;
            const int s = i - t * args.n_used;
            // a scalar load (constant address space): it is waited for only
            // where the expert's address is first needed, so in the first
            // step it overlaps the activation loads
            typedef const __attribute__((address_space(4))) int32_t cid_t;
            q.e = *(cid_t *)(uintptr_t)(args.ids + (int64_t)t * args.ld_ids + s);
            q.it.w = args.w;
            q.it.x = args.x + t * args.x_tok + s * args.x_slot;
            q.it.y = args.y + t * args.y_tok + s * args.y_slot;
            q.it.ldx = 0;
            q.it.ldy = 0;
            q.it.m = args.m;
            q.it.nb = args.nb;
        } else {
            const GemvItem &src = *item(i);
            q.e = 0;
            q.it.w = src.w;
            q.it.x = src.x;
            q.it.y = src.y;
            q.it.ldx = src.ldx;
            q.it.ldy = src.ldy;
            q.it.m = src.m;
            q.it.nb = src.nb;
        }
        q.gb0 = gbase(i);
        q.gb1 = gbase(i + 1);
        q.sub = sub_of(i);
        q.nchunks = chunks(q.it.nb, q.sub);
    };
    Pos P;
    P.g = gbeg;
    P.c = 0;
    {
        int i = 0;
        if constexpr (SRC == kSrcExpert) i = gbeg / split.gpi;
        else while (gbeg >= gbase(i + 1)) ++i;
        enter(P, i);
    }
    // The step after q within this workgroup's range (problems have at least
    // one row group each, so a step enters at most one new problem).
    auto advance = [&](const Pos &q) __attribute__((always_inline)) {
        Pos r = q;
        if (++r.c >= r.nchunks) {
            r.c = 0;
            if (++r.g >= r.gb1 && r.g < gend) enter(r, r.mi + 1);
        }
        return r;
    };
    // The problem's weights, and whether its outputs are NaN (an expert id
    // outside the stack reads expert 0 instead).
    auto bad = [&](const Pos &q) -> bool {
        if constexpr (SRC == kSrcExpert) return (unsigned)q.e >= (unsigned)args.nexp;
        else return false;
    };
    auto weights = [&](const Pos &q) -> const uint8_t * {
        if constexpr (SRC == kSrcExpert) return q.it.w + (bad(q) ? 0 : (int64_t)q.e * args.estride);
        else return q.it.w;
    };
    int staged_mi = -1, staged_w = -1;

    float acc[RWV][NC];
#pragma unroll
    for (int r = 0; r < RWV; ++r)
#pragma unroll
        for (int j = 0; j < NC; ++j) acc[r][j] = 0.0f;

    // Weight loads of step q into dst.  On the fast path every lane issues the
    // same loads with no branch around them (a lane past the last pair or row
    // reads a clamped, valid address and ignores the data), so the compiler
    // counts them and waits for exactly the loads a computation needs while
    // the prefetch stays in flight.
    auto load_step = [&](const Pos &q, uint32_t (&dst)[RWV][ND]) __attribute__((always_inline)) {
        const GemvItem &it = q.it;
        const Geo G = geo_of(q);
        const uint8_t *w = weights(q);
        const int row0 = (q.g - q.gb0) * G.rg + wave * G.rpw + G.seg * RWV;
        const int npairs = (it.nb + 1) >> 1;
        const int64_t row_bytes = (int64_t)it.nb * BS;
        const int pp = q.c * G.lpr + G.sl;
        if (FAST) {
            const int ppc = min(pp, npairs - 1);
#pragma unroll
            for (int r = 0; r < RWV; ++r) {
                const int row = min(row0 + r, it.m - 1);
                load_pair_fast<FMT>(w + (int64_t)row * row_bytes + (int64_t)ppc * (2 * BS), dst[r]);
            }
        } else if (pp < npairs) {
            const int nrows = max(0, min(RWV, it.m - row0));
            const uint8_t *p = w + (int64_t)row0 * row_bytes + (int64_t)pp * (2 * BS);
            const uint8_t *wend = w + (int64_t)it.m * row_bytes;
            const bool second = 2 * pp + 1 < it.nb;
#pragma unroll
            for (int r = 0; r < RWV; ++r) {
                if (r < nrows) {
                    const uint8_t *pr = p + r * row_bytes;
                    // whole dwords unless that would read past the matrix
                    if (pr + kPairReach<FMT> <= wend) load_pair_shift<FMT>(pr, dst[r]);
                    else load_pair_generic<FMT>(pr, second, dst[r]);
                }
            }
        }
    };

    // Columns of the first window staged through registers: their loads are
    // all issued before the weight loads, so the LDS copy waits for them
    // alone; a column copied by the loop further down waits for the weights
    // too (the counter is in order) and then takes one round trip per float4.
    // Every column on the aligned path (Q4_1 11008 x 4096 at 3 columns 14.0
    // -> 11.9 us, 4096 x 11008 at 4 / 8 columns 21.5 -> 19.1 / 38.4 -> 35.5
    // us) and on the unaligned one except Q8_0, whose registers would cost
    // it waves per SIMD (unaligned 11008 x 4096 at 3 / 4 / 8 columns: Q4_0
    // 14.8 -> 13.6 / 16.3 -> 16.4 / 29.2 -> 28.5 us, Q4_1 14.3 -> 14.5 / 19.3
    // -> 18.1 / 28.4 -> 27.2, Q5_0 16.6 -> 14.9 / 18.4 / 31.5 -> 30.0, Q5_1
    // 15.7 -> 16.0 / 20.8 -> 19.5 / 30.3 -> 28.2).
    constexpr int XR = NC <= 2 || FAST || FMT != QK_Q8_0 ? NC : 0;

    // 8-bit activations: block bi of the window (columns one after another,
    // nblk blocks each) is read from x and quantized into LDS.
    auto x8_src = [&](const GemvItem &it, int e0, int nblk, int bi) -> const float * {
        const int j = bi / nblk;
        return it.x + j * it.ldx + e0 + 32 * (bi - j * nblk);
    };
    auto x8_load = [&](const float *src, f32x4_t (&v)[8]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = *reinterpret_cast<const f32x4_a4 *>(src + 4 * i);
    };
    auto x8_put = [&](int nblk, int bi, const f32x4_t (&v)[8]) __attribute__((always_inline)) {
        const int j = bi / nblk;
        const int bb = bi - j * nblk;
        uint8_t *col = xq + j * kX8ColBytes;
        x8_block(v, col + kX8PairPitch * (bb >> 1) + 32 * (bb & 1), col + kX8ScaleOff + 8 * bb);
    };

    // Copy window `wi` of problem `it`'s activations into LDS (whole workgroup).
    auto stage_x = [&](const GemvItem &it, int wi) __attribute__((always_inline)) {
        const int e0 = wi * XW;
        if constexpr (X8) {
            const int nblk = min(XW, it.nb * 32 - e0) / 32;
            for (int bi = tid; bi < NC * nblk; bi += NT) {
                f32x4_t v[8];
                x8_load(x8_src(it, e0, nblk, bi), v);
                x8_put(nblk, bi, v);
            }
            return;
        }
        const int ce4 = min(XW, it.nb * 32 - e0) / 4;  // float4s in this window (>= 8)
        if constexpr (NC >= 3 && (FAST || FMT != QK_Q8_0)) {
            // a batch of columns' loads at a time (a tail thread repeats the
            // last float4 and skips the store), one round trip per batch
            // instead of one per float4: Q4_1 4096 x 11008 at 3 / 4 / 8
            // columns 14.8 -> 14.6, 19.1 -> 17.5, 35.5 -> 33.9 us; unaligned,
            // 15.9 -> 15.9, 19.7 -> 17.9, 35.5 -> 32.3 us (Q5_1 at 8 columns
            // 39.9 -> 33.9).  (With one column the registers cost the grouped
            // layer a wave per SIMD; the unaligned Q8_0 kernels, one to two.)
            constexpr int XU = (XW / 4 + NT - 1) / NT;  // float4s per thread and column
            // columns per batch: up to four, at most 8 float4s per thread
            constexpr int CB = (NC < 4 ? NC : 4) * XU <= 8 ? (NC < 4 ? NC : 4) : (XU < 8 ? 8 / XU : 1);
#pragma unroll
            for (int j0 = 0; j0 < NC; j0 += CB) {
                f32x4_t v[CB][XU];
#pragma unroll
                for (int jj = 0; jj < CB; ++jj)
#pragma unroll
                    for (int u = 0; u < XU; ++u)
                        if (j0 + jj < NC)
                            v[jj][u] = *reinterpret_cast<const f32x4_a4 *>(
                                it.x + (j0 + jj) * it.ldx + e0 + 4 * min(tid + u * NT, ce4 - 1));
#pragma unroll
                for (int jj = 0; jj < CB; ++jj)
#pragma unroll
                    for (int u = 0; u < XU; ++u) {
                        const int t = tid + u * NT;
                        if (j0 + jj < NC && t < ce4)
                            *reinterpret_cast<f32x4_t *>(xs + (j0 + jj) * XP + 4 * t + (t >> 4) * 4) = v[jj][u];
                    }
            }
        } else {
#pragma unroll
            for (int j = 0; j < NC; ++j) {
                const float *xj = it.x + j * it.ldx + e0;
                for (int t = tid; t < ce4; t += NT) {
                    const f32x4_t val = *reinterpret_cast<const f32x4_a4 *>(xj + 4 * t);
                    *reinterpret_cast<f32x4_t *>(xs + j * XP + 4 * t + (t >> 4) * 4) = val;
                }
            }
        }
    };

    // Steps in this workgroup's range.
    int nsteps = 0;
    if constexpr (SRC == kSrcExpert) {
        nsteps = (gend - gbeg) * P.nchunks;  // every problem has the same shape
    } else {
        int gg = gbeg, ii = P.mi;
        while (gg < gend) {
            while (gg >= gbase(ii + 1)) ++ii;
            const int nxt = min(gend, gbase(ii + 1));
            nsteps += (nxt - gg) * chunks(item(ii)->nb, sub_of(ii));
            gg = nxt;
        }
    }

    // One step computing with cur.  Each (FIRST, DEPTH) combination is its own
    // straight-line code, so the compiler waits for exactly the loads the
    // computation needs and the prefetch stays in flight.  FIRST issues the
    // activation loads before any weight load, so copying them to LDS does
    // not wait for the weights (loads complete in order).
    // DEPTH: 0 no prefetch, 1 the next step's weights requested into nxt.
    auto step = [&](auto first_tag, auto depth_tag, uint32_t (&cur)[RWV][ND],
                    uint32_t (&nxt)[RWV][ND]) __attribute__((always_inline)) {
        constexpr bool FIRST = decltype(first_tag)::value;
        constexpr int DEPTH = decltype(depth_tag)::value;
        constexpr bool PREFETCH = DEPTH > 0;
        const GemvItem &it = P.it;
        const Geo G = geo_of(P);
        const int npairs = (it.nb + 1) >> 1;
        const int swl = SUB == kSubMixed ? G.sub : cpw_log;  // log2 of the steps per window
        const int wi = P.c >> swl;  // activation window of this step

        // the next step, and what to prefetch: past the workgroup's last step
        // a prefetch repeats this step's loads
        const Pos Q = advance(P);
        const Pos PF = Q.g < gend ? Q : P;

        if constexpr (FIRST && X8) {
            // one block of activations per thread loaded first, then the
            // weights, then quantization into LDS (waits only for the
            // activations); a tail thread repeats the last block
            const int e0 = wi * XW;
            const int nblk = min(XW, it.nb * 32 - e0) / 32;
            const int tb = NC * nblk;
            const int b0 = min(tid, tb - 1);
            f32x4_t xr8[8];
            x8_load(x8_src(it, e0, nblk, b0), xr8);
            // (the empty asm statements keep the three groups of loads in
            // this order and ahead of the quantization, which then waits for
            // the activations alone; left to itself the scheduler moved
            // activation loads behind the weight loads and the prefetch
            // behind the quantization: Q4_1 11008 x 4096 at 1 / 2 columns
            // 9.1 -> 8.5 / 10.5 -> 10.3 us)
            asm volatile("" ::: "memory");
            load_step(P, cur);
            if constexpr (PREFETCH) load_step(PF, nxt);
            asm volatile("" ::: "memory");
            x8_put(nblk, b0, xr8);
            for (int bi = tid + NT; bi < tb; bi += NT) {
                f32x4_t v[8];
                x8_load(x8_src(it, e0, nblk, bi), v);
                x8_put(nblk, bi, v);
            }
            __syncthreads();
            staged_mi = P.mi;
            staged_w = wi;
        } else if constexpr (FIRST) {
            // activation loads, then this step's and the next step's weights,
            // then the LDS copy (waits only for the activations)
            constexpr int XU = (XW / 4 + NT - 1) / NT;  // registers cover the first window
            const int e0 = wi * XW;
            const int ce4 = min(XW, it.nb * 32 - e0) / 4;
            const int cr4 = min(XW / 4, ce4);
            f32x4_t xr[XR > 0 ? XR : 1][XU];
#pragma unroll
            for (int j = 0; j < XR; ++j) {
                const float *xj = it.x + j * it.ldx + e0;
#pragma unroll
                for (int u = 0; u < XU; ++u) {
                    // clamped so every lane loads (a tail lane repeats the last
                    // float4 and stores it again)
                    const int t = min(tid + u * NT, cr4 - 1);
                    xr[j][u] = *reinterpret_cast<const f32x4_a4 *>(xj + 4 * t);
                }
            }
            load_step(P, cur);
            // (keeps this step's weight loads ahead of the prefetch: the
            // scheduler interleaved the two sets in the one-row Q8_0 kernel,
            // so the first products waited for most of the prefetch too)
            asm volatile("" ::: "memory");
            if constexpr (PREFETCH) load_step(PF, nxt);
            // unconditional stores (a tail lane rewrites the last float4 with
            // the same value), so no load is moved behind the weight loads
#pragma unroll
            for (int j = 0; j < XR; ++j)
#pragma unroll
                for (int u = 0; u < XU; ++u) {
                    const int t = min(tid + u * NT, cr4 - 1);
                    *reinterpret_cast<f32x4_t *>(xs + j * XP + 4 * t + (t >> 4) * 4) = xr[j][u];
                }
            // the rest of the window (and wider activation sets) directly
#pragma unroll
            for (int j = 0; j < NC; ++j) {
                const float *xj = it.x + j * it.ldx + e0;
                for (int t = (j < XR ? cr4 : 0) + tid; t < ce4; t += NT) {
                    const f32x4_t val = *reinterpret_cast<const f32x4_a4 *>(xj + 4 * t);
                    *reinterpret_cast<f32x4_t *>(xs + j * XP + 4 * t + (t >> 4) * 4) = val;
                }
            }
            __syncthreads();
            staged_mi = P.mi;
            staged_w = wi;
        } else {
            // a new problem or window: restage the activations before the prefetch
            if (staged_mi != P.mi || staged_w != wi) {
                __syncthreads();  // readers of the previous window are done
                stage_x(it, wi);
                __syncthreads();
                staged_mi = P.mi;
                staged_w = wi;
            }
            if constexpr (PREFETCH) load_step(PF, nxt);
        }

        // compute this step
        const int row0 = (P.g - P.gb0) * G.rg + wave * G.rpw + G.seg * RWV;
        const int nrows = max(0, min(RWV, it.m - row0));
        const int pp = P.c * G.lpr + G.sl;
        if (nrows > 0 && pp < npairs) {
            const int el = (P.c - (wi << swl)) * (64 * G.lpr) + G.sl * 64;  // window element of the pair
            if constexpr (X8)
                pair_dot_x8<FMT, NC, RWV, FAST>(cur, nrows, FAST || (2 * pp + 1 < it.nb), xq, el >> 6, acc);
            else
                pair_dot<FMT, NC, RWV, FAST>(cur, nrows, FAST || (2 * pp + 1 < it.nb), xs, XP, el, acc);
        }

        // last chunk of the group: reduce across the row's lanes and store
        if (P.c == P.nchunks - 1) {
#pragma unroll
            for (int r = 0; r < RWV; ++r) {
                if (G.sub > 0 || r < nrows) {  // (uniform across the wave when the split is 0)
#pragma unroll
                    for (int j = 0; j < NC; ++j) {
                        float sum;
                        if constexpr (SUB == kSubMixed) {
                            // wave-uniform: a row group belongs to one problem
                            switch (G.sub) {
                            case 0: sum = seg_sum<64>(acc[r][j]); break;
                            case 1: sum = seg_sum<32>(acc[r][j]); break;
                            case 2: sum = seg_sum<16>(acc[r][j]); break;
                            default: sum = seg_sum<8>(acc[r][j]); break;
                            }
                        } else {
                            sum = seg_sum<(64 >> SUB)>(acc[r][j]);
                        }
                        if (G.sl == seg_store_lane(G.lpr) && r < nrows)
                            it.y[j * it.ldy + row0 + r] = bad(P) ? __builtin_nanf("") : sum;
                    }
                }
#pragma unroll
                for (int j = 0; j < NC; ++j) acc[r][j] = 0.0f;
            }
        }
        P = Q;
    };

    using T = std::true_type;
    using F = std::false_type;
    using D0 = std::integral_constant<int, 0>;
    using D1 = std::integral_constant<int, 1>;
    uint32_t va[RWV][ND], vb[RWV][ND];
    if (nsteps == 1) {
        step(T{}, D0{}, va, vb);
        return;
    }
    step(T{}, D1{}, va, vb);
    // Two steps per iteration with the register sets in swapped roles and no
    // branch between them, so the two bodies stay distinct: a merged body
    // would copy the prefetched registers into place, and that copy waits for
    // every outstanding load (the new prefetch included).  The final step's
    // prefetch repeats its own loads (clamped).
    int left = nsteps - 1;  // steps still to compute; the next one's weights are in vb
    for (; left >= 2; left -= 2) {
        step(F{}, D1{}, vb, va);
        step(F{}, D1{}, va, vb);
    }
    if (left == 1) step(F{}, D0{}, vb, va);
}

// Launch shape by column count: RWV rows per wave, WPG waves per workgroup
// sharing one LDS copy of the activations.
// Above 4 columns the staged activations (NC x 4096 floats) leave room for
// one workgroup per CU, so the workgroup itself is as wide as registers
// allow: 12 waves (3 per SIMD) for Q4_1, 8 for Q4_0, 4 for Q8_0.
#ifndef QK_GEMV_SHORT_WPG
#define QK_GEMV_SHORT_WPG 4
#endif
// The generic (unaligned) Q4_1 kernels above 4 columns need more registers
// than 12 waves leave (168): they take one row per wave in 8-wave workgroups.
// With 8-bit activations the Q8_0 kernels above 3 columns fit two rows per
// wave in 8-wave workgroups (measured 15.3 -> 12.1 us at 8 columns on
// 4096 x 4096; four rows per wave was slower for every format).
// R2: two rows per wave (activations read from LDS once for both) for a
// one-column launch of full-wave rows with more than 64 rows per CU, i.e. more
// row groups of one row per wave than the launch's 8 workgroups per CU, so
// workgroups walk several steps either way.  Measured in alternating runs on
// one box: the grouped 7B-shaped Q4_0 layer (42 496 rows) 27.1-28.1 ->
// 25.2-26.5 us.  With fewer rows each workgroup takes one step and halving the
// workgroups costs more than it saves: Q4_1 11008 x 4096 8.6 -> 9.0 us, the
// layer's 8-way tensor-parallel share (12 480 rows) 9.4 -> 11.0 us, Q8_0 4096 x
// 4096 5.3 -> 6.2 us.
//
// R2 with 2 or 3 columns (Q4_0, and aligned Q4_1: the generic Q4_1 kernel
// spills with two rows per wave) above 32 rows per CU: Q4_1 11008 x 4096
// 11.4 -> 10.6 us at 2 columns, 15.6 -> 14.0 us at 3; at 4096 rows it loses
// (5.5 -> 6.3 and 7.1 -> 7.6 us).
template <int FMT, int NC, int SUB, bool FAST, bool X8 = false, bool R2 = false> struct GemvShape {
    static_assert(!R2 || (NC <= 3 && SUB == 0 && !X8 && (NC == 1 || (FMT != QK_Q8_0 && (!kHasM<FMT> || FAST)))),
                  "two rows per wave: up to 3 columns, full-wave rows");
    static constexpr bool kWideQ41Generic = kHasM<FMT> && NC > 4 && !FAST;
    static constexpr bool kX8Q8Wide = X8 && FMT == QK_Q8_0 && NC >= 4 && SUB == 0;
    static constexpr int kRWV =
        (R2 || kX8Q8Wide) ? 2 : (NC >= 4 && FMT != QK_Q8_0 && !kWideQ41Generic ? 2 : 1);
    static constexpr int kWPG =
        SUB > 0 ? QK_GEMV_SHORT_WPG
                : (kX8Q8Wide ? 8
                             : (NC <= 4 ? 8 : (kHasM<FMT> ? (FAST ? 12 : 8) : (FMT == QK_Q8_0 ? 4 : 8))));
    static constexpr int kRowsPerGroup = SUB == kSubMixed ? kWPG : kWPG * (kRWV << SUB);  // (mixed: per problem)
};

// Rows per wave (as 2^SUB) for one-column launches whose longest row has
// `npairs` pairs: short rows share a wave instead of leaving lanes idle.
inline int gemv_sub(int npairs) {
    return npairs <= 8 ? 3 : (npairs <= 16 ? 2 : (npairs <= 32 ? 1 : 0));
}

// Workgroups launched per CU at most (when LDS allows).  Above what can be
// resident at once, the hardware dispatcher starts a workgroup as another
// finishes, which balances row groups better than giving each resident
// workgroup a longer range.
#ifndef QK_GEMV_WG_PER_CU
#define QK_GEMV_WG_PER_CU 8
#endif
constexpr int kGvMaxWgPerCu = QK_GEMV_WG_PER_CU;
// With 8-bit activations every workgroup quantizes the whole activation
// window it stages, so fewer workgroups, each walking more row groups, share
// that work.
#ifndef QK_GEMV_X8_WG_PER_CU
#define QK_GEMV_X8_WG_PER_CU 1
#endif
constexpr int kGvX8MaxWgPerCu = QK_GEMV_X8_WG_PER_CU;

// One launch over `total` row groups (gpi per problem for expert launches).
template <int FMT, int NC, int SRC, int SUB, bool FAST, bool X8, bool R2 = false>
int gemv_launch(const typename GemvSrc<SRC>::Args &args, int64_t total, int gpi, hipStream_t stream) {
    constexpr int RWV = GemvShape<FMT, NC, SUB, FAST, X8, R2>::kRWV;
    constexpr int WPG = GemvShape<FMT, NC, SUB, FAST, X8, R2>::kWPG;
    if (total <= 0) return QK_OK;
    if (total > INT32_MAX) return QK_ERR_INVALID_ARG;
    // Activation window: 4096 weights per column (17 KiB at one column).
    // Longer rows restage it per window; the small window lets more
    // workgroups share a CU, which measured faster than holding whole rows of
    // 11008 weights.
    // (8-bit activations: 6 KiB per column)
    const size_t lds = X8 ? (size_t)NC * kX8ColBytes : (size_t)NC * kGvPitch * sizeof(float);
    const int per_cu = max(1, min(X8 ? kGvX8MaxWgPerCu : kGvMaxWgPerCu, (int)((160 * 1024) / lds)));
    const int64_t cap = (int64_t)device_cus() * per_cu;
    const int nwg = (int)(total < cap ? total : cap);
    const GemvSplit split{(int)total, (int)total / nwg, (int)total % nwg, gpi};
    auto kern = gemv_kernel<FMT, NC, RWV, WPG, FAST, SRC, SUB, X8>;
    if (lds > 64 * 1024 &&
        hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return QK_ERR_LAUNCH;
    return launch_lds(kern, dim3((unsigned)nwg), dim3(64 * WPG), lds, stream, args, split);
}

template <int FMT, int NC, int SUB, bool FAST, bool X8, bool R2 = false>
int gemv_table_run(GemvArgs &a, hipStream_t stream) {
    constexpr int RG = GemvShape<FMT, NC, SUB, FAST, X8, R2>::kRowsPerGroup;
    int64_t g = 0;
    a.gbase[0] = 0;
    for (int i = 0; i < a.count; ++i) {
        const int rg = SUB == kSubMixed ? RG << a.sub[i] : RG;
        g += (a.item[i].m + rg - 1) / rg;
        if (g > INT32_MAX) return QK_ERR_INVALID_ARG;
        a.gbase[i + 1] = (int)g;
    }
    if constexpr (SUB == kSubMixed) {
        return gemv_launch<FMT, NC, kSrcTable, SUB, FAST, false, false>(a, g, 0, stream);  // count > 1
    } else {
        if (a.count == 1) return gemv_launch<FMT, NC, kSrcOne, SUB, FAST, X8, R2>(a.item[0], g, 0, stream);
        if constexpr (X8) return QK_ERR_INVALID_ARG;  // 8-bit activations: one problem per launch
        else return gemv_launch<FMT, NC, kSrcTable, SUB, FAST, false, R2>(a, g, 0, stream);
    }
}

template <int FMT, int NC, int SUB, bool X8>
int gemv_table_sub(GemvArgs &a, bool fast, hipStream_t stream) {
    if constexpr (NC <= 3 && SUB == 0 && !X8 && (NC == 1 || FMT != QK_Q8_0)) {
        int64_t rows = 0;
        for (int i = 0; i < a.count; ++i) rows += a.item[i].m;
        if (rows > (NC == 1 ? 64 : 32) * (int64_t)device_cus()) {
            if (fast) return gemv_table_run<FMT, NC, SUB, true, X8, true>(a, stream);
            if constexpr (NC == 1 || !kHasM<FMT>) return gemv_table_run<FMT, NC, SUB, false, X8, true>(a, stream);
        }
    }
    if (fast) return gemv_table_run<FMT, NC, SUB, true, X8>(a, stream);
    return gemv_table_run<FMT, NC, SUB, false, X8>(a, stream);
}

// The GEMV for 4..8 columns on the matrix cores (gemv_mfma.h): one problem,
// 4-byte aligned weights with an even block count, k <= kGvWindow.  (At 2 or
// 3 columns the vector-ALU kernel below measured faster: Q4_1 11008 x 4096
// at 2 columns 11.0 us against 14.8 us.)
template <int FMT, int NC>
int gemv_mfma_launch(const GemvItem &it, hipStream_t stream);

template <int FMT, int NC, bool X8>
int gemv_table_fmt(GemvArgs &a, bool fast, hipStream_t stream) {
    if constexpr (NC >= 4 && !X8) {
        if (a.count == 1 && fast && a.item[0].nb * kBlockElems <= kGvWindow) {
            // At 4 columns the vector-ALU kernel is the faster one when its
            // launch has a row group for every CU and at most one per resident
            // workgroup (each workgroup then takes a single step): 4096 x 4096
            // Q4_1 7.9 -> 6.9 us, Q5_1 8.2 -> 7.3, Q8_0 10.2 -> 9.2; 8192
            // rows Q4_1 11.4 -> 10.1, Q5_0 12.6 -> 11.1 us.  Outside that
            // range (fewer rows, or more row groups than workgroup slots) the
            // matrix cores measured as fast or faster.
            bool vector_alu = false;
            if constexpr (NC == 4) {
                constexpr int RG = GemvShape<FMT, NC, 0, true, false>::kRowsPerGroup;
                const int64_t groups = ((int64_t)a.item[0].m + RG - 1) / RG;
                const int slots =
                    max(1, min(kGvMaxWgPerCu, (int)((160 * 1024) / ((size_t)NC * kGvPitch * sizeof(float)))));
                const int64_t cus = device_cus();
                vector_alu = groups >= cus && groups <= slots * cus;
            }
            if (!vector_alu) return gemv_mfma_launch<FMT, NC>(a.item[0], stream);
        }
    }
    if constexpr (NC == 1) {
        int npairs = 0;
        bool mixed = false;
        for (int i = 0; i < a.count; ++i) {
            npairs = max(npairs, (a.item[i].nb + 1) / 2);
            a.sub[i] = gemv_sub((a.item[i].nb + 1) / 2);
            mixed = mixed || a.sub[i] != a.sub[0];
        }
        // problems whose rows want different splits (e.g. a layer's
        // tensor-parallel share: 8-pair and 64-pair rows) keep their own
        if constexpr (!X8) {
            if (mixed && a.count > 1) {
                if (fast) return gemv_table_run<FMT, NC, kSubMixed, true, false>(a, stream);
                return gemv_table_run<FMT, NC, kSubMixed, false, false>(a, stream);
            }
        }
        switch (gemv_sub(npairs)) {
        case 3: return gemv_table_sub<FMT, NC, 3, X8>(a, fast, stream);
        case 2: return gemv_table_sub<FMT, NC, 2, X8>(a, fast, stream);
        case 1: return gemv_table_sub<FMT, NC, 1, X8>(a, fast, stream);
        default: break;
        }
    }
    return gemv_table_sub<FMT, NC, 0, X8>(a, fast, stream);
}

template <int NC>
int gemv_table(int fmt, GemvArgs &a, bool fast, hipStream_t stream) {
    switch (fmt) {
    case QK_Q4_0: return gemv_table_fmt<QK_Q4_0, NC, false>(a, fast, stream);
    case QK_Q4_1: return gemv_table_fmt<QK_Q4_1, NC, false>(a, fast, stream);
    case QK_Q8_0: return gemv_table_fmt<QK_Q8_0, NC, false>(a, fast, stream);
    case QK_Q5_0: return gemv_table_fmt<QK_Q5_0, NC, false>(a, fast, stream);
    case QK_Q5_1: return gemv_table_fmt<QK_Q5_1, NC, false>(a, fast, stream);
    default: return QK_ERR_INVALID_ARG;
    }
}

template <int NC>
int gemv_table_x8(int fmt, GemvArgs &a, bool fast, hipStream_t stream) {
    switch (fmt) {
    case QK_Q4_0: return gemv_table_fmt<QK_Q4_0, NC, true>(a, fast, stream);
    case QK_Q4_1: return gemv_table_fmt<QK_Q4_1, NC, true>(a, fast, stream);
    case QK_Q8_0: return gemv_table_fmt<QK_Q8_0, NC, true>(a, fast, stream);
    case QK_Q5_0: return gemv_table_fmt<QK_Q5_0, NC, true>(a, fast, stream);
    case QK_Q5_1: return gemv_table_fmt<QK_Q5_1, NC, true>(a, fast, stream);
    default: return QK_ERR_INVALID_ARG;
    }
}

template <int FMT, int SUB, bool FAST>
int gemv_expert_run(const GemvExpert &e, hipStream_t stream) {
    constexpr int RG = GemvShape<FMT, 1, SUB, FAST>::kRowsPerGroup;
    const int gpi = (e.m + RG - 1) / RG;
    return gemv_launch<FMT, 1, kSrcExpert, SUB, FAST, false>(e, (int64_t)gpi * e.count, gpi, stream);
}

template <int FMT, int SUB>
int gemv_expert_sub(const GemvExpert &e, bool fast, hipStream_t stream) {
    if (fast) return gemv_expert_run<FMT, SUB, true>(e, stream);
    return gemv_expert_run<FMT, SUB, false>(e, stream);
}

template <int FMT>
int gemv_expert_fmt(const GemvExpert &e, bool fast, hipStream_t stream) {
    switch (gemv_sub((e.nb + 1) / 2)) {
    case 3: return gemv_expert_sub<FMT, 3>(e, fast, stream);
    case 2: return gemv_expert_sub<FMT, 2>(e, fast, stream);
    case 1: return gemv_expert_sub<FMT, 1>(e, fast, stream);
    default: return gemv_expert_sub<FMT, 0>(e, fast, stream);
    }
}

}  // namespace qk
