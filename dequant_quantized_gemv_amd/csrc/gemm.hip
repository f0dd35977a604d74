// gemm.hip - batched quantized GEMM: Y = f16(W) X on the gfx950 matrix cores.
//
// The reference path for more than one activation column dequantizes the
// weights to fp16 (ggml_get_to_fp16_cuda) and hands them to a BLAS GEMM;
// ggml_cuda_mul_mat picks it by the column count ("llama_cpp 0.12.1 -> 0.12.2"
// ggml-cuda.cu diff).  Here the two steps are fused: weights are dequantized to
// fp16 straight into the registers that feed v_mfma_f32_16x16x32_f16, and the
// products accumulate in fp32.  The fp16 weight is one round-to-nearest-even
// of the exact weight value, i.e. the value qk_dequantize(..., QK_F16, ...)
// produces (a Q4_0 code 8 with negative d gives -0 here, +0 there: the same
// number).
//
// Tile: 256 rows x 128 columns per workgroup of 8 waves: 4 row slices of 64
// rows x 2 k groups.  Each wave holds a 64 x 128 fp32 accumulator tile (4 x 8
// MFMA tiles of 16 x 16) and multiplies its k group's half of the pairs of
// blocks; at the end the two k groups' partial sums are combined through LDS.
// In the MFMA A operand, lane l holds row l%16 of a 16-row tile and elements
// 8(l/16)..8(l/16)+7 of a 32-element block, so each 16 x 32 operand is
// exactly one quant block of 16 rows, and each lane dequantizes its own 8
// weights per block from quant bytes staged in LDS straight into operand
// registers.  The quant bytes (row-contiguous 16-byte chunks) and the
// activation tile pass through LDS: with k % 128 == 0 and aligned operands
// they are copied global -> LDS by gfx950 direct loads into a ring of 3
// stages (Q4_0) or 2 (Q4_1, Q8_0) that many super-steps minus one ahead
// (gemm_dma_kernel); otherwise through registers one step ahead into double
// buffers (gemm_kernel).
//
// Dequantization to fp16 (Q4_0, Q8_0), packed two at a time and exact: the
// integer code is placed in the mantissa of an fp16 (0x64XX is 1024 + XX) with
// a byte permute, the bias removed with one packed fma or add (giving q - 8,
// or q, exactly), and one packed multiply by (d, d) rounds d * (q - 8) or
// d * q to fp16 once.  A lane that takes high nibbles keeps them in place
// (0x64XX with XX = 16q) and scales by 1/16 in the same fma.  Q4_1
// (d*q + m is one fp32 rounding) goes through fp32 so that the fp16 is rounded
// from exactly the fp32 dequantized value.
//
// Tiles are assigned so that the workgroups of one XCD (the hardware sends
// workgroup i to XCD i % 8) cover consecutive tiles, column tile fastest, so
// the workgroups sharing a weight row tile share that XCD's L2.
//
// Small batches: with 256 x 128 tiles a tall matrix has too few tiles to cover
// the CUs (14336 rows: 56), so up to 32 columns (128 where the large tiles
// would number fewer than the CUs) the direct-load kernel runs 64 x 32 tiles
// whose eight waves each take one pair of every eight; their partial sums are
// added through LDS in a fixed order.  Block counts that are not a multiple of
// 16 leave 4-12 blocks to a second launch of the large tile that adds its
// products to y.
#include <type_traits>

#include "qk_common.h"
#include "qk_internal.h"

namespace qk {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2g_t __attribute__((ext_vector_type(2)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4g_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x3g_a4 __attribute__((ext_vector_type(3), aligned(4)));
typedef uint32_t u32x2g_a4 __attribute__((ext_vector_type(2), aligned(4)));
typedef uint32_t u32x4g_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2g_t __attribute__((ext_vector_type(2)));

constexpr int kGmThreads = 512;  // 8 waves: 4 row slices x 2 k groups
constexpr int kBM = 256;         // rows per tile (64 per row slice)
constexpr int kBN = 128;         // columns per tile
constexpr int kBK = 64;          // elements of K per step (one pair of blocks)
constexpr int kPitch = kBK + 8;  // halves per LDS column (144 bytes: spreads columns over banks)
constexpr int kRT = 4;           // 16-row MFMA tiles per wave
constexpr int kCT = 8;           // 16-column MFMA tiles per wave
// The 64 x 32 direct-load tile takes batches of up to kGmSmallBatch columns,
// and up to kGmSmallBatchMax where 256 x 128 tiles would not cover the CUs
// (each further 32 columns decode the weights once more).  Q4_0 14336 x 4096:
// n = 16 / 33 / 64 / 96 / 128 in 15.5 / 28.5 / 30.7 / 44.3 / 58.5 us against
// 65-70 us with the large tile; at n = 256 the large tile takes 70 us.
constexpr int kGmSmallBatch = 32;
constexpr int kGmSmallBatchMax = 128;

// Quant dwords one lane loads per 16-row tile and step.  Byte offsets from the
// start of the pair (g = lane/16, h = g % 2 picks the half of a block's quant
// bytes):
//   Q4_0 (36-byte pair): 8h, 8h+4, 8h+8 | 20+8h, 24+8h | (h ? 0 : 16), the last
//     one from the partner lane's registers, not from LDS (gm_partner_scale)
//   Q4_1 (40-byte pair): 0 | 4+8h, 8+8h | 20 | 24+8h, 28+8h
//   Q8_0 (68-byte pair): 8g, 8g+4, 8g+8 | 36+8g, 40+8g | 0 | 32
//   Q5_0 (44-byte pair; block 0 = d at 0, qh at 2-5, quant bytes 6-21; block
//     1 = d at 22, qh 24-27, quant bytes 28-43): 0, 4, 4+8h, 8+8h, 12+8h |
//     20, 24, 28+8h, 32+8h
//   Q5_1 (48-byte pair; d, m, qh, quant bytes at 0, 2, 4, 8 and 24, 26, 28,
//     32): 0, 4, 8+8h, 12+8h | 24, 28, 32+8h, 36+8h
template <int FMT> struct GmQ;
template <> struct GmQ<QK_Q4_0> { static constexpr int kN = 6; };
template <> struct GmQ<QK_Q4_1> { static constexpr int kN = 6; };
template <> struct GmQ<QK_Q8_0> { static constexpr int kN = 7; };
template <> struct GmQ<QK_Q5_0> { static constexpr int kN = 9; };
template <> struct GmQ<QK_Q5_1> { static constexpr int kN = 8; };

template <int FMT>
__device__ __forceinline__ int gm_offset(int slot, int g) {
    const int h = g & 1;
    if constexpr (FMT == QK_Q4_0) {
        constexpr int base[6] = {0, 4, 8, 20, 24, 0};
        return slot < 5 ? base[slot] + 8 * h : (h ? 0 : 16);
    } else if constexpr (FMT == QK_Q4_1) {
        constexpr int base[6] = {0, 4, 8, 20, 24, 28};
        return (slot == 0 || slot == 3) ? base[slot] : base[slot] + 8 * h;
    } else if constexpr (FMT == QK_Q5_0) {
        constexpr int base[9] = {0, 4, 4, 8, 12, 20, 24, 28, 32};
        constexpr bool by_half[9] = {false, false, true, true, true, false, false, true, true};
        return base[slot] + (by_half[slot] ? 8 * h : 0);
    } else if constexpr (FMT == QK_Q5_1) {
        constexpr int base[8] = {0, 4, 8, 12, 24, 28, 32, 36};
        constexpr bool by_half[8] = {false, false, true, true, false, false, true, true};
        return base[slot] + (by_half[slot] ? 8 * h : 0);
    } else {
        constexpr int base[7] = {0, 4, 8, 36, 40, 0, 32};
        return slot < 5 ? base[slot] + 8 * g : base[slot];
    }
}

__device__ __forceinline__ uint32_t gm_perm_lo(uint32_t src) {
    return __builtin_amdgcn_perm(0x64646464u, src, 0x04010400u);  // [b0, 64, b1, 64]
}
__device__ __forceinline__ uint32_t gm_perm_hi(uint32_t src) {
    return __builtin_amdgcn_perm(0x64646464u, src, 0x04030402u);  // [b2, 64, b3, 64]
}
__device__ __forceinline__ uint32_t gm_pk_add(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2g_t, a) + __builtin_bit_cast(half2g_t, b));
}
__device__ __forceinline__ uint32_t gm_pk_fma(uint32_t a, uint32_t s, uint32_t t) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(half2g_t, a),
                                                                  __builtin_bit_cast(half2g_t, s),
                                                                  __builtin_bit_cast(half2g_t, t)));
}
__device__ __forceinline__ uint32_t gm_pk_mul(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2g_t, a) * __builtin_bit_cast(half2g_t, b));
}
__device__ __forceinline__ uint32_t gm_pack2(float a, float b) {
    return (uint32_t)f2h(a) | ((uint32_t)f2h(b) << 16);
}
// The fp32 weight d*q + m (one rounding), then its fp16 (a second rounding).
// The fp32 value is made opaque first: otherwise the compiler fuses the fma
// and the conversion into one mixed-precision fma that rounds the exact sum
// straight to fp16, which differs where the fp32 rounding lands on an fp16
// tie (d = 0x3556, m = 0x0001, q = 3: 1.0 by the definition, 1.0009765625
// fused).
__device__ __forceinline__ float gm_q41_weight(float d, float q, float m) {
    float v = __builtin_fmaf(d, q, m);
    asm volatile("" : "+v"(v));
    return v;
}
__device__ __forceinline__ uint32_t gm_h2(float v) {
    const uint32_t b = f2h(v);
    return b | (b << 16);
}

// Per-lane constants of the dequantization.
struct GmLaneConst {
    uint32_t mask;   // Q4_x: nibble mask of this lane's half (low, or high in place)
    uint32_t s, t;   // Q4_0: packed fp16 scale and offset taking 0x64XX to q - 8
    uint32_t sel0;   // Q4_0: perm selector giving (d, d) of block 0
    uint32_t sel1;   // Q4_0: perm selector giving (d, d) of block 1
    float dscale;    // Q4_1: 1, or 1/16 for high nibbles kept in place (16q)
    uint32_t nsh;    // Q5: shift bringing this lane's nibbles to the low four bits (0 or 4)
    uint32_t qsh;    // Q5: shift bringing this lane's eight qh bits (elements 8g..8g+7) to bits 0-7
};

template <int FMT>
__device__ __forceinline__ GmLaneConst gm_lane_const(int g) {
    GmLaneConst c;
    const bool hi = (g >> 1) != 0;
    const bool h = (g & 1) != 0;
    c.mask = hi ? 0xF0F0F0F0u : 0x0F0F0F0Fu;
    c.s = hi ? gm_h2(0.0625f) : gm_h2(1.0f);
    c.t = hi ? gm_h2(-72.0f) : gm_h2(-1032.0f);
    // Q4_0: d of block 0 is pair bytes 0-1, d of block 1 bytes 18-19.  With
    // h = 0 they sit in slot 0 (offset 0, low half) and slot 5 (offset 16,
    // high half); with h = 1 in slot 5 (offset 0, low) and slot 2 (offset 16,
    // high).  perm(src0, src1, sel) takes selector values 4-7 from src0.
    c.sel0 = h ? 0x05040504u : 0x01000100u;  // perm(q5, q0)
    c.sel1 = h ? 0x07060706u : 0x03020302u;  // perm(q2, q5)
    c.dscale = hi ? 0.0625f : 1.0f;
    c.nsh = hi ? 4u : 0u;
    c.qsh = 8u * (uint32_t)g;
    return c;
}

// Two quant dwords (8 weights of this lane) -> 4 packed fp16 (one A operand).
template <int FMT>
__device__ __forceinline__ u32x4g_t gm_decode8(uint32_t qa, uint32_t qb, uint32_t dd, float d, float mm,
                                               const GmLaneConst &c) {
    if constexpr (FMT == QK_Q4_0) {
        const uint32_t ua = qa & c.mask, ub = qb & c.mask;
        return u32x4g_t{gm_pk_mul(gm_pk_fma(gm_perm_lo(ua), c.s, c.t), dd),
                        gm_pk_mul(gm_pk_fma(gm_perm_hi(ua), c.s, c.t), dd),
                        gm_pk_mul(gm_pk_fma(gm_perm_lo(ub), c.s, c.t), dd),
                        gm_pk_mul(gm_pk_fma(gm_perm_hi(ub), c.s, c.t), dd)};
    } else if constexpr (FMT == QK_Q8_0) {
        // c + 128 is the byte of (c ^ 0x80): 1024 + c + 128 - 1152 = c
        const uint32_t ua = qa ^ 0x80808080u, ub = qb ^ 0x80808080u;
        const uint32_t bias = 0xE480E480u;  // (-1152, -1152)
        return u32x4g_t{gm_pk_mul(gm_pk_add(gm_perm_lo(ua), bias), dd),
                        gm_pk_mul(gm_pk_add(gm_perm_hi(ua), bias), dd),
                        gm_pk_mul(gm_pk_add(gm_perm_lo(ub), bias), dd),
                        gm_pk_mul(gm_pk_add(gm_perm_hi(ub), bias), dd)};
    } else {
        // d here is d or d/16 (exact in fp32); times the in-place code it is
        // d * q exactly, so the fma rounds d*q + m once, as the definition does
        const uint32_t ua = qa & c.mask, ub = qb & c.mask;
        return u32x4g_t{gm_pack2(gm_q41_weight(d, ubyte_f<0>(ua), mm), gm_q41_weight(d, ubyte_f<1>(ua), mm)),
                        gm_pack2(gm_q41_weight(d, ubyte_f<2>(ua), mm), gm_q41_weight(d, ubyte_f<3>(ua), mm)),
                        gm_pack2(gm_q41_weight(d, ubyte_f<0>(ub), mm), gm_q41_weight(d, ubyte_f<1>(ub), mm)),
                        gm_pack2(gm_q41_weight(d, ubyte_f<2>(ub), mm), gm_q41_weight(d, ubyte_f<3>(ub), mm))};
    }
}

// Q5: two quant dwords and the block's qh word -> 4 packed fp16 (one A
// operand).  The lane's nibbles are brought to the low four bits of each
// byte and bit 4 of each code comes from its qh bit (elements 8g..8g+7 are
// qh bits 8g..8g+7), so each byte is the 5-bit code q.  Q5_0: 1024 + q as
// fp16, minus 1040 is q - 16 exactly, times (d, d) is the one rounding of the
// exact weight; Q5_1: the fp32 weight d*q + m, then its fp16 (as Q4_1).
template <int FMT>
__device__ __forceinline__ u32x4g_t gm_decode8_q5(uint32_t qa, uint32_t qb, uint32_t qh, uint32_t dd, float d,
                                                  float mm, const GmLaneConst &c) {
    const uint32_t hb = (qh >> c.qsh) & 0xFFu;
    const uint32_t ua = ((qa >> c.nsh) & 0x0F0F0F0Fu) | q5_high4(hb & 0xFu);
    const uint32_t ub = ((qb >> c.nsh) & 0x0F0F0F0Fu) | q5_high4(hb >> 4);
    if constexpr (FMT == QK_Q5_0) {
        const uint32_t bias = 0xE410E410u;  // (-1040, -1040)
        return u32x4g_t{gm_pk_mul(gm_pk_add(gm_perm_lo(ua), bias), dd),
                        gm_pk_mul(gm_pk_add(gm_perm_hi(ua), bias), dd),
                        gm_pk_mul(gm_pk_add(gm_perm_lo(ub), bias), dd),
                        gm_pk_mul(gm_pk_add(gm_perm_hi(ub), bias), dd)};
    } else {
        return u32x4g_t{gm_pack2(gm_q41_weight(d, ubyte_f<0>(ua), mm), gm_q41_weight(d, ubyte_f<1>(ua), mm)),
                        gm_pack2(gm_q41_weight(d, ubyte_f<2>(ua), mm), gm_q41_weight(d, ubyte_f<3>(ua), mm)),
                        gm_pack2(gm_q41_weight(d, ubyte_f<0>(ub), mm), gm_q41_weight(d, ubyte_f<1>(ub), mm)),
                        gm_pack2(gm_q41_weight(d, ubyte_f<2>(ub), mm), gm_q41_weight(d, ubyte_f<3>(ub), mm))};
    }
}

// The lane's A operands of one 16-row tile and step: block 0 -> a0, block 1 -> a1.
template <int FMT>
__device__ __forceinline__ void gm_decode(const uint32_t (&q)[GmQ<FMT>::kN], const GmLaneConst &c,
                                          u32x4g_t &a0, u32x4g_t &a1) {
    if constexpr (FMT == QK_Q4_0) {
        const uint32_t dd0 = __builtin_amdgcn_perm(q[5], q[0], c.sel0);
        const uint32_t dd1 = __builtin_amdgcn_perm(q[2], q[5], c.sel1);
        a0 = gm_decode8<FMT>(__builtin_amdgcn_alignbyte(q[1], q[0], 2), __builtin_amdgcn_alignbyte(q[2], q[1], 2),
                             dd0, 0.0f, 0.0f, c);
        a1 = gm_decode8<FMT>(q[3], q[4], dd1, 0.0f, 0.0f, c);
    } else if constexpr (FMT == QK_Q8_0) {
        const uint32_t dd0 = __builtin_amdgcn_perm(0u, q[5], 0x01000100u);
        const uint32_t dd1 = __builtin_amdgcn_perm(0u, q[6], 0x03020302u);
        a0 = gm_decode8<FMT>(__builtin_amdgcn_alignbyte(q[1], q[0], 2), __builtin_amdgcn_alignbyte(q[2], q[1], 2),
                             dd0, 0.0f, 0.0f, c);
        a1 = gm_decode8<FMT>(q[3], q[4], dd1, 0.0f, 0.0f, c);
    } else if constexpr (FMT == QK_Q5_0) {
        // block 0: d in the low half of dword 0, qh two bytes further, its
        // quant half 2 bytes past dwords 4+8h..; block 1: d in the high half
        // of dword 20, qh and quant bytes aligned
        const uint32_t dd0 = __builtin_amdgcn_perm(0u, q[0], 0x01000100u);
        const uint32_t dd1 = __builtin_amdgcn_perm(0u, q[5], 0x03020302u);
        a0 = gm_decode8_q5<FMT>(__builtin_amdgcn_alignbyte(q[3], q[2], 2), __builtin_amdgcn_alignbyte(q[4], q[3], 2),
                                __builtin_amdgcn_alignbyte(q[1], q[0], 2), dd0, 0.0f, 0.0f, c);
        a1 = gm_decode8_q5<FMT>(q[7], q[8], q[6], dd1, 0.0f, 0.0f, c);
    } else if constexpr (FMT == QK_Q5_1) {
        const float d0 = h2f(q[0] & 0xFFFFu), m0 = h2f(q[0] >> 16);
        const float d1 = h2f(q[4] & 0xFFFFu), m1 = h2f(q[4] >> 16);
        a0 = gm_decode8_q5<FMT>(q[2], q[3], q[1], 0u, d0, m0, c);
        a1 = gm_decode8_q5<FMT>(q[6], q[7], q[5], 0u, d1, m1, c);
    } else {
        const float d0 = h2f(q[0] & 0xFFFFu) * c.dscale, m0 = h2f(q[0] >> 16);
        const float d1 = h2f(q[3] & 0xFFFFu) * c.dscale, m1 = h2f(q[3] >> 16);
        a0 = gm_decode8<FMT>(q[1], q[2], 0u, d0, m0, c);
        a1 = gm_decode8<FMT>(q[4], q[5], 0u, d1, m1, c);
    }
}

// Quant dwords a lane reads from LDS per 16-row tile and step.  For Q4_0 the
// last one (the dword holding the scale of the block whose quant bytes the
// lane does not otherwise read) is taken from the lane 16 away instead: the
// same row, other half of the quant bytes, which has block 0's scale in its
// slot 0 (h = 0) or block 1's in its slot 2 (h = 1).  Read from LDS, the two
// halves' scale dwords fall on the same banks for rows 8 apart.
template <int FMT> constexpr int gm_lds_slots() { return FMT == QK_Q4_0 ? 5 : GmQ<FMT>::kN; }

template <int FMT>
__device__ __forceinline__ void gm_partner_scale(uint32_t (&q)[GmQ<FMT>::kN], int g) {
    if constexpr (FMT == QK_Q4_0) {
        const bool odd = (g & 1) != 0;
        const uint32_t s = odd ? q[2] : q[0];
        // rows of 16 lanes: the odd rows of the first operand trade places
        // with the even rows of the second
        const auto r = __builtin_amdgcn_permlane16_swap(s, s, false, false);
        q[5] = odd ? r[0] : r[1];
    }
}

// Combine the two k groups of a 256 x 128 tile and store it: group KG
// finishes columns 64KG..64KG+63.  In two rounds (row tiles 0-1, then 2-3),
// each wave hands the partial sums of the other group's columns to its
// partner through LDS (8 waves x 8 tiles x 64 lanes x 16 bytes).  Column
// indices are compile-time constants so that the accumulators stay in
// registers, hence one instance per group.
template <int KG, bool YALIGNED, bool ACC = false>
__device__ __forceinline__ void gm_finish(floatx4_t (&acc)[kRT][kCT], uint8_t *lds, int wave, int lane,
                                          int row0, int col0, int m, int n, float *__restrict__ y,
                                          int64_t ldy) {
    const int wm = wave & 3, g = lane >> 4;
    float4 *red = reinterpret_cast<float4 *>(lds);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
#pragma unroll
        for (int il = 0; il < 2; ++il)
#pragma unroll
            for (int jl = 0; jl < 4; ++jl) {
                const int i = 2 * r + il;
                constexpr int jo = 4 * (1 - KG);
                const int owner = (1 - KG) * 4 + wm;
                red[((owner * 2 + il) * 4 + jl) * 64 + lane] =
                    make_float4(acc[i][jo + jl][0], acc[i][jo + jl][1], acc[i][jo + jl][2], acc[i][jo + jl][3]);
            }
        __syncthreads();
#pragma unroll
        for (int il = 0; il < 2; ++il)
#pragma unroll
            for (int jl = 0; jl < 4; ++jl) {
                const int i = 2 * r + il;
                constexpr int jm = 4 * KG;
                const float4 o = red[((wave * 2 + il) * 4 + jl) * 64 + lane];
                acc[i][jm + jl][0] += o.x;
                acc[i][jm + jl][1] += o.y;
                acc[i][jm + jl][2] += o.z;
                acc[i][jm + jl][3] += o.w;
            }
        __syncthreads();
    }

    // acc[i][j][e] is row 64*wm + 16i + 4*(lane/16) + e, column 16j + lane%16
    // of the tile; this group stores j = 4KG..4KG+3.  Row tiles i and i+1 of
    // a column tile go out as two stores that each cover 32 rows (one 128-byte
    // line) of 8 columns: within each row of 16 lanes, lanes 0-7 hand their
    // rows 16-31 to lanes 8-15 and take those lanes' rows 0-15 (DPP rotation
    // by 8).  Stores of 16 rows of 16 columns would write every line in two
    // halves, which costs about half as many bytes again in HBM writes.
    const int c8 = lane & 7;
    const bool up = (lane & 8) != 0;
    // ACC: add to the outputs already in y (the second launch of a split K)
    auto put = [&](const floatx4_t &v, int col, int row) {
        if (col >= n) return;
        float *p = y + (int64_t)col * ldy + row;
        if (YALIGNED && row + 3 < m) {
            floatx4_t o = v;
            if constexpr (ACC) o += *reinterpret_cast<const floatx4_t *>(p);
            // non-temporal: every tile writes its outputs at the end, all at once
            __builtin_nontemporal_store(o, reinterpret_cast<floatx4_t *>(p));
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (row + e < m) p[e] = ACC ? p[e] + v[e] : v[e];
        }
    };
#pragma unroll
    for (int jl = 0; jl < 4; ++jl) {
        constexpr int jm = 4 * KG;
        const int colt = col0 + (jm + jl) * 16;
#pragma unroll
        for (int ip = 0; ip < kRT / 2; ++ip) {
            const floatx4_t a = acc[2 * ip][jm + jl], b = acc[2 * ip + 1][jm + jl];
            floatx4_t r;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float s = up ? a[e] : b[e];
                r[e] = __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, s), 0x128, 0xF,
                                                                          0xF, false));  // row_ror:8
            }
            const int row = row0 + wm * 64 + ip * 32 + (up ? 16 : 0) + 4 * g;
            put(up ? r : a, colt + c8, row);
            put(up ? b : r, colt + 8 + c8, row);
        }
    }
}

// Combine the eight k groups of a 64 x 32 tile (the small-batch shape) and
// store it: every wave writes its 8 partial 16 x 16 tiles to LDS (8 waves x 8
// tiles x 64 lanes x 16 bytes), then wave w adds tile w of all eight groups,
// in group order, and stores it.
template <bool YALIGNED>
__device__ __forceinline__ void gm_finish8(floatx4_t (&acc)[kRT][2], uint8_t *lds, int wave, int lane, int row0,
                                           int col0, int m, int n, float *__restrict__ y, int64_t ldy) {
    floatx4_t *red = reinterpret_cast<floatx4_t *>(lds);
#pragma unroll
    for (int i = 0; i < kRT; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) red[(wave * 8 + i * 2 + j) * 64 + lane] = acc[i][j];
    __syncthreads();
    floatx4_t v = red[wave * 64 + lane];
#pragma unroll
    for (int grp = 1; grp < 8; ++grp) v += red[(grp * 8 + wave) * 64 + lane];
    // tile `wave` is row tile wave / 2, column tile wave % 2; the lane holds
    // rows 4 (lane / 16) .. + 3 of column lane % 16
    const int col = col0 + (wave & 1) * 16 + (lane & 15);
    const int row = row0 + (wave >> 1) * 16 + 4 * (lane >> 4);
    if (col < n) {
        float *p = y + (int64_t)col * ldy + row;
        if (YALIGNED && row + 3 < m) {
            __builtin_nontemporal_store(v, reinterpret_cast<floatx4_t *>(p));
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (row + e < m) p[e] = v[e];
        }
    }
}

// LDS bytes per weight row and step in the quant stage (the pair, padded so
// that rows start on 16 bytes; the pitch in dwords is 4 mod 8 or 8 mod 16,
// which spreads 16 consecutive rows over distinct banks).
template <int FMT> struct GmStage;
template <> struct GmStage<QK_Q4_0> { static constexpr int kPitch = 48; };
template <> struct GmStage<QK_Q4_1> { static constexpr int kPitch = 48; };
template <> struct GmStage<QK_Q8_0> { static constexpr int kPitch = 80; };
template <> struct GmStage<QK_Q5_0> { static constexpr int kPitch = 48; };
template <> struct GmStage<QK_Q5_1> { static constexpr int kPitch = 48; };

template <int FMT>
constexpr size_t gm_group_lds() {
    return 2 * (size_t)kBN * kPitch * 2 + 2 * (size_t)kBM * GmStage<FMT>::kPitch;
}
template <int FMT>
constexpr size_t gm_lds_bytes() {
    // two k groups; the partial-sum exchange (8 waves x 8 tiles x 64 lanes x
    // 16 bytes) reuses the same memory after the k loop
    return 2 * gm_group_lds<FMT>() > 8 * 8 * 64 * 16 ? 2 * gm_group_lds<FMT>() : 8 * 8 * 64 * 16;
}

// FAST: w 4-byte aligned and an even number of blocks per row (every pair
// starts on 4 bytes and both of its blocks exist).  XFAST: x 16-byte aligned
// and ldx % 8 == 0; otherwise each thread's 64 activation bytes are read as
// the 17 dwords from the 4-byte boundary below them and shifted into place
// (a 2-byte aligned column starts 2 bytes into its first dword and ends 2
// bytes into its last, so nothing outside those dwords is read).
// YALIGNED: y 16-byte aligned and ldy % 4 == 0.
template <int FMT, bool FAST, bool XFAST, bool YALIGNED>
__global__ __launch_bounds__(kGmThreads) void gemm_kernel(
    const uint8_t *__restrict__ w, int m, int nb, const uint16_t *__restrict__ x, int64_t ldx,
    int n, float *__restrict__ y, int64_t ldy, int mtiles, int ntiles) {
    using F = Format<FMT>;
    constexpr int NQ = GmQ<FMT>::kN;
    constexpr int kPairBytes = 2 * F::kBytes;
    constexpr int kNC = kPairBytes / 16;        // 16-byte chunks of a pair
    constexpr int kTail = kPairBytes % 16;      // remaining 4 or 8 bytes
    constexpr int kAP = GmStage<FMT>::kPitch;
    constexpr int kBufHalves = kBN * kPitch;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    // XCD-aware tile order: XCD x (= id % 8) takes a contiguous range of tiles.
    const int ntot = mtiles * ntiles;
    const int id = blockIdx.x;
    const int xcd = id & 7, slot = id >> 3;
    const int per = ntot >> 3, rem = ntot & 7;
    const int L = (xcd < rem) ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
    const int mt = L / ntiles;
    const int nt = L - mt * ntiles;
    const int row0 = mt * kBM;
    const int col0 = nt * kBN;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int g = lane >> 4;
    const int wm = wave & 3;     // 64-row slice of the tile
    const int kg = wave >> 2;    // k group: first or second half of the pairs
    const int gtid = tid & 255;  // thread index within the k group
    const int k = nb * 32;
    const int npairs = (nb + 1) / 2;
    const int nsteps = (npairs + 1) / 2;   // steps of group 0; group 1 has npairs - nsteps
    const int pbase = kg * nsteps;
    const int gsteps = kg ? npairs - nsteps : nsteps;
    const int64_t row_bytes = (int64_t)nb * F::kBytes;
    const GmLaneConst lc = gm_lane_const<FMT>(g);

    // this group's LDS: activation tiles [2][kBN][kPitch] halves, then the
    // quant stages [2][kBM][kAP] bytes
    uint8_t *const glds = lds + kg * gm_group_lds<FMT>();
    uint16_t *const bsm = reinterpret_cast<uint16_t *>(glds);
    uint8_t *const asm_ = glds + 2 * (size_t)kBufHalves * 2;

    // Quant staging role: 16-byte chunk u of thread gtid is chunk c of row r
    // (e = gtid + 256u, r = e / kNC, c = e % kNC), and the tail of row gtid.
    // Rows past the matrix read a clamped, valid row: output (i, j) depends
    // only on weight row i and activation column j, and such rows are never
    // stored.
    const uint8_t *arow[kNC + 1];
#pragma unroll
    for (int u = 0; u < kNC; ++u) {
        const int e = gtid + 256 * u;
        arow[u] = w + (int64_t)min(row0 + e / kNC, m - 1) * row_bytes + 16 * (e % kNC);
    }
    arow[kNC] = w + (int64_t)min(row0 + gtid, m - 1) * row_bytes + 16 * kNC;

    // activation staging role: column gtid/2 of the tile, k-half gtid%2 of the step
    const int bcol = gtid >> 1, bhalf = gtid & 1;
    const uint16_t *__restrict__ xcol = x + (int64_t)min(col0 + bcol, n - 1) * ldx + 32 * bhalf;

    typedef u32x4g_t ASet[kRT][2];
    typedef uint32_t QStage[kNC * 4 + kTail / 4];
    typedef u32x4g_t XSet[4];

    // Global -> registers: the quant bytes and activations of local step s
    // (clamped to the group's last pair; the data of a clamped step is unused).
    auto load_a = [&](int s, QStage &qa) __attribute__((always_inline)) {
        const int pair = pbase + min(s, gsteps - 1);
        const int64_t off = (int64_t)pair * kPairBytes;
        if constexpr (FAST) {
#pragma unroll
            for (int u = 0; u < kNC; ++u) {
                const u32x4g_a4 t = *reinterpret_cast<const u32x4g_a4 *>(arow[u] + off);
                qa[4 * u] = t.x; qa[4 * u + 1] = t.y; qa[4 * u + 2] = t.z; qa[4 * u + 3] = t.w;
            }
            if constexpr (kTail >= 8) {
                const u32x2g_a4 t = *reinterpret_cast<const u32x2g_a4 *>(arow[kNC] + off);
                qa[4 * kNC] = t.x; qa[4 * kNC + 1] = t.y;
                if constexpr (kTail == 12) qa[4 * kNC + 2] = *reinterpret_cast<const uint32_t *>(arow[kNC] + off + 8);
            } else if constexpr (kTail == 4) {
                qa[4 * kNC] = *reinterpret_cast<const uint32_t *>(arow[kNC] + off);
            }
        } else {
            // A pair may start 2 bytes past a dword (2-byte aligned w, or
            // every other row of an odd block count).  A chunk whose bytes all
            // belong to the row is read as the dwords from the boundary below
            // it and shifted into place (the extra dword of a 2-byte offset
            // holds the chunk's last two bytes, so nothing outside the row's
            // dwords is read); a chunk reaching past a missing second block
            // (the last pair of an odd block count) takes 2-byte loads, the
            // missing bytes reading as zeros (scale 0, weights 0).
            const bool second = 2 * pair + 1 < nb;
#pragma unroll
            for (int u = 0; u < kNC + (kTail > 0 ? 1 : 0); ++u) {
                const int nd = u < kNC ? 4 : kTail / 4;
                const int pos0 = u < kNC ? 16 * ((gtid + 256 * u) % kNC) : 16 * kNC;
                const uint8_t *a = arow[u] + off;
                if (second || pos0 + 4 * nd <= F::kBytes) {
                    const uintptr_t ai = reinterpret_cast<uintptr_t>(a);
                    const uint32_t *base = reinterpret_cast<const uint32_t *>(ai & ~uintptr_t(3));
                    const uint32_t sh = (uint32_t)(ai & 3);  // 0 or 2
                    uint32_t d[5];
                    if (nd == 4) {
                        const u32x4g_a4 t = *reinterpret_cast<const u32x4g_a4 *>(base);
                        d[0] = t.x; d[1] = t.y; d[2] = t.z; d[3] = t.w;
                    } else if (nd == 3) {
                        const u32x2g_a4 t = *reinterpret_cast<const u32x2g_a4 *>(base);
                        d[0] = t.x; d[1] = t.y; d[2] = base[2]; d[3] = 0u;
                    } else if (nd == 2) {
                        const u32x2g_a4 t = *reinterpret_cast<const u32x2g_a4 *>(base);
                        d[0] = t.x; d[1] = t.y; d[2] = 0u; d[3] = 0u;
                    } else {
                        d[0] = base[0]; d[1] = 0u; d[2] = 0u; d[3] = 0u;
                    }
                    d[4] = 0u;
                    if (sh) d[nd] = base[nd];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (e < nd) qa[4 * u + e] = __builtin_amdgcn_alignbyte(d[e + 1], d[e], sh);
                } else {
                    const uint16_t *hp = reinterpret_cast<const uint16_t *>(a);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (e < nd) {
                            const int o = pos0 + 4 * e;
                            const uint32_t lo = o < F::kBytes ? (uint32_t)hp[2 * e] : 0u;
                            const uint32_t hi = o + 2 < F::kBytes ? (uint32_t)hp[2 * e + 1] : 0u;
                            qa[4 * u + e] = lo | (hi << 16);
                        }
                    }
                }
            }
        }
    };
    auto store_a = [&](const QStage &qa, int buf) __attribute__((always_inline)) {
        uint8_t *st = asm_ + buf * (kBM * kAP);
#pragma unroll
        for (int u = 0; u < kNC; ++u) {
            const int e = gtid + 256 * u;
            *reinterpret_cast<u32x4g_t *>(st + (e / kNC) * kAP + 16 * (e % kNC)) =
                u32x4g_t{qa[4 * u], qa[4 * u + 1], qa[4 * u + 2], qa[4 * u + 3]};
        }
        if constexpr (kTail >= 8) {
            *reinterpret_cast<u32x2g_t *>(st + gtid * kAP + 16 * kNC) = u32x2g_t{qa[4 * kNC], qa[4 * kNC + 1]};
            if constexpr (kTail == 12) *reinterpret_cast<uint32_t *>(st + gtid * kAP + 16 * kNC + 8) = qa[4 * kNC + 2];
        } else if constexpr (kTail == 4) {
            *reinterpret_cast<uint32_t *>(st + gtid * kAP + 16 * kNC) = qa[4 * kNC];
        }
    };

    auto load_b = [&](int s, XSet &xb) __attribute__((always_inline)) {
        const int pair = pbase + min(s, gsteps - 1);
        const uint16_t *p = xcol + pair * kBK;
        // k is a multiple of 32: a thread's 32 activations are all in the
        // column or all past it (the missing second block of an odd block
        // count), and those past it are zeros, never loaded: for the last
        // column they would lie past the end of x
        if (pair * kBK + 32 * bhalf >= k) {
#pragma unroll
            for (int u = 0; u < 4; ++u) xb[u] = u32x4g_t{0u, 0u, 0u, 0u};
        } else if constexpr (XFAST) {
#pragma unroll
            for (int u = 0; u < 4; ++u) xb[u] = *reinterpret_cast<const u32x4g_t *>(p + 8 * u);
        } else {
            const uintptr_t a = reinterpret_cast<uintptr_t>(p);
            const uint32_t *base = reinterpret_cast<const uint32_t *>(a & ~uintptr_t(3));
            const uint32_t sh = (uint32_t)(a & 3);  // 0 or 2
            uint32_t d[17];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const u32x4g_a4 t = *reinterpret_cast<const u32x4g_a4 *>(base + 4 * u);
                d[4 * u] = t.x; d[4 * u + 1] = t.y; d[4 * u + 2] = t.z; d[4 * u + 3] = t.w;
            }
            d[16] = sh ? base[16] : 0u;  // only a 2-byte offset reaches into a 17th dword
#pragma unroll
            for (int u = 0; u < 4; ++u)
                xb[u] = u32x4g_t{__builtin_amdgcn_alignbyte(d[4 * u + 1], d[4 * u], sh),
                                 __builtin_amdgcn_alignbyte(d[4 * u + 2], d[4 * u + 1], sh),
                                 __builtin_amdgcn_alignbyte(d[4 * u + 3], d[4 * u + 2], sh),
                                 __builtin_amdgcn_alignbyte(d[4 * u + 4], d[4 * u + 3], sh)};
        }
    };
    auto store_b = [&](const XSet &xb, int buf) __attribute__((always_inline)) {
        u32x4g_t *dst = reinterpret_cast<u32x4g_t *>(bsm + buf * kBufHalves + bcol * kPitch + 32 * bhalf);
#pragma unroll
        for (int u = 0; u < 4; ++u) dst[u] = xb[u];
    };

    // LDS quant stage -> this lane's A operands (16-row tile i: rows
    // 64wm + 16i + lane%16, the lane's 8 elements of each block).
    auto decode = [&](int buf, ASet &a) __attribute__((always_inline)) {
        const uint8_t *st = asm_ + buf * (kBM * kAP) + (wm * 64 + (lane & 15)) * kAP;
#pragma unroll
        for (int i = 0; i < kRT; ++i) {
            uint32_t q[NQ];
#pragma unroll
            for (int t = 0; t < gm_lds_slots<FMT>(); ++t)
                q[t] = *reinterpret_cast<const uint32_t *>(st + i * 16 * kAP + gm_offset<FMT>(t, g));
            gm_partner_scale<FMT>(q, g);
            gm_decode<FMT>(q, lc, a[i][0], a[i][1]);
        }
    };

    floatx4_t acc[kRT][kCT];
#pragma unroll
    for (int i = 0; i < kRT; ++i)
#pragma unroll
        for (int j = 0; j < kCT; ++j) acc[i][j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // (activation fragments read one group of eight products ahead; two
    // groups, as in the direct-load kernel, spill registers here)
    auto mma = [&](const ASet &a, int buf) __attribute__((always_inline)) {
        const uint16_t *bb = bsm + buf * kBufHalves + (lane & 15) * kPitch + 8 * g;
        auto frag = [&](int q, int h) -> half8_t {
            const int ks = q >> 2, j = 2 * (q & 3) + h;
            return *reinterpret_cast<const half8_t *>(bb + j * 16 * kPitch + 32 * ks);
        };
        constexpr int FA = 1;
        half8_t fr[FA + 1][2];
#pragma unroll
        for (int u = 0; u < FA; ++u) {
            fr[u][0] = frag(u, 0);
            fr[u][1] = frag(u, 1);
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int ks = q >> 2, j = 2 * (q & 3);
            if (q + FA < 8) {
                fr[(q + FA) % (FA + 1)][0] = frag(q + FA, 0);
                fr[(q + FA) % (FA + 1)][1] = frag(q + FA, 1);
            }
            const half8_t c0 = fr[q % (FA + 1)][0], c1 = fr[q % (FA + 1)][1];
#pragma unroll
            for (int i = 0; i < kRT; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a[i][ks]), c0,
                                                                   acc[i][j], 0, 0, 0);
#pragma unroll
            for (int i = 0; i < kRT; ++i)
                acc[i][j + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a[i][ks]), c1,
                                                                       acc[i][j + 1], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    if (nsteps > 0) {
        QStage qa;
        XSet xb;
        load_a(0, qa);
        load_b(0, xb);
        store_a(qa, 0);
        store_b(xb, 0);
        __syncthreads();
        // Local step s (both groups step together; group 1 skips the multiply
        // of a step past its last pair): prefetch step s+1 into registers,
        // dequantize step s from LDS, multiply, then stage step s+1 into the
        // other LDS buffers.
        for (int s = 0; s < nsteps; ++s) {
            const int buf = s & 1;
            load_a(s + 1, qa);
            load_b(s + 1, xb);
            if (s < gsteps) {
                ASet f;
                decode(buf, f);
                mma(f, buf);
            }
            store_a(qa, buf ^ 1);
            store_b(xb, buf ^ 1);
            __syncthreads();
        }
    }

    if (kg == 0)
        gm_finish<0, YALIGNED>(acc, lds, wave, lane, row0, col0, m, n, y, ldy);
    else
        gm_finish<1, YALIGNED>(acc, lds, wave, lane, row0, col0, m, n, y, ldy);
}

// ---------------------------------------------------------------------------
// Aligned path: the same tile, waves and arithmetic, with the operands copied
// global -> LDS by the gfx950 direct loads (global_load_lds, no registers in
// between) into a ring of stages, kDmaLead super-steps ahead of their use.
// A super-step is two consecutive pairs: k group 0 multiplies the first and
// k group 1 the second, so one stage holds, per weight row, 72 / 80 / 136
// contiguous quant bytes, and two 128 x 64 activation tiles.
//
// Quant stage: the row's bytes as 16-byte chunks, row pitch 16 * kDmaChunks;
// a row length that is not a multiple of 16 (Q4_0 72, Q8_0 136) is covered by
// a last chunk that overlaps the one before it (global bytes R-16..R-1), so
// global byte o >= 16 (kDmaChunks - 1) sits at o + kDmaPad in LDS.
// Activation tile: column c's eight 16-byte chunks at c*128 + 16 (q ^ ((c/2)
// % 8)) (an XOR swizzle in place of padding: the direct loads write lane after
// lane, and 16 consecutive columns of a fragment read then fall on distinct
// banks).
// ---------------------------------------------------------------------------
// Tile shapes of the direct-load kernel: KG k groups of waves and 8 / KG row
// slices of 64 rows.  KG = 2: 256 x 128 tiles (a super-step is two pairs);
// KG = 8: 64 x 32 tiles for batches of up to 32 columns, where 256-row tiles
// leave most CUs idle (14336 rows: 56 tiles, against 224 of 64 rows); a
// super-step is then eight pairs, one per wave.
template <int KG> struct GmTile {
    static_assert(KG == 2 || KG == 8, "tile shape");
    static constexpr int kSlices = 8 / KG;
    static constexpr int kRows = 64 * kSlices;
    static constexpr int kCols = KG == 2 ? 128 : 32;
    static constexpr int kColTiles = kCols / 16;
};

template <int FMT, int KG = 2> struct GmDma {
    using T = GmTile<KG>;
    static constexpr int kRow = 2 * KG * Format<FMT>::kBytes;       // quant bytes per row and super-step
    // Rows that fill their chunks exactly get one more chunk, which gives the
    // spare bytes for the row shift below: Q4_1 at KG = 2 (80 bytes, at the
    // price of a 2-stage ring: measured 2-6 % faster than 3 stages without the
    // shift), Q5_1 at KG = 2 (96 bytes; two stages either way), and every
    // format at KG = 8 (288 / 320 / 544 / 352 / 384 bytes; Q4_1's three stages
    // take 162 816 of the 163 840 bytes, Q5's take two).
    static constexpr int kChunks =
        (kRow + 15) / 16 + (((kRow % 16) == 0 && (KG == 8 || FMT == QK_Q4_1 || FMT == QK_Q5_1)) ? 1 : 0);
    static constexpr int kPad = 16 * kChunks - kRow;
    // Rows 8-15 of every 16-row tile are stored 4 bytes later in their LDS
    // row (their chunks are loaded from 4 bytes earlier), so that the dwords
    // the lanes of rows r and r + 8 read in one instruction fall on
    // different banks.  Needs 4 spare bytes in the row.
    static constexpr bool kShift = kPad >= 4;
    static constexpr int kAStage = T::kRows * 16 * kChunks;         // bytes
    static constexpr int kBStage = KG * T::kCols * kBK * 2;         // bytes (one tile per k group)
    static constexpr int kStage = kAStage + kBStage;
    static constexpr int kStages = 3 * kStage <= 160 * 1024 ? 3 : 2;
    static constexpr int kLead = kStages - 1;                       // super-steps loaded ahead
    static constexpr int kAPerThread = (T::kRows * kChunks + kGmThreads - 1) / kGmThreads;
    static constexpr int kBPerThread = kBStage / 16 / kGmThreads;  // 4
    // Direct loads a wave issues per stage.  Wave v issues quant chunk u when
    // 512u + 64v < kBM * kChunks, so the last waves may issue one fewer; the
    // count used in the waits is the smallest one (wave 7's): leaving that
    // many newer loads outstanding completes the older stage for every wave
    // (a wave with more newer loads merely waits for one of them as well).
    static constexpr int kAMin = (T::kRows * kChunks - 64 * 7 + kGmThreads - 1) / kGmThreads;
    static_assert((T::kRows * kChunks) % 64 == 0, "whole waves of quant chunks");
    static constexpr int kLoadsPerStage = kAMin + kBPerThread;
};

template <int FMT, int KG>
constexpr size_t gm_dma_lds_bytes() {
    // the partial-sum exchange after the k loop takes 8 waves x 8 tiles x 64
    // lanes x 16 bytes for either shape
    return (size_t)GmDma<FMT, KG>::kStages * GmDma<FMT, KG>::kStage > 8 * 8 * 64 * 16
               ? (size_t)GmDma<FMT, KG>::kStages * GmDma<FMT, KG>::kStage
               : 8 * 8 * 64 * 16;
}

typedef __attribute__((address_space(3))) void gm_lds_void;
typedef __attribute__((address_space(1))) void gm_glb_void;

__device__ __forceinline__ void gm_dma16(const void *src, void *lds_wave_base) {
    __builtin_amdgcn_global_load_lds((gm_glb_void *)src, (gm_lds_void *)lds_wave_base, 16, 0, 0);
}

// s_waitcnt vmcnt(N) lgkmcnt(0), then the workgroup barrier; a
// compiler-level memory barrier as well.
template <int N>
__device__ __forceinline__ void gm_wait_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt immediate");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// nb blocks of each row are multiplied; rows are row_nb blocks apart (row_nb >
// nb when a second launch takes the rest of K, with ACC adding its products to
// y).
template <int FMT, bool YALIGNED, int KG, bool ACC>
__global__ __launch_bounds__(kGmThreads) void gemm_dma_kernel(
    const uint8_t *__restrict__ w, int m, int nb, const uint16_t *__restrict__ x, int64_t ldx,
    int n, float *__restrict__ y, int64_t ldy, int mtiles, int ntiles, int row_nb) {
    static_assert(!ACC || KG == 2, "only the 256 x 128 tile accumulates");
    using F = Format<FMT>;
    using D = GmDma<FMT, KG>;
    using T = GmTile<KG>;
    constexpr int CT = T::kColTiles;
    constexpr int NQ = GmQ<FMT>::kN;
    constexpr int kPairBytes = 2 * F::kBytes;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    // XCD-aware tile order: XCD x (= id % 8) takes a contiguous range of tiles.
    const int ntot = mtiles * ntiles;
    const int id = blockIdx.x;
    const int xcd = id & 7, slot = id >> 3;
    const int per = ntot >> 3, rem = ntot & 7;
    const int L = (xcd < rem) ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
    const int mt = L / ntiles;
    const int nt = L - mt * ntiles;
    const int row0 = mt * T::kRows;
    const int col0 = nt * T::kCols;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches on the k group
    const int lane = tid & 63;
    const int g = lane >> 4;
    const int wm = wave % T::kSlices;  // 64-row slice of the tile
    const int kg = wave / T::kSlices;  // k group: pair kg of each super-step
    const int npairs = nb / 2;         // whole super-steps here (nb % (2 KG) == 0)
    const int nsup = (npairs + KG - 1) / KG;
    const int64_t row_bytes = (int64_t)row_nb * F::kBytes;
    const GmLaneConst lc = gm_lane_const<FMT>(g);

    // Direct-load roles.  Quant chunk u of this thread: linear chunk
    // e = 512u + tid of the stage, row e / kChunks, chunk e % kChunks (rows
    // past the matrix are clamped: their outputs are never stored).
    const uint8_t *asrc[D::kAPerThread];
#pragma unroll
    for (int u = 0; u < D::kAPerThread; ++u) {
        const int e = min(kGmThreads * u + tid, T::kRows * D::kChunks - 1);
        const int r = e / D::kChunks, c = e % D::kChunks;
        const int sh = (D::kShift && (r & 8)) ? 4 : 0;
        const int R = min(row0 + r, m - 1);
        // the last chunk keeps its place at the end of the super-step's bytes;
        // a shifted first chunk reaches 4 bytes into the previous super-step or
        // row, which exists unless the row is a clamped copy of row 0 (m == 1,
        // never stored): that one starts at 0
        int off = c < D::kChunks - 1 ? 16 * c - sh : D::kRow - 16;
        if (R == 0 && off < 0) off = 0;
        asrc[u] = w + (int64_t)R * row_bytes + off;
    }
    // Activation chunk u: linear chunk e = 512u + tid, tile e / (8 kCols) (the
    // k group), column (e / 8) % kCols, stored slot e % 8 holding logical
    // 16-byte chunk (e % 8) ^ ((column / 2) % 8).
    const uint16_t *bsrc[D::kBPerThread];
    int bgrp[D::kBPerThread];
#pragma unroll
    for (int u = 0; u < D::kBPerThread; ++u) {
        const int e = kGmThreads * u + tid;
        const int grp = e / (8 * T::kCols), col = (e >> 3) & (T::kCols - 1), p = e & 7;
        const int q = p ^ ((col >> 1) & 7);
        bgrp[u] = grp;
        bsrc[u] = x + (int64_t)min(col0 + col, n - 1) * ldx + 8 * q;
    }

    // Issue the direct loads of super-step t (clamped to the last one) into
    // stage buffer `buf`.
    auto issue = [&](int t, int buf) __attribute__((always_inline)) {
        t = min(t, nsup - 1);
        uint8_t *st = lds + buf * D::kStage;
        const int64_t aoff = (int64_t)(KG * t) * kPairBytes;
#pragma unroll
        for (int u = 0; u < D::kAPerThread; ++u) {
            if (kGmThreads * u + wave * 64 < T::kRows * D::kChunks)  // wave-uniform
                gm_dma16(asrc[u] + aoff, st + 16 * (kGmThreads * u + wave * 64));
        }
        uint8_t *bst = st + D::kAStage;
#pragma unroll
        for (int u = 0; u < D::kBPerThread; ++u) {
            const int pair = min(KG * t + bgrp[u], npairs - 1);
            gm_dma16(bsrc[u] + pair * kBK, bst + 16 * (kGmThreads * u + wave * 64));
        }
    };

    // LDS byte offset of quant byte o (of the super-step's row bytes) in this
    // lane's row: the last chunk holds the row's last 16 bytes
    const int lsh = (D::kShift && (lane & 8)) ? 4 : 0;
    auto aoff_lds = [&](int o) __attribute__((always_inline)) {
        return o < 16 * (D::kChunks - 1) - lsh ? o + lsh : o + D::kPad;
    };
    int qoff[NQ];
#pragma unroll
    for (int t = 0; t < NQ; ++t) qoff[t] = aoff_lds(kg * kPairBytes + gm_offset<FMT>(t, g));
    const int arow = (wm * 64 + (lane & 15)) * 16 * D::kChunks;
    // activation fragment: column 16j + lane%16 of this group's tile, logical
    // chunk 4ks + g, stored at slot (4ks + g) ^ ((lane%16) / 2)
    const int bcol = (lane & 15) * 128;
    const int bslot0 = 16 * ((0 * 4 + g) ^ ((lane & 15) >> 1));
    const int bslot1 = 16 * ((1 * 4 + g) ^ ((lane & 15) >> 1));

    typedef u32x4g_t ASet[kRT][2];
    floatx4_t acc[kRT][CT];
#pragma unroll
    for (int i = 0; i < kRT; ++i)
#pragma unroll
        for (int j = 0; j < CT; ++j) acc[i][j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // The lane's A operands of stage `buf` (this k group's pair).
    auto decode_stage = [&](int buf, ASet &f) __attribute__((always_inline)) {
        const uint8_t *st = lds + buf * D::kStage;
#pragma unroll
        for (int i = 0; i < kRT; ++i) {
            const uint8_t *ar = st + arow + i * 16 * (16 * D::kChunks);
            uint32_t q[NQ];
#pragma unroll
            for (int t2 = 0; t2 < gm_lds_slots<FMT>(); ++t2) q[t2] = *reinterpret_cast<const uint32_t *>(ar + qoff[t2]);
            gm_partner_scale<FMT>(q, g);
            gm_decode<FMT>(q, lc, f[i][0], f[i][1]);
        }
    };
    // The products of stage `buf` (2 k halves x CT column tiles x 4 row
    // tiles), in groups of two column tiles.  The activation fragments are
    // read two at a time, two groups ahead of their use, so the matrix cores
    // wait less for the LDS.
    constexpr int GH = CT / 2;  // groups per k half
    auto mma_stage = [&](int buf, const ASet &f) __attribute__((always_inline)) {
        const uint8_t *bb = lds + buf * D::kStage + D::kAStage + kg * (T::kCols * kBK * 2) + bcol;
        auto frag = [&](int q, int h) -> half8_t {
            const int ks = q / GH, j = 2 * (q % GH) + h;
            return *reinterpret_cast<const half8_t *>(bb + j * 16 * 128 + (ks ? bslot1 : bslot0));
        };
        // groups of fragments in flight (one: 77-81 us on the Q4_0
        // 14336 x 4096 x 512 workload; two: 74-80 us; three: no better)
        constexpr int FA = 2;
        constexpr int NG = 2 * GH;  // groups per stage
        half8_t fr[FA + 1][2];
#pragma unroll
        for (int u = 0; u < FA && u < NG; ++u) {
            fr[u][0] = frag(u, 0);
            fr[u][1] = frag(u, 1);
        }
#pragma unroll
        for (int q = 0; q < NG; ++q) {
            const int ks = q / GH, j = 2 * (q % GH);
            if (q + FA < NG) {
                fr[(q + FA) % (FA + 1)][0] = frag(q + FA, 0);
                fr[(q + FA) % (FA + 1)][1] = frag(q + FA, 1);
            }
            const half8_t c0 = fr[q % (FA + 1)][0], c1 = fr[q % (FA + 1)][1];
#pragma unroll
            for (int i = 0; i < kRT; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, f[i][ks]), c0,
                                                                   acc[i][j], 0, 0, 0);
#pragma unroll
            for (int i = 0; i < kRT; ++i)
                acc[i][j + 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, f[i][ks]), c1,
                                                                       acc[i][j + 1], 0, 0, 0);
            // keep the later groups' reads ahead of these products
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    if (nsup > 0) {
#pragma unroll
        for (int t = 0; t < D::kLead; ++t) issue(t, t);
        gm_wait_barrier<(D::kLead - 1) * D::kLoadsPerStage>();

        int buf = 0;
        for (int t = 0; t < nsup; ++t) {
            int nbuf = buf + D::kLead;
            if (nbuf >= D::kStages) nbuf -= D::kStages;
            issue(t + D::kLead, nbuf);
            if (KG * t + kg < npairs) {  // wave-uniform
                ASet f;
                decode_stage(buf, f);
                mma_stage(buf, f);
            }
            // stage t+1 (issued kLead-1 super-steps ago) complete for every
            // wave before anyone reads it; the kLead-1 newer stages may still
            // be in flight
            gm_wait_barrier<(D::kLead - 1) * D::kLoadsPerStage>();
            buf = buf + 1 == D::kStages ? 0 : buf + 1;
        }
        // drain the clamped prefetches before the LDS is reused
        gm_wait_barrier<0>();
    }

    if constexpr (KG == 8) {
        gm_finish8<YALIGNED>(acc, lds, wave, lane, row0, col0, m, n, y, ldy);
    } else if (kg == 0) {
        gm_finish<0, YALIGNED, ACC>(acc, lds, wave, lane, row0, col0, m, n, y, ldy);
    } else {
        gm_finish<1, YALIGNED, ACC>(acc, lds, wave, lane, row0, col0, m, n, y, ldy);
    }
}

template <int FMT, bool YA, int KG, bool ACC = false>
static int launch_gemm_dma(const uint8_t *w, int m, int nb, const uint16_t *x, int64_t ldx, int n,
                           float *y, int64_t ldy, hipStream_t stream, int row_nb) {
    using T = GmTile<KG>;
    const int mtiles = (m + T::kRows - 1) / T::kRows;
    const int ntiles = (n + T::kCols - 1) / T::kCols;
    auto kern = gemm_dma_kernel<FMT, YA, KG, ACC>;
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)gm_dma_lds_bytes<FMT, KG>()) != hipSuccess)
        return QK_ERR_LAUNCH;
    return launch_lds(kern, dim3((unsigned)(mtiles * ntiles)), dim3(kGmThreads), gm_dma_lds_bytes<FMT, KG>(),
                      stream, w, m, nb, x, ldx, n, y, ldy, mtiles, ntiles, row_nb);
}

template <int FMT, bool FAST, bool XFAST, bool YA>
static int launch_gemm(const uint8_t *w, int m, int nb, const uint16_t *x, int64_t ldx, int n,
                       float *y, int64_t ldy, int mtiles, int ntiles, hipStream_t stream) {
    auto kern = gemm_kernel<FMT, FAST, XFAST, YA>;
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)gm_lds_bytes<FMT>()) != hipSuccess)
        return QK_ERR_LAUNCH;
    return launch_lds(kern, dim3((unsigned)(mtiles * ntiles)), dim3(kGmThreads), gm_lds_bytes<FMT>(), stream, w, m, nb,
                      x, ldx, n, y, ldy, mtiles, ntiles);
}

template <int FMT>
static int dispatch_gemm(const uint8_t *w, int m, int nb, const uint16_t *x, int64_t ldx, int n,
                         float *y, int64_t ldy, hipStream_t stream) {
    const int mtiles = (m + kBM - 1) / kBM;
    const int ntiles = (n + kBN - 1) / kBN;
    const bool fast = ((uintptr_t)w % 4) == 0 && (nb % 2) == 0;
    const bool xfast = ((uintptr_t)x % 16) == 0 && (ldx % 8) == 0;
    const bool ya = ((uintptr_t)y % 16) == 0 && (ldy % 4) == 0;
    // the direct-load path moves whole super-steps (two pairs, or eight for
    // the small-batch tile): k % 128 == 0, or k % 512 == 0
    constexpr bool kDmaFormat = true;
    const bool dma = kDmaFormat && fast && xfast && (nb % 4) == 0;
    const bool small = dma && nb >= 16 &&
                       (n <= kGmSmallBatch || (n <= kGmSmallBatchMax && mtiles * ntiles < device_cus()));
    if constexpr (kDmaFormat) {
        if (small) {
            // the small-batch tile takes whole eight-pair super-steps; the 4, 8 or
            // 12 blocks left over go to a second launch that adds its products
            const int nb16 = nb - nb % 16;
            int st = ya ? launch_gemm_dma<FMT, true, 8>(w, m, nb16, x, ldx, n, y, ldy, stream, nb)
                        : launch_gemm_dma<FMT, false, 8>(w, m, nb16, x, ldx, n, y, ldy, stream, nb);
            if (st != QK_OK || nb16 == nb) return st;
            const uint8_t *wr = w + (size_t)nb16 * Format<FMT>::kBytes;
            const uint16_t *xr = x + (size_t)nb16 * kBlockElems;
            return ya ? launch_gemm_dma<FMT, true, 2, true>(wr, m, nb - nb16, xr, ldx, n, y, ldy, stream, nb)
                      : launch_gemm_dma<FMT, false, 2, true>(wr, m, nb - nb16, xr, ldx, n, y, ldy, stream, nb);
        }
        if (dma)
            return ya ? launch_gemm_dma<FMT, true, 2>(w, m, nb, x, ldx, n, y, ldy, stream, nb)
                      : launch_gemm_dma<FMT, false, 2>(w, m, nb, x, ldx, n, y, ldy, stream, nb);
    }
    auto run = [&](auto fw, auto fx) {
        if (ya) return launch_gemm<FMT, decltype(fw)::value, decltype(fx)::value, true>(w, m, nb, x, ldx, n, y, ldy,
                                                                                        mtiles, ntiles, stream);
        return launch_gemm<FMT, decltype(fw)::value, decltype(fx)::value, false>(w, m, nb, x, ldx, n, y, ldy, mtiles,
                                                                                 ntiles, stream);
    };
    using T = std::true_type;
    using F = std::false_type;
    if (fast) return xfast ? run(T{}, T{}) : run(T{}, F{});
    return xfast ? run(F{}, T{}) : run(F{}, F{});
}

int launch_mul_mat(int fmt, const void *w, int64_t m, int64_t k, const uint16_t *x, int64_t n,
                   int64_t ldx, float *y, int64_t ldy, hipStream_t stream) {
    const uint8_t *wb = static_cast<const uint8_t *>(w);
    const int nb = (int)(k / kBlockElems);
    switch (fmt) {
    case QK_Q4_0: return dispatch_gemm<QK_Q4_0>(wb, (int)m, nb, x, ldx, (int)n, y, ldy, stream);
    case QK_Q4_1: return dispatch_gemm<QK_Q4_1>(wb, (int)m, nb, x, ldx, (int)n, y, ldy, stream);
    case QK_Q8_0: return dispatch_gemm<QK_Q8_0>(wb, (int)m, nb, x, ldx, (int)n, y, ldy, stream);
    case QK_Q5_0: return dispatch_gemm<QK_Q5_0>(wb, (int)m, nb, x, ldx, (int)n, y, ldy, stream);
    case QK_Q5_1: return dispatch_gemm<QK_Q5_1>(wb, (int)m, nb, x, ldx, (int)n, y, ldy, stream);
    default: return QK_ERR_UNSUPPORTED;
    }
}

}  // namespace qk
