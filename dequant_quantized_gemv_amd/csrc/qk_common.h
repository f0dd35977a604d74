// qk_common.h - format traits and device helpers shared by the gfx950 kernels.
//
// Block formats (from the "llama_cpp 0.12.1 -> 0.12.2" diff of ggml-cuda.cu,
// hunks adding dequantize_block_q4_0 / _q4_1 / _q8_0_f16):
//   Q4_0: d (fp16) then 16 quant bytes; byte j = element j (low nibble) and
//         element j+16 (high nibble); value d*q + (-8*d).
//   Q4_1: d, m (fp16) then 16 quant bytes as above; value d*q + m.
//   Q8_0: d (fp16) then 32 int8; value d*q.
//   Q5_0: d, qh (4 bytes, bit t = bit 4 of code t), 16 quant bytes as Q4_0;
//         value (q - 16) * d.  Q5_1: d, m, qh, 16 quant bytes; value d*q + m.
//         (Named only in the diff's to_fp16 / to_fp32 dispatch; ggml's block
//         format.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qk.h"

namespace qk {

constexpr int kBlockElems = 32;

template <int FMT> struct Format;
template <> struct Format<QK_Q4_0> { static constexpr int kBytes = 18, kQsOffset = 2, kQsBytes = 16; };
template <> struct Format<QK_Q4_1> { static constexpr int kBytes = 20, kQsOffset = 4, kQsBytes = 16; };
template <> struct Format<QK_Q8_0> { static constexpr int kBytes = 34, kQsOffset = 2, kQsBytes = 32; };
template <> struct Format<QK_Q5_0> {
    static constexpr int kBytes = 22, kQhOffset = 2, kQsOffset = 6, kQsBytes = 16;
};
template <> struct Format<QK_Q5_1> {
    static constexpr int kBytes = 24, kQhOffset = 4, kQsOffset = 8, kQsBytes = 16;
};

// Bit 4 of four consecutive Q5 codes: bits b (0..3) of `four` -> bit 4 of
// byte b (the multiply places bit b at bit 8b, with no carries between the
// shifted copies, which sit 7 bits apart).
__device__ __forceinline__ uint32_t q5_high4(uint32_t four) {
    return ((four * 0x00204081u) & 0x01010101u) << 4;
}

inline int block_bytes_host(int fmt) {
    switch (fmt) {
    case QK_Q4_0: return Format<QK_Q4_0>::kBytes;
    case QK_Q4_1: return Format<QK_Q4_1>::kBytes;
    case QK_Q8_0: return Format<QK_Q8_0>::kBytes;
    case QK_Q5_0: return Format<QK_Q5_0>::kBytes;
    case QK_Q5_1: return Format<QK_Q5_1>::kBytes;
    default: return 0;
    }
}

// binary16 bits -> fp32 (v_cvt_f32_f16: exact, fp16 subnormals kept).
__device__ __forceinline__ float h2f(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// fp32 -> binary16 bits, round to nearest even (v_cvt_f16_f32 in the default
// rounding mode; overflow to inf, fp16 subnormals kept).
__device__ __forceinline__ uint16_t f2h(float v) {
    return __builtin_bit_cast(uint16_t, (_Float16)v);
}

// Unsigned byte i of a word as float (v_cvt_f32_ubyte{i}).
template <int I>
__device__ __forceinline__ float ubyte_f(uint32_t w) {
    return (float)((w >> (8 * I)) & 0xFFu);
}

// Exact fp32 weight from a code held as float.  d*c is exact for every fp16
// d and |c| <= 255 (11 + 8 significant bits), so one fused multiply-add
// rounds exactly like the separate multiply and add of the definition.
__device__ __forceinline__ float wval(float d, float c, float off) {
    return __builtin_fmaf(d, c, off);
}

// Byte-addressed 16-bit read from LDS (address must be even).
__device__ __forceinline__ uint32_t lds_u16(const uint8_t *base, int byte_off) {
    return *reinterpret_cast<const uint16_t *>(base + byte_off);
}

// 32-bit word from a 2-byte-aligned LDS address.
__device__ __forceinline__ uint32_t lds_u32_a2(const uint8_t *base, int byte_off) {
    const uint16_t *p = reinterpret_cast<const uint16_t *>(base + byte_off);
    return (uint32_t)p[0] | ((uint32_t)p[1] << 16);
}

// DPP lane-shuffle of a float (rows of 16 lanes; lanes outside row_mask
// read 0).
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 ROW_MASK, 0xF, false));
}

// Sum over the 64 lanes of a wave with DPP, returned to every lane:
// xor 1 and xor 2 within quads, half-row and row mirrors give every lane its
// 16-lane row sum, then two row broadcasts fold rows 0..3 into lane 63.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp<0xB1>(v);         // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);         // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);        // row_half_mirror
    v += dpp<0x140>(v);        // row_mirror
    v += dpp<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
    v += dpp<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

}  // namespace qk
