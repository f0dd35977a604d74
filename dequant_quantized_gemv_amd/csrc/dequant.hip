// dequant.hip - standalone dequantize of ggml Q4_0 / Q4_1 / Q8_0 to fp32 / fp16.
//
// Follows the dequantize_block_q4_0 / _q4_1 and dequantize_block_q8_0_f16
// kernels of the "llama_cpp 0.12.1 -> 0.12.2" ggml-cuda.cu diff in what is
// computed (fp32 value d*q + (-8*d), d*q + m, d*q; fp16 = one rounding of it)
// and in the idea of staging the misaligned blocks through shared memory with
// wide coalesced loads (the q8_0 kernel's shared-memory copy).  The layout
// here is gfx950's: a 256-lane workgroup owns 256 consecutive blocks, copies
// their bytes to LDS with 16-byte loads, and each lane then writes 16-byte
// vectors of output, so every wave store covers 1 KiB of contiguous output.
//
// The matrix is a flat run of blocks (rows are back to back with no padding
// and k % 32 == 0), so block b always produces outputs [32b, 32b + 32).
#include "qk_common.h"
#include "qk_internal.h"

namespace qk {

constexpr int kDqThreads = 256;
constexpr int kDqBlocks = 256;  // quant blocks per workgroup

// Copy `bytes` (even) from global memory to LDS.  ALIGNED16: src and dst are
// 16-byte aligned, so whole 16-byte pieces move with one load each and only a
// tail of fewer than 16 bytes falls back to 2-byte loads.
template <bool ALIGNED16>
__device__ __forceinline__ void stage_to_lds(uint8_t *dst, const uint8_t *__restrict__ src,
                                             int bytes) {
    int done = 0;
    if (ALIGNED16) {
        const int n16 = bytes >> 4;
        const uint4 *s = reinterpret_cast<const uint4 *>(src);
        uint4 *d = reinterpret_cast<uint4 *>(dst);
        for (int i = threadIdx.x; i < n16; i += kDqThreads) d[i] = s[i];
        done = n16 << 4;
    }
    const int n2 = (bytes - done) >> 1;
    const uint16_t *s2 = reinterpret_cast<const uint16_t *>(src + done);
    uint16_t *d2 = reinterpret_cast<uint16_t *>(dst + done);
    for (int i = threadIdx.x; i < n2; i += kDqThreads) d2[i] = s2[i];
}

// Four consecutive elements j0..j0+3 (j0 % 4 == 0) of the block at LDS offset
// boff, as fp32 in the definition's operation order.
template <int FMT>
__device__ __forceinline__ void decode4(const uint8_t *lds, int boff, int j0, float v[4]) {
    using F = Format<FMT>;
    const float d = h2f(lds_u16(lds, boff));
    if constexpr (FMT == QK_Q8_0) {
        const uint32_t q = lds_u32_a2(lds, boff + F::kQsOffset + j0);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = d * (float)(int8_t)(q >> (8 * i));
    } else {
        uint32_t q = lds_u32_a2(lds, boff + F::kQsOffset + (j0 & 15));
        if (j0 >= 16) q >>= 4;
        q &= 0x0F0F0F0Fu;
        const float off = (FMT == QK_Q4_0) ? -8.0f * d : h2f(lds_u16(lds, boff + 2));
        v[0] = d * ubyte_f<0>(q) + off;
        v[1] = d * ubyte_f<1>(q) + off;
        v[2] = d * ubyte_f<2>(q) + off;
        v[3] = d * ubyte_f<3>(q) + off;
    }
}

template <int FMT, bool ALIGNED_IN, bool ALIGNED_OUT>
__global__ __launch_bounds__(kDqThreads) void dequant_f32_kernel(
    const uint8_t *__restrict__ w, int64_t nblocks, float *__restrict__ out) {
    using F = Format<FMT>;
    __shared__ __attribute__((aligned(16))) uint8_t lds[kDqBlocks * F::kBytes];
    const int64_t blk0 = (int64_t)blockIdx.x * kDqBlocks;
    const int nb = (int)min((int64_t)kDqBlocks, nblocks - blk0);
    stage_to_lds<ALIGNED_IN>(lds, w + blk0 * F::kBytes, nb * F::kBytes);
    __syncthreads();
    float *o = out + blk0 * kBlockElems;
    const int ngroups = nb * 8;  // 4-element groups
    for (int g = threadIdx.x; g < ngroups; g += kDqThreads) {
        float v[4];
        decode4<FMT>(lds, (g >> 3) * F::kBytes, (g & 7) * 4, v);
        if (ALIGNED_OUT) {
            *reinterpret_cast<float4 *>(o + 4 * g) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) o[4 * g + i] = v[i];
        }
    }
}

template <int FMT, bool ALIGNED_IN, bool ALIGNED_OUT>
__global__ __launch_bounds__(kDqThreads) void dequant_f16_kernel(
    const uint8_t *__restrict__ w, int64_t nblocks, uint16_t *__restrict__ out) {
    using F = Format<FMT>;
    __shared__ __attribute__((aligned(16))) uint8_t lds[kDqBlocks * F::kBytes];
    const int64_t blk0 = (int64_t)blockIdx.x * kDqBlocks;
    const int nb = (int)min((int64_t)kDqBlocks, nblocks - blk0);
    stage_to_lds<ALIGNED_IN>(lds, w + blk0 * F::kBytes, nb * F::kBytes);
    __syncthreads();
    uint16_t *o = out + blk0 * kBlockElems;
    const int ngroups = nb * 4;  // 8-element groups
    for (int g = threadIdx.x; g < ngroups; g += kDqThreads) {
        const int boff = (g >> 2) * F::kBytes;
        const int j0 = (g & 3) * 8;
        float v[8];
        decode4<FMT>(lds, boff, j0, v);
        decode4<FMT>(lds, boff, j0 + 4, v + 4);
        uint16_t h[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) h[i] = f2h(v[i]);
        if (ALIGNED_OUT) {
            uint4 p;
            p.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
            p.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
            p.z = (uint32_t)h[4] | ((uint32_t)h[5] << 16);
            p.w = (uint32_t)h[6] | ((uint32_t)h[7] << 16);
            *reinterpret_cast<uint4 *>(o + 8 * g) = p;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) o[8 * g + i] = h[i];
        }
    }
}

template <int FMT>
static int dispatch_dequant(const uint8_t *w, int64_t nblocks, int out_dtype, void *out,
                            hipStream_t stream) {
    const dim3 grid((unsigned)((nblocks + kDqBlocks - 1) / kDqBlocks));
    const dim3 block(kDqThreads);
    const bool ain = ((uintptr_t)w % 16) == 0;
    const bool aout = ((uintptr_t)out % 16) == 0;
    if (out_dtype == QK_F32) {
        float *o = static_cast<float *>(out);
        if (ain && aout) return launch(dequant_f32_kernel<FMT, true, true>, grid, block, stream, w, nblocks, o);
        if (ain) return launch(dequant_f32_kernel<FMT, true, false>, grid, block, stream, w, nblocks, o);
        if (aout) return launch(dequant_f32_kernel<FMT, false, true>, grid, block, stream, w, nblocks, o);
        return launch(dequant_f32_kernel<FMT, false, false>, grid, block, stream, w, nblocks, o);
    }
    uint16_t *o = static_cast<uint16_t *>(out);
    if (ain && aout) return launch(dequant_f16_kernel<FMT, true, true>, grid, block, stream, w, nblocks, o);
    if (ain) return launch(dequant_f16_kernel<FMT, true, false>, grid, block, stream, w, nblocks, o);
    if (aout) return launch(dequant_f16_kernel<FMT, false, true>, grid, block, stream, w, nblocks, o);
    return launch(dequant_f16_kernel<FMT, false, false>, grid, block, stream, w, nblocks, o);
}

int launch_dequantize(int fmt, const void *w, int64_t nblocks, int out_dtype, void *out,
                      hipStream_t stream) {
    const uint8_t *wb = static_cast<const uint8_t *>(w);
    switch (fmt) {
    case QK_Q4_0: return dispatch_dequant<QK_Q4_0>(wb, nblocks, out_dtype, out, stream);
    case QK_Q4_1: return dispatch_dequant<QK_Q4_1>(wb, nblocks, out_dtype, out, stream);
    case QK_Q8_0: return dispatch_dequant<QK_Q8_0>(wb, nblocks, out_dtype, out, stream);
    default: return QK_ERR_UNSUPPORTED;
    }
}

}  // namespace qk
