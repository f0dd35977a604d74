// dequant.hip - standalone dequantize of ggml Q4_0 / Q4_1 / Q8_0 / Q5_0 / Q5_1
// to fp32 / fp16.
//
// Follows the dequantize_block_q4_0 / _q4_1 and dequantize_block_q8_0_f16
// kernels of the "llama_cpp 0.12.1 -> 0.12.2" ggml-cuda.cu diff in what is
// computed (fp32 value d*q + (-8*d), d*q + m, d*q; fp16 = one rounding of it)
// and in the idea of staging the misaligned blocks through shared memory with
// wide coalesced loads (the q8_0 kernel's shared-memory copy).  The layout
// here is gfx950's: a 256-lane workgroup takes chunks of 128 consecutive
// blocks, copies their bytes to LDS with 16-byte loads, and each lane then
// writes 16-byte vectors of output, so every wave store covers 1 KiB of
// contiguous output.
//
// The matrix is a flat run of blocks (rows are back to back with no padding
// and k % 32 == 0), so block b always produces outputs [32b, 32b + 32).
#include <type_traits>

#include "qk_common.h"
#include "qk_internal.h"

namespace qk {

constexpr int kDqThreads = 256;
// quant blocks per chunk (128 measured 2-3 % faster than 256 on a 4096 x
// 4096 Q4_0 -> fp32 dequantize: each workgroup then takes two chunks)
constexpr int kDqBlocks = 128;

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
        if constexpr (FMT == QK_Q5_0 || FMT == QK_Q5_1)
            q |= q5_high4((lds_u32_a2(lds, boff + Format<FMT>::kQhOffset) >> j0) & 0xFu);
        if constexpr (FMT == QK_Q5_0) {
            // (q - 16) * d: the difference is exact, the product rounds once
            v[0] = (ubyte_f<0>(q) - 16.0f) * d;
            v[1] = (ubyte_f<1>(q) - 16.0f) * d;
            v[2] = (ubyte_f<2>(q) - 16.0f) * d;
            v[3] = (ubyte_f<3>(q) - 16.0f) * d;
        } else {
            const float off = (FMT == QK_Q4_0) ? -8.0f * d : h2f(lds_u16(lds, boff + 2));
            v[0] = d * ubyte_f<0>(q) + off;
            v[1] = d * ubyte_f<1>(q) + off;
            v[2] = d * ubyte_f<2>(q) + off;
            v[3] = d * ubyte_f<3>(q) + off;
        }
    }
}

// A workgroup walks chunks of 128 blocks c, c + gridDim.x, ... and requests
// the next chunk's bytes into registers before it writes the current chunk's
// outputs, so the reads of one chunk overlap the writes of the one before.
// Chunks are 2304 / 2560 / 4352 / 2816 / 3072 bytes, multiples of 16, so every 16-byte
// piece of every chunk has the alignment of w.  A16: w 16-byte aligned, one
// 16-byte load per piece.  Otherwise (w 2- or 4-byte aligned) a piece is read
// as the four dwords from the 4-byte boundary at or below it, plus for a
// 2-byte offset the dword holding its last two bytes, and shifted into place
// when it is written to LDS (every dword read holds bytes of the piece).
// Outputs are written with non-temporal 16-byte stores (the output is not
// read again by this kernel; streaming it past the caches measured 14.3 ->
// 12.9 us on a 4096 x 4096 Q4_0 -> fp32 dequantize).
constexpr int kDqWgPerCu = 8;

typedef float f32x4v_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4v_t __attribute__((ext_vector_type(4)));

template <int FMT, bool F16, bool ALIGNED_OUT, bool A16>
__global__ __launch_bounds__(kDqThreads) void dequant_loop_kernel(
    const uint8_t *__restrict__ w, int64_t nblocks, void *__restrict__ out_) {
    using F = Format<FMT>;
    constexpr int kChunkBytes = kDqBlocks * F::kBytes;
    constexpr int kU = (kChunkBytes / 16 + kDqThreads - 1) / kDqThreads;  // 16-byte pieces per thread
    static_assert(kU <= 3, "pieces per thread");
    __shared__ __attribute__((aligned(16))) uint8_t lds[kChunkBytes];
    const int64_t nchunks = (nblocks + kDqBlocks - 1) / kDqBlocks;
    const int tid = threadIdx.x;
    int64_t c = blockIdx.x;
    // (named registers rather than arrays: a loop-carried private array is
    // moved to LDS by the compiler, with a wait after every load)
    typedef uint32_t u32x4a4_t __attribute__((ext_vector_type(4), aligned(4)));
    const uint32_t sh = A16 ? 0u : (uint32_t)(reinterpret_cast<uintptr_t>(w) & 3);  // 0 or 2
    const uint8_t *const wb = w - sh;  // 4-byte aligned
    u32x4a4_t r0, r1, r2;
    uint32_t e0 = 0u, e1 = 0u, e2 = 0u;  // last dword of a 2-byte offset piece
    auto piece = [&](const uint8_t *cb, int i, u32x4a4_t &r, uint32_t &e) __attribute__((always_inline)) {
        if constexpr (A16) {
            r = *reinterpret_cast<const u32x4a4_t *>(reinterpret_cast<const uint4 *>(cb) + i);
        } else {
            r = *reinterpret_cast<const u32x4a4_t *>(cb + 16 * i);
            if (sh) e = *reinterpret_cast<const uint32_t *>(cb + 16 * i + 16);
        }
    };
    auto fetch = [&](int64_t ch) __attribute__((always_inline)) {
        const int nb = (int)min((int64_t)kDqBlocks, nblocks - ch * kDqBlocks);
        const int n16 = (nb * F::kBytes) >> 4;
        const uint8_t *cb = wb + ch * kChunkBytes;
        // every thread loads (a piece past the chunk's end repeats its last one)
        piece(cb, min(tid, n16 - 1), r0, e0);
        if constexpr (kU > 1) piece(cb, min(tid + kDqThreads, n16 - 1), r1, e1);
        if constexpr (kU > 2) piece(cb, min(tid + 2 * kDqThreads, n16 - 1), r2, e2);
    };
    auto placed = [&](const u32x4a4_t &r, uint32_t e) -> uint4 {
        if constexpr (A16) return make_uint4(r.x, r.y, r.z, r.w);
        else return make_uint4(__builtin_amdgcn_alignbyte(r.y, r.x, sh), __builtin_amdgcn_alignbyte(r.z, r.y, sh),
                               __builtin_amdgcn_alignbyte(r.w, r.z, sh), __builtin_amdgcn_alignbyte(e, r.w, sh));
    };
    fetch(c);
    for (;;) {
        const int nb = (int)min((int64_t)kDqBlocks, nblocks - c * kDqBlocks);
        const int bytes = nb * F::kBytes;
        const int n16 = bytes >> 4;
        uint4 *l16 = reinterpret_cast<uint4 *>(lds);
        if (tid < n16) l16[tid] = placed(r0, e0);
        if constexpr (kU > 1) if (tid + kDqThreads < n16) l16[tid + kDqThreads] = placed(r1, e1);
        if constexpr (kU > 2) if (tid + 2 * kDqThreads < n16) l16[tid + 2 * kDqThreads] = placed(r2, e2);
        // a partial last chunk may end with fewer than 16 bytes
        if ((bytes & 15) != 0) {
            const uint16_t *s2 = reinterpret_cast<const uint16_t *>(w + c * kChunkBytes + (n16 << 4));
            uint16_t *d2 = reinterpret_cast<uint16_t *>(lds + (n16 << 4));
            for (int i = tid; i < ((bytes & 15) >> 1); i += kDqThreads) d2[i] = s2[i];
        }
        __syncthreads();
        const int64_t cn = c + gridDim.x;
        if (cn < nchunks) fetch(cn);
        if constexpr (!F16) {
            float *o = static_cast<float *>(out_) + c * kDqBlocks * kBlockElems;
            for (int g = tid; g < nb * 8; g += kDqThreads) {  // 4-element groups
                float v[4];
                decode4<FMT>(lds, (g >> 3) * F::kBytes, (g & 7) * 4, v);
                if (ALIGNED_OUT) {
                    __builtin_nontemporal_store(f32x4v_t{v[0], v[1], v[2], v[3]},
                                                reinterpret_cast<f32x4v_t *>(o + 4 * g));
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) o[4 * g + i] = v[i];
                }
            }
        } else {
            uint16_t *o = static_cast<uint16_t *>(out_) + c * kDqBlocks * kBlockElems;
            for (int g = tid; g < nb * 4; g += kDqThreads) {  // 8-element groups
                float v[8];
                decode4<FMT>(lds, (g >> 2) * F::kBytes, (g & 3) * 8, v);
                decode4<FMT>(lds, (g >> 2) * F::kBytes, (g & 3) * 8 + 4, v + 4);
                uint16_t h[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    // opaque: the compiler otherwise folds a product and its
                    // conversion into v_fma_mix*_f16 with a +0 addend, which
                    // turns a -0 product (Q5_0 with q = 16, d < 0) into +0
                    asm volatile("" : "+v"(v[i]));
                    h[i] = f2h(v[i]);
                }
                if (ALIGNED_OUT) {
                    __builtin_nontemporal_store(
                        u32x4v_t{(uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16),
                                 (uint32_t)h[4] | ((uint32_t)h[5] << 16), (uint32_t)h[6] | ((uint32_t)h[7] << 16)},
                        reinterpret_cast<u32x4v_t *>(o + 8 * g));
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) o[8 * g + i] = h[i];
                }
            }
        }
        if (cn >= nchunks) break;
        __syncthreads();  // every read of this chunk done before the next one is written
        c = cn;
    }
}

template <int FMT>
static int dispatch_dequant(const uint8_t *w, int64_t nblocks, int out_dtype, void *out,
                            hipStream_t stream) {
    const dim3 block(kDqThreads);
    const bool a16 = ((uintptr_t)w % 16) == 0;
    const bool aout = ((uintptr_t)out % 16) == 0;
    const bool f32 = out_dtype == QK_F32;
    const int64_t nchunks = (nblocks + kDqBlocks - 1) / kDqBlocks;
    const int64_t cap = (int64_t)device_cus() * kDqWgPerCu;
    const dim3 grid((unsigned)(nchunks < cap ? nchunks : cap));
    auto run = [&](auto f16, auto ao, auto in16) {
        return launch(dequant_loop_kernel<FMT, decltype(f16)::value, decltype(ao)::value, decltype(in16)::value>,
                      grid, block, stream, w, nblocks, out);
    };
    using T = std::true_type;
    using Fl = std::false_type;
    if (f32) {
        if (a16) return aout ? run(Fl{}, T{}, T{}) : run(Fl{}, Fl{}, T{});
        return aout ? run(Fl{}, T{}, Fl{}) : run(Fl{}, Fl{}, Fl{});
    }
    if (a16) return aout ? run(T{}, T{}, T{}) : run(T{}, Fl{}, T{});
    return aout ? run(T{}, T{}, Fl{}) : run(T{}, Fl{}, Fl{});
}

int launch_dequantize(int fmt, const void *w, int64_t nblocks, int out_dtype, void *out,
                      hipStream_t stream) {
    const uint8_t *wb = static_cast<const uint8_t *>(w);
    switch (fmt) {
    case QK_Q4_0: return dispatch_dequant<QK_Q4_0>(wb, nblocks, out_dtype, out, stream);
    case QK_Q4_1: return dispatch_dequant<QK_Q4_1>(wb, nblocks, out_dtype, out, stream);
    case QK_Q8_0: return dispatch_dequant<QK_Q8_0>(wb, nblocks, out_dtype, out, stream);
    case QK_Q5_0: return dispatch_dequant<QK_Q5_0>(wb, nblocks, out_dtype, out, stream);
    case QK_Q5_1: return dispatch_dequant<QK_Q5_1>(wb, nblocks, out_dtype, out, stream);
    default: return QK_ERR_UNSUPPORTED;
    }
}

}  // namespace qk
