// gemm.hip - batched quantized GEMM: Y = f16(W) X on the gfx950 matrix cores.
//
// The reference path for more than one activation column dequantizes the
// weights to fp16 (ggml_get_to_fp16_cuda) and hands them to a BLAS GEMM;
// ggml_cuda_mul_mat picks it by the column count ("llama_cpp 0.12.1 -> 0.12.2"
// ggml-cuda.cu diff).  Here the two steps are fused: each 128 x 128 output tile
// dequantizes its weight rows straight into LDS as fp16 and feeds them, with
// the fp16 activation tile, to v_mfma_f32_16x16x32_f16, accumulating in fp32.
// The fp16 weight is one round-to-nearest-even of the exact weight value, i.e.
// the value qk_dequantize(..., QK_F16, ...) produces (a Q4_0 code 8 with
// negative d gives -0 here, +0 there: the same number).
//
// Workgroup: 256 lanes = 4 waves in a 2 x 2 grid, each wave a 64 x 64 sub-tile
// (4 x 4 MFMA tiles of 16 x 16).  K advances 64 (two quant blocks, one "pair")
// per step.  Lane t stages row t/2 of the weight tile: it loads the row's pair
// (36 / 40 / 68 bytes, dword aligned when the block count is even) and
// dequantizes block t%2 of it; it also loads 64 bytes of activations (column
// t/2, k-half t%2).  The next step's loads are issued into registers before the
// matrix cores work on the current step.
//
// Dequantization to fp16 (Q4_0, Q8_0), packed two at a time and exact: the
// integer code is placed in the mantissa of an fp16 (0x64XX is 1024 + XX) with
// a byte permute, the bias removed with one packed add (q - 8, or q, exactly),
// and one packed multiply by (d, d) rounds d * (q - 8) or d * q to fp16 once.
// Q4_1 (d*q + m is one fp32 rounding) goes through fp32 so that the fp16 is
// rounded from exactly the fp32 dequantized value.
//
// Tiles are assigned so that the workgroups of one XCD (the hardware sends
// workgroup i to XCD i % 8) cover consecutive tiles, column tile fastest, so
// the workgroups sharing a weight row tile share that XCD's L2.
#include "qk_common.h"
#include "qk_internal.h"

namespace qk {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2g_t __attribute__((ext_vector_type(2)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4g_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4g_a4 __attribute__((ext_vector_type(4), aligned(4)));

constexpr int kGmThreads = 256;
constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kBK = 64;
constexpr int kPitch = kBK + 8;  // halves per LDS row (144 bytes: spreads rows over banks)

template <int FMT> struct GmPair;
template <> struct GmPair<QK_Q4_0> { static constexpr int kDwords = 9; };
template <> struct GmPair<QK_Q4_1> { static constexpr int kDwords = 10; };
template <> struct GmPair<QK_Q8_0> { static constexpr int kDwords = 17; };

__device__ __forceinline__ uint32_t gm_perm_lo(uint32_t src) {
    return __builtin_amdgcn_perm(0x64646464u, src, 0x04010400u);  // [b0, 64, b1, 64]
}
__device__ __forceinline__ uint32_t gm_perm_hi(uint32_t src) {
    return __builtin_amdgcn_perm(0x64646464u, src, 0x04030402u);  // [b2, 64, b3, 64]
}
__device__ __forceinline__ uint32_t gm_pk_add(uint32_t a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2g_t, a) + half2g_t{(_Float16)b, (_Float16)b});
}
__device__ __forceinline__ uint32_t gm_pk_fma(uint32_t a, float s, float t) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(half2g_t, a),
                                                                  half2g_t{(_Float16)s, (_Float16)s},
                                                                  half2g_t{(_Float16)t, (_Float16)t}));
}
__device__ __forceinline__ uint32_t gm_pk_mul(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2g_t, a) * __builtin_bit_cast(half2g_t, b));
}
__device__ __forceinline__ uint32_t gm_pack2(float a, float b) {
    return (uint32_t)f2h(a) | ((uint32_t)f2h(b) << 16);
}

// Block b (0/1) of a pair held in registers: d bits, m bits, quant word i.
template <int FMT>
__device__ __forceinline__ uint32_t gm_d(const uint32_t (&v)[GmPair<FMT>::kDwords], int b) {
    if constexpr (FMT == QK_Q4_0) return b == 0 ? (v[0] & 0xFFFFu) : (v[4] >> 16);
    if constexpr (FMT == QK_Q4_1) return b == 0 ? (v[0] & 0xFFFFu) : (v[5] & 0xFFFFu);
    return b == 0 ? (v[0] & 0xFFFFu) : (v[8] >> 16);
}
template <int FMT>
__device__ __forceinline__ uint32_t gm_qs(const uint32_t (&v)[GmPair<FMT>::kDwords], int b, int i) {
    if constexpr (FMT == QK_Q4_0) return b == 0 ? __builtin_amdgcn_alignbyte(v[i + 1], v[i], 2) : v[5 + i];
    if constexpr (FMT == QK_Q4_1) return b == 0 ? v[1 + i] : v[6 + i];
    return b == 0 ? __builtin_amdgcn_alignbyte(v[i + 1], v[i], 2) : v[9 + i];
}

// Dequantize block b of the pair to 32 fp16 (out[g] = elements 8g..8g+7).
template <int FMT>
__device__ __forceinline__ void gm_dequant(const uint32_t (&v)[GmPair<FMT>::kDwords], int b, u32x4g_t (&out)[4]) {
    const uint32_t db = gm_d<FMT>(v, b);
    if constexpr (FMT == QK_Q4_1) {
        const float d = h2f(db);
        const float mm = h2f(b == 0 ? (v[0] >> 16) : (v[5] >> 16));
        // word i: low nibbles -> elements 4i..4i+3, high -> 16+4i..16+4i+3
        uint32_t lo[4][2], hi[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t q = gm_qs<FMT>(v, b, i);
            const uint32_t l = q & 0x0F0F0F0Fu, h = (q >> 4) & 0x0F0F0F0Fu;
            lo[i][0] = gm_pack2(d * ubyte_f<0>(l) + mm, d * ubyte_f<1>(l) + mm);
            lo[i][1] = gm_pack2(d * ubyte_f<2>(l) + mm, d * ubyte_f<3>(l) + mm);
            hi[i][0] = gm_pack2(d * ubyte_f<0>(h) + mm, d * ubyte_f<1>(h) + mm);
            hi[i][1] = gm_pack2(d * ubyte_f<2>(h) + mm, d * ubyte_f<3>(h) + mm);
        }
        out[0] = u32x4g_t{lo[0][0], lo[0][1], lo[1][0], lo[1][1]};
        out[1] = u32x4g_t{lo[2][0], lo[2][1], lo[3][0], lo[3][1]};
        out[2] = u32x4g_t{hi[0][0], hi[0][1], hi[1][0], hi[1][1]};
        out[3] = u32x4g_t{hi[2][0], hi[2][1], hi[3][0], hi[3][1]};
    } else if constexpr (FMT == QK_Q4_0) {
        const uint32_t dd = db | (db << 16);
        uint32_t lo[4][2], hi[4][2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t q = gm_qs<FMT>(v, b, i);
            const uint32_t l = q & 0x0F0F0F0Fu, h = q & 0xF0F0F0F0u;
            // 1024 + c - 1032 = c - 8; (1024 + 16c) / 16 - 72 = c - 8; then * d
            lo[i][0] = gm_pk_mul(gm_pk_add(gm_perm_lo(l), -1032.0f), dd);
            lo[i][1] = gm_pk_mul(gm_pk_add(gm_perm_hi(l), -1032.0f), dd);
            hi[i][0] = gm_pk_mul(gm_pk_fma(gm_perm_lo(h), 0.0625f, -72.0f), dd);
            hi[i][1] = gm_pk_mul(gm_pk_fma(gm_perm_hi(h), 0.0625f, -72.0f), dd);
        }
        out[0] = u32x4g_t{lo[0][0], lo[0][1], lo[1][0], lo[1][1]};
        out[1] = u32x4g_t{lo[2][0], lo[2][1], lo[3][0], lo[3][1]};
        out[2] = u32x4g_t{hi[0][0], hi[0][1], hi[1][0], hi[1][1]};
        out[3] = u32x4g_t{hi[2][0], hi[2][1], hi[3][0], hi[3][1]};
    } else {
        const uint32_t dd = db | (db << 16);
        uint32_t p[8][2];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            // c + 128 is the byte of (c ^ 0x80): 1024 + c + 128 - 1152 = c; then * d
            const uint32_t u = gm_qs<FMT>(v, b, i) ^ 0x80808080u;
            p[i][0] = gm_pk_mul(gm_pk_add(gm_perm_lo(u), -1152.0f), dd);
            p[i][1] = gm_pk_mul(gm_pk_add(gm_perm_hi(u), -1152.0f), dd);
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) out[g] = u32x4g_t{p[2 * g][0], p[2 * g][1], p[2 * g + 1][0], p[2 * g + 1][1]};
    }
}

// FAST: w 4-byte aligned and an even number of blocks per row (so every pair
// starts on 4 bytes and both of its blocks exist), x 16-byte aligned and
// ldx % 8 == 0.  YALIGNED: y 16-byte aligned and ldy % 4 == 0.
template <int FMT, bool FAST, bool YALIGNED>
__global__ __launch_bounds__(kGmThreads) void gemm_kernel(
    const uint8_t *__restrict__ w, int m, int nb, const uint16_t *__restrict__ x, int64_t ldx,
    int n, float *__restrict__ y, int64_t ldy, int mtiles, int ntiles) {
    using F = Format<FMT>;
    constexpr int ND = GmPair<FMT>::kDwords;
    __shared__ __attribute__((aligned(16))) uint16_t As[kBM * kPitch];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[kBN * kPitch];

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
    const int wr = wave >> 1;
    const int wc = wave & 1;
    const int k = nb * 32;

    // loader roles
    const int lr = tid >> 1;   // weight row / activation column within the tile
    const int lh = tid & 1;    // block of the pair / k-half of the step
    const int64_t row_bytes = (int64_t)nb * F::kBytes;
    // Rows and columns past the matrix load a clamped, valid row or column.
    // Output (i, j) depends only on weight row i and activation column j, and
    // such rows and columns are never stored, so their values do not matter.
    const uint8_t *__restrict__ wrow = w + (int64_t)min(row0 + lr, m - 1) * row_bytes;
    const uint16_t *__restrict__ xcol = x + (int64_t)min(col0 + lr, n - 1) * ldx;

    uint32_t wv[ND];
    u32x4g_t xv[4];

    auto load_step = [&](int it) {
        const uint8_t *p = wrow + (int64_t)it * (2 * F::kBytes);
        if (FAST) {
#pragma unroll
            for (int i = 0; i + 4 <= ND; i += 4) {
                const u32x4g_a4 t = *reinterpret_cast<const u32x4g_a4 *>(p + 4 * i);
                wv[i] = t.x; wv[i + 1] = t.y; wv[i + 2] = t.z; wv[i + 3] = t.w;
            }
#pragma unroll
            for (int i = ND & ~3; i < ND; ++i) wv[i] = *reinterpret_cast<const uint32_t *>(p + 4 * i);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                xv[i] = *reinterpret_cast<const u32x4g_t *>(xcol + it * kBK + 32 * lh + 8 * i);
        } else {
            // 2-byte loads; a missing second block (odd block count) reads as
            // zeros (d = m = 0, weights 0), activations past K as 0
            const bool second = 2 * it + 1 < nb;
            const uint16_t *h = reinterpret_cast<const uint16_t *>(p);
#pragma unroll
            for (int i = 0; i < ND; ++i) {
                const uint32_t a = (4 * i < F::kBytes || second) ? (uint32_t)h[2 * i] : 0u;
                const uint32_t b = (4 * i + 2 < F::kBytes || second) ? (uint32_t)h[2 * i + 1] : 0u;
                wv[i] = a | (b << 16);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int kk = it * kBK + 32 * lh + 8 * i;
                uint32_t e[4] = {0u, 0u, 0u, 0u};
                if (kk < k) {
                    const uint16_t *q = xcol + kk;
#pragma unroll
                    for (int u = 0; u < 4; ++u) e[u] = (uint32_t)q[2 * u] | ((uint32_t)q[2 * u + 1] << 16);
                }
                xv[i] = u32x4g_t{e[0], e[1], e[2], e[3]};
            }
        }
    };

    floatx4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

    const int nsteps = (nb + 1) / 2;
    if (nsteps > 0) load_step(0);
    for (int it = 0; it < nsteps; ++it) {
        // stage: dequantized weights and activations of this step into LDS
        u32x4g_t a4[4];
        // (a block missing from the last pair of an odd row was loaded as
        // zeros: its weights are 0 and the activations past K are 0 too)
        gm_dequant<FMT>(wv, lh, a4);
        u32x4g_t *adst = reinterpret_cast<u32x4g_t *>(As + lr * kPitch + 32 * lh);
        u32x4g_t *bdst = reinterpret_cast<u32x4g_t *>(Bs + lr * kPitch + 32 * lh);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            adst[g] = a4[g];
            bdst[g] = xv[g];
        }
        __syncthreads();
        if (it + 1 < nsteps) load_step(it + 1);

#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            half8_t af[4], bf[4];
            const int kofs = ks * 32 + (lane >> 4) * 8;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                af[i] = *reinterpret_cast<const half8_t *>(As + (wr * 64 + i * 16 + (lane & 15)) * kPitch + kofs);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bf[j] = *reinterpret_cast<const half8_t *>(Bs + (wc * 64 + j * 16 + (lane & 15)) * kPitch + kofs);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }

    // Epilogue: acc[i][j][e] is row wr*64 + 16i + 4*(lane/16) + e, column
    // wc*64 + 16j + lane%16 of the tile.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int col = col0 + wc * 64 + j * 16 + (lane & 15);
        if (col >= n) continue;
        float *ycol = y + (int64_t)col * ldy;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = row0 + wr * 64 + i * 16 + 4 * (lane >> 4);
            if (YALIGNED && row + 3 < m) {
                *reinterpret_cast<float4 *>(ycol + row) =
                    make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (row + e < m) ycol[row + e] = acc[i][j][e];
            }
        }
    }
}

template <int FMT>
static int dispatch_gemm(const uint8_t *w, int m, int nb, const uint16_t *x, int64_t ldx, int n,
                         float *y, int64_t ldy, hipStream_t stream) {
    const int mtiles = (m + kBM - 1) / kBM;
    const int ntiles = (n + kBN - 1) / kBN;
    const dim3 grid((unsigned)(mtiles * ntiles));
    const dim3 block(kGmThreads);
    const bool fast = ((uintptr_t)w % 4) == 0 && (nb % 2) == 0 && ((uintptr_t)x % 16) == 0 &&
                      (ldx % 8) == 0;
    const bool ya = ((uintptr_t)y % 16) == 0 && (ldy % 4) == 0;
    if (fast && ya)
        return launch(gemm_kernel<FMT, true, true>, grid, block, stream, w, m, nb, x, ldx, n, y, ldy, mtiles, ntiles);
    if (fast)
        return launch(gemm_kernel<FMT, true, false>, grid, block, stream, w, m, nb, x, ldx, n, y, ldy, mtiles, ntiles);
    if (ya)
        return launch(gemm_kernel<FMT, false, true>, grid, block, stream, w, m, nb, x, ldx, n, y, ldy, mtiles, ntiles);
    return launch(gemm_kernel<FMT, false, false>, grid, block, stream, w, m, nb, x, ldx, n, y, ldy, mtiles, ntiles);
}

int launch_mul_mat(int fmt, const void *w, int64_t m, int64_t k, const uint16_t *x, int64_t n,
                   int64_t ldx, float *y, int64_t ldy, hipStream_t stream) {
    const uint8_t *wb = static_cast<const uint8_t *>(w);
    const int nb = (int)(k / kBlockElems);
    switch (fmt) {
    case QK_Q4_0: return dispatch_gemm<QK_Q4_0>(wb, (int)m, nb, x, ldx, (int)n, y, ldy, stream);
    case QK_Q4_1: return dispatch_gemm<QK_Q4_1>(wb, (int)m, nb, x, ldx, (int)n, y, ldy, stream);
    case QK_Q8_0: return dispatch_gemm<QK_Q8_0>(wb, (int)m, nb, x, ldx, (int)n, y, ldy, stream);
    default: return QK_ERR_UNSUPPORTED;
    }
}

}  // namespace qk
