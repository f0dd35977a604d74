// gemm.hip - batched quantized GEMM: Y = f16(W) X on the gfx950 matrix cores.
//
// The reference path for more than one activation column dequantizes the
// weights to fp16 (ggml_get_to_fp16_cuda) and hands them to a BLAS GEMM;
// ggml_cuda_mul_mat picks it by the column count ("llama_cpp 0.12.1 -> 0.12.2"
// ggml-cuda.cu diff).  Here the two steps are fused: each 128 x 128 output tile
// dequantizes its weight rows straight into LDS as fp16 and feeds them, with
// the fp16 activation tile, to v_mfma_f32_16x16x32_f16, accumulating in fp32.
// The fp16 weight is one round-to-nearest-even of the exact fp32 value, i.e.
// the same bits qk_dequantize(..., QK_F16, ...) produces.
//
// Workgroup: 256 lanes = 4 waves in a 2 x 2 grid, each wave a 64 x 64 sub-tile
// (4 x 4 MFMA tiles of 16 x 16).  K advances 64 (two quant blocks) per step:
//   lane t loads one quant block (row t/2, block t%2 of the step) and 64 bytes
//   of activations (column t/2, k-half t%2) into registers for the next step
//   while the matrix cores work on the current one.
// Tiles are assigned so that the workgroups of one XCD (the hardware sends
// workgroup i to XCD i % 8) cover consecutive tiles, column tile fastest, so
// the workgroups sharing a weight row tile share that XCD's L2.
#include "qk_common.h"
#include "qk_internal.h"

namespace qk {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kGmThreads = 256;
constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kBK = 64;
constexpr int kPitch = kBK + 8;  // halves per LDS row (144 bytes: spreads rows over banks)

template <int FMT>
struct BlockRegs {
    uint32_t d;                            // fp16 d bits
    uint32_t mb;                           // fp16 m bits (Q4_1)
    uint32_t qs[Format<FMT>::kQsBytes / 4];
};

template <int FMT>
__device__ __forceinline__ void load_block(const uint8_t *__restrict__ p, BlockRegs<FMT> &b) {
    using F = Format<FMT>;
    const uint16_t *h = reinterpret_cast<const uint16_t *>(p);
    b.d = h[0];
    b.mb = (FMT == QK_Q4_1) ? h[1] : 0u;
    const uint16_t *qs = reinterpret_cast<const uint16_t *>(p + F::kQsOffset);
#pragma unroll
    for (int i = 0; i < F::kQsBytes / 4; ++i)
        b.qs[i] = (uint32_t)qs[2 * i] | ((uint32_t)qs[2 * i + 1] << 16);
}

__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return (uint32_t)f2h(a) | ((uint32_t)f2h(b) << 16);
}

// Dequantize one block (32 weights) to fp16 and store it as 4 x 16 bytes.
template <int FMT>
__device__ __forceinline__ void store_block_f16(uint16_t *dst, const BlockRegs<FMT> &b) {
    const float d = h2f(b.d);
    uint4 out[4];
    if constexpr (FMT == QK_Q8_0) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const uint32_t q0 = b.qs[2 * g], q1 = b.qs[2 * g + 1];
            out[g].x = pack2(d * (float)(int8_t)q0, d * (float)(int8_t)(q0 >> 8));
            out[g].y = pack2(d * (float)(int8_t)(q0 >> 16), d * (float)(int8_t)(q0 >> 24));
            out[g].z = pack2(d * (float)(int8_t)q1, d * (float)(int8_t)(q1 >> 8));
            out[g].w = pack2(d * (float)(int8_t)(q1 >> 16), d * (float)(int8_t)(q1 >> 24));
        }
    } else {
        const float off = (FMT == QK_Q4_0) ? -8.0f * d : h2f(b.mb);
        // group g: elements 8g..8g+7; g < 2 low nibbles of bytes 8g.., g >= 2 high
        // nibbles of bytes 8(g-2)..
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            uint32_t q0 = b.qs[2 * (g & 1)], q1 = b.qs[2 * (g & 1) + 1];
            if (g >= 2) {
                q0 >>= 4;
                q1 >>= 4;
            }
            q0 &= 0x0F0F0F0Fu;
            q1 &= 0x0F0F0F0Fu;
            out[g].x = pack2(d * ubyte_f<0>(q0) + off, d * ubyte_f<1>(q0) + off);
            out[g].y = pack2(d * ubyte_f<2>(q0) + off, d * ubyte_f<3>(q0) + off);
            out[g].z = pack2(d * ubyte_f<0>(q1) + off, d * ubyte_f<1>(q1) + off);
            out[g].w = pack2(d * ubyte_f<2>(q1) + off, d * ubyte_f<3>(q1) + off);
        }
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) reinterpret_cast<uint4 *>(dst)[g] = out[g];
}

// XALIGNED: x 16-byte aligned and ldx % 8 == 0.  YALIGNED: y 16-byte aligned
// and ldy % 4 == 0.
template <int FMT, bool XALIGNED, bool YALIGNED>
__global__ __launch_bounds__(kGmThreads) void gemm_kernel(
    const uint8_t *__restrict__ w, int m, int nbk, const uint16_t *__restrict__ x, int64_t ldx,
    int n, float *__restrict__ y, int64_t ldy, int mtiles, int ntiles) {
    using F = Format<FMT>;
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
    const int k = nbk * 32;

    // loader roles
    const int lr = tid >> 1;   // weight row / activation column within the tile
    const int lh = tid & 1;    // block within the step / k-half within the step
    const int64_t row_bytes = (int64_t)nbk * F::kBytes;
    const bool wrow_ok = row0 + lr < m;
    const uint8_t *__restrict__ wrow = w + (int64_t)(row0 + lr) * row_bytes;
    const bool xcol_ok = col0 + lr < n;
    const uint16_t *__restrict__ xcol = x + (int64_t)(col0 + lr) * ldx;

    BlockRegs<FMT> wreg;
    uint4 xreg[4];
    bool wvalid = false;

    auto load_step = [&](int it) {
        const int kb = 2 * it + lh;
        wvalid = wrow_ok && kb < nbk;
        if (wvalid) load_block<FMT>(wrow + (int64_t)kb * F::kBytes, wreg);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int kk = it * kBK + 32 * lh + 8 * i;
            if (xcol_ok && kk < k) {
                if (XALIGNED) {
                    xreg[i] = *reinterpret_cast<const uint4 *>(xcol + kk);
                } else {
                    const uint16_t *p = xcol + kk;
                    xreg[i].x = (uint32_t)p[0] | ((uint32_t)p[1] << 16);
                    xreg[i].y = (uint32_t)p[2] | ((uint32_t)p[3] << 16);
                    xreg[i].z = (uint32_t)p[4] | ((uint32_t)p[5] << 16);
                    xreg[i].w = (uint32_t)p[6] | ((uint32_t)p[7] << 16);
                }
            } else {
                xreg[i] = make_uint4(0u, 0u, 0u, 0u);
            }
        }
    };

    floatx4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

    const int nsteps = (nbk + 1) / 2;
    if (nsteps > 0) load_step(0);
    for (int it = 0; it < nsteps; ++it) {
        uint16_t *adst = As + lr * kPitch + 32 * lh;
        if (wvalid) {
            store_block_f16<FMT>(adst, wreg);
        } else {
#pragma unroll
            for (int g = 0; g < 4; ++g) reinterpret_cast<uint4 *>(adst)[g] = make_uint4(0u, 0u, 0u, 0u);
        }
        uint16_t *bdst = Bs + lr * kPitch + 32 * lh;
#pragma unroll
        for (int i = 0; i < 4; ++i) reinterpret_cast<uint4 *>(bdst)[i] = xreg[i];
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
static int dispatch_gemm(const uint8_t *w, int m, int nbk, const uint16_t *x, int64_t ldx, int n,
                         float *y, int64_t ldy, hipStream_t stream) {
    const int mtiles = (m + kBM - 1) / kBM;
    const int ntiles = (n + kBN - 1) / kBN;
    const dim3 grid((unsigned)(mtiles * ntiles));
    const dim3 block(kGmThreads);
    const bool xa = ((uintptr_t)x % 16) == 0 && (ldx % 8) == 0;
    const bool ya = ((uintptr_t)y % 16) == 0 && (ldy % 4) == 0;
    if (xa && ya)
        return launch(gemm_kernel<FMT, true, true>, grid, block, stream, w, m, nbk, x, ldx, n, y, ldy, mtiles, ntiles);
    if (xa)
        return launch(gemm_kernel<FMT, true, false>, grid, block, stream, w, m, nbk, x, ldx, n, y, ldy, mtiles, ntiles);
    if (ya)
        return launch(gemm_kernel<FMT, false, true>, grid, block, stream, w, m, nbk, x, ldx, n, y, ldy, mtiles, ntiles);
    return launch(gemm_kernel<FMT, false, false>, grid, block, stream, w, m, nbk, x, ldx, n, y, ldy, mtiles, ntiles);
}

int launch_mul_mat(int fmt, const void *w, int64_t m, int64_t k, const uint16_t *x, int64_t n,
                   int64_t ldx, float *y, int64_t ldy, hipStream_t stream) {
    const uint8_t *wb = static_cast<const uint8_t *>(w);
    const int nbk = (int)(k / kBlockElems);
    switch (fmt) {
    case QK_Q4_0: return dispatch_gemm<QK_Q4_0>(wb, (int)m, nbk, x, ldx, (int)n, y, ldy, stream);
    case QK_Q4_1: return dispatch_gemm<QK_Q4_1>(wb, (int)m, nbk, x, ldx, (int)n, y, ldy, stream);
    case QK_Q8_0: return dispatch_gemm<QK_Q8_0>(wb, (int)m, nbk, x, ldx, (int)n, y, ldy, stream);
    default: return QK_ERR_UNSUPPORTED;
    }
}

}  // namespace qk
