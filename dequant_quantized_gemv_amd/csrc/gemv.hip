// gemv.hip - fused quantized GEMV for decode: y = W x for 1..8 fp32 columns.
//
// What is computed follows dequantize_mul_mat_vec ("dmmv", named in the
// "llama_cpp 0.12.1 -> 0.12.2" ggml-cuda.cu diff with its tuning block) and the
// ggml_cuda_op_mul_mat driver (a row range times a column count): each output
// is the dot product of one dequantized weight row with one activation column,
// reduced across lanes (the diff's warp_reduce_sum).  The kernel body is not on
// that page; this one is designed for gfx950:
//
//  * A 256-lane workgroup owns RT consecutive rows.  The K dimension is walked
//    in chunks of 64 blocks.  The chunk's bytes for all RT rows are copied to
//    LDS with 16-byte coalesced loads (rows are contiguous, so the copy is a
//    few long runs), the next chunk's loads are issued into registers before
//    the current chunk is computed.
//  * Compute: wave w takes blocks 16w..16w+15 of the chunk; lane = 4*slot + q
//    takes quarter q of block `slot`: 8 weights (Q4: quant bytes 4q..4q+3,
//    low nibbles -> elements 4q+i, high nibbles -> 16+4q+i; Q8: bytes 8q..8q+7).
//    Its 8*NC activations are loaded once and reused for all RT rows.
//  * Each weight is rebuilt exactly in fp32 (one FMA on the integer code, see
//    wval) and multiplied into fp32 accumulators, so every term of the sum is
//    the exact weight times x.
//  * Row reduction: wave-wide butterfly over 64 lanes, then the 4 waves'
//    partials are summed through LDS and one lane per (row, column) writes y.
#include "qk_common.h"
#include "qk_internal.h"

namespace qk {

constexpr int kGvThreads = 256;
constexpr int kGvChunk = 64;  // quant blocks per chunk and row (16 per wave)

template <int FMT, int RT>
struct GemvCfg {
    static constexpr int kBS = Format<FMT>::kBytes;
    static constexpr int kSegMax = kGvChunk * kBS;               // bytes per row per chunk
    static constexpr int kLds = RT * kSegMax;                    // LDS bytes
    static constexpr int kPref = (kLds / 16 + kGvThreads - 1) / kGvThreads;  // 16-B loads per lane
};

// Eight exact fp32 weights of quarter q of the block at LDS offset boff.
template <int FMT>
__device__ __forceinline__ void weights8(const uint8_t *lds, int boff, int q, float wv[8]) {
    using F = Format<FMT>;
    const float d = h2f(lds_u16(lds, boff));
    if constexpr (FMT == QK_Q8_0) {
        // c + 128 = unsigned byte of (c ^ 0x80); d*(c+128) - 128*d is exactly d*c.
        const uint32_t q0 = lds_u32_a2(lds, boff + F::kQsOffset + 8 * q) ^ 0x80808080u;
        const uint32_t q1 = lds_u32_a2(lds, boff + F::kQsOffset + 8 * q + 4) ^ 0x80808080u;
        const float off = -128.0f * d;
        wv[0] = wval(d, ubyte_f<0>(q0), off);
        wv[1] = wval(d, ubyte_f<1>(q0), off);
        wv[2] = wval(d, ubyte_f<2>(q0), off);
        wv[3] = wval(d, ubyte_f<3>(q0), off);
        wv[4] = wval(d, ubyte_f<0>(q1), off);
        wv[5] = wval(d, ubyte_f<1>(q1), off);
        wv[6] = wval(d, ubyte_f<2>(q1), off);
        wv[7] = wval(d, ubyte_f<3>(q1), off);
    } else {
        const uint32_t qw = lds_u32_a2(lds, boff + F::kQsOffset + 4 * q);
        const uint32_t lo = qw & 0x0F0F0F0Fu;
        const uint32_t hi = (qw >> 4) & 0x0F0F0F0Fu;
        const float off = (FMT == QK_Q4_0) ? -8.0f * d : h2f(lds_u16(lds, boff + 2));
        wv[0] = wval(d, ubyte_f<0>(lo), off);
        wv[1] = wval(d, ubyte_f<1>(lo), off);
        wv[2] = wval(d, ubyte_f<2>(lo), off);
        wv[3] = wval(d, ubyte_f<3>(lo), off);
        wv[4] = wval(d, ubyte_f<0>(hi), off);
        wv[5] = wval(d, ubyte_f<1>(hi), off);
        wv[6] = wval(d, ubyte_f<2>(hi), off);
        wv[7] = wval(d, ubyte_f<3>(hi), off);
    }
}

// The 8 activations of column j matching weights8's element order.
template <int FMT, bool ALIGNED>
__device__ __forceinline__ void acts8(const float *__restrict__ xj, int kg, int q, float xv[8]) {
    const float *p0, *p1;
    if constexpr (FMT == QK_Q8_0) {
        p0 = xj + 32 * kg + 8 * q;
        p1 = p0 + 4;
    } else {
        p0 = xj + 32 * kg + 4 * q;
        p1 = p0 + 16;
    }
    if (ALIGNED) {
        const float4 a = *reinterpret_cast<const float4 *>(p0);
        const float4 b = *reinterpret_cast<const float4 *>(p1);
        xv[0] = a.x; xv[1] = a.y; xv[2] = a.z; xv[3] = a.w;
        xv[4] = b.x; xv[5] = b.y; xv[6] = b.z; xv[7] = b.w;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            xv[i] = p0[i];
            xv[4 + i] = p1[i];
        }
    }
}

// ALIGNED: w 16-byte aligned, blocks per row % 8 == 0 (so every row and every
// chunk segment starts on 16 bytes), x 16-byte aligned and ldx % 4 == 0.
template <int FMT, int NC, int RT, bool ALIGNED>
__global__ __launch_bounds__(kGvThreads) void gemv_kernel(
    const uint8_t *__restrict__ w, int m, int nbk, const float *__restrict__ x, int64_t ldx,
    float *__restrict__ y, int64_t ldy) {
    using C = GemvCfg<FMT, RT>;
    constexpr int BS = C::kBS;
    __shared__ __attribute__((aligned(16))) uint8_t lds[C::kLds];
    __shared__ float red[4][RT * NC];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int slot = lane >> 2;
    const int q = lane & 3;
    const int row0 = blockIdx.x * RT;
    const int nrows = min(RT, m - row0);
    const int64_t row_bytes = (int64_t)nbk * BS;
    const uint8_t *__restrict__ wrows = w + (int64_t)row0 * row_bytes;

    float acc[RT][NC];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int j = 0; j < NC; ++j) acc[r][j] = 0.0f;

    uint4 pref[C::kPref];
    // Issue the 16-byte loads of chunk kb0 into registers.
    auto prefetch = [&](int kb0) {
        const int seg16 = min(kGvChunk, nbk - kb0) * BS / 16;
        const int total = nrows * seg16;
#pragma unroll
        for (int l = 0; l < C::kPref; ++l) {
            const int i = tid + l * kGvThreads;
            if (i < total) {
                const int r = i / seg16;
                const int c = i - r * seg16;
                pref[l] = *reinterpret_cast<const uint4 *>(wrows + r * row_bytes +
                                                           (int64_t)kb0 * BS + 16 * c);
            }
        }
    };
    if (ALIGNED && nbk > 0) prefetch(0);

    for (int kb0 = 0; kb0 < nbk; kb0 += kGvChunk) {
        const int kc = min(kGvChunk, nbk - kb0);
        const int seg = kc * BS;
        if (ALIGNED) {
            const int seg16 = seg / 16;
            const int total = nrows * seg16;
#pragma unroll
            for (int l = 0; l < C::kPref; ++l) {
                const int i = tid + l * kGvThreads;
                if (i < total) reinterpret_cast<uint4 *>(lds)[i] = pref[l];
            }
        } else {
            const int seg2 = seg / 2;
            const int total = nrows * seg2;
            for (int i = tid; i < total; i += kGvThreads) {
                const int r = i / seg2;
                const int c = i - r * seg2;
                reinterpret_cast<uint16_t *>(lds)[i] = *reinterpret_cast<const uint16_t *>(
                    wrows + r * row_bytes + (int64_t)kb0 * BS + 2 * c);
            }
        }
        __syncthreads();
        if (ALIGNED && kb0 + kGvChunk < nbk) prefetch(kb0 + kGvChunk);

        const int b = wave * 16 + slot;
        if (b < kc) {
            const int kg = kb0 + b;
            float xv[NC][8];
#pragma unroll
            for (int j = 0; j < NC; ++j) acts8<FMT, ALIGNED>(x + j * ldx, kg, q, xv[j]);
#pragma unroll
            for (int r = 0; r < RT; ++r) {
                if (r < nrows) {
                    float wv[8];
                    weights8<FMT>(lds, r * seg + b * BS, q, wv);
#pragma unroll
                    for (int j = 0; j < NC; ++j)
#pragma unroll
                        for (int t = 0; t < 8; ++t)
                            acc[r][j] = __builtin_fmaf(wv[t], xv[j][t], acc[r][j]);
                }
            }
        }
        __syncthreads();
    }

#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            const float v = wave_sum(acc[r][j]);
            if (lane == 0) red[wave][r * NC + j] = v;
        }
    __syncthreads();
    if (tid < RT * NC) {
        const int r = tid / NC;
        const int j = tid - r * NC;
        if (r < nrows)
            y[j * ldy + row0 + r] = (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
    }
}

template <int FMT, int NC>
static int dispatch_gemv_nc(const uint8_t *w, int m, int nbk, const float *x, int64_t ldx,
                            float *y, int64_t ldy, hipStream_t stream) {
    constexpr int RT = 8;
    const dim3 grid((unsigned)((m + RT - 1) / RT));
    const dim3 block(kGvThreads);
    const bool aligned = ((uintptr_t)w % 16) == 0 && (nbk % 8) == 0 &&
                         ((uintptr_t)x % 16) == 0 && (ldx % 4) == 0;
    if (aligned)
        return launch(gemv_kernel<FMT, NC, RT, true>, grid, block, stream, w, m, nbk, x, ldx, y, ldy);
    return launch(gemv_kernel<FMT, NC, RT, false>, grid, block, stream, w, m, nbk, x, ldx, y, ldy);
}

template <int FMT>
static int dispatch_gemv(const uint8_t *w, int m, int nbk, const float *x, int n, int64_t ldx,
                         float *y, int64_t ldy, hipStream_t stream) {
    switch (n) {
    case 1: return dispatch_gemv_nc<FMT, 1>(w, m, nbk, x, ldx, y, ldy, stream);
    case 2: return dispatch_gemv_nc<FMT, 2>(w, m, nbk, x, ldx, y, ldy, stream);
    case 3: return dispatch_gemv_nc<FMT, 3>(w, m, nbk, x, ldx, y, ldy, stream);
    case 4: return dispatch_gemv_nc<FMT, 4>(w, m, nbk, x, ldx, y, ldy, stream);
    case 5: return dispatch_gemv_nc<FMT, 5>(w, m, nbk, x, ldx, y, ldy, stream);
    case 6: return dispatch_gemv_nc<FMT, 6>(w, m, nbk, x, ldx, y, ldy, stream);
    case 7: return dispatch_gemv_nc<FMT, 7>(w, m, nbk, x, ldx, y, ldy, stream);
    case 8: return dispatch_gemv_nc<FMT, 8>(w, m, nbk, x, ldx, y, ldy, stream);
    default: return QK_ERR_INVALID_ARG;
    }
}

int launch_mul_mat_vec(int fmt, const void *w, int64_t m, int64_t k, const float *x,
                       int64_t n, int64_t ldx, float *y, int64_t ldy, hipStream_t stream) {
    const uint8_t *wb = static_cast<const uint8_t *>(w);
    const int nbk = (int)(k / kBlockElems);
    switch (fmt) {
    case QK_Q4_0: return dispatch_gemv<QK_Q4_0>(wb, (int)m, nbk, x, (int)n, ldx, y, ldy, stream);
    case QK_Q4_1: return dispatch_gemv<QK_Q4_1>(wb, (int)m, nbk, x, (int)n, ldx, y, ldy, stream);
    case QK_Q8_0: return dispatch_gemv<QK_Q8_0>(wb, (int)m, nbk, x, (int)n, ldx, y, ldy, stream);
    default: return QK_ERR_UNSUPPORTED;
    }
}

}  // namespace qk
