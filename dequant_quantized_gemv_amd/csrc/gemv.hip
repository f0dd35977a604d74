// gemv.hip - fused quantized GEMV for decode: y = W x for 1..8 fp32 columns.
//
// What is computed follows dequantize_mul_mat_vec ("dmmv", named with its
// tuning block in the "llama_cpp 0.12.1 -> 0.12.2" ggml-cuda.cu diff) and the
// ggml_cuda_op_mul_mat driver (a row range times a column count): each output
// is the dot product of one dequantized weight row with one activation column,
// reduced across lanes (the diff's warp_reduce_sum).  That kernel's body is not
// on the page; this one is designed for gfx950.
//
// Work split.  A workgroup of WPG waves owns WPG*RWV consecutive rows, RWV
// per wave.  K is walked in chunks of 128 blocks (4096 weights).  Within a
// chunk, lane p of every wave owns "pair" p: two consecutive blocks, 64
// weights.  A pair of Q4_0 / Q4_1 / Q8_0 blocks is 36 / 40 / 68 bytes, a whole
// number of dwords, so with an even block count per row every pair starts on
// 4 bytes and comes straight into registers with dword-aligned 16-byte loads
// (plain loads: streaming hints measured slower on this chip).
//
// Activations are the expensive side: every row needs all of x.  The chunk of
// x (4096 x NC floats) is copied once per workgroup into LDS and read from
// there by all of its rows; its global loads are issued before the weight
// loads so the copy never waits behind HBM.  In LDS each run of 64 floats is
// followed by 4 floats of padding, so the 16-byte reads of lanes p = 0..15 (at
// float offset 68p + 4t) fall in distinct banks.  A workgroup may take several
// row groups (grid-stride) and keeps its staged x when K fits one chunk.
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
// Reduction: a 64-lane DPP butterfly per (row, column); lane 0 writes y.
#include "qk_common.h"
#include "qk_internal.h"

namespace qk {

constexpr int kGvChunkPairs = 64;                   // pairs per chunk (one per lane)
constexpr int kGvChunkElems = kGvChunkPairs * 64;   // 4096 weights per chunk
constexpr int kGvXPitch = kGvChunkElems + kGvChunkElems / 16;  // floats per column in LDS (padded)

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int FMT> struct Pair;
template <> struct Pair<QK_Q4_0> { static constexpr int kDwords = 9; };
template <> struct Pair<QK_Q4_1> { static constexpr int kDwords = 10; };
template <> struct Pair<QK_Q8_0> { static constexpr int kDwords = 17; };

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

// fp16 bits of d (and m) of block b of the pair.
template <int FMT>
__device__ __forceinline__ uint32_t pair_d(const uint32_t (&v)[Pair<FMT>::kDwords], int b) {
    if constexpr (FMT == QK_Q4_0) return b == 0 ? (v[0] & 0xFFFFu) : (v[4] >> 16);
    if constexpr (FMT == QK_Q4_1) return b == 0 ? (v[0] & 0xFFFFu) : (v[5] & 0xFFFFu);
    return b == 0 ? (v[0] & 0xFFFFu) : (v[8] >> 16);
}
__device__ __forceinline__ uint32_t pair_m_q41(const uint32_t (&v)[10], int b) {
    return b == 0 ? (v[0] >> 16) : (v[5] >> 16);
}

// Quant word i of block b (Q4: i < 4, bytes 4i..4i+3; Q8: i < 8).
template <int FMT>
__device__ __forceinline__ uint32_t pair_qs(const uint32_t (&v)[Pair<FMT>::kDwords], int b, int i) {
    if constexpr (FMT == QK_Q4_0) return b == 0 ? shift2(v[i], v[i + 1]) : v[5 + i];
    if constexpr (FMT == QK_Q4_1) return b == 0 ? v[1 + i] : v[6 + i];
    return b == 0 ? shift2(v[i], v[i + 1]) : v[9 + i];
}

// ---------------------------------------------------------------------------
// Per-group products.  A group is quant word i of block b: Q4 elements
// 4i..4i+3 (low nibbles) and 16+4i..16+4i+3 (high nibbles); Q8 elements
// 4i..4i+3 (i < 8).  xa / xb are the matching activations.
// ---------------------------------------------------------------------------

// Q4_0 group: sum over the 8 elements of (q - 8) * x, added to s.
__device__ __forceinline__ float group_q4_0(uint32_t qw, const float4 &xa, const float4 &xb, float s) {
    // low nibbles: 1024 + c - 1032 = c - 8; high nibbles left in place:
    // (1024 + 16c) / 16 - 72 = c - 8 (one fused, exact operation)
    const uint32_t lo = qw & 0x0F0F0F0Fu;
    const uint32_t hi = qw & 0xF0F0F0F0u;
    const uint32_t l01 = pk_add_f16(bytes_to_f16_lo(lo), -1032.0f);
    const uint32_t l23 = pk_add_f16(bytes_to_f16_hi(lo), -1032.0f);
    const uint32_t h01 = pk_fma_f16(bytes_to_f16_lo(hi), 0.0625f, -72.0f);
    const uint32_t h23 = pk_fma_f16(bytes_to_f16_hi(hi), 0.0625f, -72.0f);
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

// float4 of x (column j) at chunk-relative element e (e % 4 == 0) from LDS.
__device__ __forceinline__ float4 x_lds(const float *xs, int j, int e) {
    return *reinterpret_cast<const float4 *>(xs + j * kGvXPitch + e + (e >> 6) * 4);
}

// FAST: w 4-byte aligned, an even number of blocks per row, x 16-byte aligned
// and ldx % 4 == 0.
//
// The grid walks row groups of 4*RWV rows: workgroup g takes groups g,
// g + gridDim.x, ...  When K fits in one chunk, x is staged once and reused by
// every group the workgroup takes.
template <int FMT, int NC, int RWV, int WPG, bool FAST>
__global__ __launch_bounds__(64 * WPG) void gemv_kernel(
    const uint8_t *__restrict__ w, int m, int nb, const float *__restrict__ x, int64_t ldx,
    float *__restrict__ y, int64_t ldy) {
    constexpr int BS = Format<FMT>::kBytes;
    constexpr int ND = Pair<FMT>::kDwords;
    constexpr int RG = WPG * RWV;  // rows per group
    constexpr int NT = 64 * WPG;   // lanes per workgroup
    __shared__ __attribute__((aligned(16))) float xs[NC * kGvXPitch];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int npairs = (nb + 1) >> 1;
    const int k = nb * 32;
    const int64_t row_bytes = (int64_t)nb * BS;
    const int ngroups = (m + RG - 1) / RG;
    int staged = -1;  // chunk currently in LDS (uniform across the workgroup)

    for (int g = blockIdx.x; g < ngroups; g += gridDim.x) {
        const int row0 = g * RG + wave * RWV;
        const int nrows = max(0, min(RWV, m - row0));  // rows of this wave (uniform)
        const uint8_t *__restrict__ wr0 = w + (int64_t)row0 * row_bytes;

        float acc[RWV][NC];
#pragma unroll
        for (int r = 0; r < RWV; ++r)
#pragma unroll
            for (int j = 0; j < NC; ++j) acc[r][j] = 0.0f;

        for (int p0 = 0; p0 < npairs; p0 += kGvChunkPairs) {
            const int pp = p0 + lane;  // this lane's pair
            const bool have = pp < npairs;
            const bool second = FAST || (2 * pp + 1 < nb);

            // Activations of this chunk go to LDS once per workgroup and chunk.
            // Their loads are issued before the weight loads, so writing them
            // to LDS does not wait for the weights (loads complete in order).
            const int chunk = p0 / kGvChunkPairs;
            const bool stage = staged != chunk;
            const int e0 = p0 * 64;
            const int ce4 = min(kGvChunkElems, k - e0) / 4;  // float4s in this chunk
            constexpr int XR = NC <= 2 ? NC : 0;  // columns staged through registers
            constexpr int XU = (kGvChunkElems / 4 + NT - 1) / NT;  // float4s per lane and column
            f32x4_t xr[XR > 0 ? XR : 1][XU];
            if (stage) {
                if (staged >= 0) __syncthreads();  // readers of the previous chunk are done
#pragma unroll
                for (int j = 0; j < XR; ++j) {
                    const float *xj = x + j * ldx + e0;
#pragma unroll
                    for (int u = 0; u < XU; ++u) {
                        // clamped so every lane loads (a tail lane repeats the
                        // last float4 and does not store it)
                        const int t = min(tid + u * NT, ce4 - 1);
                        if (FAST) {
                            xr[j][u] = *reinterpret_cast<const f32x4_t *>(xj + 4 * t);
                        } else {
                            xr[j][u] = f32x4_t{xj[4 * t], xj[4 * t + 1], xj[4 * t + 2], xj[4 * t + 3]};
                        }
                    }
                }
            }

            // weights of this chunk for the wave's rows, straight to registers
            uint32_t v[RWV][ND];
#pragma unroll
            for (int r = 0; r < RWV; ++r) {
                if (r < nrows && have) {
                    const uint8_t *p = wr0 + r * row_bytes + (int64_t)pp * (2 * BS);
                    if (FAST) load_pair_fast<FMT>(p, v[r]);
                    else load_pair_generic<FMT>(p, second, v[r]);
                }
            }

            if (stage) {
#pragma unroll
                for (int j = 0; j < XR; ++j)
#pragma unroll
                    for (int u = 0; u < XU; ++u) {
                        const int t = tid + u * NT;
                        if (t < ce4) *reinterpret_cast<f32x4_t *>(xs + j * kGvXPitch + 4 * t + (t >> 4) * 4) = xr[j][u];
                    }
#pragma unroll
                for (int j = XR; j < NC; ++j) {
                    const float *xj = x + j * ldx + e0;
                    for (int t = tid; t < ce4; t += NT) {
                        float4 val;
                        if (FAST) {
                            val = *reinterpret_cast<const float4 *>(xj + 4 * t);
                        } else {
                            val = make_float4(xj[4 * t], xj[4 * t + 1], xj[4 * t + 2], xj[4 * t + 3]);
                        }
                        *reinterpret_cast<float4 *>(xs + j * kGvXPitch + 4 * t + (t >> 4) * 4) = val;
                    }
                }
                __syncthreads();
                staged = chunk;
            }

            if (have && nrows > 0) {
                const int el = lane * 64;  // chunk-relative element of this lane's pair
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    if (!FAST && b == 1 && !second) break;
                    if constexpr (FMT == QK_Q4_1) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            float4 xa[NC], xb[NC];
#pragma unroll
                            for (int j = 0; j < NC; ++j) {
                                xa[j] = x_lds(xs, j, el + 32 * b + 4 * i);
                                xb[j] = x_lds(xs, j, el + 32 * b + 16 + 4 * i);
                            }
#pragma unroll
                            for (int r = 0; r < RWV; ++r) {
                                if (r < nrows) {
                                    const float d = h2f(pair_d<FMT>(v[r], b));
                                    const float mm = h2f(pair_m_q41(v[r], b));
                                    const uint32_t qw = pair_qs<FMT>(v[r], b, i);
                                    const uint32_t lo = qw & 0x0F0F0F0Fu;
                                    const uint32_t hi = (qw >> 4) & 0x0F0F0F0Fu;
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
                            // keep the next group's LDS reads from being hoisted
                            // above this one (bounds the live activations)
                            if constexpr (NC >= 2) __builtin_amdgcn_sched_barrier(0);
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
                                xa[j] = x_lds(xs, j, el + 32 * b + 4 * i);
                                if (FMT == QK_Q4_0) xb[j] = x_lds(xs, j, el + 32 * b + 16 + 4 * i);
                            }
#pragma unroll
                            for (int r = 0; r < RWV; ++r) {
                                if (r < nrows) {
#pragma unroll
                                    for (int j = 0; j < NC; ++j) {
                                        if constexpr (FMT == QK_Q4_0) {
                                            s[r][j] = group_q4_0(pair_qs<FMT>(v[r], b, i), xa[j], xb[j], s[r][j]);
                                        } else if (b == 0) {
                                            s[r][j] = group_q8_0_split(v[r][i], v[r][i + 1], xa[j], s[r][j]);
                                        } else {
                                            s[r][j] = group_q8_0(v[r][9 + i], xa[j], s[r][j]);
                                        }
                                    }
                                }
                            }
                            if constexpr (NC >= 3) __builtin_amdgcn_sched_barrier(0);
                        }
#pragma unroll
                        for (int r = 0; r < RWV; ++r) {
                            if (r < nrows) {
                                const float d = h2f(pair_d<FMT>(v[r], b));
#pragma unroll
                                for (int j = 0; j < NC; ++j) acc[r][j] = __builtin_fmaf(d, s[r][j], acc[r][j]);
                            }
                        }
                    }
                }
            }
        }

#pragma unroll
        for (int r = 0; r < RWV; ++r) {
            if (r < nrows) {
#pragma unroll
                for (int j = 0; j < NC; ++j) {
                    const float sum = wave_sum(acc[r][j]);
                    if (lane == 0) y[j * ldy + row0 + r] = sum;
                }
            }
        }
    }
}

// Launch shape by column count: RWV rows per wave (registers hold RWV pairs
// of weights and RWV * NC partial sums), WPG waves per workgroup sharing one
// LDS copy of the activations.
template <int NC> struct GemvShape {
    static constexpr int kRWV = 1;
    static constexpr int kWPG = NC <= 4 ? 8 : 4;
};

template <int FMT, int NC>
static int dispatch_gemv_nc(const uint8_t *w, int m, int nb, const float *x, int64_t ldx,
                            float *y, int64_t ldy, hipStream_t stream) {
    constexpr int RWV = GemvShape<NC>::kRWV;
    constexpr int WPG = GemvShape<NC>::kWPG;
    constexpr int RG = WPG * RWV;
    const int ngroups = (m + RG - 1) / RG;
    // Enough workgroups to cover the chip several times over; beyond that a
    // workgroup takes several row groups and reuses its staged activations.
    int cus = 256;
    int dev = 0;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0) cus = v;
    }
    const int per_cu = NC <= 2 ? 4 : (NC <= 4 ? 2 : 1);  // LDS holds NC * 17 KiB of activations
    const dim3 grid((unsigned)min(ngroups, cus * per_cu));
    const dim3 block(64 * WPG);
    const bool fast = ((uintptr_t)w % 4) == 0 && (nb % 2) == 0 &&
                      ((uintptr_t)x % 16) == 0 && (ldx % 4) == 0;
    if (fast)
        return launch(gemv_kernel<FMT, NC, RWV, WPG, true>, grid, block, stream, w, m, nb, x, ldx, y, ldy);
    return launch(gemv_kernel<FMT, NC, RWV, WPG, false>, grid, block, stream, w, m, nb, x, ldx, y, ldy);
}

template <int FMT>
static int dispatch_gemv(const uint8_t *w, int m, int nb, const float *x, int n, int64_t ldx,
                         float *y, int64_t ldy, hipStream_t stream) {
    switch (n) {
    case 1: return dispatch_gemv_nc<FMT, 1>(w, m, nb, x, ldx, y, ldy, stream);
    case 2: return dispatch_gemv_nc<FMT, 2>(w, m, nb, x, ldx, y, ldy, stream);
    case 3: return dispatch_gemv_nc<FMT, 3>(w, m, nb, x, ldx, y, ldy, stream);
    case 4: return dispatch_gemv_nc<FMT, 4>(w, m, nb, x, ldx, y, ldy, stream);
    case 5: return dispatch_gemv_nc<FMT, 5>(w, m, nb, x, ldx, y, ldy, stream);
    case 6: return dispatch_gemv_nc<FMT, 6>(w, m, nb, x, ldx, y, ldy, stream);
    case 7: return dispatch_gemv_nc<FMT, 7>(w, m, nb, x, ldx, y, ldy, stream);
    case 8: return dispatch_gemv_nc<FMT, 8>(w, m, nb, x, ldx, y, ldy, stream);
    default: return QK_ERR_INVALID_ARG;
    }
}

int launch_mul_mat_vec(int fmt, const void *w, int64_t m, int64_t k, const float *x,
                       int64_t n, int64_t ldx, float *y, int64_t ldy, hipStream_t stream) {
    const uint8_t *wb = static_cast<const uint8_t *>(w);
    const int nb = (int)(k / kBlockElems);
    switch (fmt) {
    case QK_Q4_0: return dispatch_gemv<QK_Q4_0>(wb, (int)m, nb, x, (int)n, ldx, y, ldy, stream);
    case QK_Q4_1: return dispatch_gemv<QK_Q4_1>(wb, (int)m, nb, x, (int)n, ldx, y, ldy, stream);
    case QK_Q8_0: return dispatch_gemv<QK_Q8_0>(wb, (int)m, nb, x, (int)n, ldx, y, ldy, stream);
    default: return QK_ERR_INVALID_ARG;
    }
}

}  // namespace qk
