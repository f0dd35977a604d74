// gemv_mfma.h - the fused quantized GEMV for 4..8 fp32 columns with the
// products on the matrix cores (v_mfma_f32_4x4x1_16b_f32).
//
// What is computed is the GEMV of gemv_impl.h (dequantize_mul_mat_vec under
// the ggml_cuda_op_mul_mat row-range x column-count driver of the
// "llama_cpp 0.12.1 -> 0.12.2" ggml-cuda.cu diff): y[j][i] = sum_c W[i,c]
// x[j][c], each term the exact fp32 weight (the dequantize definition: d*q
// + (-8*d), d*q + m, d*q) times the fp32 activation.  With several columns
// the per-weight work of the vector ALU is dominated by the n multiply-adds;
// here they run on the matrix cores instead, and the vector ALU only rebuilds
// each fp32 weight once for all columns.
//
// The fp32 4x4x1 MFMA does 16 independent 4x4 outer-product updates,
// D_g += A_g (4 values) x B_g (4 values), g = lane / 4; on gfx950 each
// update is a fused multiply-add per element (one rounding, fp32 denormals
// kept), so every term is rounded exactly as an FMA on the vector ALU rounds
// it.  The 16 updates are used as 16 k-streams of one row-quad: lane (g, c)
// (c = lane % 4) supplies the weight of row c of the quad and the activation
// of column c at the same k, and block g accumulates the 4 x 4 partial sums
// of its stream.  A row-quad's pairs are split over KQ waves (1, 2 or 4, as
// k needs): lane group g of wave kq takes pair g + 16 kq of each of the four
// rows (a pair is two blocks, 64 weights: 36 / 40 / 68 bytes, dword aligned,
// loaded straight into registers).  A stream is two or four fp32 FMA chains
// of at most 32 terms (elements t % 2 or t % 4); the chains and the 16
// streams are added in trees (2 + 4 levels), and the KQ waves' sums in
// sequence, so |y - exact| <= (32 + 6 + 3) * 2^-24 * S to first order.
//
// Activations: the row's whole activation window (k <= 4096 weights, up to
// 8 columns) is staged once per workgroup in LDS, column c at c * kMfPitch
// floats and element e at e + 4 * (e / 64): the 16 reads of a quarter-wave
// (4 lane groups x 4 columns, 16 bytes each) then fall in distinct banks.
// Workgroups are one per CU when the window is large (8 columns: 140 KB) and
// walk a contiguous range of row-quads in rounds, so the window is staged once
// per workgroup.  In a round each row-quad is split over KQ waves (pairs
// g + 16 kq), whose partial sums meet in LDS and are added in a fixed order
// by the first of them: deterministic, with no atomics.
#pragma once

#include "gemv_impl.h"

namespace qk {

typedef float f32x4m_t __attribute__((ext_vector_type(4)));

// LDS floats per staged column: 4096 weights + 4 floats of padding per 64,
// and 16 more so consecutive columns start 16 banks apart.
constexpr int kMfPitch = kGvWindow + kGvWindow / 16 + 16;
// Largest k (weights per row) the matrix-core GEMV takes: one staged window.
constexpr int kMfMaxK = kGvWindow;

// The value of lane l ^ 16 or l ^ 32, from gfx950's row-swap instructions:
// v_permlane16_swap exchanges the odd 16-lane rows of its first operand with
// the even rows of its second (v_permlane32_swap: the upper half of the
// first with the lower half of the second), so with x in both, the first
// holds the partner's value in odd rows (upper half), the second in even
// rows (lower half).  Written as inline asm so that the compiler sees both
// registers change; the two wait states before it cover a vector write of
// either operand just ahead (the hazard the compiler itself pads for these
// instructions).  Vector-ALU operations, no LDS access.
__device__ __forceinline__ float lane_xor16(float x, bool odd_row) {
    uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
    return __builtin_bit_cast(float, odd_row ? a : b);
}
__device__ __forceinline__ float lane_xor32(float x, bool upper_half) {
    uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
    return __builtin_bit_cast(float, upper_half ? a : b);
}

template <int FMT>
__device__ __forceinline__ void word_weights(const uint32_t (&v)[Pair<FMT>::kDwords], int b, int i,
                                             float d, float mm, float (&w)[8]) {
    if constexpr (FMT == QK_Q8_0) {
        const uint32_t qw = b == 0 ? shift2(v[i], v[i + 1]) : v[9 + i];
        w[0] = d * (float)(int8_t)(qw);
        w[1] = d * (float)(int8_t)(qw >> 8);
        w[2] = d * (float)(int8_t)(qw >> 16);
        w[3] = d * (float)(int8_t)(qw >> 24);
    } else {
        uint32_t lo, hi;
        pair_codes<FMT>(v, b, i, lo, hi);
        // opaque, so each nibble converts with one byte-select convert
        // (v_cvt_f32_ubyte1..3) instead of a field extract and a convert
        asm volatile("" : "+v"(lo), "+v"(hi));
        w[0] = wval(d, ubyte_f<0>(lo), mm);
        w[1] = wval(d, ubyte_f<1>(lo), mm);
        w[2] = wval(d, ubyte_f<2>(lo), mm);
        w[3] = wval(d, ubyte_f<3>(lo), mm);
        w[4] = wval(d, ubyte_f<0>(hi), mm);
        w[5] = wval(d, ubyte_f<1>(hi), mm);
        w[6] = wval(d, ubyte_f<2>(hi), mm);
        w[7] = wval(d, ubyte_f<3>(hi), mm);
    }
}

template <int FMT, int NC, int WPG, int KQ, bool CNT>
__global__ __launch_bounds__(64 * WPG) __attribute__((amdgpu_waves_per_eu(4))) void gemv_mfma_kernel(
    const GemvItem it, const int qper, const int qrem) {
    static_assert(NC >= 1 && NC <= 8, "1..8 columns");
    static_assert((KQ == 1 || KQ == 2 || KQ == 4) && WPG % KQ == 0, "K split");
    constexpr int CG = (NC + 3) / 4;  // column groups of 4 (one MFMA each per k)
    // At 5 or 6 columns the columns past the fourth go to the vector ALU (one
    // FMA per weight and column, fused like the MFMA's updates) instead of a
    // second, mostly idle MFMA group: Q4_1 11008 x 4096 at 5 / 6 columns
    // 17.5 -> 15.5 / 17.3 -> 16.7 us, Q5_1 at 6 19.4 -> 17.8, Q8_0 21.6 ->
    // 21.0; at 7 columns it measured 17.8 -> 21.9 us, so 7 and 8 keep it.
    constexpr int NV = (NC == 5 || NC == 6) ? NC - 4 : 0;
    constexpr int CGM = NV > 0 ? 1 : CG;  // column groups on the matrix cores
    constexpr int ND = Pair<FMT>::kDwords;
    constexpr int BS = Format<FMT>::kBytes;
    constexpr int NT = 64 * WPG;
    constexpr int RPR = WPG / KQ;  // row-quads per round
    extern __shared__ __attribute__((aligned(16))) float xs[];
    // per wave, its partial sums of one round: [cg][column c][row r], in two
    // sets used by alternate rounds
    float *const part = xs + NC * kMfPitch;
    // CNT: one set of slots per round, never reused, and an LDS counter per
    // row-quad of each round; the last of the row-quad's KQ waves to arrive
    // adds the partial sums, so the rounds need no barrier
    const int nsets = (qper + (qrem > 0 ? 1 : 0) + RPR - 1) / RPR;
    uint32_t *const cnt = reinterpret_cast<uint32_t *>(part + (CNT ? nsets : 2) * (WPG * CG * 16));

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // (made uniform for two column groups: the round's branches are then
    // scalar; measured 19.7 -> 19.1 us at 8 columns, 14.7 -> 15.0 at 4)
    const int wave = CG == 2 ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
    const int kq = wave % KQ;    // which pair of the row this wave's lanes take
    const int slot = wave / KQ;  // which row-quad of the round
    const int g = lane >> 2;     // k-stream (lane group)
    const int c = lane & 3;      // row of the quad (A) and column of the group (B)
    const int b = blockIdx.x;
    const int q0 = b * qper + min(b, qrem);
    const int q1 = q0 + qper + (b < qrem ? 1 : 0);
    const int npairs = it.nb >> 1;  // an even block count on this path
    const int kk = it.nb * 32;
    const int64_t row_bytes = (int64_t)it.nb * BS;
    const int p = g + 16 * kq;       // the lane's pair of every row it reads
    const bool valid = p < npairs;   // a pair past the row: weights 0

    // the lane's pair of row-quad q (a row past m, or a pair past the row,
    // reads a clamped valid address; its weights are zeroed below)
    auto load = [&](int q, uint32_t (&dst)[ND]) __attribute__((always_inline)) {
        const int row = min(4 * q + c, it.m - 1);
        load_pair_fast<FMT>(it.w + (int64_t)row * row_bytes + (int64_t)min(p, npairs - 1) * (2 * BS), dst);
    };

    // The activations go to LDS: NC columns of KQ * 1024 elements, zero past
    // k (every lane then reads finite values).  Their loads are issued first,
    // unconditionally (a clamped address, the value zeroed after), then the
    // first row-quad's weight loads: loads complete in order, so the LDS
    // stores wait only for the activations and the weights' HBM latency
    // overlaps the staging.
    constexpr int PER_COL = KQ * 256;  // float4s per column
    constexpr int TOT = NC * PER_COL;
    constexpr int IT = (TOT + NT - 1) / NT;
    f32x4m_t tmp[IT];
#pragma unroll
    for (int u = 0; u < IT; ++u) {
        const int idx = min(tid + u * NT, TOT - 1);
        const int j = idx / PER_COL;
        const int e = (idx % PER_COL) << 2;
        tmp[u] = *reinterpret_cast<const f32x4_a4 *>(it.x + j * it.ldx + min(e, kk - 4));
    }
    // the wave's pairs of its first D rounds (unconditional, clamped, so the
    // waits that follow are counted exactly); each round then requests the
    // round D ahead into the registers it has just used.  Two rounds ahead;
    // three for Q4_1 at four columns with each row-quad over four waves and
    // counters between the rounds (11008 x 4096: 14.26-14.33 -> 13.58-13.67
    // us, 12000 x 3072: 14.29 -> 13.74-13.83 us).  Elsewhere three measured
    // slower: with a barrier per round, at 8 columns (the extra registers:
    // 6-19 %), for Q8_0 and with two waves per row-quad (1-2 %), and for
    // Q4_0 / Q5_0 / Q5_1 it was within -2..+2 %.
    constexpr int D = CNT && CG == 1 && KQ == 4 && FMT == QK_Q4_1 ? 3 : 2;
    uint32_t v[D][ND];
#pragma unroll
    for (int r = 0; r < D; ++r) load(min(q0 + slot + r * RPR, q1 - 1), v[r]);
    // The staged values pass through an empty asm here, unconditionally:
    // otherwise the compiler may sink an activation load into the branch of
    // the zero fill below, behind the weight loads, and the LDS copy then
    // waits for every weight load too (Q4_1 11008 x 4096 at 8 columns 19.0
    // -> 17.9 us, 4096 x 4096 at 4 / 8 columns 8.5 -> 8.0 / 11.1 -> 10.4 us).
#pragma unroll
    for (int u = 0; u < IT; ++u) asm volatile("" : "+v"(tmp[u]));
#pragma unroll
    for (int u = 0; u < IT; ++u) {
        const int idx = tid + u * NT;
        const int j = idx / PER_COL;
        const int e = (idx % PER_COL) << 2;
        const f32x4m_t z = {0.0f, 0.0f, 0.0f, 0.0f};
        if (TOT % NT == 0 || idx < TOT)
            *reinterpret_cast<f32x4m_t *>(xs + j * kMfPitch + e + (e >> 6) * 4) = e < kk ? tmp[u] : z;
    }
    if constexpr (CNT)
        for (int i = tid; i < nsets * RPR; i += NT) cnt[i] = 0u;
    __syncthreads();

    // partial sum of (wave w, column group cg, column c, row r) in a slot set
    auto part_at = [](float *set, int w, int cg, int cc, int r) -> float & {
        return set[((w * CG + cg) * 4 + cc) * 4 + r];
    };

    // the B operand of column group cg: column cg*4 + c (a lane whose column
    // is past NC reads column NC-1; its sums are never stored)
    int colo[CG];
#pragma unroll
    for (int cg = 0; cg < CG; ++cg) colo[cg] = min(cg * 4 + c, NC - 1) * kMfPitch;

    // One round: RPR row-quads, each split over KQ waves (one pair per lane);
    // its partial sums go to set `ps` of the partial slots.
    auto round = [&](const int qb, uint32_t (&cur)[ND], const int ps) __attribute__((always_inline)) {
        const int q = qb + slot;
        // CH independent accumulation chains per column group (element
        // t % CH), added at the end: four for one group, two for two
        constexpr int CH = CGM == 1 ? 4 : 2;
        // (with two column groups each chain's first product takes a zero
        // accumulator operand instead of registers cleared beforehand; with
        // one, clearing them first measured faster)
        const f32x4m_t zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
        f32x4m_t acc[CGM][CH];
        if constexpr (CGM == 1) {
#pragma unroll
            for (int u = 0; u < CH; ++u) acc[0][u] = zero4;
        }
        // the vector-ALU columns: two chains per column (element t % 2)
        float accv[NV > 0 ? NV : 1][2];
#pragma unroll
        for (int j = 0; j < NV; ++j) accv[j][0] = accv[j][1] = 0.0f;
        float *const pw = part + ps * (WPG * CG * 16);
        if (q < q1) {
#pragma unroll
            for (int bk = 0; bk < 2; ++bk) {
                float d = h2f(pair_d<FMT>(cur, bk));
                float mm = 0.0f;
                // (d*q + mm: exact for the offset formats, -8d and -16d
                // being exact and (q - 8) d, (q - 16) d representable)
                if constexpr (kHasM<FMT>) mm = h2f(pair_m<FMT>(cur, bk));
                else if constexpr (FMT == QK_Q4_0) mm = -8.0f * d;
                else if constexpr (FMT == QK_Q5_0) mm = -16.0f * d;
                d = valid ? d : 0.0f;
                mm = valid ? mm : 0.0f;
                constexpr int NW = FMT == QK_Q8_0 ? 8 : 4;  // quant words per block
#pragma unroll
                for (int wi = 0; wi < NW; ++wi) {
                    float wt[8];
                    word_weights<FMT>(cur, bk, wi, d, mm, wt);
#pragma unroll
                    for (int h = 0; h < (FMT == QK_Q8_0 ? 1 : 2); ++h) {
                        // elements 4wi..4wi+3 (h = 0) or 16+4wi.. (h = 1) of the block
                        const int e = 64 * p + 32 * bk + 16 * h + 4 * wi;
                        const int eo = e + (e >> 6) * 4;
                        f32x4m_t xb[CGM];
#pragma unroll
                        for (int cg = 0; cg < CGM; ++cg)
                            xb[cg] = *reinterpret_cast<const f32x4m_t *>(xs + colo[cg] + eo);
                        // (column 4 + j at the lane's own k, as for its row's weight)
                        f32x4m_t xv[NV > 0 ? NV : 1];
#pragma unroll
                        for (int j = 0; j < NV; ++j)
                            xv[j] = *reinterpret_cast<const f32x4m_t *>(xs + (4 + j) * kMfPitch + eo);
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            const bool first = CGM == 2 && bk == 0 && wi == 0 && h == 0 && u < CH;
#pragma unroll
                            for (int cg = 0; cg < CGM; ++cg)
                                acc[cg][u % CH] = __builtin_amdgcn_mfma_f32_4x4x1f32(
                                    wt[4 * h + u], xb[cg][u], first ? zero4 : acc[cg][u % CH], 0, 0, 0);
#pragma unroll
                            for (int j = 0; j < NV; ++j)
                                accv[j][u & 1] = __builtin_fmaf(wt[4 * h + u], xv[j][u], accv[j][u & 1]);
                        }
                    }
                    // keep the next word's LDS reads from being hoisted above
                    // this one (bounds the live activations)
                    asm volatile("" ::: "memory");
                }
            }
        }
        // the pair of the wave's round D ahead into the registers just used
        if (q + D * RPR < q1) load(q + D * RPR, cur);
        // a row-quad past the range has no sums, and none are read: with two
        // column groups its reduction is skipped (with one, running it on
        // the cleared accumulators measured faster than the branch)
        if (CG == 1 || q < q1) {
            // The 16 streams of each (row r, column c) are lanes c, c + 4, ...,
            // c + 60: a DPP tree within each 16-lane row (every lane of the row
            // then holds its column's row sums for all four r), then across the
            // rows with the four values shared out: rows 0 and 1 (2 and 3) trade
            // halves so that each keeps two of the r, then the two halves of the
            // wave so that row R keeps one, r = 2 (R & 1) + (R >> 1).  Lanes 0..3
            // of each row write it.
            const int R = lane >> 4;
            const bool odd = (R & 1) != 0;
            const bool upper = R >= 2;
#pragma unroll
            for (int cg = 0; cg < CGM; ++cg) {
                float v4[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float sm = acc[cg][0][r] + acc[cg][1][r];
                    if constexpr (CH == 4) sm += acc[cg][2][r] + acc[cg][3][r];
                    sm += dpp<0x124>(sm);  // row_ror:4
                    sm += dpp<0x128>(sm);  // row_ror:8
                    v4[r] = sm;
                }
                // the pair this row keeps (r = 2 (R & 1) + {0, 1}) and the pair it hands over
                const float k0 = odd ? v4[2] : v4[0], k1 = odd ? v4[3] : v4[1];
                const float s0 = odd ? v4[0] : v4[2], s1 = odd ? v4[1] : v4[3];
                const float t0 = k0 + lane_xor16(s0, odd), t1 = k1 + lane_xor16(s1, odd);
                const float sm = (upper ? t1 : t0) + lane_xor32(upper ? t0 : t1, upper);
                if ((lane & 15) < 4) part_at(pw, wave, cg, c, 2 * (R & 1) + (R >> 1)) = sm;
            }
            // a vector-ALU column: lane (g, c) holds row c's sum over its
            // k-stream g; the same tree adds the 16 streams (lanes c, c + 4,
            // ..., c + 60), every lane ends with its row's sum, lanes 0..3 write
#pragma unroll
            for (int j = 0; j < NV; ++j) {
                float sm = accv[j][0] + accv[j][1];
                sm += dpp<0x124>(sm);  // row_ror:4
                sm += dpp<0x128>(sm);  // row_ror:8
                sm += lane_xor16(sm, odd);
                sm += lane_xor32(sm, upper);
                if (lane < 4) part_at(pw, wave, 1, j, c) = sm;
            }
        }
        if constexpr (CNT) {
            // LDS operations of one wave are performed in order, so the
            // partial sums written above precede this wave's increment; the
            // wave that sees KQ - 1 comes after every other wave's increment
            // and reads their sums (in wave order, as below: the same bits
            // whichever wave adds them)
            asm volatile("" ::: "memory");
            uint32_t old = 0;
            if (lane == 0)
                old = __hip_atomic_fetch_add(&cnt[ps * RPR + slot], 1u, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_WORKGROUP);
            old = __builtin_amdgcn_readfirstlane(old);
            asm volatile("" ::: "memory");
            if (old == KQ - 1 && q < q1 && lane < 16 * CG) {
                const int r = lane & 3;
                const int cc = (lane >> 2) & 3;
                const int cg = lane >> 4;
                const int col = cg * 4 + cc;
                float sm = part_at(pw, slot * KQ, cg, cc, r);
#pragma unroll
                for (int k2 = 1; k2 < KQ; ++k2) sm += part_at(pw, slot * KQ + k2, cg, cc, r);
                const int ro = 4 * q + r;
                if (col < NC && ro < it.m) it.y[col * it.ldy + ro] = sm;
            }
            return;
        }
        // one barrier per round: a set of slots is written again two rounds
        // later, after every wave has passed the next round's barrier, by
        // which time its readers are done with it
        __syncthreads();
        // the KQ waves of a row-quad in order: the first one adds and stores
        if (kq == 0 && q < q1 && lane < 16 * CG) {
            const int r = lane & 3;
            const int cc = (lane >> 2) & 3;
            const int cg = lane >> 4;
            const int col = cg * 4 + cc;
            float sm = part_at(pw, wave, cg, cc, r);
#pragma unroll
            for (int k2 = 1; k2 < KQ; ++k2) sm += part_at(pw, wave + k2, cg, cc, r);
            const int ro = 4 * q + r;
            if (col < NC && ro < it.m) it.y[col * it.ldy + ro] = sm;
        }
    };
    static_assert(CNT || D == 2, "without CNT the rounds alternate between two sets of partial slots");
    for (int qb = q0; qb < q1; qb += D * RPR) {
#pragma unroll
        for (int r = 0; r < D; ++r)
            if (qb + r * RPR < q1)  // (uniform across the workgroup)
                round(qb + r * RPR, v[r], CNT ? (qb - q0) / RPR + r : r);
    }
}

// Waves per workgroup by column count: the staged window takes NC * 17.5 KB
// of LDS, so 8 columns fit one workgroup per CU (16 waves), 4 columns two (8
// waves each), 2 or 3 columns four (4 waves each): 16 waves per CU in all.
template <int NC> struct MfShape {
    static constexpr int kWPG = NC > 4 ? 16 : (NC > 2 ? 8 : 4);
};

template <int FMT, int NC, int KQ>
int gemv_mfma_run(const GemvItem &it, hipStream_t stream) {
    constexpr int WPG = MfShape<NC>::kWPG;
    constexpr int RPR = WPG / KQ;
    const size_t set_floats = (size_t)WPG * ((NC + 3) / 4) * 16;
    size_t lds = ((size_t)NC * kMfPitch + 2 * set_floats) * sizeof(float);
    const int per_cu = max(1, (int)((160 * 1024) / lds));
    const int64_t quads = ((int64_t)it.m + 3) / 4;
    if (quads > INT32_MAX) return QK_ERR_INVALID_ARG;
    const int64_t cap = (int64_t)device_cus() * per_cu;
    const int nwg = (int)(quads < cap ? quads : cap);
    // Counters instead of a barrier per round where workgroups run two or
    // more rounds and the extra slot sets leave as many workgroups per CU
    // (Q4_1 11008 x 4096 at 4 / 5 / 6 / 8 columns 14.39 -> 14.27, 17.91 ->
    // 17.56, 17.95 -> 17.34, 17.97 -> 17.77 us, bitwise equal; with a single
    // round, e.g. 4096 x 4096 at 8 columns, the counter cost 1 % more)
    const int64_t rounds = ((quads + nwg - 1) / nwg + RPR - 1) / RPR;
    const size_t lds_cnt = ((size_t)NC * kMfPitch + (size_t)rounds * (set_floats + RPR)) * sizeof(float);
    const bool use_cnt = rounds >= 2 && lds_cnt * per_cu <= 160 * 1024;
    if (use_cnt) lds = lds_cnt;
    auto kern = use_cnt ? gemv_mfma_kernel<FMT, NC, WPG, KQ, true> : gemv_mfma_kernel<FMT, NC, WPG, KQ, false>;
    if (lds > 64 * 1024 &&
        hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
        return QK_ERR_LAUNCH;
    return launch_lds(kern, dim3((unsigned)nwg), dim3(64 * WPG), lds, stream, it, (int)(quads / nwg),
                      (int)(quads % nwg));
}

// y = W x for NC = 4..8 columns on the matrix cores: one problem, weights
// 4-byte aligned with an even block count, k <= kMfMaxK.  Each row-quad is
// split over KQ waves, one pair of blocks per lane.
template <int FMT, int NC>
int gemv_mfma_launch(const GemvItem &it, hipStream_t stream) {
    const int npairs = it.nb >> 1;
    if (npairs <= 16) return gemv_mfma_run<FMT, NC, 1>(it, stream);
    if (npairs <= 32) return gemv_mfma_run<FMT, NC, 2>(it, stream);
    return gemv_mfma_run<FMT, NC, 4>(it, stream);
}

}  // namespace qk
