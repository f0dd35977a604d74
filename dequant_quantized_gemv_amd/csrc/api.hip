// api.hip - the C ABI: argument validation, then dispatch to the launchers.
//
// Validation happens entirely on the host before any HIP call, so every error
// path returns a status with nothing enqueued.
#include <stdint.h>
#include <stddef.h>

#include "qk.h"
#include "qk_common.h"
#include "qk_internal.h"

namespace {

constexpr int64_t kMaxDim = INT32_MAX;  // kernels index rows and columns in 32 bits

bool fmt_ok(int fmt) { return qk::block_bytes_host(fmt) != 0; }

// Half-open byte ranges [a, a+na) and [b, b+nb) intersect.
bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    if (na == 0 || nb == 0) return false;
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + nb && y < x + na;
}

// Bytes spanned by n columns of length len with stride ld (elements of size es).
size_t span_bytes(int64_t n, int64_t ld, int64_t len, size_t es) {
    if (n <= 0 || len <= 0) return 0;
    return (size_t)((n - 1) * ld + len) * es;
}

}  // namespace

extern "C" {

size_t qk_block_bytes(int fmt) { return (size_t)qk::block_bytes_host(fmt); }

size_t qk_row_bytes(int fmt, int64_t k) {
    if (!fmt_ok(fmt) || k < 0 || k % 32 != 0) return 0;
    return (size_t)(k / 32) * (size_t)qk::block_bytes_host(fmt);
}

const char *qk_status_string(int status) {
    switch (status) {
    case QK_OK: return "ok";
    case QK_ERR_INVALID_ARG: return "invalid argument";
    case QK_ERR_UNSUPPORTED: return "unsupported format or dtype";
    case QK_ERR_ALIGNMENT: return "misaligned pointer";
    case QK_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
    }
}

int qk_version(void) { return 200; }

int qk_dequantize(int fmt, const void *w, int64_t rows, int64_t k, int out_dtype, void *out,
                  void *stream) {
    if (!fmt_ok(fmt)) return QK_ERR_UNSUPPORTED;
    if (out_dtype != QK_F32 && out_dtype != QK_F16) return QK_ERR_UNSUPPORTED;
    if (rows < 0 || k < 0 || k % 32 != 0) return QK_ERR_INVALID_ARG;
    if (rows == 0 || k == 0) return QK_OK;
    if (k > kMaxDim || rows > INT64_MAX / (k / 32)) return QK_ERR_INVALID_ARG;
    // chunks of 128 blocks are numbered in 32 bits on the device side
    if ((rows * (k / 32) + 127) / 128 > (int64_t)INT32_MAX) return QK_ERR_INVALID_ARG;
    if (w == nullptr || out == nullptr) return QK_ERR_INVALID_ARG;
    const size_t es = out_dtype == QK_F32 ? 4 : 2;
    if ((uintptr_t)w % 2 != 0 || (uintptr_t)out % es != 0) return QK_ERR_ALIGNMENT;
    const int64_t nblocks = rows * (k / 32);
    const size_t wbytes = (size_t)nblocks * qk::block_bytes_host(fmt);
    const size_t obytes = (size_t)(rows * k) * es;
    if (overlaps(w, wbytes, out, obytes)) return QK_ERR_INVALID_ARG;
    return qk::launch_dequantize(fmt, w, nblocks, out_dtype, out,
                                 static_cast<hipStream_t>(stream));
}

// Checks one GEMV problem (n already known to be 1..8); QK_OK if valid.
static int check_gemv_item(int fmt, const qk_mat_vec_item &it, int64_t n) {
    if (it.m < 0 || it.k < 0 || it.k % 32 != 0) return QK_ERR_INVALID_ARG;
    if (it.m == 0) return QK_OK;
    if (it.m > kMaxDim || it.k > kMaxDim || it.ldx < it.k || it.ldy < it.m) return QK_ERR_INVALID_ARG;
    if (it.y == nullptr || (it.k > 0 && (it.w == nullptr || it.x == nullptr))) return QK_ERR_INVALID_ARG;
    if ((uintptr_t)it.w % 2 != 0 || (uintptr_t)it.x % 4 != 0 || (uintptr_t)it.y % 4 != 0)
        return QK_ERR_ALIGNMENT;
    const size_t wbytes = (size_t)it.m * (size_t)(it.k / 32) * qk::block_bytes_host(fmt);
    const size_t xbytes = span_bytes(n, it.ldx, it.k, 4);
    const size_t ybytes = span_bytes(n, it.ldy, it.m, 4);
    if (overlaps(it.y, ybytes, it.w, wbytes) || overlaps(it.y, ybytes, it.x, xbytes))
        return QK_ERR_INVALID_ARG;
    return QK_OK;
}

int qk_mul_mat_vec(int fmt, const void *w, int64_t m, int64_t k, const float *x, int64_t n,
                   int64_t ldx, float *y, int64_t ldy, void *stream) {
    if (!fmt_ok(fmt)) return QK_ERR_UNSUPPORTED;
    if (m < 0 || k < 0 || k % 32 != 0 || n < 0 || n > 8) return QK_ERR_INVALID_ARG;
    if (m == 0 || n == 0) return QK_OK;
    const qk_mat_vec_item it{w, m, k, x, ldx, y, ldy};
    const int st = check_gemv_item(fmt, it, n);
    if (st != QK_OK) return st;
    return qk::launch_mul_mat_vec(fmt, w, m, k, x, n, ldx, y, ldy, static_cast<hipStream_t>(stream));
}

int qk_mul_mat_vec_x8(int fmt, const void *w, int64_t m, int64_t k, const float *x, int64_t n,
                      int64_t ldx, float *y, int64_t ldy, void *stream) {
    if (!fmt_ok(fmt)) return QK_ERR_UNSUPPORTED;
    if (m < 0 || k < 0 || k % 32 != 0 || n < 0 || n > 8) return QK_ERR_INVALID_ARG;
    if (m == 0 || n == 0) return QK_OK;
    const qk_mat_vec_item it{w, m, k, x, ldx, y, ldy};
    const int st = check_gemv_item(fmt, it, n);
    if (st != QK_OK) return st;
    return qk::launch_mul_mat_vec_x8(fmt, w, m, k, x, n, ldx, y, ldy, static_cast<hipStream_t>(stream));
}

int qk_mul_mat_vec_batched(int fmt, const qk_mat_vec_item *items, int count, int64_t n,
                           void *stream) {
    if (!fmt_ok(fmt)) return QK_ERR_UNSUPPORTED;
    if (count < 0 || count > QK_MAX_BATCH || n < 0 || n > 8) return QK_ERR_INVALID_ARG;
    if (count == 0 || n == 0) return QK_OK;
    if (items == nullptr) return QK_ERR_INVALID_ARG;
    for (int i = 0; i < count; ++i) {
        const int st = check_gemv_item(fmt, items[i], n);
        if (st != QK_OK) return st;
    }
    // no output may overlap another item's inputs or output
    for (int i = 0; i < count; ++i) {
        const qk_mat_vec_item &a = items[i];
        if (a.m == 0) continue;
        const size_t ya = span_bytes(n, a.ldy, a.m, 4);
        for (int j = 0; j < count; ++j) {
            const qk_mat_vec_item &b = items[j];
            if (j == i || b.m == 0) continue;
            const size_t wb = (size_t)b.m * (size_t)(b.k / 32) * qk::block_bytes_host(fmt);
            if (overlaps(a.y, ya, b.w, wb) || overlaps(a.y, ya, b.x, span_bytes(n, b.ldx, b.k, 4)) ||
                overlaps(a.y, ya, b.y, span_bytes(n, b.ldy, b.m, 4)))
                return QK_ERR_INVALID_ARG;
        }
    }
    return qk::launch_mul_mat_vec_batched(fmt, items, count, n, static_cast<hipStream_t>(stream));
}

// (n - 1) * ld stays below 2^58, so a sum of a few such spans (and its size
// in bytes) cannot overflow.
static bool span_fits(int64_t n, int64_t ld) {
    return n <= 1 || ld == 0 || (n - 1) <= (int64_t(1) << 58) / ld;
}

// Outputs [p, p+m) at p = i*inner_ld + o*outer_ld (i < inner_n, o < outer_n)
// are pairwise disjoint when each inner run fits inside one outer stride.
static bool nested_disjoint(int64_t m, int64_t inner_n, int64_t inner_ld, int64_t outer_n,
                            int64_t outer_ld) {
    const int64_t inner_span = inner_n > 1 ? (inner_n - 1) * inner_ld + m : m;
    return (inner_n <= 1 || inner_ld >= m) && (outer_n <= 1 || outer_ld >= inner_span);
}

int qk_mul_mat_vec_id(int fmt, const void *w, int64_t n_experts, int64_t expert_stride,
                      int64_t m, int64_t k, const int32_t *ids, int64_t ld_ids,
                      int64_t n_used, int64_t n_tokens, const float *x, int64_t x_slot,
                      int64_t x_tok, float *y, int64_t y_slot, int64_t y_tok, void *stream) {
    if (!fmt_ok(fmt)) return QK_ERR_UNSUPPORTED;
    if (m < 0 || k < 0 || k % 32 != 0 || n_used < 0 || n_tokens < 0) return QK_ERR_INVALID_ARG;
    if (m == 0 || n_used == 0 || n_tokens == 0) return QK_OK;
    if (m > kMaxDim || k > kMaxDim || n_experts < 1 || n_experts > kMaxDim ||
        n_used > kMaxDim || n_tokens > kMaxDim)
        return QK_ERR_INVALID_ARG;
    const int64_t es = n_experts > 1 ? expert_stride : 0;
    const int64_t li = n_tokens > 1 ? ld_ids : 0;
    const int64_t xs = n_used > 1 ? x_slot : 0, xt = n_tokens > 1 ? x_tok : 0;
    const int64_t ys = n_used > 1 ? y_slot : 0, yt = n_tokens > 1 ? y_tok : 0;
    if (es < 0 || li < 0 || xs < 0 || xt < 0 || ys < 0 || yt < 0) return QK_ERR_INVALID_ARG;
    if (!span_fits(n_experts, es) || !span_fits(n_tokens, li) || !span_fits(n_tokens, xt) ||
        !span_fits(n_used, xs) || !span_fits(n_tokens, yt) || !span_fits(n_used, ys))
        return QK_ERR_INVALID_ARG;
    const size_t ebytes = (size_t)m * (size_t)(k / 32) * qk::block_bytes_host(fmt);
    if (n_experts > 1 && (size_t)es < ebytes) return QK_ERR_INVALID_ARG;
    if (n_tokens > 1 && li < n_used) return QK_ERR_INVALID_ARG;
    if (n_used * n_tokens > (int64_t)INT32_MAX / ((m + 7) / 8)) return QK_ERR_INVALID_ARG;
    if (!nested_disjoint(m, n_used, ys, n_tokens, yt) && !nested_disjoint(m, n_tokens, yt, n_used, ys))
        return QK_ERR_INVALID_ARG;
    if (w == nullptr || ids == nullptr || x == nullptr || y == nullptr) return QK_ERR_INVALID_ARG;
    if ((uintptr_t)w % 2 != 0 || es % 2 != 0 || (uintptr_t)ids % 4 != 0 || (uintptr_t)x % 4 != 0 ||
        (uintptr_t)y % 4 != 0)
        return QK_ERR_ALIGNMENT;
    const size_t wbytes = (size_t)(n_experts - 1) * (size_t)es + ebytes;
    const size_t ibytes = (size_t)((n_tokens - 1) * li + n_used) * 4;
    const size_t xbytes = (size_t)((n_tokens - 1) * xt + (n_used - 1) * xs + k) * 4;
    const size_t ybytes = (size_t)((n_tokens - 1) * yt + (n_used - 1) * ys + m) * 4;
    if (overlaps(y, ybytes, w, wbytes) || overlaps(y, ybytes, ids, ibytes) ||
        overlaps(y, ybytes, x, xbytes))
        return QK_ERR_INVALID_ARG;
    return qk::launch_mul_mat_vec_id(fmt, w, n_experts, es, m, k, ids, li, n_used, n_tokens, x,
                                     xs, xt, y, ys, yt, static_cast<hipStream_t>(stream));
}

int qk_mul_mat(int fmt, const void *w, int64_t m, int64_t k, const void *x_f16, int64_t n,
               int64_t ldx, float *y, int64_t ldy, void *stream) {
    if (!fmt_ok(fmt)) return QK_ERR_UNSUPPORTED;
    if (m < 0 || k < 0 || k % 32 != 0 || n < 0) return QK_ERR_INVALID_ARG;
    if (m == 0 || n == 0) return QK_OK;
    if (m > kMaxDim || k > kMaxDim || n > kMaxDim || ldx < k || ldy < m) return QK_ERR_INVALID_ARG;
    // the tile grid is one dimension of 128 x 128 tiles
    if (((m + 127) / 128) * ((n + 127) / 128) > (int64_t)INT32_MAX) return QK_ERR_INVALID_ARG;
    if (y == nullptr || (k > 0 && (w == nullptr || x_f16 == nullptr))) return QK_ERR_INVALID_ARG;
    if ((uintptr_t)w % 2 != 0 || (uintptr_t)x_f16 % 2 != 0 || (uintptr_t)y % 4 != 0)
        return QK_ERR_ALIGNMENT;
    const size_t wbytes = (size_t)m * (size_t)(k / 32) * qk::block_bytes_host(fmt);
    const size_t xbytes = span_bytes(n, ldx, k, 2);
    const size_t ybytes = span_bytes(n, ldy, m, 4);
    if (overlaps(y, ybytes, w, wbytes) || overlaps(y, ybytes, x_f16, xbytes)) return QK_ERR_INVALID_ARG;
    return qk::launch_mul_mat(fmt, w, m, k, static_cast<const uint16_t *>(x_f16), n, ldx, y, ldy,
                              static_cast<hipStream_t>(stream));
}

}  // extern "C"
