// gemv.hip - host side of the fused quantized GEMV: builds the launch
// descriptors (gemv.h) from validated C-ABI arguments and picks the instance
// by column count.  The kernels are in gemv_impl.h.
#include "gemv.h"
#include "qk_common.h"
#include "qk_internal.h"

#include <algorithm>

namespace qk {

// Outputs of problems with no weights per row (k == 0): the empty sum, 0, or
// NaN where an expert id falls outside the stack.  `e` describes `count`
// columns (slots) of m outputs each; ids == nullptr marks every column valid.
__global__ __launch_bounds__(256) void gemv_empty_kernel(const GemvExpert e, const int64_t total) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total; idx += stride) {
        const int64_t p = idx / e.m;
        const int i = (int)(idx - p * e.m);
        const int t = (int)(p / e.n_used);
        const int s = (int)(p - (int64_t)t * e.n_used);
        bool bad = false;
        if (e.ids != nullptr) {
            const int id = e.ids[(int64_t)t * e.ld_ids + s];
            bad = (unsigned)id >= (unsigned)e.nexp;
        }
        e.y[t * e.y_tok + s * e.y_slot + i] = bad ? __builtin_nanf("") : 0.0f;
    }
}

static int launch_empty(const GemvExpert &e, hipStream_t stream) {
    const int64_t total = (int64_t)e.count * e.m;
    if (total <= 0) return QK_OK;
    const int64_t nwg = std::min<int64_t>((total + 255) / 256, 4096);
    return launch(gemv_empty_kernel, dim3((unsigned)nwg), dim3(256), stream, e, total);
}

static int gemv_by_columns(int fmt, GemvArgs &a, int n, bool fast, hipStream_t stream) {
    switch (n) {
    case 1: return gemv_table<1>(fmt, a, fast, stream);
    case 2: return gemv_table<2>(fmt, a, fast, stream);
    case 3: return gemv_table<3>(fmt, a, fast, stream);
    case 4: return gemv_table<4>(fmt, a, fast, stream);
    case 5: return gemv_table<5>(fmt, a, fast, stream);
    case 6: return gemv_table<6>(fmt, a, fast, stream);
    case 7: return gemv_table<7>(fmt, a, fast, stream);
    case 8: return gemv_table<8>(fmt, a, fast, stream);
    default: return QK_ERR_INVALID_ARG;
    }
}

int launch_mul_mat_vec_batched(int fmt, const qk_mat_vec_item *items, int count, int64_t n,
                               hipStream_t stream) {
    GemvArgs a{};
    bool fast = true;
    int used = 0;
    for (int i = 0; i < count; ++i) {
        const qk_mat_vec_item &src = items[i];
        if (src.m == 0) continue;
        if (src.k == 0) {
            // no weights: every output is the empty sum
            GemvExpert z{};
            z.y = src.y;
            z.y_slot = src.ldy;
            z.m = (int)src.m;
            z.n_used = (int)n;
            z.count = (int)n;
            const int st = launch_empty(z, stream);
            if (st != QK_OK) return st;
            continue;
        }
        GemvItem &d = a.item[used++];
        d.w = static_cast<const uint8_t *>(src.w);
        d.x = src.x;
        d.y = src.y;
        d.ldx = src.ldx;
        d.ldy = src.ldy;
        d.m = (int)src.m;
        d.nb = (int)(src.k / kBlockElems);
        fast = fast && ((uintptr_t)d.w % 4) == 0 && (d.nb % 2) == 0;
    }
    a.count = used;
    if (used == 0) return QK_OK;
    // Longest rows first: items are independent, and a row group of a long
    // row is several steps, so starting those first keeps them from being the
    // stragglers at the end of the launch (insertion sort, at most 16 items,
    // stable so equal lengths keep the caller's order).
    for (int i = 1; i < used; ++i) {
        const GemvItem t = a.item[i];
        int j = i;
        for (; j > 0 && a.item[j - 1].nb < t.nb; --j) a.item[j] = a.item[j - 1];
        a.item[j] = t;
    }
    return gemv_by_columns(fmt, a, (int)n, fast, stream);
}

int launch_mul_mat_vec_x8(int fmt, const void *w, int64_t m, int64_t k, const float *x,
                          int64_t n, int64_t ldx, float *y, int64_t ldy, hipStream_t stream) {
    if (k == 0) {
        // no weights: every output is the empty sum
        GemvExpert z{};
        z.y = y;
        z.y_slot = ldy;
        z.m = (int)m;
        z.n_used = (int)n;
        z.count = (int)n;
        return launch_empty(z, stream);
    }
    GemvArgs a{};
    GemvItem &d = a.item[0];
    d.w = static_cast<const uint8_t *>(w);
    d.x = x;
    d.y = y;
    d.ldx = ldx;
    d.ldy = ldy;
    d.m = (int)m;
    d.nb = (int)(k / kBlockElems);
    a.count = 1;
    const bool fast = ((uintptr_t)d.w % 4) == 0 && (d.nb % 2) == 0;
    switch (n) {
    case 1: return gemv_table_x8<1>(fmt, a, fast, stream);
    case 2: return gemv_table_x8<2>(fmt, a, fast, stream);
    case 3: return gemv_table_x8<3>(fmt, a, fast, stream);
    case 4: return gemv_table_x8<4>(fmt, a, fast, stream);
    case 5: return gemv_table_x8<5>(fmt, a, fast, stream);
    case 6: return gemv_table_x8<6>(fmt, a, fast, stream);
    case 7: return gemv_table_x8<7>(fmt, a, fast, stream);
    case 8: return gemv_table_x8<8>(fmt, a, fast, stream);
    default: return QK_ERR_INVALID_ARG;
    }
}

int launch_mul_mat_vec(int fmt, const void *w, int64_t m, int64_t k, const float *x,
                       int64_t n, int64_t ldx, float *y, int64_t ldy, hipStream_t stream) {
    qk_mat_vec_item item{w, m, k, x, ldx, y, ldy};
    return launch_mul_mat_vec_batched(fmt, &item, 1, n, stream);
}

int launch_mul_mat_vec_id(int fmt, const void *w, int64_t n_experts, int64_t expert_stride,
                          int64_t m, int64_t k, const int32_t *ids, int64_t ld_ids,
                          int64_t n_used, int64_t n_tokens, const float *x, int64_t x_slot,
                          int64_t x_tok, float *y, int64_t y_slot, int64_t y_tok,
                          hipStream_t stream) {
    GemvExpert e{};
    e.w = static_cast<const uint8_t *>(w);
    e.estride = n_experts > 1 ? expert_stride : 0;
    e.ids = ids;
    e.ld_ids = n_tokens > 1 ? ld_ids : 0;
    e.x = x;
    e.x_slot = n_used > 1 ? x_slot : 0;
    e.x_tok = n_tokens > 1 ? x_tok : 0;
    e.y = y;
    e.y_slot = n_used > 1 ? y_slot : 0;
    e.y_tok = n_tokens > 1 ? y_tok : 0;
    e.m = (int)m;
    e.nb = (int)(k / kBlockElems);
    e.nexp = (int)n_experts;
    e.n_used = (int)n_used;
    e.count = (int)(n_used * n_tokens);
    if (e.nb == 0) return launch_empty(e, stream);
    const bool fast = (uintptr_t)e.w % 4 == 0 && e.estride % 4 == 0 && e.nb % 2 == 0;
    return gemv_expert(fmt, e, fast, stream);
}

}  // namespace qk
