// qk_internal.h - launchers behind the C ABI (validated arguments only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <tuple>
#include <utility>

#include "qk.h"

namespace qk {

// Launch a kernel with hipLaunchKernel and map the runtime's answer to a
// status code (no global error state is read or cleared).
template <typename... KArgs, typename... Args>
inline int launch_lds(void (*kern)(KArgs...), dim3 grid, dim3 block, size_t lds_bytes,
                      hipStream_t stream, Args... args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "kernel arity");
    std::tuple<KArgs...> vals(static_cast<KArgs>(args)...);
    void *argv[sizeof...(KArgs)];
    std::apply([&](auto &...v) {
        int i = 0;
        ((argv[i++] = static_cast<void *>(&v)), ...);
    }, vals);
    const hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(kern), grid, block,
                                         argv, lds_bytes, stream);
    return e == hipSuccess ? QK_OK : QK_ERR_LAUNCH;
}

template <typename... KArgs, typename... Args>
inline int launch(void (*kern)(KArgs...), dim3 grid, dim3 block, hipStream_t stream,
                  Args... args) {
    return launch_lds(kern, grid, block, 0, stream, args...);
}

// Compute units of the current device (256 on MI355X if the query fails),
// queried once per device and kept (launch shapes ask for it on every call).
inline int device_cus() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cached[kMaxDevices] = {};
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (dev >= 0 && dev < kMaxDevices && (v = cached[dev].load(std::memory_order_relaxed)) > 0) return v;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) return 256;
    if (dev >= 0 && dev < kMaxDevices) cached[dev].store(v, std::memory_order_relaxed);
    return v;
}

int launch_dequantize(int fmt, const void *w, int64_t nblocks, int out_dtype, void *out,
                      hipStream_t stream);

int launch_mul_mat_vec(int fmt, const void *w, int64_t m, int64_t k, const float *x,
                       int64_t n, int64_t ldx, float *y, int64_t ldy, hipStream_t stream);

int launch_mul_mat_vec_x8(int fmt, const void *w, int64_t m, int64_t k, const float *x,
                          int64_t n, int64_t ldx, float *y, int64_t ldy, hipStream_t stream);

int launch_mul_mat_vec_batched(int fmt, const qk_mat_vec_item *items, int count, int64_t n,
                               hipStream_t stream);

int launch_mul_mat_vec_id(int fmt, const void *w, int64_t n_experts, int64_t expert_stride,
                          int64_t m, int64_t k, const int32_t *ids, int64_t ld_ids,
                          int64_t n_used, int64_t n_tokens, const float *x, int64_t x_slot,
                          int64_t x_tok, float *y, int64_t y_slot, int64_t y_tok,
                          hipStream_t stream);

int launch_mul_mat(int fmt, const void *w, int64_t m, int64_t k, const uint16_t *x,
                   int64_t n, int64_t ldx, float *y, int64_t ldy, hipStream_t stream);

}  // namespace qk
