// gemv_id.hip - instances of the fused quantized GEMV for expert-indexed
// problems (kernels in gemv_impl.h).
#include "gemv_impl.h"

namespace qk {

int gemv_expert(int fmt, const GemvExpert &e, bool fast, hipStream_t stream) {
    switch (fmt) {
    case QK_Q4_0: return gemv_expert_fmt<QK_Q4_0>(e, fast, stream);
    case QK_Q4_1: return gemv_expert_fmt<QK_Q4_1>(e, fast, stream);
    case QK_Q8_0: return gemv_expert_fmt<QK_Q8_0>(e, fast, stream);
    case QK_Q5_0: return gemv_expert_fmt<QK_Q5_0>(e, fast, stream);
    case QK_Q5_1: return gemv_expert_fmt<QK_Q5_1>(e, fast, stream);
    default: return QK_ERR_INVALID_ARG;
    }
}

}  // namespace qk
