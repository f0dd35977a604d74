// gemv_x8_n24.hip - instances of the fused quantized GEMV with 8-bit activations
// for 2, 3, 4 column(s) (kernels in gemv_impl.h).
#include "gemv_impl.h"

namespace qk {

template int gemv_table_x8<2>(int fmt, GemvArgs &a, bool fast, hipStream_t stream);
template int gemv_table_x8<3>(int fmt, GemvArgs &a, bool fast, hipStream_t stream);
template int gemv_table_x8<4>(int fmt, GemvArgs &a, bool fast, hipStream_t stream);

}  // namespace qk
