// gemv_x8_n1.hip - instances of the fused quantized GEMV with 8-bit activations
// for 1 column(s) (kernels in gemv_impl.h).
#include "gemv_impl.h"

namespace qk {

template int gemv_table_x8<1>(int fmt, GemvArgs &a, bool fast, hipStream_t stream);

}  // namespace qk
