// gemv_x8_n58.hip - instances of the fused quantized GEMV with 8-bit activations
// for 5, 6, 7, 8 column(s) (kernels in gemv_impl.h).
#include "gemv_impl.h"

namespace qk {

template int gemv_table_x8<5>(int fmt, GemvArgs &a, bool fast, hipStream_t stream);
template int gemv_table_x8<6>(int fmt, GemvArgs &a, bool fast, hipStream_t stream);
template int gemv_table_x8<7>(int fmt, GemvArgs &a, bool fast, hipStream_t stream);
template int gemv_table_x8<8>(int fmt, GemvArgs &a, bool fast, hipStream_t stream);

}  // namespace qk
