// gemv_n2.hip - instances of the fused quantized GEMV for 2 column(s)
// (kernels in gemv_impl.h; one file per column count so they build in parallel).
#include "gemv_impl.h"

namespace qk {

template int gemv_table<2>(int fmt, GemvArgs &a, bool fast, hipStream_t stream);

}  // namespace qk
