// gemv_n34.hip - instances of the fused quantized GEMV for 3 and 4 column(s)
// (kernels in gemv_impl.h; one file per column count so they build in parallel).
#include "gemv_mfma.h"

namespace qk {

template int gemv_table<3>(int fmt, GemvArgs &a, bool fast, hipStream_t stream);
template int gemv_table<4>(int fmt, GemvArgs &a, bool fast, hipStream_t stream);

}  // namespace qk
