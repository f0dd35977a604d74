// gemv_n78.hip - instances of the fused quantized GEMV for 7 and 8 column(s)
// (kernels in gemv_impl.h; one file per column count so they build in parallel).
#include "gemv_mfma.h"

namespace qk {

template int gemv_table<7>(int fmt, GemvArgs &a, bool fast, hipStream_t stream);
template int gemv_table<8>(int fmt, GemvArgs &a, bool fast, hipStream_t stream);

}  // namespace qk
