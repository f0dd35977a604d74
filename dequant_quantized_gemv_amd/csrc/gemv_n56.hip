// gemv_n56.hip - instances of the fused quantized GEMV for 5 and 6 column(s)
// (kernels in gemv_impl.h; one file per column count so they build in parallel).
#include "gemv_mfma.h"

namespace qk {

template int gemv_table<5>(int fmt, GemvArgs &a, bool fast, hipStream_t stream);
template int gemv_table<6>(int fmt, GemvArgs &a, bool fast, hipStream_t stream);

}  // namespace qk
