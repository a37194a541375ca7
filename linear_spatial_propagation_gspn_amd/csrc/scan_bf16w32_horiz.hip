// scan_bf16w32_horiz.hip -- instantiates the horizontal (L2R, R2L) line-scan kernels for bf16 storage with fp32 weights.
#include "scan_kernel.hpp"

namespace gspn {

template hipError_t launch_family<bf16_t, float, true>(const ScanConfig&, bool, bool, const ScanK&, int64_t,
                                                 int, hipStream_t);

}  // namespace gspn
