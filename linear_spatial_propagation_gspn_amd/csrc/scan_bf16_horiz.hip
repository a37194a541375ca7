// scan_bf16_horiz.hip -- instantiates the horizontal (L2R, R2L) line-scan kernels for bf16 storage with bf16 weights.
#include "scan_kernel.hpp"

namespace gspn {

template hipError_t launch_family<bf16_t, bf16_t, true>(const ScanConfig&, bool, bool, const ScanK&, int64_t,
                                                 int, hipStream_t);

}  // namespace gspn
