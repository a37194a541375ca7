// scan_bf16_vert.hip -- instantiates the vertical (T2B, B2T) line-scan kernels for bf16 storage with bf16 weights.
#include "scan_kernel.hpp"

namespace gspn {

template hipError_t launch_family<bf16_t, bf16_t, false>(const ScanConfig&, bool, bool, const ScanK&, int64_t,
                                                 int, hipStream_t);

}  // namespace gspn
