// scan_f32_vert.hip -- instantiates the vertical (T2B, B2T) line-scan kernels for f32 storage.
#include "scan_kernel.hpp"

namespace gspn {

template hipError_t launch_family<float, false>(const ScanConfig&, bool, const ScanK&, int64_t, int,
                                          hipStream_t);

}  // namespace gspn
