// scan_bf16pair_vert.hip -- instantiates the vertical (T2B, B2T) line-scan kernels for bf16 storage with channel-shared weights pre-normalised as packed half pairs.
#include "scan_kernel.hpp"

namespace gspn {

template hipError_t launch_family<bf16_t, WPair, false>(const ScanConfig&, bool, bool, const ScanK&, int64_t,
                                                 int, hipStream_t);

}  // namespace gspn
