// scan_bf16pair_horiz.hip -- instantiates the horizontal (L2R, R2L) line-scan kernels for bf16 storage with channel-shared weights pre-normalised as packed half pairs.
#include "scan_kernel.hpp"

namespace gspn {

template hipError_t launch_family<bf16_t, WPair, true>(const ScanConfig&, bool, bool, const ScanK&, int64_t,
                                                 int, hipStream_t);

}  // namespace gspn
