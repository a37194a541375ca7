// scan4_f32.hip -- instantiates the four-scans-in-one-launch kernels for fp32 storage with fp32 weights.
#include "scan_kernel.hpp"
#include "scan_band.hpp"
#include "scan_lp.hpp"

namespace gspn {

template hipError_t launch_fused4<float, float>(const Scan4K&, int, int, int, hipStream_t);
template hipError_t launch_fused4v<float, float>(const Scan4K&, int, int, int, hipStream_t);
template hipError_t launch_fused4lp<float, float, true>(const Scan4K&, int, hipStream_t);
template hipError_t launch_fused4lp<float, float, false>(const Scan4K&, int, hipStream_t);

// the banded kernel for very few long lines
template hipError_t launch_band4<float, float, true>(const BandK&, hipStream_t);
template hipError_t launch_band4<float, float, false>(const BandK&, hipStream_t);

}  // namespace gspn
