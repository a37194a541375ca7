// scan4_bf16.hip -- instantiates the four-scans-in-one-launch kernels for bf16 storage with bf16 weights.
#include "scan_kernel.hpp"
#include "scan_band.hpp"
#include "scan_lp.hpp"

namespace gspn {

template hipError_t launch_fused4<bf16_t, bf16_t>(const Scan4K&, int, int, int, hipStream_t);
template hipError_t launch_fused4v<bf16_t, bf16_t>(const Scan4K&, int, int, int, hipStream_t);
template hipError_t launch_fused4lp<bf16_t, bf16_t, true>(const Scan4K&, int, hipStream_t);
// fp32 states (the backward pass's recomputed forward)
template hipError_t launch_fused4v<bf16_t, bf16_t, float>(const Scan4K&, int, int, int, hipStream_t);
template hipError_t launch_fused4lp<bf16_t, bf16_t, true, float>(const Scan4K&, int, hipStream_t);

// the banded kernel for very few long lines
template hipError_t launch_band4<bf16_t, bf16_t, true>(const BandK&, hipStream_t);
template hipError_t launch_band4<bf16_t, bf16_t, true, float>(const BandK&, hipStream_t);

}  // namespace gspn
