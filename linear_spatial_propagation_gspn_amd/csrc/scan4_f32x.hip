// scan4_f32x.hip -- instantiates the long-line four-direction kernel for fp32
// storage whose horizontal directions read x through LDS column tiles.
#include "scan_kernel.hpp"
#include "scan_lp.hpp"

namespace gspn {

template hipError_t launch_fused4lp<float, float, true, float, true>(const Scan4K&, int, hipStream_t);
template hipError_t launch_fused4lp<float, float, false, float, true>(const Scan4K&, int, hipStream_t);

}  // namespace gspn
