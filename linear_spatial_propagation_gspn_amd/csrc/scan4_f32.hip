// scan4_f32.hip -- instantiates the four-directions-in-one-launch scan for f32 storage.
#include "scan_kernel.hpp"

namespace gspn {

template hipError_t launch_fused4<float>(const Scan4K&, int, int, int, hipStream_t);

}  // namespace gspn
