// scan4_bf16.hip -- instantiates the four-directions-in-one-launch scan for bf16 storage.
#include "scan_kernel.hpp"

namespace gspn {

template hipError_t launch_fused4<bf16_t>(const Scan4K&, int, int, int, hipStream_t);

}  // namespace gspn
