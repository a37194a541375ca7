// project.hip -- the 1x1 projection between channel spaces (GSPN-2 notes,
// "Optimisation 2", compressive channel proxy):
//   out[n][o][p] = sum_c weight[o][c] * in[n][c][p]   (no bias, fp32 accumulate)
//
// Generic VALU kernel: one lane per pixel, OB output channels accumulated in
// registers per pass over the input channels.  The weight index is uniform
// across the wavefront, so weights come through the scalar cache.
#include "device.hpp"
#include "launch.hpp"

namespace gspn {
namespace {

template <typename T, int OB>
__global__ __launch_bounds__(256) void project_kernel(const T* __restrict__ in, const T* __restrict__ wt,
                                                      T* __restrict__ out, int64_t n, int64_t cin,
                                                      int64_t hw, int64_t cout) {
    const int64_t total = n * hw;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
         e += stride) {
        const int64_t ni = e / hw;
        const int64_t pix = e - ni * hw;
        const T* src = in + ni * cin * hw + pix;
        T* dst = out + ni * cout * hw + pix;
        for (int64_t o0 = 0; o0 < cout; o0 += OB) {
            float acc[OB];
#pragma unroll
            for (int oo = 0; oo < OB; ++oo) acc[oo] = 0.0f;
            for (int64_t ci = 0; ci < cin; ++ci) {
                const float v = Store<T>::ld(src + ci * hw);
#pragma unroll
                for (int oo = 0; oo < OB; ++oo) {
                    if (o0 + oo < cout)
                        acc[oo] = __builtin_fmaf(Store<T>::ld(wt + (o0 + oo) * cin + ci), v, acc[oo]);
                }
            }
#pragma unroll
            for (int oo = 0; oo < OB; ++oo)
                if (o0 + oo < cout) Store<T>::st(dst + (o0 + oo) * hw, acc[oo]);
        }
    }
}

}  // namespace

hipError_t launch_project(int64_t n, int64_t c_in, int64_t hw, int64_t c_out, const void* in,
                          const void* weight, void* out, int dtype, hipStream_t stream) {
    const int64_t total = n * hw;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 256 * 32) blocks = 256 * 32;
    if (blocks < 1) blocks = 1;
    const dim3 grid(static_cast<unsigned>(blocks));
    if (dtype == kF32) {
        hipLaunchKernelGGL((project_kernel<float, 8>), grid, dim3(256), 0, stream,
                           static_cast<const float*>(in), static_cast<const float*>(weight),
                           static_cast<float*>(out), n, c_in, hw, c_out);
    } else {
        hipLaunchKernelGGL((project_kernel<bf16_t, 8>), grid, dim3(256), 0, stream,
                           static_cast<const bf16_t*>(in), static_cast<const bf16_t*>(weight),
                           static_cast<bf16_t*>(out), n, c_in, hw, c_out);
    }
    return hipGetLastError();
}

}  // namespace gspn
