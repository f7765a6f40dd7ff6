// 3D-form kernels with head_dim 256 (one translation unit per head_dim, built in parallel).
#include "qkrope_kernel_impl.h"

namespace qkrope {

hipError_t launch_3d_d256(const KernelKey &k, const LaunchShape &s, const KernelArgs &a, hipStream_t st)
{
    return dev::launch_3d<256>(k, s, a, st);
}

}  // namespace qkrope
