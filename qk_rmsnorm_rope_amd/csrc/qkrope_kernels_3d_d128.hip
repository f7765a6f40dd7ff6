// 3D-form kernels with head_dim 128 (one translation unit per head_dim, built in parallel).
#include "qkrope_kernel_impl.h"

namespace qkrope {

hipError_t launch_3d_d128(const KernelKey &k, const LaunchShape &s, const KernelArgs &a, hipStream_t st)
{
    return dev::launch_3d<128>(k, s, a, st);
}

}  // namespace qkrope
