// Table-form kernels, halfsplit pairing.
#include "qkrope_kernel_impl.h"

namespace qkrope {

hipError_t launch_table_halfsplit(const KernelKey &k, const LaunchShape &s, const KernelArgs &a, hipStream_t st)
{
    return dev::launch_table<true>(k, s, a, st);
}

}  // namespace qkrope
