// Table-form kernels, interleaved pairing.
#include "qkrope_kernel_impl.h"

namespace qkrope {

hipError_t launch_table_interleaved(const KernelKey &k, const LaunchShape &s, const KernelArgs &a, hipStream_t st)
{
    return dev::launch_table<false>(k, s, a, st);
}

}  // namespace qkrope
