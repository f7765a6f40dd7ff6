// Table-form kernels: halfsplit pairing, f16 activations.
#include "qkrope_kernel_impl.h"

namespace qkrope {

hipError_t launch_table_halfsplit_f16(const KernelKey &k, const LaunchShape &s, const KernelArgs &a, hipStream_t st)
{
    return dev::launch_table<kPairHalf, kActF16>(k, s, a, st);
}

}  // namespace qkrope
