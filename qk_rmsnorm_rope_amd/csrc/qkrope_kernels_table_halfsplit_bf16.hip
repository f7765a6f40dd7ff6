// Table-form kernels: halfsplit pairing, bf16 activations.
#include "qkrope_kernel_impl.h"

namespace qkrope {

hipError_t launch_table_halfsplit_bf16(const KernelKey &k, const LaunchShape &s, const KernelArgs &a, hipStream_t st)
{
    return dev::launch_table<kPairHalf, kActBF16>(k, s, a, st);
}

}  // namespace qkrope
