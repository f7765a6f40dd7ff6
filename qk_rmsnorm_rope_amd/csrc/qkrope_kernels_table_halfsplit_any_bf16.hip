// Table-form kernels: half-split pairing with any even rotary_dim (partners through LDS),
// bf16 activations.
#include "qkrope_kernel_impl.h"

namespace qkrope {

hipError_t launch_table_halfsplit_any_bf16(const KernelKey &k, const LaunchShape &s, const KernelArgs &a, hipStream_t st)
{
    return dev::launch_table<kPairHalfAny, kActBF16>(k, s, a, st);
}

}  // namespace qkrope
