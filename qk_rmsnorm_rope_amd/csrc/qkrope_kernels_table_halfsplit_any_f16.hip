// Table-form kernels: half-split pairing with any even rotary_dim (partners through LDS),
// f16 activations.
#include "qkrope_kernel_impl.h"

namespace qkrope {

hipError_t launch_table_halfsplit_any_f16(const KernelKey &k, const LaunchShape &s, const KernelArgs &a, hipStream_t st)
{
    return dev::launch_table<kPairHalfAny, kActF16>(k, s, a, st);
}

}  // namespace qkrope
