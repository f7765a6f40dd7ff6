// Per-token Q/K sums of squares of packed QKV (first phase of a head-sharded across-heads norm).
#include "qkrope_kernel_impl.h"

namespace qkrope {

hipError_t launch_sumsq(const SumsqArgs &a, int64_t tokens, int threads, hipStream_t st)
{
    return dev::launch_sumsq_impl(a, tokens, threads, st);
}

}  // namespace qkrope
