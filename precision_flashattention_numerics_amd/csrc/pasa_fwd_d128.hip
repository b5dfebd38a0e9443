// PASA forward (prefill) at head_dim 128: the kernels of pasa_fwd.hpp, in a
// translation unit of their own so that the build can schedule them with
// their own compiler options.  The naive fp16 exhibit at this head dim is in
// pasa_fwd_d128_naive.hip, built with the default options.
#include "pasa_fwd.hpp"

namespace pasa {

hipError_t launch_fwd_d128(const FwdArgs& a, int variant, hipStream_t stream) {
    if (variant == kVarNaive) return launch_fwd_d128_naive(a, stream);
    if (variant == kVarStrict) return launch_causal_or_not<128, kVarStrict>(a, stream);
    if (variant == kVarFp8) return launch_causal_or_not<128, kVarFp8>(a, stream);
    return launch_causal_or_not<128, kVarPasa>(a, stream);
}

}  // namespace pasa
