// PASA forward (prefill) at head_dim 128: the kernels of pasa_fwd.hpp, in a
// translation unit of their own so that the build can schedule them with
// their own compiler options.
#include "pasa_fwd.hpp"

namespace pasa {

hipError_t launch_fwd_d128(const FwdArgs& a, int variant, hipStream_t stream) {
    return launch_var<128>(a, variant, stream);
}

}  // namespace pasa
