// The naive fp16 Flash-Attention exhibit at head_dim 128 (kernels of
// pasa_fwd.hpp), separate from the PASA kernels of that head dim so that the
// build can schedule the two with different compiler options.
#include "pasa_fwd.hpp"

namespace pasa {

hipError_t launch_fwd_d128_naive(const FwdArgs& a, hipStream_t stream) {
    return launch_causal_or_not<128, kVarNaive>(a, stream);
}

}  // namespace pasa
