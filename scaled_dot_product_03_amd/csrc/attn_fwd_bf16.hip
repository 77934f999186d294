// The bf16 forward kernels: explicit instantiations of the per-type launches
// (with and without a bias) declared in attn_fwd_kernels.h.

#include "attn_fwd_kernels.h"

namespace sdpa03 {

template int launch_fwd_dtype<__bf16, false>(const FwdArgs&, int, int, bool, hipStream_t);
template int launch_fwd_dtype<__bf16, true>(const FwdArgs&, int, int, bool, hipStream_t);

}  // namespace sdpa03
