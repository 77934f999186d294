// Launcher of the flash-attention forward with an additive bias (the kernels
// are in attn_fwd_kernels.h; a separate translation unit so that the biased
// instantiations compile in parallel with the others).

#include "attn_fwd_kernels.h"

namespace sdpa03 {

int launch_attn_fwd_bias(const FwdArgs& a, int dtype, int head_dim, int mode, bool causal,
                         void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (dtype) {
    case DT_F32: return launch_dim<float, true>(a, head_dim, mode, causal, s);
    case DT_F16: return launch_dim<_Float16, true>(a, head_dim, mode, causal, s);
    default: return launch_dim<__bf16, true>(a, head_dim, mode, causal, s);
  }
}

}  // namespace sdpa03
