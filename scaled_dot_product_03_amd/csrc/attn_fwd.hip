// Entry of the flash-attention forward launches (plain, with a bias, split;
// the kernels are in attn_fwd_kernels.h, the per-type launches in
// attn_fwd_{bf16,f16,f32}.hip) and the compiled-in kernel choice.

#include "attn_fwd_kernels.h"

namespace sdpa03 {

bool kernel_config(int dtype, int head_dim, int seqlen_q, int seqlen_k, bool causal, int mode,
                   bool single_group, KernelConfig* cfg) {
  if (head_dim != 64 && head_dim != 128) return false;
  const int b = seq_bucket(seqlen_q, seqlen_k);
  const int v = mask_variant(causal, mode);
  auto pick = [&](auto tag) {
    using T = decltype(tag);
    if (head_dim == 64) {
      return single_group ? entry_for<T, 64, true>(b, v) : entry_for<T, 64, false>(b, v);
    }
    return single_group ? entry_for<T, 128, true>(b, v) : entry_for<T, 128, false>(b, v);
  };
  TableEntry e;
  switch (dtype) {
    case DT_F32: e = pick(float{}); break;
    case DT_F16: e = pick(_Float16{}); break;
    case DT_BF16: e = pick(__bf16{}); break;
    default: return false;
  }
  cfg->block_m = block_m_of(e);
  cfg->block_n = e.block_n;
  cfg->waves = e.waves;
  return true;
}

int launch_attn_fwd_split(const FwdArgs& a, const MergeArgs& mg, int dtype, int head_dim,
                          bool causal, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto by_dim = [&](auto tag) {
    using T = decltype(tag);
    if (head_dim == 64) {
      return causal ? launch_split_typed<T, 64, true>(a, mg, s) : launch_split_typed<T, 64, false>(a, mg, s);
    }
    return causal ? launch_split_typed<T, 128, true>(a, mg, s) : launch_split_typed<T, 128, false>(a, mg, s);
  };
  switch (dtype) {
    case DT_F32: return by_dim(float{});
    case DT_F16: return by_dim(_Float16{});
    default: return by_dim(__bf16{});
  }
}

int launch_attn_fwd(const FwdArgs& a, int dtype, int head_dim, int mode, bool causal, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (dtype) {
    case DT_F32: return launch_fwd_dtype<float, false>(a, head_dim, mode, causal, s);
    case DT_F16: return launch_fwd_dtype<_Float16, false>(a, head_dim, mode, causal, s);
    default: return launch_fwd_dtype<__bf16, false>(a, head_dim, mode, causal, s);
  }
}

int launch_attn_fwd_bias(const FwdArgs& a, int dtype, int head_dim, int mode, bool causal,
                         void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (dtype) {
    case DT_F32: return launch_fwd_dtype<float, true>(a, head_dim, mode, causal, s);
    case DT_F16: return launch_fwd_dtype<_Float16, true>(a, head_dim, mode, causal, s);
    default: return launch_fwd_dtype<__bf16, true>(a, head_dim, mode, causal, s);
  }
}

}  // namespace sdpa03
