// Launchers of the plain and split flash-attention forward (the kernels are
// in attn_fwd_kernels.h) and the compiled-in kernel choice.

#include "attn_fwd_kernels.h"

namespace sdpa03 {

bool kernel_config(int dtype, int head_dim, bool causal, int mode, KernelConfig* cfg) {
  (void)causal;
  (void)mode;
  if (head_dim != 64 && head_dim != 128) return false;
  TableEntry e;
  switch (dtype) {
    case DT_F32: e = head_dim == 64 ? table_entry<float, 64>() : table_entry<float, 128>(); break;
    case DT_F16: e = head_dim == 64 ? table_entry<_Float16, 64>() : table_entry<_Float16, 128>(); break;
    case DT_BF16: e = head_dim == 64 ? table_entry<__bf16, 64>() : table_entry<__bf16, 128>(); break;
    default: return false;
  }
  cfg->block_m = e.waves * 32;
  cfg->block_n = e.block_n;
  cfg->waves = e.waves;
  return true;
}

bool split_kernel_config(int dtype, int head_dim, KernelConfig* cfg) {
  if (head_dim != 64 && head_dim != 128) return false;
  TableEntry e;
  switch (dtype) {
    case DT_F32: e = head_dim == 64 ? single_group_entry<float, 64>() : single_group_entry<float, 128>(); break;
    case DT_F16: e = head_dim == 64 ? single_group_entry<_Float16, 64>() : single_group_entry<_Float16, 128>(); break;
    case DT_BF16: e = head_dim == 64 ? single_group_entry<__bf16, 64>() : single_group_entry<__bf16, 128>(); break;
    default: return false;
  }
  cfg->block_m = e.waves * 32;
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
    case DT_F32: return launch_dim<float, false>(a, head_dim, mode, causal, s);
    case DT_F16: return launch_dim<_Float16, false>(a, head_dim, mode, causal, s);
    default: return launch_dim<__bf16, false>(a, head_dim, mode, causal, s);
  }
}

}  // namespace sdpa03
