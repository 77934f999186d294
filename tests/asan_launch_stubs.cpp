// Stand-ins for the kernel launchers and the dispatch table, linked with an
// AddressSanitizer build of the host code in api.cpp (tests/test_host_asan.py).
// They touch no memory and launch nothing: the validation paths of the C ABI
// run under the sanitizer without a GPU and without compiling the kernels.
// Every launch reports success; the kernel shape is one fixed tile for every
// supported (dtype, head_dim), so only the argument checks are exercised.
#include "bwd_args.h"
#include "fwd_args.h"

namespace sdpa03 {

bool kernel_config(int dtype, int head_dim, int, int, bool, int, bool, KernelConfig* cfg) {
  if (dtype != DT_F32 && dtype != DT_F16 && dtype != DT_BF16) return false;
  if (head_dim != 64 && head_dim != 128) return false;
  cfg->block_m = 128;
  cfg->block_n = 64;
  cfg->waves = 4;
  return true;
}

int launch_attn_fwd(const FwdArgs&, int, int, int, bool, void*) { return 0; }

int launch_attn_fwd_bias(const FwdArgs&, int, int, int, bool, void*) { return 0; }

int launch_attn_fwd_split(const FwdArgs&, const MergeArgs&, int, int, bool, void*) { return 0; }

int launch_attn_bwd(const BwdArgs&, int, int, int, bool, void*) { return 0; }

}  // namespace sdpa03
