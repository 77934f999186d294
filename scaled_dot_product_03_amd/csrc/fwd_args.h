// Internal kernel arguments of the attention forward (not part of the C ABI).
#pragma once

#include <stdint.h>

namespace sdpa03 {

enum Mode : int { MODE_DENSE = 0, MODE_COMPACT = 1, MODE_PADDED = 2 };
enum DType : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

// Everything a workgroup needs, passed by value in the kernel-argument
// segment.  Strides are in elements; lse rows are contiguous.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* cu_q;  // device cu_seqlens (varlen modes), else nullptr
  const int32_t* cu_k;
  int64_t q_sb, q_sh, q_ss;
  int64_t k_sb, k_sh, k_ss;
  int64_t v_sb, v_sh, v_ss;
  int64_t o_sb, o_sh, o_ss;
  int64_t lse_sb, lse_sh;
  int32_t seqlen_q;   // dense: Sq; compact: max_seqlen_q; padded: Sq_max
  int32_t seqlen_k;   // dense: Sk; compact: max_seqlen_k; padded: Sk_max
  int32_t total_q;    // rows addressable along seq: compact total_q, else seqlen_q
  int32_t total_k;    // likewise for keys
  int32_t num_heads;
  int32_t num_z;      // batches (dense, padded) or sequences (compact)
  int32_t m_tiles;    // ceil(seqlen_q / block_m)
  float scale_log2;   // scale * log2(e): scores go straight into exp2
  // Additive bias (nullptr: none), same element type as q, indexed like the
  // scores of the rank-4 view: (b, h, row, key) with key stride 1.
  const void* bias;
  int64_t bias_sb, bias_sh, bias_sq;
  float scale;        // the bias is added to scale * q.k before the softmax
  // Key-parallel (split) dense forward only: split s of a query tile covers
  // key tiles [s * split_tiles, (s + 1) * split_tiles) and writes its
  // normalised fp32 partial output and its logsumexp to the workspace.
  int32_t num_splits;     // 1 outside split mode
  int32_t split_tiles;
  float* ws_o;            // [split][z][h][row][head_dim]
  float* ws_lse;          // [split][z][h][row]
  int64_t ws_rows;        // rows per split: num_z * num_heads * seqlen_q
  // Causal launch order (unsplit): (batch or sequence, head) groups per part
  // of an XCD's work; 0 keeps the order without parts.  Set by the launcher.
  int32_t causal_span = 0;
};

// Arguments of the kernel that merges the partial results of a split
// forward into O and LSE.
struct MergeArgs {
  const float* ws_o;
  const float* ws_lse;
  void* o;
  float* lse;
  int64_t o_sb, o_sh, o_ss;
  int64_t lse_sb, lse_sh;
  int64_t ws_rows;
  int32_t num_heads;
  int32_t seqlen_q;
  int32_t num_splits;
};

// One compiled kernel shape.
struct KernelConfig {
  int block_m;
  int block_n;
  int waves;
};

// The compiled kernel shape a launch uses for (dtype, head_dim), the
// sequence extents (seqlen_q and seqlen_k of FwdArgs), the mask and the
// layout (mode); single_group for the split forward (which takes the dense
// non-causal entry for both masks) and the forward with a bias.  False if
// unsupported.
bool kernel_config(int dtype, int head_dim, int seqlen_q, int seqlen_k, bool causal, int mode,
                   bool single_group, KernelConfig* cfg);

// Launches the forward on `stream` (a hipStream_t).  Returns the HIP error
// code of the launch (0 on success).  Arguments are assumed validated.
int launch_attn_fwd(const FwdArgs& args, int dtype, int head_dim, int mode, bool causal,
                    void* stream);

// The same with the additive bias of args.bias (non-null).
int launch_attn_fwd_bias(const FwdArgs& args, int dtype, int head_dim, int mode, bool causal,
                         void* stream);

// Split dense forward: the partial kernel (grid m_tiles * heads * batches *
// splits), then the merge kernel, both on `stream`.
int launch_attn_fwd_split(const FwdArgs& args, const MergeArgs& merge, int dtype, int head_dim,
                          bool causal, void* stream);

}  // namespace sdpa03
