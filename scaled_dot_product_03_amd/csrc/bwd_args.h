// Internal kernel arguments of the attention backward (not part of the C ABI).
#pragma once

#include <stdint.h>

namespace sdpa03 {

// Everything the backward kernels need, passed by value.  Strides are in
// elements; dq, dk and dv use the strides of q, k and v.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  const int32_t* cu_q;  // device cu_seqlens (varlen modes), else nullptr
  const int32_t* cu_k;
  void* dq;
  void* dk;
  void* dv;
  // Workspace: per query row rowsum(dO * O) and LSE * log2(e), laid out
  // [b][h][row] over the rank-4 view's rows with ws_rows_pad rows per
  // (b, h): a multiple of 64 with 64 rows to spare past the last one, so a
  // whole query tile starting at any row can be read without bounds checks.
  float* ws_delta;
  float* ws_lse2;
  int64_t q_sb, q_sh, q_ss;
  int64_t k_sb, k_sh, k_ss;
  int64_t v_sb, v_sh, v_ss;
  int64_t o_sb, o_sh, o_ss;
  int64_t do_sb, do_sh, do_ss;
  int64_t lse_sb, lse_sh;
  int32_t seqlen_q;   // dense: Sq; compact: max_seqlen_q; padded: Sq_max
  int32_t seqlen_k;   // dense: Sk; compact: max_seqlen_k; padded: Sk_max
  int32_t total_q;    // rows of the rank-4 view along seq (compact: total_q)
  int32_t total_k;
  int32_t num_heads;
  int32_t num_b;      // batches of the rank-4 view (1 in compact mode)
  int32_t num_z;      // batches (dense, padded) or sequences (compact)
  int32_t ws_rows_pad;
  int32_t q_tiles;    // query tiles of the dQ kernel
  int32_t k_tiles;    // key tiles of the dK/dV kernel
  float scale;        // dQ and dK carry the softmax scale
  float scale_log2;   // scale * log2(e)
  // Causal launch order: groups per part of an XCD's work for the dQ and
  // the dK/dV kernels (0: no parts).  Set by the launcher.
  int32_t span_q = 0;
  int32_t span_k = 0;
};

// Workspace rows per (b, h) for a rank-4 view of `rows` query rows.
constexpr int64_t bwd_ws_rows_pad(int64_t rows) { return (rows + 63) / 64 * 64 + 64; }

// Query rows per dQ workgroup and keys per dK/dV workgroup.
constexpr int kBwdDqRows = 256;
constexpr int kBwdDkvKeys = 128;

// Launches the two backward kernels (dQ, then dK/dV) on `stream`; returns
// the HIP error of the first launch that fails (0 on success).  Arguments are
// assumed validated; dtype is 16-bit.
int launch_attn_bwd(const BwdArgs& args, int dtype, int head_dim, int mode, bool causal,
                    void* stream);

}  // namespace sdpa03
