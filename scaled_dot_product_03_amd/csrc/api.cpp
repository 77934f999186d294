// C-ABI entry points of libsdpa03.so: argument validation on the host, then
// one kernel launch.  The declarations and the contract are in sdpa03.h.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "../../include/sdpa03.h"
#include "bwd_args.h"
#include "fwd_args.h"

// Scratch of attn_fwd_splitk_noalloc, for callers that cannot allocate: the
// split forward's partial outputs and logsumexps.  Every GPU the library
// runs on holds its own copy from the first call there until the process
// ends.  In host code `scratch` is only the handle hipGetSymbolAddress
// resolves (scratch_address below); kernels get the per-device address it
// returns, never the name.
static __device__ __align__(256) unsigned char scratch[SDPA_NOALLOC_SCRATCH_BYTES];

namespace {

using sdpa03::FwdArgs;

constexpr int64_t kMaxGrid = (int64_t(1) << 32) / 256 - 1;  // workgroups per launch

int elem_size(sdpa_dtype dt) { return dt == SDPA_F32 ? 4 : 2; }

bool dtype_ok(int dt) { return dt == SDPA_F32 || dt == SDPA_F16 || dt == SDPA_BF16; }

// One rank-4 view: (batch, head, seq, dim) sizes and element strides.
struct View {
  const void* ptr;
  int64_t size[4];
  const int64_t* stride;
};

// Largest element offset the view can reach, or -1 on overflow.
int64_t max_offset(const View& v) {
  int64_t off = 0;
  for (int i = 0; i < 4; ++i) {
    if (v.size[i] == 0) return 0;
    const int64_t span = v.size[i] - 1;
    if (v.stride[i] != 0 && span > INT64_MAX / 4 / v.stride[i]) return -1;
    off += span * v.stride[i];
    if (off > INT64_MAX / 4) return -1;
  }
  return off;
}

// K and V tiles are fetched with 32-bit buffer offsets of up to 64 rows:
// their row stride is limited to 16 MiB.
constexpr int64_t kMaxKvRowBytes = int64_t(1) << 24;

sdpa_status check_view(const View& v, int esize, bool key_side) {
  if (v.stride == nullptr) return SDPA_ERR_NULL;
  if (v.ptr == nullptr) return SDPA_OK;  // empty tensor (checked by check_pointers)
  if (v.stride[3] != 1) return SDPA_ERR_STRIDE;
  if (v.size[2] > 1 && v.stride[2] < v.size[3]) return SDPA_ERR_STRIDE;  // rows must not overlap
  if (key_side && v.stride[2] * esize > kMaxKvRowBytes) return SDPA_ERR_STRIDE;
  for (int i = 0; i < 3; ++i) {
    if (v.stride[i] < 0) return SDPA_ERR_STRIDE;
    if ((v.stride[i] * esize) % 16 != 0) return SDPA_ERR_ALIGN;
  }
  if (reinterpret_cast<uintptr_t>(v.ptr) % 16 != 0) return SDPA_ERR_ALIGN;
  if (max_offset(v) < 0) return SDPA_ERR_STRIDE;
  return SDPA_OK;
}

// Shared checks of dtype, head_dim and scale.
sdpa_status check_common(int dtype, int32_t head_dim, float scale) {
  if (!dtype_ok(dtype)) return SDPA_ERR_DTYPE;
  if (head_dim != 64 && head_dim != 128) return SDPA_ERR_HEAD_DIM;
  if (!(isfinite(scale) && scale > 0.f)) return SDPA_ERR_SCALE;
  return SDPA_OK;
}

// q, o and lse are always required; k and v only when they hold any row
// (an empty key axis is legal and its pointers are never dereferenced).
sdpa_status check_pointers(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, int64_t key_rows) {
  if (!q || !o || !lse) return SDPA_ERR_NULL;
  if (key_rows > 0 && (!k || !v)) return SDPA_ERR_NULL;
  return SDPA_OK;
}

void set_strides(const int64_t* s, int64_t& sb, int64_t& sh, int64_t& ss) {
  sb = s[0];
  sh = s[1];
  ss = s[2];
}

// Argument checks and kernel arguments of a dense call (attn_fwd and the
// split forward).  *empty is set when there is no query row to produce.
sdpa_status dense_args(const void* q, const void* k, const void* v, void* o, float* lse,
                       sdpa_dtype dtype, int32_t B, int32_t H, int32_t seqlen_q, int32_t seqlen_k,
                       int32_t head_dim, const int64_t q_stride[4], const int64_t k_stride[4],
                       const int64_t v_stride[4], const int64_t o_stride[4], float scale,
                       FwdArgs* a, bool* empty) {
  *empty = false;
  sdpa_status st = check_common(dtype, head_dim, scale);
  if (st != SDPA_OK) return st;
  if (B < 0 || H < 0 || seqlen_q < 0 || seqlen_k < 0) return SDPA_ERR_SHAPE;
  if (static_cast<int64_t>(B) * H * seqlen_q == 0) {
    *empty = true;
    return SDPA_OK;
  }
  if ((st = check_pointers(q, k, v, o, lse, seqlen_k)) != SDPA_OK) return st;
  const int es = elem_size(dtype);
  const View vq{q, {B, H, seqlen_q, head_dim}, q_stride};
  const View vk{k, {B, H, seqlen_k, head_dim}, k_stride};
  const View vv{v, {B, H, seqlen_k, head_dim}, v_stride};
  const View vo{o, {B, H, seqlen_q, head_dim}, o_stride};
  if ((st = check_view(vq, es, false)) != SDPA_OK || (st = check_view(vk, es, true)) != SDPA_OK ||
      (st = check_view(vv, es, true)) != SDPA_OK || (st = check_view(vo, es, false)) != SDPA_OK)
    return st;
  if (reinterpret_cast<uintptr_t>(lse) % 4 != 0) return SDPA_ERR_ALIGN;

  *a = FwdArgs{};
  a->q = q; a->k = k; a->v = v; a->o = o; a->lse = lse;
  a->cu_q = nullptr; a->cu_k = nullptr;
  set_strides(q_stride, a->q_sb, a->q_sh, a->q_ss);
  set_strides(k_stride, a->k_sb, a->k_sh, a->k_ss);
  set_strides(v_stride, a->v_sb, a->v_sh, a->v_ss);
  set_strides(o_stride, a->o_sb, a->o_sh, a->o_ss);
  a->lse_sh = seqlen_q;
  a->lse_sb = static_cast<int64_t>(H) * seqlen_q;
  a->seqlen_q = seqlen_q;
  a->seqlen_k = seqlen_k;
  a->total_q = seqlen_q;
  a->total_k = seqlen_k;
  a->num_heads = H;
  a->num_z = B;
  a->scale_log2 = scale * 1.4426950408889634f;
  a->scale = scale;
  a->num_splits = 1;
  return SDPA_OK;
}

// The bias view (num_b, H, rows_q, rows_k), read-only: key stride 1, other
// strides >= 0 (0 broadcasts) and multiples of 4 elements, base 16-byte
// aligned, every offset within 64-bit addressing.
sdpa_status check_bias(const void* bias, int64_t num_b, int64_t H, int64_t rows_q,
                       int64_t rows_k, const int64_t* stride, int esize) {
  if (bias == nullptr || stride == nullptr) return SDPA_ERR_NULL;
  if (stride[3] != 1) return SDPA_ERR_STRIDE;
  for (int i = 0; i < 3; ++i) {
    if (stride[i] < 0) return SDPA_ERR_STRIDE;
    if (stride[i] % 4 != 0) return SDPA_ERR_ALIGN;
  }
  if (reinterpret_cast<uintptr_t>(bias) % 16 != 0) return SDPA_ERR_ALIGN;
  const View vb{bias, {num_b, H, rows_q, rows_k}, stride};
  if (max_offset(vb) < 0 || max_offset(vb) > INT64_MAX / esize) return SDPA_ERR_STRIDE;
  return SDPA_OK;
}

void set_bias(FwdArgs& a, const void* bias, const int64_t* stride) {
  a.bias = bias;
  a.bias_sb = stride[0];
  a.bias_sh = stride[1];
  a.bias_sq = stride[2];
}

// Key ranges of a split forward and the workspace they need.  The library
// aims at two workgroups per compute unit of a 256-CU MI355X and at least
// kMinTilesPerSplit key tiles per range; the key tiles are then dealt out
// evenly (every range but possibly the last gets split_tiles tiles).
constexpr int64_t kSplitTargetWorkgroups = 512;
constexpr int64_t kMinTilesPerSplit = 4;
constexpr int64_t kMaxSplits = 256;

struct SplitPlan {
  int32_t splits;
  int32_t split_tiles;
  int32_t m_tiles;
  int64_t rows;       // B * H * seqlen_q
  uint64_t o_bytes;   // partial outputs, padded to 256 bytes
  uint64_t bytes;     // o_bytes + partial logsumexps
};

sdpa_status split_plan(int dtype, int32_t B, int32_t H, int32_t seqlen_q, int32_t seqlen_k,
                       int32_t head_dim, int32_t request, SplitPlan* p) {
  if (!dtype_ok(dtype)) return SDPA_ERR_DTYPE;
  if (head_dim != 64 && head_dim != 128) return SDPA_ERR_HEAD_DIM;
  if (B < 0 || H < 0 || seqlen_q < 0 || seqlen_k < 0) return SDPA_ERR_SHAPE;
  sdpa03::KernelConfig cfg;
  if (!sdpa03::kernel_config(dtype, head_dim, seqlen_q, seqlen_k, false, sdpa03::MODE_DENSE, true,
                             &cfg))
    return SDPA_ERR_HEAD_DIM;
  const int64_t key_tiles = (static_cast<int64_t>(seqlen_k) + cfg.block_n - 1) / cfg.block_n;
  const int64_t m_tiles = (static_cast<int64_t>(seqlen_q) + cfg.block_m - 1) / cfg.block_m;
  const int64_t base = m_tiles * H * B;
  int64_t splits;
  if (request <= 0) {
    splits = base > 0 ? (kSplitTargetWorkgroups + base - 1) / base : 1;
    splits = std::min(splits, std::max<int64_t>(1, key_tiles / kMinTilesPerSplit));
  } else {
    splits = std::min<int64_t>(request, std::max<int64_t>(1, key_tiles));
  }
  splits = std::max<int64_t>(1, std::min(splits, kMaxSplits));
  int64_t split_tiles = 1;
  if (key_tiles > 0) {
    split_tiles = (key_tiles + splits - 1) / splits;
    splits = (key_tiles + split_tiles - 1) / split_tiles;  // no range left empty
  }
  const int64_t rows = static_cast<int64_t>(B) * H * seqlen_q;
  if (rows > (int64_t(1) << 40) / (splits * (head_dim + 1))) return SDPA_ERR_SHAPE;
  if (base * splits > kMaxGrid) return SDPA_ERR_SHAPE;
  p->splits = static_cast<int32_t>(splits);
  p->split_tiles = static_cast<int32_t>(split_tiles);
  p->m_tiles = static_cast<int32_t>(m_tiles);
  p->rows = rows;
  p->o_bytes = (static_cast<uint64_t>(splits * rows * head_dim) * 4 + 255) / 256 * 256;
  p->bytes = p->o_bytes + static_cast<uint64_t>(splits * rows) * 4;
  return SDPA_OK;
}

// Argument checks and kernel arguments of a compact varlen call.
sdpa_status compact_args(const void* q, const void* k, const void* v, void* o, float* lse,
                         sdpa_dtype dtype, int32_t B, int32_t H, int32_t total_q, int32_t total_k,
                         int32_t head_dim, const int32_t* cu_seqlens_q,
                         const int32_t* cu_seqlens_k, int32_t num_seqs, int32_t max_seqlen_q,
                         int32_t max_seqlen_k, const int64_t q_stride[4],
                         const int64_t k_stride[4], const int64_t v_stride[4],
                         const int64_t o_stride[4], float scale, FwdArgs* a, bool* empty) {
  *empty = false;
  sdpa_status st = check_common(dtype, head_dim, scale);
  if (st != SDPA_OK) return st;
  if (B != 1) return SDPA_ERR_BATCH;
  if (H < 0 || total_q < 0 || total_k < 0) return SDPA_ERR_SHAPE;
  if (num_seqs < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || max_seqlen_q > total_q ||
      max_seqlen_k > total_k)
    return SDPA_ERR_SEQLEN;
  if (static_cast<int64_t>(H) * num_seqs * max_seqlen_q == 0) {
    *empty = true;
    return SDPA_OK;
  }
  if ((st = check_pointers(q, k, v, o, lse, total_k)) != SDPA_OK) return st;
  if (!cu_seqlens_q || !cu_seqlens_k) return SDPA_ERR_NULL;
  const int es = elem_size(dtype);
  const View vq{q, {1, H, total_q, head_dim}, q_stride};
  const View vk{k, {1, H, total_k, head_dim}, k_stride};
  const View vv{v, {1, H, total_k, head_dim}, v_stride};
  const View vo{o, {1, H, total_q, head_dim}, o_stride};
  if ((st = check_view(vq, es, false)) != SDPA_OK || (st = check_view(vk, es, true)) != SDPA_OK ||
      (st = check_view(vv, es, true)) != SDPA_OK || (st = check_view(vo, es, false)) != SDPA_OK)
    return st;
  if (reinterpret_cast<uintptr_t>(lse) % 4 != 0) return SDPA_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(cu_seqlens_q) % 4 != 0 ||
      reinterpret_cast<uintptr_t>(cu_seqlens_k) % 4 != 0)
    return SDPA_ERR_ALIGN;

  *a = FwdArgs{};
  a->q = q; a->k = k; a->v = v; a->o = o; a->lse = lse;
  a->cu_q = cu_seqlens_q; a->cu_k = cu_seqlens_k;
  set_strides(q_stride, a->q_sb, a->q_sh, a->q_ss);
  set_strides(k_stride, a->k_sb, a->k_sh, a->k_ss);
  set_strides(v_stride, a->v_sb, a->v_sh, a->v_ss);
  set_strides(o_stride, a->o_sb, a->o_sh, a->o_ss);
  a->lse_sh = total_q;
  a->lse_sb = static_cast<int64_t>(H) * total_q;
  a->seqlen_q = max_seqlen_q;
  a->seqlen_k = max_seqlen_k;
  a->total_q = total_q;
  a->total_k = total_k;
  a->num_heads = H;
  a->num_z = num_seqs;
  a->scale_log2 = scale * 1.4426950408889634f;
  a->scale = scale;
  a->num_splits = 1;
  return SDPA_OK;
}

// Argument checks and kernel arguments of a padded varlen call.
sdpa_status padded_args(const void* q, const void* k, const void* v, void* o, float* lse,
                        sdpa_dtype dtype, int32_t B, int32_t H, int32_t seqlen_q_max,
                        int32_t seqlen_k_max, int32_t head_dim, const int32_t* cu_seqlens_q,
                        const int32_t* cu_seqlens_k, const int64_t q_stride[4],
                        const int64_t k_stride[4], const int64_t v_stride[4],
                        const int64_t o_stride[4], float scale, FwdArgs* a, bool* empty) {
  *empty = false;
  sdpa_status st = check_common(dtype, head_dim, scale);
  if (st != SDPA_OK) return st;
  if (B < 0 || H < 0 || seqlen_q_max < 0 || seqlen_k_max < 0) return SDPA_ERR_SHAPE;
  if (static_cast<int64_t>(B) * H * seqlen_q_max == 0) {
    *empty = true;
    return SDPA_OK;
  }
  if ((st = check_pointers(q, k, v, o, lse, seqlen_k_max)) != SDPA_OK) return st;
  if (!cu_seqlens_q || !cu_seqlens_k) return SDPA_ERR_NULL;
  const int es = elem_size(dtype);
  const View vq{q, {B, H, seqlen_q_max, head_dim}, q_stride};
  const View vk{k, {B, H, seqlen_k_max, head_dim}, k_stride};
  const View vv{v, {B, H, seqlen_k_max, head_dim}, v_stride};
  const View vo{o, {B, H, seqlen_q_max, head_dim}, o_stride};
  if ((st = check_view(vq, es, false)) != SDPA_OK || (st = check_view(vk, es, true)) != SDPA_OK ||
      (st = check_view(vv, es, true)) != SDPA_OK || (st = check_view(vo, es, false)) != SDPA_OK)
    return st;
  if (reinterpret_cast<uintptr_t>(lse) % 4 != 0) return SDPA_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(cu_seqlens_q) % 4 != 0 ||
      reinterpret_cast<uintptr_t>(cu_seqlens_k) % 4 != 0)
    return SDPA_ERR_ALIGN;

  *a = FwdArgs{};
  a->q = q; a->k = k; a->v = v; a->o = o; a->lse = lse;
  a->cu_q = cu_seqlens_q; a->cu_k = cu_seqlens_k;
  set_strides(q_stride, a->q_sb, a->q_sh, a->q_ss);
  set_strides(k_stride, a->k_sb, a->k_sh, a->k_ss);
  set_strides(v_stride, a->v_sb, a->v_sh, a->v_ss);
  set_strides(o_stride, a->o_sb, a->o_sh, a->o_ss);
  a->lse_sh = seqlen_q_max;
  a->lse_sb = static_cast<int64_t>(H) * seqlen_q_max;
  a->seqlen_q = seqlen_q_max;
  a->seqlen_k = seqlen_k_max;
  a->total_q = seqlen_q_max;
  a->total_k = seqlen_k_max;
  a->num_heads = H;
  a->num_z = B;
  a->scale_log2 = scale * 1.4426950408889634f;
  a->scale = scale;
  a->num_splits = 1;
  return SDPA_OK;
}

// The two launches of a split forward whose arguments are validated and
// whose workspace (partial outputs, then partial logsumexps, as the plan
// lays them out) is at `workspace`.
sdpa_status launch_split(FwdArgs& a, const SplitPlan& p, void* workspace, void* o, float* lse,
                         sdpa_dtype dtype, int32_t H, int32_t seqlen_q, int32_t head_dim,
                         int32_t causal, void* stream) {
  a.m_tiles = p.m_tiles;
  a.num_splits = p.splits;
  a.split_tiles = p.split_tiles;
  a.ws_o = static_cast<float*>(workspace);
  a.ws_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.o_bytes);
  a.ws_rows = p.rows;
  sdpa03::MergeArgs mg{};
  mg.ws_o = a.ws_o;
  mg.ws_lse = a.ws_lse;
  mg.o = o;
  mg.lse = lse;
  mg.o_sb = a.o_sb;
  mg.o_sh = a.o_sh;
  mg.o_ss = a.o_ss;
  mg.lse_sb = a.lse_sb;
  mg.lse_sh = a.lse_sh;
  mg.ws_rows = p.rows;
  mg.num_heads = H;
  mg.seqlen_q = seqlen_q;
  mg.num_splits = p.splits;
  const int err = sdpa03::launch_attn_fwd_split(a, mg, dtype, head_dim, causal != 0, stream);
  return err == 0 ? SDPA_OK : SDPA_ERR_HIP;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_addr[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up once per
// device (that device current) on its first call.  The stream must belong to
// the current device.
sdpa_status scratch_address(void* stream, void** addr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SDPA_ERR_HIP;
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess || sdev != dev)
      return SDPA_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return SDPA_ERR_HIP;
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return SDPA_OK;
}

sdpa_status finish_and_launch(FwdArgs& a, sdpa_dtype dtype, int32_t head_dim, int mode,
                              int32_t causal, void* stream) {
  sdpa03::KernelConfig cfg;
  if (!sdpa03::kernel_config(dtype, head_dim, a.seqlen_q, a.seqlen_k, causal != 0, mode,
                             a.bias != nullptr, &cfg))
    return SDPA_ERR_HEAD_DIM;
  const int64_t m_tiles = (static_cast<int64_t>(a.seqlen_q) + cfg.block_m - 1) / cfg.block_m;
  const int64_t grid = m_tiles * a.num_heads * static_cast<int64_t>(a.num_z);
  if (grid > kMaxGrid) return SDPA_ERR_SHAPE;
  if (grid == 0) return SDPA_OK;
  a.m_tiles = static_cast<int32_t>(m_tiles);
  const int err = a.bias != nullptr
                      ? sdpa03::launch_attn_fwd_bias(a, dtype, head_dim, mode, causal != 0, stream)
                      : sdpa03::launch_attn_fwd(a, dtype, head_dim, mode, causal != 0, stream);
  return err == 0 ? SDPA_OK : SDPA_ERR_HIP;
}

// One backward call.  The rank-4 views are (num_b, H, rows_q or rows_k, D);
// mode, num_z and the per-sequence bounds (seqlen_q, seqlen_k, cu_q, cu_k)
// select the sequences inside them, as in the forward.
struct BwdCall {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  sdpa_dtype dtype;
  int32_t num_b, num_heads, rows_q, rows_k, head_dim;
  const int64_t* q_stride;
  const int64_t* k_stride;
  const int64_t* v_stride;
  const int64_t* o_stride;
  const int64_t* dout_stride;
  float scale;
  int32_t causal;
  void* workspace;
  uint64_t workspace_bytes;
  void* stream;
  int mode;
  int32_t num_z, seqlen_q, seqlen_k;
  const int32_t* cu_q;
  const int32_t* cu_k;
};

// Checks shared by the three backward entry points (sizes are already known
// to be non-negative), then the launches.
sdpa_status run_bwd(const BwdCall& c) {
  sdpa_status st = check_common(c.dtype, c.head_dim, c.scale);
  if (st != SDPA_OK) return st;
  if (c.dtype == SDPA_F32) return SDPA_ERR_DTYPE;
  const int32_t H = c.num_heads;
  // Nothing to write when no sequence has a query row or a key.
  if (static_cast<int64_t>(c.num_b) * H * c.num_z == 0 || (c.seqlen_q == 0 && c.seqlen_k == 0))
    return SDPA_OK;
  // Query side (q, o, dout, lse, dq) is needed when the view has query rows;
  // key side (k, v, dk, dv) when it has keys.
  if (c.rows_q > 0 && (!c.q || !c.o || !c.dout || !c.lse || !c.dq)) return SDPA_ERR_NULL;
  if (c.rows_k > 0 && (!c.k || !c.v || !c.dk || !c.dv)) return SDPA_ERR_NULL;
  if (c.mode != sdpa03::MODE_DENSE) {
    if (!c.cu_q || !c.cu_k) return SDPA_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(c.cu_q) % 4 != 0 ||
        reinterpret_cast<uintptr_t>(c.cu_k) % 4 != 0)
      return SDPA_ERR_ALIGN;
  }
  const int es = elem_size(c.dtype);
  const int64_t nb = c.num_b, hd = c.head_dim;
  const View views[] = {
      {c.q, {nb, H, c.rows_q, hd}, c.q_stride},    {c.dq, {nb, H, c.rows_q, hd}, c.q_stride},
      {c.o, {nb, H, c.rows_q, hd}, c.o_stride},    {c.dout, {nb, H, c.rows_q, hd}, c.dout_stride},
      {c.k, {nb, H, c.rows_k, hd}, c.k_stride},    {c.dk, {nb, H, c.rows_k, hd}, c.k_stride},
      {c.v, {nb, H, c.rows_k, hd}, c.v_stride},    {c.dv, {nb, H, c.rows_k, hd}, c.v_stride},
  };
  for (int i = 0; i < 8; ++i) {
    const bool key_side = i >= 4;
    if ((key_side ? c.rows_k : c.rows_q) == 0) continue;
    if ((st = check_view(views[i], es, true)) != SDPA_OK) return st;
  }
  if (reinterpret_cast<uintptr_t>(c.lse) % 4 != 0) return SDPA_ERR_ALIGN;
  const int64_t pad = sdpa03::bwd_ws_rows_pad(c.rows_q);
  const int64_t ws_groups = nb * H;  // workspace (b, h) blocks
  const int64_t q_tiles = (static_cast<int64_t>(c.seqlen_q) + sdpa03::kBwdDqRows - 1) / sdpa03::kBwdDqRows;
  const int64_t k_tiles = (static_cast<int64_t>(c.seqlen_k) + sdpa03::kBwdDkvKeys - 1) / sdpa03::kBwdDkvKeys;
  const int64_t groups = static_cast<int64_t>(c.num_z) * H;  // (sequence, head) pairs
  if (pad > INT32_MAX || q_tiles * groups > kMaxGrid || k_tiles * groups > kMaxGrid ||
      ws_groups * pad > (int64_t(1) << 40))
    return SDPA_ERR_SHAPE;
  const uint64_t need = 2ull * static_cast<uint64_t>(ws_groups * pad) * 4ull;
  if (q_tiles > 0 && (c.workspace == nullptr ||
                      reinterpret_cast<uintptr_t>(c.workspace) % 16 != 0 ||
                      c.workspace_bytes < need))
    return SDPA_ERR_WORKSPACE;

  sdpa03::BwdArgs a{};
  a.q = c.q; a.k = c.k; a.v = c.v; a.o = c.o; a.dout = c.dout; a.lse = c.lse;
  a.cu_q = c.cu_q; a.cu_k = c.cu_k;
  a.dq = c.dq; a.dk = c.dk; a.dv = c.dv;
  a.ws_delta = static_cast<float*>(c.workspace);
  a.ws_lse2 = q_tiles > 0 ? static_cast<float*>(c.workspace) + ws_groups * pad : nullptr;
  set_strides(c.q_stride, a.q_sb, a.q_sh, a.q_ss);
  set_strides(c.k_stride, a.k_sb, a.k_sh, a.k_ss);
  set_strides(c.v_stride, a.v_sb, a.v_sh, a.v_ss);
  set_strides(c.o_stride, a.o_sb, a.o_sh, a.o_ss);
  set_strides(c.dout_stride, a.do_sb, a.do_sh, a.do_ss);
  // The forward's logsumexp layout: (num_b, H, rows_q), contiguous.
  a.lse_sh = c.rows_q;
  a.lse_sb = static_cast<int64_t>(H) * c.rows_q;
  a.seqlen_q = c.seqlen_q;
  a.seqlen_k = c.seqlen_k;
  a.total_q = c.rows_q;
  a.total_k = c.rows_k;
  a.num_heads = H;
  a.num_b = c.num_b;
  a.num_z = c.num_z;
  a.ws_rows_pad = static_cast<int32_t>(pad);
  a.q_tiles = static_cast<int32_t>(q_tiles);
  a.k_tiles = static_cast<int32_t>(k_tiles);
  a.scale = c.scale;
  a.scale_log2 = c.scale * 1.4426950408889634f;
  const int err = sdpa03::launch_attn_bwd(a, c.dtype, c.head_dim, c.mode, c.causal != 0, c.stream);
  return err == 0 ? SDPA_OK : SDPA_ERR_HIP;
}

}  // namespace

extern "C" {

const char* sdpa_status_string(sdpa_status status) {
  switch (status) {
    case SDPA_OK: return "ok";
    case SDPA_ERR_NULL: return "a required pointer is NULL";
    case SDPA_ERR_DTYPE: return "unsupported dtype (expected fp32, fp16 or bf16)";
    case SDPA_ERR_HEAD_DIM: return "unsupported head_dim (expected 64 or 128)";
    case SDPA_ERR_SHAPE: return "invalid or too large sizes";
    case SDPA_ERR_STRIDE: return "invalid strides (dim stride must be 1, no negative or overflowing strides)";
    case SDPA_ERR_ALIGN: return "base pointers and strides must be 16-byte aligned";
    case SDPA_ERR_BATCH: return "compact varlen needs batch size exactly 1";
    case SDPA_ERR_SEQLEN: return "invalid sequence-length arguments";
    case SDPA_ERR_SCALE: return "scale must be finite and positive";
    case SDPA_ERR_HIP: return "the HIP runtime rejected the kernel launch";
    case SDPA_ERR_WORKSPACE:
      return "split forward workspace is NULL, not 16-byte aligned or smaller than the plan";
    case SDPA_ERR_SCRATCH:
      return "the problem needs more split-forward scratch than the library's static buffer "
             "(SDPA_NOALLOC_SCRATCH_BYTES) holds";
  }
  return "unknown status";
}

sdpa_status sdpa_bwd_workspace_bytes(int32_t B, int32_t H, int32_t seqlen_q,
                                     uint64_t* workspace_bytes) {
  if (B < 0 || H < 0 || seqlen_q < 0) return SDPA_ERR_SHAPE;
  if (workspace_bytes) {
    *workspace_bytes = 2ull * static_cast<uint64_t>(B) * static_cast<uint64_t>(H) *
                       static_cast<uint64_t>(sdpa03::bwd_ws_rows_pad(seqlen_q)) * 4ull;
  }
  return SDPA_OK;
}

sdpa_status attn_bwd(const void* q, const void* k, const void* v, const void* o,
                     const void* dout, const float* lse, void* dq, void* dk, void* dv,
                     sdpa_dtype dtype, int32_t B, int32_t H, int32_t seqlen_q,
                     int32_t seqlen_k, int32_t head_dim, const int64_t q_stride[4],
                     const int64_t k_stride[4], const int64_t v_stride[4],
                     const int64_t o_stride[4], const int64_t dout_stride[4], float scale,
                     int32_t causal, void* workspace, uint64_t workspace_bytes,
                     void* hip_stream) {
  BwdCall c{q, k, v, o, dout, lse, dq, dk, dv, dtype, B, H, seqlen_q, seqlen_k, head_dim,
            q_stride, k_stride, v_stride, o_stride, dout_stride, scale, causal, workspace,
            workspace_bytes, hip_stream, sdpa03::MODE_DENSE, B, seqlen_q, seqlen_k,
            nullptr, nullptr};
  if (B < 0 || H < 0 || seqlen_q < 0 || seqlen_k < 0) return SDPA_ERR_SHAPE;
  return run_bwd(c);
}

sdpa_status attn_bwd_compact_varlen(const void* q, const void* k, const void* v, const void* o,
                                    const void* dout, const float* lse, void* dq, void* dk,
                                    void* dv, sdpa_dtype dtype, int32_t B, int32_t H,
                                    int32_t total_q, int32_t total_k, int32_t head_dim,
                                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                    int32_t num_seqs, int32_t max_seqlen_q,
                                    int32_t max_seqlen_k, const int64_t q_stride[4],
                                    const int64_t k_stride[4], const int64_t v_stride[4],
                                    const int64_t o_stride[4], const int64_t dout_stride[4],
                                    float scale, int32_t causal, void* workspace,
                                    uint64_t workspace_bytes, void* hip_stream) {
  if (B != 1) return SDPA_ERR_BATCH;
  if (H < 0 || total_q < 0 || total_k < 0) return SDPA_ERR_SHAPE;
  if (num_seqs < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || max_seqlen_q > total_q ||
      max_seqlen_k > total_k)
    return SDPA_ERR_SEQLEN;
  BwdCall c{q, k, v, o, dout, lse, dq, dk, dv, dtype, 1, H, total_q, total_k, head_dim,
            q_stride, k_stride, v_stride, o_stride, dout_stride, scale, causal, workspace,
            workspace_bytes, hip_stream, sdpa03::MODE_COMPACT, num_seqs, max_seqlen_q,
            max_seqlen_k, cu_seqlens_q, cu_seqlens_k};
  return run_bwd(c);
}

sdpa_status attn_bwd_padded_varlen(const void* q, const void* k, const void* v, const void* o,
                                   const void* dout, const float* lse, void* dq, void* dk,
                                   void* dv, sdpa_dtype dtype, int32_t B, int32_t H,
                                   int32_t seqlen_q_max, int32_t seqlen_k_max,
                                   int32_t head_dim, const int32_t* cu_seqlens_q,
                                   const int32_t* cu_seqlens_k, const int64_t q_stride[4],
                                   const int64_t k_stride[4], const int64_t v_stride[4],
                                   const int64_t o_stride[4], const int64_t dout_stride[4],
                                   float scale, int32_t causal, void* workspace,
                                   uint64_t workspace_bytes, void* hip_stream) {
  if (B < 0 || H < 0 || seqlen_q_max < 0 || seqlen_k_max < 0) return SDPA_ERR_SHAPE;
  BwdCall c{q, k, v, o, dout, lse, dq, dk, dv, dtype, B, H, seqlen_q_max, seqlen_k_max,
            head_dim, q_stride, k_stride, v_stride, o_stride, dout_stride, scale, causal,
            workspace, workspace_bytes, hip_stream, sdpa03::MODE_PADDED, B, seqlen_q_max,
            seqlen_k_max, cu_seqlens_q, cu_seqlens_k};
  return run_bwd(c);
}

sdpa_status sdpa_check_cu_seqlens_host(const int32_t* cu, int32_t n, int32_t total,
                                       int32_t max_len) {
  if (cu == nullptr) return SDPA_ERR_NULL;
  if (n < 0 || total < 0 || max_len < 0) return SDPA_ERR_SEQLEN;
  if (cu[0] != 0) return SDPA_ERR_SEQLEN;
  for (int32_t i = 0; i < n; ++i) {
    const int64_t len = static_cast<int64_t>(cu[i + 1]) - cu[i];
    if (len < 0 || len > max_len) return SDPA_ERR_SEQLEN;
  }
  if (cu[n] > total) return SDPA_ERR_SEQLEN;
  return SDPA_OK;
}

sdpa_status sdpa_kernel_config(sdpa_dtype dtype, int32_t head_dim, int32_t causal, int32_t mode,
                               int32_t seqlen_q, int32_t seqlen_k, int32_t single_group,
                               int32_t* block_m, int32_t* block_n, int32_t* waves) {
  if (!dtype_ok(dtype)) return SDPA_ERR_DTYPE;
  if (mode < 0 || mode > 2) return SDPA_ERR_SHAPE;
  if (seqlen_q < 0 || seqlen_k < 0) return SDPA_ERR_SHAPE;
  sdpa03::KernelConfig cfg;
  if (!sdpa03::kernel_config(dtype, head_dim, seqlen_q, seqlen_k, causal != 0, mode,
                             single_group != 0, &cfg))
    return SDPA_ERR_HEAD_DIM;
  if (block_m) *block_m = cfg.block_m;
  if (block_n) *block_n = cfg.block_n;
  if (waves) *waves = cfg.waves;
  return SDPA_OK;
}

sdpa_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     sdpa_dtype dtype, int32_t B, int32_t H, int32_t seqlen_q,
                     int32_t seqlen_k, int32_t head_dim, const int64_t q_stride[4],
                     const int64_t k_stride[4], const int64_t v_stride[4],
                     const int64_t o_stride[4], float scale, int32_t causal, void* hip_stream) {
  FwdArgs a;
  bool empty;
  const sdpa_status st = dense_args(q, k, v, o, lse, dtype, B, H, seqlen_q, seqlen_k, head_dim,
                                    q_stride, k_stride, v_stride, o_stride, scale, &a, &empty);
  if (st != SDPA_OK || empty) return st;
  return finish_and_launch(a, dtype, head_dim, sdpa03::MODE_DENSE, causal, hip_stream);
}

sdpa_status sdpa_fwd_splitk_plan(sdpa_dtype dtype, int32_t B, int32_t H, int32_t seqlen_q,
                                 int32_t seqlen_k, int32_t head_dim, int32_t num_splits,
                                 int32_t* num_splits_used, uint64_t* workspace_bytes) {
  SplitPlan p;
  const sdpa_status st = split_plan(dtype, B, H, seqlen_q, seqlen_k, head_dim, num_splits, &p);
  if (st != SDPA_OK) return st;
  if (num_splits_used) *num_splits_used = p.splits;
  if (workspace_bytes) *workspace_bytes = p.bytes;
  return SDPA_OK;
}

sdpa_status attn_fwd_splitk(const void* q, const void* k, const void* v, void* o, float* lse,
                            sdpa_dtype dtype, int32_t B, int32_t H, int32_t seqlen_q,
                            int32_t seqlen_k, int32_t head_dim, const int64_t q_stride[4],
                            const int64_t k_stride[4], const int64_t v_stride[4],
                            const int64_t o_stride[4], float scale, int32_t causal,
                            int32_t num_splits, void* workspace, uint64_t workspace_bytes,
                            void* hip_stream) {
  FwdArgs a;
  bool empty;
  sdpa_status st = dense_args(q, k, v, o, lse, dtype, B, H, seqlen_q, seqlen_k, head_dim,
                              q_stride, k_stride, v_stride, o_stride, scale, &a, &empty);
  if (st != SDPA_OK || empty) return st;
  SplitPlan p;
  if ((st = split_plan(dtype, B, H, seqlen_q, seqlen_k, head_dim, num_splits, &p)) != SDPA_OK)
    return st;
  if (workspace == nullptr || reinterpret_cast<uintptr_t>(workspace) % 16 != 0 ||
      workspace_bytes < p.bytes)
    return SDPA_ERR_WORKSPACE;
  return launch_split(a, p, workspace, o, lse, dtype, H, seqlen_q, head_dim, causal, hip_stream);
}

sdpa_status attn_fwd_splitk_noalloc(const void* q, const void* k, const void* v, void* o,
                                    float* lse, sdpa_dtype dtype, int32_t B, int32_t H,
                                    int32_t seqlen_q, int32_t seqlen_k, int32_t head_dim,
                                    const int64_t q_stride[4], const int64_t k_stride[4],
                                    const int64_t v_stride[4], const int64_t o_stride[4],
                                    float scale, int32_t causal, int32_t num_splits,
                                    void* hip_stream) {
  FwdArgs a;
  bool empty;
  sdpa_status st = dense_args(q, k, v, o, lse, dtype, B, H, seqlen_q, seqlen_k, head_dim,
                              q_stride, k_stride, v_stride, o_stride, scale, &a, &empty);
  if (st != SDPA_OK || empty) return st;
  SplitPlan p;
  if ((st = split_plan(dtype, B, H, seqlen_q, seqlen_k, head_dim, num_splits, &p)) != SDPA_OK)
    return st;
  if (p.bytes > SDPA_NOALLOC_SCRATCH_BYTES) return SDPA_ERR_SCRATCH;
  void* ws = nullptr;
  if ((st = scratch_address(hip_stream, &ws)) != SDPA_OK) return st;
  return launch_split(a, p, ws, o, lse, dtype, H, seqlen_q, head_dim, causal, hip_stream);
}

sdpa_status attn_fwd_compact_varlen(const void* q, const void* k, const void* v, void* o,
                                    float* lse, sdpa_dtype dtype, int32_t B, int32_t H,
                                    int32_t total_q, int32_t total_k, int32_t head_dim,
                                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                    int32_t num_seqs, int32_t max_seqlen_q,
                                    int32_t max_seqlen_k, const int64_t q_stride[4],
                                    const int64_t k_stride[4], const int64_t v_stride[4],
                                    const int64_t o_stride[4], float scale, int32_t causal,
                                    void* hip_stream) {
  FwdArgs a;
  bool empty;
  const sdpa_status st = compact_args(q, k, v, o, lse, dtype, B, H, total_q, total_k, head_dim,
                                      cu_seqlens_q, cu_seqlens_k, num_seqs, max_seqlen_q,
                                      max_seqlen_k, q_stride, k_stride, v_stride, o_stride, scale,
                                      &a, &empty);
  if (st != SDPA_OK || empty) return st;
  return finish_and_launch(a, dtype, head_dim, sdpa03::MODE_COMPACT, causal, hip_stream);
}

sdpa_status attn_fwd_padded_varlen(const void* q, const void* k, const void* v, void* o,
                                   float* lse, sdpa_dtype dtype, int32_t B, int32_t H,
                                   int32_t seqlen_q_max, int32_t seqlen_k_max,
                                   int32_t head_dim, const int32_t* cu_seqlens_q,
                                   const int32_t* cu_seqlens_k, const int64_t q_stride[4],
                                   const int64_t k_stride[4], const int64_t v_stride[4],
                                   const int64_t o_stride[4], float scale, int32_t causal,
                                   void* hip_stream) {
  FwdArgs a;
  bool empty;
  const sdpa_status st = padded_args(q, k, v, o, lse, dtype, B, H, seqlen_q_max, seqlen_k_max,
                                     head_dim, cu_seqlens_q, cu_seqlens_k, q_stride, k_stride,
                                     v_stride, o_stride, scale, &a, &empty);
  if (st != SDPA_OK || empty) return st;
  return finish_and_launch(a, dtype, head_dim, sdpa03::MODE_PADDED, causal, hip_stream);
}

sdpa_status attn_fwd_bias(const void* q, const void* k, const void* v, const void* bias,
                          void* o, float* lse, sdpa_dtype dtype, int32_t B, int32_t H,
                          int32_t seqlen_q, int32_t seqlen_k, int32_t head_dim,
                          const int64_t q_stride[4], const int64_t k_stride[4],
                          const int64_t v_stride[4], const int64_t bias_stride[4],
                          const int64_t o_stride[4], float scale, int32_t causal,
                          void* hip_stream) {
  FwdArgs a;
  bool empty;
  sdpa_status st = dense_args(q, k, v, o, lse, dtype, B, H, seqlen_q, seqlen_k, head_dim,
                              q_stride, k_stride, v_stride, o_stride, scale, &a, &empty);
  if (st != SDPA_OK || empty) return st;
  if ((st = check_bias(bias, B, H, seqlen_q, seqlen_k, bias_stride, elem_size(dtype))) != SDPA_OK)
    return st;
  set_bias(a, bias, bias_stride);
  return finish_and_launch(a, dtype, head_dim, sdpa03::MODE_DENSE, causal, hip_stream);
}

sdpa_status attn_fwd_compact_varlen_bias(
    const void* q, const void* k, const void* v, const void* bias, void* o, float* lse,
    sdpa_dtype dtype, int32_t B, int32_t H, int32_t total_q, int32_t total_k, int32_t head_dim,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t num_seqs,
    int32_t max_seqlen_q, int32_t max_seqlen_k, const int64_t q_stride[4],
    const int64_t k_stride[4], const int64_t v_stride[4], const int64_t bias_stride[4],
    const int64_t o_stride[4], float scale, int32_t causal, void* hip_stream) {
  FwdArgs a;
  bool empty;
  sdpa_status st = compact_args(q, k, v, o, lse, dtype, B, H, total_q, total_k, head_dim,
                                cu_seqlens_q, cu_seqlens_k, num_seqs, max_seqlen_q, max_seqlen_k,
                                q_stride, k_stride, v_stride, o_stride, scale, &a, &empty);
  if (st != SDPA_OK || empty) return st;
  if ((st = check_bias(bias, 1, H, total_q, total_k, bias_stride, elem_size(dtype))) != SDPA_OK)
    return st;
  set_bias(a, bias, bias_stride);
  return finish_and_launch(a, dtype, head_dim, sdpa03::MODE_COMPACT, causal, hip_stream);
}

sdpa_status attn_fwd_padded_varlen_bias(
    const void* q, const void* k, const void* v, const void* bias, void* o, float* lse,
    sdpa_dtype dtype, int32_t B, int32_t H, int32_t seqlen_q_max, int32_t seqlen_k_max,
    int32_t head_dim, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
    const int64_t q_stride[4], const int64_t k_stride[4], const int64_t v_stride[4],
    const int64_t bias_stride[4], const int64_t o_stride[4], float scale, int32_t causal,
    void* hip_stream) {
  FwdArgs a;
  bool empty;
  sdpa_status st = padded_args(q, k, v, o, lse, dtype, B, H, seqlen_q_max, seqlen_k_max, head_dim,
                               cu_seqlens_q, cu_seqlens_k, q_stride, k_stride, v_stride, o_stride,
                               scale, &a, &empty);
  if (st != SDPA_OK || empty) return st;
  if ((st = check_bias(bias, B, H, seqlen_q_max, seqlen_k_max, bias_stride, elem_size(dtype))) !=
      SDPA_OK)
    return st;
  set_bias(a, bias, bias_stride);
  return finish_and_launch(a, dtype, head_dim, sdpa03::MODE_PADDED, causal, hip_stream);
}

}  // extern "C"
