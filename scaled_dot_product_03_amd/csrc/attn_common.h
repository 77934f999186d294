// Device helpers shared by the attention kernels (forward and backward):
// vector types, MFMA wrappers, wave reductions, memory waits, the LDS-only
// workgroup barrier and the HBM -> LDS tile copy (namespace sdpa03).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fwd_args.h"  // Mode

namespace sdpa03 {

using f32x16 = float __attribute__((ext_vector_type(16)));
using f32x4 = float __attribute__((ext_vector_type(4)));
using bf16x8 = __bf16 __attribute__((ext_vector_type(8)));
using f16x8 = _Float16 __attribute__((ext_vector_type(8)));
using lds_void_ptr = __attribute__((address_space(3))) void*;

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2e = 1.4426950408889634f;
// Fourth dword of a raw buffer descriptor on gfx9 (32-bit data format).
constexpr int kBufferFlags = 0x00020000;

__device__ __forceinline__ float max_across_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_across_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Workgroup barrier for LDS hand-offs.  __syncthreads() (and any release
// fence covering LDS) waits for every outstanding vector-memory load first
// (vmcnt(0)), because a buffer load into LDS counts as an LDS write -- which
// would drain tile loads that are meant to stay in flight across the barrier.
// Here each wave waits for its own tile loads explicitly (wait_vmem_allow)
// before it arrives; the barrier itself waits only for the wave's LDS reads
// (so no later load can overwrite a buffer still being read), and the memory
// clobber and the scheduling barriers keep the compiler from moving LDS
// accesses -- or any other instruction -- across it.
__device__ __forceinline__ void barrier_lds() {
  __builtin_amdgcn_sched_barrier(0);  // no instruction moves across
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// s_waitcnt vmcnt(N): wait until at most N of this wave's vector-memory
// loads are still in flight (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem_allow() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 0xF) | ((N >> 4) << 14));
}

// ---------------------------------------------------------------------------
// Matrix-core paths.  Each provides: Q fragments held in registers, the
// S^T = K Q^T product from a K tile in LDS, the probabilities P of a score
// tile, and O^T += V^T P^T from a V tile in LDS.  Tiles in LDS are row-major
// [key][dim]: 16-bit tiles of head dim 128 with their 16-byte chunks
// XOR-swizzled per row (swizzle_of below), the others with padded rows.
// ---------------------------------------------------------------------------

template <typename T>
struct Mma16;

template <>
struct Mma16<__bf16> {
  using frag = bf16x8;
  __device__ static __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Mma16<_Float16> {
  using frag = f16x8;
  __device__ static __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

// Sum of the 16 floats of an accumulator as a balanced tree (short
// dependency chains for the in-order VALU).
__device__ __forceinline__ float tree_sum16(const float (&x)[16]) {
  float a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = x[2 * i] + x[2 * i + 1];
  float b0 = (a[0] + a[1]) + (a[2] + a[3]);
  float b1 = (a[4] + a[5]) + (a[6] + a[7]);
  return b0 + b1;
}

// ---------------------------------------------------------------------------
// Tile copies: buffer loads straight into LDS
// ---------------------------------------------------------------------------
// buffer_load_dwordx4 ... lds writes lane L's 16 bytes to (wave-uniform LDS
// base + 16 L): one instruction fills a 1 KiB block of LDS from 64
// independent source offsets.  A tile of BN rows at LDS row stride ROW
// occupies BN * ROW bytes; every wave issues the same number of blocks
// (the last ones may lie past the tile, inside the array).  A lane whose
// 16 bytes fall on row padding, or past the tile, gets an offset outside
// the descriptor's range and writes zeros.  The descriptor starts at the
// tile's first row and covers only the rows that exist, so rows past the
// sequence read back as zeros too, with no bounds arithmetic in the loop.
// Source offsets are 32-bit: the host limits row strides accordingly.

// XOR swizzle of the 16-byte chunks of a 16-bit tile whose rows are exactly
// D * 2 bytes long and that is read both as 16-row MFMA operands
// (ds_read_b128: a pass reads one chunk of 16 aligned consecutive rows) and
// transposed (ds_read_b64_tr_b16: a 32-lane pass reads one aligned 64-byte
// block of 4 aligned consecutive rows).  Chunk c of row r is stored at chunk
// c ^ swizzle_of<D>(r).  Over 16 aligned rows the XOR puts a chunk in 16
// distinct bank groups (for D = 64, rows of one parity share a half of the
// banks and take 8 distinct values each); over 4 aligned rows it gives a
// 64-byte block 4 distinct block positions.  So both passes touch every
// bank once.  No row padding does both: the first needs the stride / 16 to
// be odd, the second a stride of +-64 modulo 256 bytes.
template <int D>
__host__ __device__ constexpr int swizzle_of(int r) {
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3))
                  : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// SWIZZLE: rows of exactly D * 2 bytes (ROW == D * 2), chunks stored as
// swizzle_of<D> says; each lane fetches the source chunk that belongs at
// its (lane-linear) LDS position.
template <typename T, int D, int BN, int NW, int ROW, bool SWIZZLE = false>
struct TileCopy {
  static_assert(!SWIZZLE || (sizeof(T) == 2 && ROW == D * 2), "swizzled tiles: 16-bit, unpadded");
  static_assert(!SWIZZLE || D == 64 || D == 128, "swizzle_of covers head_dim 64 and 128");
  static constexpr int kDataBytes = D * static_cast<int>(sizeof(T));  // payload per row
  static constexpr int kBlocks = (BN * ROW + 1023) / 1024;
  static constexpr int kInstPerWave = (kBlocks + NW - 1) / NW;
  static constexpr int kArrayBytes = kInstPerWave * NW * 1024;  // LDS array size per tile
  static constexpr uint32_t kNowhere = 0x80000000u;  // past any descriptor range

  uint32_t voff[kInstPerWave];

  __device__ __forceinline__ void init(int wave, int lane, int64_t row_bytes) {
#pragma unroll
    for (int i = 0; i < kInstPerWave; ++i) {
      const int pos = (i * NW + wave) * 1024 + lane * 16;
      const int r = pos / ROW;
      const int col = SWIZZLE ? ((((pos % ROW) >> 4) ^ swizzle_of<D>(r)) << 4) : pos % ROW;
      const bool data = r < BN && col < kDataBytes;
      voff[i] = data ? static_cast<uint32_t>(r * row_bytes) + static_cast<uint32_t>(col) : kNowhere;
    }
  }

  // Rows [0, valid_rows) of the tile starting at `tile` land in `lds_tile`.
  __device__ __forceinline__ void issue(const char* tile, int valid_rows, int64_t row_bytes,
                                        T* lds_tile, int wave) const {
    // hipcc's host (x86) pass parses this body too but has no buffer-resource
    // type; left visible there, it stops the host pass from emitting the
    // launch stubs of later kernel instantiations.
#if defined(__HIP_DEVICE_COMPILE__)
    const int rows = valid_rows < 0 ? 0 : (valid_rows > BN ? BN : valid_rows);
    const uint32_t bytes = static_cast<uint32_t>(rows * row_bytes);  // <= 2^30
    // Every input of the descriptor is wave-uniform; saying so explicitly
    // keeps the descriptor in SGPRs.  (Left in VGPRs, the compiler wraps each
    // buffer load in a loop over the distinct descriptor values of the wave.)
    // readfirstlane returns int: keep both halves unsigned 32-bit before
    // widening, or a low half with bit 31 set would sign-extend into the
    // high half of the address.
    const uint64_t addr = reinterpret_cast<uint64_t>(tile);
    const uint32_t hi = static_cast<uint32_t>(
        __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(addr >> 32))));
    const uint32_t lo = static_cast<uint32_t>(
        __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(addr))));
    const uint64_t base = (static_cast<uint64_t>(hi) << 32) | static_cast<uint64_t>(lo);
    const int nrec = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(base), 0, nrec, kBufferFlags);
    char* lds = reinterpret_cast<char*>(lds_tile);
#pragma unroll
    for (int i = 0; i < kInstPerWave; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (lds_void_ptr)(lds + (i * NW + wave) * 1024), 16, voff[i], 0, 0, 0);
    }
#endif
  }

  // The same copy written as inline assembly.  The compiler neither moves
  // these loads nor counts them, so it inserts no waits of its own for them
  // (its tracking of which LDS buffer a load writes is lost across the
  // ping-pong loop and would make it drain every load in flight); the caller
  // waits with explicit vmcnt counts, and must have no compiler-issued
  // vector-memory load outstanding that it relies on the compiler to wait
  // for.  The memory clobber keeps LDS reads of earlier code before the
  // loads.  M0 (the LDS destination) is an input bound to the register, so
  // the compiler writes it and knows its value; s_nop 4 covers the wait
  // states between a VALU write of a descriptor SGPR (readfirstlane) and its
  // use by a vector-memory instruction, and with them the one between
  // writing M0 and an LDS load.
  __device__ __forceinline__ void issue_untracked(const char* tile, int valid_rows,
                                                  int64_t row_bytes, T* lds_tile, int wave) const {
#if defined(__HIP_DEVICE_COMPILE__)
    using i32x4 = int __attribute__((ext_vector_type(4)));
    const int rows = valid_rows < 0 ? 0 : (valid_rows > BN ? BN : valid_rows);
    const uint32_t bytes = static_cast<uint32_t>(rows * row_bytes);  // <= 2^30
    const uint64_t addr = reinterpret_cast<uint64_t>(tile);
    const int hi = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(addr >> 32)));
    const int lo = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(addr)));
    const int nrec = __builtin_amdgcn_readfirstlane(static_cast<int>(bytes));
    // Raw descriptor: base (48 bits, stride 0), num_records, format/flags.
    const i32x4 rsrc = {lo, hi & 0xFFFF, nrec, kBufferFlags};
    const uint32_t lds = (uint32_t)(uintptr_t)(lds_void_ptr)(lds_tile);  // LDS byte address
#pragma unroll
    for (int i = 0; i < kInstPerWave; ++i) {
      const uint32_t m0v = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(
          static_cast<int>(lds + static_cast<uint32_t>((i * NW + wave) * 1024))));
      asm volatile(
          "s_nop 4\n\t"
          "buffer_load_dwordx4 %0, %1, 0 offen lds"
          :
          : "v"(voff[i]), "s"(rsrc), "{m0}"(m0v)
          : "memory");
    }
#endif
  }
};

struct SeqRange {
  int64_t b;    // batch index into the rank-4 view
  int q_start;  // first token of the sequence along seq (compact), else 0
  int k_start;
  int len_q;
  int len_k;
};

// Rows and keys of program z (forward and backward kernels).  seqlen_q and seqlen_k are
// the rank-4 view's sequence lengths (dense), the maximum lengths (compact)
// or the padded lengths (padded).  Dense: batch z, all rows.  Compact: batch 0,
// tokens [cu[z], cu[z+1]).  Padded: batch z, lengths cu[z+1] - cu[z] from
// offset 0 (the padded branch of the fwd_kernel.py excerpt quoted in
// AOTriton PR #31).  Ranges are clamped to the addressable rows so that
// malformed cu_seqlens can never move an access out of bounds: compact
// token ranges to [0, total), padded lengths to [0, padded length].
template <int MODE>
__device__ __forceinline__ SeqRange seq_range_of(const int32_t* cu_q, const int32_t* cu_k,
                                                 int total_q, int total_k, int seqlen_q,
                                                 int seqlen_k, int z) {
  SeqRange r;
  if constexpr (MODE == MODE_DENSE) {
    r.b = z;
    r.q_start = 0;
    r.k_start = 0;
    r.len_q = seqlen_q;
    r.len_k = seqlen_k;
  } else if constexpr (MODE == MODE_COMPACT) {
    const int q0 = min(max(cu_q[z], 0), total_q);
    const int q1 = min(max(cu_q[z + 1], q0), total_q);
    const int k0 = min(max(cu_k[z], 0), total_k);
    const int k1 = min(max(cu_k[z + 1], k0), total_k);
    r.b = 0;
    r.q_start = q0;
    r.k_start = k0;
    r.len_q = min(q1 - q0, seqlen_q);
    r.len_k = min(k1 - k0, seqlen_k);
  } else {
    const int64_t lq = static_cast<int64_t>(cu_q[z + 1]) - cu_q[z];
    const int64_t lk = static_cast<int64_t>(cu_k[z + 1]) - cu_k[z];
    r.b = z;
    r.q_start = 0;
    r.k_start = 0;
    r.len_q = static_cast<int>(min(max(lq, int64_t(0)), static_cast<int64_t>(seqlen_q)));
    r.len_k = static_cast<int>(min(max(lk, int64_t(0)), static_cast<int64_t>(seqlen_k)));
  }
  return r;
}

// An XCD holds 256 waves at two per SIMD (32 CUs x 4 SIMDs).  A part of the
// causal launch order gets at least four times that many waves of
// workgroups; measured on the causal forward workloads (S 2048 dense, THD varlen
// with sequences up to 4096, padded varlen up to 8192), more parts than
// that left the long tiles of the last part unbalanced, fewer kept more
// heads' keys in flight.
constexpr int64_t kCausalPartWaves = 1024;
// Compact (THD) sequences are short on average and their heads' key tiles
// few: parts of one XCD's worth of waves keep fewer heads' keys in flight.
// Measured on the THD workload (16 sequences up to 4096, H 16, D 128):
// 562 against 598 us for parts of 1024 waves; the padded workload (up to
// 8192) ran 3 % slower with 256, so it keeps 1024.
constexpr int64_t kCausalPartWavesCompact = 256;

// Groups per part (a divisor of the groups each XCD gets) for a causal
// launch of `groups` (batch or sequence, head) groups of m_tiles workgroups
// of `waves` waves; 0 when the groups do not split evenly over 8 XCDs.
// Workgroup n runs on XCD n % 8; the forward and backward launch orders
// deal group g to XCD g % 8 and take each XCD's groups `span` at a time.
inline int32_t causal_span(int64_t groups, int32_t m_tiles, int waves,
                           int64_t part_waves = kCausalPartWaves) {
  if (groups <= 0 || groups % 8 != 0 || m_tiles <= 0) return 0;
  const int64_t per_xcd = groups / 8;
  for (int64_t d = 1; d < per_xcd; ++d) {
    if (per_xcd % d == 0 && d * m_tiles * waves >= part_waves) return static_cast<int32_t>(d);
  }
  return static_cast<int32_t>(per_xcd);
}

// Launch order of the backward kernels: workgroup n of groups x tiles
// workgroups -> (group g, tile rank t).  Without a causal mask each XCD runs
// a contiguous range of groups-major ranks (whole heads share its L2).
// Under the mask rank 0 is a group's most expensive tile; ranks run from 0
// up, over the XCD's groups in parts of `span` as in the forward (span 0:
// over all groups fastest).
__device__ __forceinline__ void bwd_launch_order(bool causal, uint32_t tiles, uint32_t groups,
                                                 int span, uint32_t& g, uint32_t& t) {
  const uint32_t n = blockIdx.x;
  if (!causal) {
    const uint32_t per_xcd = gridDim.x >> 3;
    uint32_t logical = n;
    if (n < (per_xcd << 3)) logical = (n & 7u) * per_xcd + (n >> 3);
    t = logical % tiles;
    g = logical / tiles;
  } else if (span > 0) {
    const uint32_t xcd = n & 7u, i = n >> 3;
    const uint32_t per_part = static_cast<uint32_t>(span);
    const uint32_t part_wgs = per_part * tiles;
    const uint32_t part = i / part_wgs, r = i % part_wgs;
    t = r / per_part;
    g = xcd + 8u * (part * per_part + r % per_part);
  } else {
    g = n % groups;
    t = n / groups;
  }
}

}  // namespace sdpa03
