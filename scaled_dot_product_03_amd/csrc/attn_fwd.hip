// Flash-attention forward kernels for CDNA4 (gfx950).
//
// One workgroup computes block_m = 32 * waves query rows of one
// (batch or sequence, head); each wavefront owns 32 rows.  The workgroup
// walks the key axis in tiles of block_n keys.  K and V tiles go from HBM
// straight into LDS with buffer loads (double-buffered, no register
// staging, rows past the sequence read back as zeros).  Every wave keeps its
// Q rows in VGPRs for the whole loop, multiplies them against the K tile on
// the matrix cores, folds the tile into a running max and running sum
// (online softmax) and accumulates P.V on the matrix cores.  The score
// matrix never leaves registers.  This is the forward pass behind the
// scaled-dot-product attention node of nvFuser issue #2278 "Investigate a
// new SDPA IR node", with the variable-length modes of AOTriton PR #31 "Add
// varlen support to AOTriton's Flash Attention".
//
// Register layout.  The kernel computes S^T = K . Q^T and O^T = V^T . P^T
// with v_mfma_f32_32x32x16_{bf16,f16} (v_mfma_f32_32x32x2_f32 for fp32
// inputs).  In a 32x32 accumulator lane l holds column l % 32, so in both
// products every lane holds values of ONE query row (i = l % 32): the row
// max, the row sum and the per-row rescale of O are in-lane, apart from one
// v_permlane32_swap to combine the two half-waves (lanes l and l ^ 32 share
// a row).  The accumulator of S^T therefore feeds the second product as its
// B operand directly.  Accumulator register r of lane l holds row
// rho = 8*(r/4) + 4*(l/32) + r%4; K rows are loaded in the order
// key_of(rho) = 16*(l/32) + r so that each half-wave holds 16 consecutive
// keys of its query row.
//
// Software pipeline.  Iteration t turns the scores of tile t into
// probabilities (VALU) while the matrix cores compute the scores of tile
// t+1, then accumulates P(t).V(t) (matrix cores) while the VALU takes the row
// max of tile t+1.  Tile t+2's K and tile t+1's V are in flight meanwhile.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fwd_args.h"

namespace sdpa03 {

using f32x16 = float __attribute__((ext_vector_type(16)));
using f32x4 = float __attribute__((ext_vector_type(4)));
using bf16x8 = __bf16 __attribute__((ext_vector_type(8)));
using f16x8 = _Float16 __attribute__((ext_vector_type(8)));
using lds_void_ptr = __attribute__((address_space(3))) void*;

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.6931471805599453f;
// O and l are rescaled only when a row max grows by more than this many
// powers of two (a wave-uniform decision); until then exponents are taken
// against the stale max, so p <= 2^8 and the fp32 sums stay exact enough.
constexpr float kRescaleLog2 = 8.0f;
// Fourth dword of a raw buffer descriptor on gfx9 (32-bit data format).
constexpr int kBufferFlags = 0x00020000;

// Key index (within a 32-key block) loaded into accumulator row rho.
__device__ __forceinline__ int key_of(int rho) {
  return ((rho >> 2) & 1) * 16 + (rho >> 3) * 4 + (rho & 3);
}

// XOR swizzle of the 16-byte chunks of a K row in LDS, chosen so that the
// 128-bit fragment reads of key_of() rows hit distinct banks.
template <int NCH>
__device__ __forceinline__ int chunk_swizzle(int r) {
  if constexpr (NCH == 8) {
    return ((r >> 1) & 1) | (((r ^ (r >> 2)) & 1) << 1) | (((r >> 4) & 1) << 2);
  } else {
    return (r & 3) | (((r >> 4) & 1) << 2) | (((r >> 2) & 1) << 3);
  }
}

__device__ __forceinline__ float max_across_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_across_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// ---------------------------------------------------------------------------
// Matrix-core paths.  Each provides: Q fragments held in registers, the
// S^T = K Q^T product from a K tile in LDS, the probabilities P of a score
// tile, and O^T += V^T P^T from a V tile in LDS.  Tiles in LDS are row-major
// [key][dim] with 16-byte chunks XOR-swizzled per row.
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

// bf16 / fp16: one 32x32x16 product per 16 elements of the contraction.
template <typename T, int D>
struct Path16 {
  static constexpr int kChunks = D / 8;  // 16-byte chunks per row
  static constexpr int kQFrags = D / 16;
  using frag = typename Mma16<T>::frag;
  struct QRegs {
    frag f[kQFrags];
  };
  template <int NB>
  struct PRegs {
    frag f[NB][2];
  };

  // Q^T operand of k-step ks: lane (i, h) holds Q[i][16ks + 8h .. +8].
  __device__ static __forceinline__ void load_q(const T* row, bool ok, int lh, QRegs& q) {
#pragma unroll
    for (int ks = 0; ks < kQFrags; ++ks) {
      q.f[ks] = ok ? *reinterpret_cast<const frag*>(row + 16 * ks + 8 * lh) : frag{};
    }
  }

  template <int NB>
  __device__ static __forceinline__ void qk(const T* k_tile, const QRegs& q, int li, int lh,
                                            f32x16 (&s)[NB]) {
#pragma unroll
    for (int ks = 0; ks < kQFrags; ++ks) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int r = nb * 32 + key_of(li);
        const int ch = 2 * ks + lh;
        const frag a = *reinterpret_cast<const frag*>(
            k_tile + r * D + ((ch ^ chunk_swizzle<kChunks>(r)) * 8));
        s[nb] = Mma16<T>::mma(a, q.f[ks], s[nb]);
      }
    }
  }

  // V rows keep their 16-byte chunks XOR-swizzled too, so that the
  // transposing reads in pv() (4 rows x 32 bytes per 16 lanes) hit distinct
  // banks.
  __device__ static __forceinline__ int v_swizzle(int r) {
    if constexpr (kChunks == 16) {
      return (r & 3) << 2;
    } else {
      return ((r >> 1) & 1) << 2;
    }
  }

  // p = 2^(s*c2 - m) for every score, rounded to T for the second product;
  // returns this half-wave's fp32 sum of the tile's p.
  template <int NB>
  __device__ static __forceinline__ float softmax_p(const f32x16 (&s)[NB], float c2, float m_sub,
                                                    PRegs<NB>& p) {
    float tile_sum = 0.f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = __builtin_amdgcn_exp2f(fmaf(s[nb][r], c2, -m_sub));
#pragma unroll
      for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int e = 0; e < 8; ++e) p.f[nb][half][e] = static_cast<T>(x[half * 8 + e]);
      }
      tile_sum += tree_sum16(x);
    }
    return tile_sum;
  }

  // O^T += V^T P^T.  p.f[nb][half] holds the weights of keys
  // 32nb + 16h + 8half .. +8 for this lane's row (the B operand of one
  // k-step).  The A operand needs V[key .. key+7][d] (eight keys, one column
  // d = the lane's li) -- a transposed access.  ds_read_b64_tr_b16 serves it:
  // within each group of 16 lanes, lane i receives element (i & 3) of the
  // 64-bit words read by lanes 4j + (i >> 2), j = 0..3.  If lane t of the
  // group points at row R0 + t/4, column C0 + 4(t & 3), lane i therefore
  // receives V[R0 + j][C0 + i] for j = 0..3: four consecutive keys of its
  // own column.  Two such reads (R0 and R0 + 4) give the eight keys of one
  // operand.
  template <int NB, int DB>
  __device__ static __forceinline__ void pv(const T* v_tile, const PRegs<NB>& p, int lane,
                                            f32x16 (&acc)[DB]) {
    using s16x4 = short __attribute__((ext_vector_type(4)));
    const int t = lane & 15;
    const int grp = lane >> 4;
    const int row_lane = (grp >> 1) * 16 + (t >> 2);    // + 32nb + 8half + 4sub
    const int col_lane = (grp & 1) * 16 + 4 * (t & 3);  // + 32db
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          s16x4 w[2];
#pragma unroll
          for (int sub = 0; sub < 2; ++sub) {
            const int row = nb * 32 + half * 8 + sub * 4 + row_lane;
            const int col = db * 32 + col_lane;
            const T* src = v_tile + row * D + (((col >> 3) ^ v_swizzle(row)) << 3) + (col & 7);
            w[sub] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)(src));
          }
          frag vf;
          __builtin_memcpy(&vf, w, sizeof(vf));
          acc[db] = Mma16<T>::mma(vf, p.f[nb][half], acc[db]);
        }
      }
    }
  }
};

// fp32: one 32x32x2 product per 2 elements of the contraction; P stays fp32.
template <int D>
struct Path32 {
  static constexpr int kChunks = D / 4;
  static constexpr int kGroups = D / 8;  // groups of 4 k-steps = 8 dims
  struct QRegs {
    f32x4 f[kGroups];
  };
  template <int NB>
  struct PRegs {
    f32x16 f[NB];
  };

  // k-step 4g + e covers dims 8g + e (lanes 0..31) and 8g + 4 + e (32..63).
  __device__ static __forceinline__ void load_q(const float* row, bool ok, int lh, QRegs& q) {
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
      q.f[g] = ok ? *reinterpret_cast<const f32x4*>(row + 8 * g + 4 * lh) : f32x4{};
    }
  }

  template <int NB>
  __device__ static __forceinline__ void qk(const float* k_tile, const QRegs& q, int li, int lh,
                                            f32x16 (&s)[NB]) {
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int r = nb * 32 + key_of(li);
        const int ch = 2 * g + lh;
        const f32x4 a = *reinterpret_cast<const f32x4*>(
            k_tile + r * D + ((ch ^ chunk_swizzle<kChunks>(r)) * 4));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], q.f[g][e], s[nb], 0, 0, 0);
        }
      }
    }
  }

  // V rows are stored unswizzled; each lane reads single fp32 elements.
  __device__ static __forceinline__ int v_swizzle(int) { return 0; }

  template <int NB>
  __device__ static __forceinline__ float softmax_p(const f32x16 (&s)[NB], float c2, float m_sub,
                                                    PRegs<NB>& p) {
    float tile_sum = 0.f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        x[r] = __builtin_amdgcn_exp2f(fmaf(s[nb][r], c2, -m_sub));
        p.f[nb][r] = x[r];
      }
      tile_sum += tree_sum16(x);
    }
    return tile_sum;
  }

  // O^T += V^T P^T with one key per k-step: lane (i, h) supplies p[nb][r]
  // (key 32nb + 16h + r) and V[32nb + 16h + r][32db + i].
  template <int NB, int DB>
  __device__ static __forceinline__ void pv(const float* v_tile, const PRegs<NB>& p, int lane,
                                            f32x16 (&acc)[DB]) {
    const int li = lane & 31;
    const int lh = lane >> 5;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float* vrow = v_tile + (nb * 32 + lh * 16 + r) * D + li;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vrow[db * 32], p.f[nb][r], acc[db], 0, 0, 0);
        }
      }
    }
  }
};

template <typename T, int D>
struct PathFor {
  using type = Path16<T, D>;
};
template <int D>
struct PathFor<float, D> {
  using type = Path32<D>;
};

// ---------------------------------------------------------------------------
// Tile copies: buffer loads straight into LDS
// ---------------------------------------------------------------------------
// buffer_load_dwordx4 ... lds writes lane L's 16 bytes to (wave-uniform LDS
// base + 16 L): one instruction fills 1 KiB of LDS from 64 independent
// source offsets.  A K or V tile is BN rows of D elements and each wave
// issues its share of the tile's 1 KiB blocks.  The swizzled LDS layout
// comes from choosing, for LDS position p of row r, the source chunk
// p ^ swizzle(r).  The buffer descriptor starts at the tile's first row and
// covers only the rows that exist, so rows past the sequence read back as
// zeros with no bounds arithmetic.  Source offsets are 32-bit: the host
// limits row strides accordingly.

template <typename T, int D, int BN, int NW>
struct TileCopy {
  static constexpr int kRowBytes = D * static_cast<int>(sizeof(T));
  static constexpr int kRowsPerInst = 1024 / kRowBytes;
  static constexpr int kInstPerTile = BN * kRowBytes / 1024;
  static_assert(kInstPerTile % NW == 0, "tile copy must split evenly over the waves");
  static constexpr int kInstPerWave = kInstPerTile / NW;
  static constexpr int kChunks = kRowBytes / 16;

  uint32_t voff[kInstPerWave];

  // Source offsets of this lane's chunks; Path supplies the row swizzle of K
  // (for_v false) or of V (for_v true).
  template <typename Path, bool for_v>
  __device__ __forceinline__ void init(int wave, int lane, int64_t row_bytes) {
    const int lr = lane / kChunks;
    const int lp = lane % kChunks;
#pragma unroll
    for (int i = 0; i < kInstPerWave; ++i) {
      const int r = (wave * kInstPerWave + i) * kRowsPerInst + lr;
      const int swz = for_v ? Path::v_swizzle(r) : chunk_swizzle<Path::kChunks>(r);
      voff[i] = static_cast<uint32_t>(r * row_bytes) + static_cast<uint32_t>((lp ^ swz) << 4);
    }
  }

  // Rows [0, valid_rows) of the tile starting at `tile` land in `lds_tile`.
  __device__ __forceinline__ void issue(const char* tile, int64_t valid_rows, int64_t row_bytes,
                                        T* lds_tile, int wave) const {
    // hipcc's host (x86) pass parses this body too but has no buffer-resource
    // type; left visible there, it stops the host pass from emitting the
    // launch stubs of later kernel instantiations.
#if defined(__HIP_DEVICE_COMPILE__)
    int64_t bytes = valid_rows * row_bytes;
    bytes = bytes < 0 ? 0 : (bytes > 0xFFFFFFFFll ? 0xFFFFFFFFll : bytes);
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(tile), 0, static_cast<int>(static_cast<uint32_t>(bytes)), kBufferFlags);
    char* lds = reinterpret_cast<char*>(lds_tile) + wave * kInstPerWave * 1024;
#pragma unroll
    for (int i = 0; i < kInstPerWave; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_ptr)(lds + i * 1024), 16, voff[i],
                                               0, 0, 0);
    }
#endif
  }
};

// ---------------------------------------------------------------------------
// Tile bookkeeping
// ---------------------------------------------------------------------------

// Workgroups are dealt round-robin to the 8 XCDs.  Remap the launch index so
// each XCD runs a contiguous range of logical tiles (whole heads, sharing
// that XCD's L2), and within a head start with the last query tile (the
// heaviest one under a causal mask).
__device__ __forceinline__ void decode_tile(int m_tiles, int num_heads, int& z, int& h, int& m) {
  const uint32_t n = blockIdx.x;
  const uint32_t per_xcd = gridDim.x >> 3;
  uint32_t logical = n;
  if (n < (per_xcd << 3)) logical = (n & 7u) * per_xcd + (n >> 3);
  const uint32_t mt = logical % static_cast<uint32_t>(m_tiles);
  const uint32_t rest = logical / static_cast<uint32_t>(m_tiles);
  m = m_tiles - 1 - static_cast<int>(mt);
  h = static_cast<int>(rest % static_cast<uint32_t>(num_heads));
  z = static_cast<int>(rest / static_cast<uint32_t>(num_heads));
}

struct SeqRange {
  int64_t b;    // batch index into the rank-4 view
  int q_start;  // first token of the sequence along seq (compact), else 0
  int k_start;
  int len_q;
  int len_k;
};

// Rows and keys of program z.  Dense: batch z, all rows.  Compact: batch 0,
// tokens [cu[z], cu[z+1]).  Padded: batch z, lengths cu[z+1] - cu[z] from
// offset 0 (the padded branch of the fwd_kernel.py excerpt quoted in
// AOTriton PR #31).  Ranges are clamped to the addressable rows so that
// malformed cu_seqlens can never move an access out of bounds: compact
// token ranges to [0, total), padded lengths to [0, padded length].
template <int MODE>
__device__ __forceinline__ SeqRange seq_range(const FwdArgs& a, int z) {
  SeqRange r;
  if constexpr (MODE == MODE_DENSE) {
    r.b = z;
    r.q_start = 0;
    r.k_start = 0;
    r.len_q = a.seqlen_q;
    r.len_k = a.seqlen_k;
  } else if constexpr (MODE == MODE_COMPACT) {
    const int q0 = min(max(a.cu_q[z], 0), a.total_q);
    const int q1 = min(max(a.cu_q[z + 1], q0), a.total_q);
    const int k0 = min(max(a.cu_k[z], 0), a.total_k);
    const int k1 = min(max(a.cu_k[z + 1], k0), a.total_k);
    r.b = 0;
    r.q_start = q0;
    r.k_start = k0;
    r.len_q = min(q1 - q0, a.seqlen_q);
    r.len_k = min(k1 - k0, a.seqlen_k);
  } else {
    const int64_t lq = static_cast<int64_t>(a.cu_q[z + 1]) - a.cu_q[z];
    const int64_t lk = static_cast<int64_t>(a.cu_k[z + 1]) - a.cu_k[z];
    r.b = z;
    r.q_start = 0;
    r.k_start = 0;
    r.len_q = static_cast<int>(min(max(lq, int64_t(0)), static_cast<int64_t>(a.seqlen_q)));
    r.len_k = static_cast<int>(min(max(lk, int64_t(0)), static_cast<int64_t>(a.seqlen_k)));
  }
  return r;
}

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------

template <typename T, int D, int NW, int BN, int MODE, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 2) void attn_fwd_kernel(FwdArgs a) {
  using Path = typename PathFor<T, D>::type;
  using Copy = TileCopy<T, D, BN, NW>;
  using PRegs = typename Path::template PRegs<BN / 32>;
  constexpr int BM = NW * 32;
  constexpr int NB = BN / 32;
  constexpr int DB = D / 32;

  // Four separate LDS arrays (not one [2][...] array): each gets its own
  // alias scope, so the compiler can see that fragment reads of one buffer do
  // not depend on the buffer loads still landing in the other one, and need
  // not wait for them.
  __shared__ __attribute__((aligned(1024))) T k_lds0[BN * D];
  __shared__ __attribute__((aligned(1024))) T k_lds1[BN * D];
  __shared__ __attribute__((aligned(1024))) T v_lds0[BN * D];
  __shared__ __attribute__((aligned(1024))) T v_lds1[BN * D];

  int z, h, m;
  decode_tile(a.m_tiles, a.num_heads, z, h, m);
  const SeqRange sr = seq_range<MODE>(a, z);
  const int m0 = m * BM;
  if (m0 >= sr.len_q) return;  // uniform over the workgroup

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 31;
  const int lh = lane >> 5;

  const T* qp = static_cast<const T*>(a.q) + sr.b * a.q_sb + h * a.q_sh +
                static_cast<int64_t>(sr.q_start) * a.q_ss;
  const char* kp = reinterpret_cast<const char*>(
      static_cast<const T*>(a.k) + sr.b * a.k_sb + h * a.k_sh +
      static_cast<int64_t>(sr.k_start) * a.k_ss);
  const char* vp = reinterpret_cast<const char*>(
      static_cast<const T*>(a.v) + sr.b * a.v_sb + h * a.v_sh +
      static_cast<int64_t>(sr.k_start) * a.v_ss);
  T* op = static_cast<T*>(a.o) + sr.b * a.o_sb + h * a.o_sh +
          static_cast<int64_t>(sr.q_start) * a.o_ss;
  float* lsep = a.lse + sr.b * a.lse_sb + h * a.lse_sh + sr.q_start;

  const int row0 = m0 + wave * 32;  // first query row of this wave
  const int qi = row0 + li;         // this lane's query row
  const bool row_ok = qi < sr.len_q;

  int kend = sr.len_k;
  if constexpr (CAUSAL) kend = min(kend, min(m0 + BM, sr.len_q));
  const int n_tiles = (kend + BN - 1) / BN;

  const int64_t k_row_bytes = a.k_ss * static_cast<int64_t>(sizeof(T));
  const int64_t v_row_bytes = a.v_ss * static_cast<int64_t>(sizeof(T));
  Copy kcopy, vcopy;
  kcopy.template init<Path, false>(wave, lane, k_row_bytes);
  vcopy.template init<Path, true>(wave, lane, v_row_bytes);
  // Tile t lives in buffer t & 1.  Every call below names its buffers
  // directly (the loop is unrolled by two), so after inlining each LDS access
  // refers to a known array.
  auto issue_k = [&](int t, T* buf) {
    const int j0 = t * BN;
    kcopy.issue(kp + j0 * k_row_bytes, sr.len_k - j0, k_row_bytes, buf, wave);
  };
  auto issue_v = [&](int t, T* buf) {
    const int j0 = t * BN;
    vcopy.issue(vp + j0 * v_row_bytes, sr.len_k - j0, v_row_bytes, buf, wave);
  };

  typename Path::QRegs qr;
  Path::load_q(qp + static_cast<int64_t>(qi) * a.q_ss, row_ok, lh, qr);

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  float m_run = kNegInf;  // running max of scale*log2(e)*s, this row
  float l_run = 0.f;      // running sum of this half-wave's weights
  float alpha = 1.f;      // pending rescale of acc and l (when rescale is set)
  bool rescale = false;
  const float c2 = a.scale_log2;

  // Scores of tile t (masked where needed) into s; k_tile holds K(t).
  auto scores = [&](int t, const T* k_tile, f32x16 (&s)[NB]) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) s[nb] = f32x16{};
    Path::template qk<NB>(k_tile, qr, li, lh, s);
    const int j0 = t * BN;
    const bool need_mask = (j0 + BN > sr.len_k) || (CAUSAL && j0 + BN - 1 > row0);
    if (need_mask) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + nb * 32 + lh * 16 + r;
          const bool ok = key < sr.len_k && (!CAUSAL || key <= qi);
          if (!ok) s[nb][r] = kNegInf;
        }
      }
    }
  };
  // Fold the row max of s into m_run; a growth beyond the threshold in any
  // row of the wave schedules a rescale of acc and l.
  auto update_max = [&](const f32x16 (&s)[NB]) {
    float mx = kNegInf;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[nb][r]);
    }
    mx = max_across_halves(mx) * c2;  // scale > 0, so max commutes with it
    const bool grow = mx > m_run + kRescaleLog2;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float m_new = fmaxf(m_run, mx);
      alpha = (m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      rescale = true;
      m_run = m_new;
    }
  };

  f32x16 s[NB];
  if (n_tiles > 0) {
    issue_k(0, k_lds0);
    issue_v(0, v_lds0);
    if (n_tiles > 1) issue_k(1, k_lds1);
    wait_vmem();
    __syncthreads();
    scores(0, k_lds0, s);
    update_max(s);
    __syncthreads();  // every wave is done with K(0) before K(2) replaces it
  }

  // One pipeline step for tile t: (k_cur, v_cur) are the buffers of parity
  // t & 1 (K(t+2) and V(t) live there), (k_nxt, v_nxt) the other parity
  // (K(t+1) and V(t+1)).
  auto step = [&](int t, T* k_cur, T* v_cur, T* k_nxt, T* v_nxt) {
    const bool has_next = t + 1 < n_tiles;
    if (t + 2 < n_tiles) issue_k(t + 2, k_cur);
    if (has_next) issue_v(t + 1, v_nxt);

    if (rescale) {  // the max grew at tile t: bring acc and l to the new base
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
      rescale = false;
    }
    const float m_sub = (m_run == kNegInf) ? 0.f : m_run;

    // Phase A: probabilities of tile t (VALU) || scores of tile t+1 (MFMA).
    PRegs p;
    l_run += Path::template softmax_p<NB>(s, c2, m_sub, p);
    f32x16 s_next[NB];
    if (has_next) scores(t + 1, k_nxt, s_next);

    // Phase B: O += P(t) V(t) (MFMA) || row max of tile t+1 (VALU).
    Path::template pv<NB, DB>(v_cur, p, lane, acc);
    if (has_next) {
      update_max(s_next);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) s[nb] = s_next[nb];
    }

    wait_vmem();
    __syncthreads();
  };
  for (int t = 0; t < n_tiles; t += 2) {
    step(t, k_lds0, v_lds0, k_lds1, v_lds1);
    if (t + 1 < n_tiles) step(t + 1, k_lds1, v_lds1, k_lds0, v_lds0);
  }

  // Epilogue: O = acc / l, LSE = (m + log2 l) * ln 2, valid rows only.
  const float l_tot = sum_across_halves(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (row_ok) {
    T* orow = op + static_cast<int64_t>(qi) * a.o_ss;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        T out4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) out4[e] = static_cast<T>(acc[db][4 * g + e] * inv);
        T* dst = orow + db * 32 + g * 8 + lh * 4;
        if constexpr (sizeof(T) == 4) {
          *reinterpret_cast<f32x4*>(dst) = f32x4{out4[0], out4[1], out4[2], out4[3]};
        } else {
          uint2 packed;
          __builtin_memcpy(&packed, out4, 8);
          *reinterpret_cast<uint2*>(dst) = packed;
        }
      }
    }
    if (lh == 0) {
      lsep[qi] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : kNegInf;
    }
  }
}

// ---------------------------------------------------------------------------
// Dispatch: the compiled-in table and the launcher
// ---------------------------------------------------------------------------

#include "dispatch_table.inc"

namespace {

template <typename T, int D, int MODE, bool CAUSAL>
int launch_typed(const FwdArgs& a, hipStream_t stream) {
  constexpr TableEntry e = table_entry<T, D>();
  const uint32_t grid = static_cast<uint32_t>(a.m_tiles) * a.num_heads * a.num_z;
  hipLaunchKernelGGL((attn_fwd_kernel<T, D, e.waves, e.block_n, MODE, CAUSAL>), dim3(grid),
                     dim3(e.waves * 64), 0, stream, a);
  return static_cast<int>(hipGetLastError());
}

template <typename T, int D>
int launch_mode(const FwdArgs& a, int mode, bool causal, hipStream_t s) {
  switch (mode) {
    case MODE_DENSE:
      return causal ? launch_typed<T, D, MODE_DENSE, true>(a, s) : launch_typed<T, D, MODE_DENSE, false>(a, s);
    case MODE_COMPACT:
      return causal ? launch_typed<T, D, MODE_COMPACT, true>(a, s) : launch_typed<T, D, MODE_COMPACT, false>(a, s);
    default:
      return causal ? launch_typed<T, D, MODE_PADDED, true>(a, s) : launch_typed<T, D, MODE_PADDED, false>(a, s);
  }
}

template <typename T>
int launch_dim(const FwdArgs& a, int head_dim, int mode, bool causal, hipStream_t s) {
  return head_dim == 64 ? launch_mode<T, 64>(a, mode, causal, s) : launch_mode<T, 128>(a, mode, causal, s);
}

}  // namespace

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

int launch_attn_fwd(const FwdArgs& a, int dtype, int head_dim, int mode, bool causal, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  switch (dtype) {
    case DT_F32: return launch_dim<float>(a, head_dim, mode, causal, s);
    case DT_F16: return launch_dim<_Float16>(a, head_dim, mode, causal, s);
    default: return launch_dim<__bf16>(a, head_dim, mode, causal, s);
  }
}

}  // namespace sdpa03
