// Flash-attention forward kernels for CDNA4 (gfx950).
//
// One workgroup computes block_m = 32 * waves query rows of one
// (batch or sequence, head); each wavefront owns 32 rows.  The workgroup
// walks the key axis in tiles of block_n keys: K and V tiles are copied from
// HBM into LDS (double-buffered, 128-bit loads), every wave multiplies its Q
// rows (held in VGPRs for the whole loop) against the K tile on the matrix
// cores, folds the tile into a running max and running sum (online softmax),
// and accumulates P.V on the matrix cores.  The score matrix never leaves
// registers.  This is the forward pass behind the scaled-dot-product
// attention node of nvFuser issue #2278 "Investigate a new SDPA IR node",
// with the variable-length modes of AOTriton PR #31 "Add varlen support to
// AOTriton's Flash Attention".
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

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fwd_args.h"

namespace sdpa03 {

using f32x16 = float __attribute__((ext_vector_type(16)));
using f32x4 = float __attribute__((ext_vector_type(4)));
using bf16x8 = __bf16 __attribute__((ext_vector_type(8)));
using f16x8 = _Float16 __attribute__((ext_vector_type(8)));

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.6931471805599453f;
// O and l are rescaled only when a row max grows by more than this many
// powers of two (a wave-uniform decision); until then exponents are taken
// against the stale max, so p <= 2^8 and the fp32 sums stay exact enough.
constexpr float kRescaleLog2 = 8.0f;

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

// ---------------------------------------------------------------------------
// Matrix-core paths.  Each provides: Q fragments held in registers, the
// S^T = K Q^T product from a K tile in LDS, and O^T += V^T P^T from a V tile
// in LDS.  Tiles in LDS are row-major [key][dim]; K rows have their 16-byte
// chunks XOR-swizzled by chunk_swizzle(row).
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

// bf16 / fp16: one 32x32x16 product per 16 elements of the contraction.
template <typename T, int D>
struct Path16 {
  static constexpr int kElemsPerChunk = 8;
  static constexpr int kChunks = D / 8;
  static constexpr int kQFrags = D / 16;
  using frag = typename Mma16<T>::frag;
  struct QRegs {
    frag f[kQFrags];
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
            k_tile + r * D + ((ch ^ chunk_swizzle<kChunks>(r)) * kElemsPerChunk));
        s[nb] = Mma16<T>::mma(a, q.f[ks], s[nb]);
      }
    }
  }

  // V rows keep their 16-byte chunks XOR-swizzled too, so that the
  // transposing reads below (4 rows x 32 bytes per 16 lanes) hit distinct banks.
  __device__ static __forceinline__ int v_swizzle(int r) {
    if constexpr (kChunks == 16) {
      return (r & 3) << 2;
    } else {
      return ((r >> 1) & 1) << 2;
    }
  }

  // O^T += V^T P^T.  p[nb][r] is the weight of key 32nb + 16h + r for this
  // lane's row, so the B operand of k-step (nb, half) is p[nb][8half ..+8].
  // The A operand needs V[key .. key+7][d] (eight keys, one column d = the
  // lane's li) -- a transposed access.  ds_read_b64_tr_b16 serves it: within
  // each group of 16 lanes, lane i receives element (i & 3) of the 64-bit
  // words read by lanes 4j + (i >> 2), j = 0..3.  If lane t of the group
  // points at row R0 + t/4, column C0 + 4(t & 3), lane i therefore receives
  // V[R0 + j][C0 + i] for j = 0..3: four consecutive keys of its own column.
  // Two such reads (R0 and R0 + 4) give the eight keys of one operand.
  template <int NB, int DB>
  __device__ static __forceinline__ void pv(const T* v_tile, const f32x16 (&p)[NB], int lane,
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
        frag pf;
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[e] = static_cast<T>(p[nb][half * 8 + e]);
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
          acc[db] = Mma16<T>::mma(vf, pf, acc[db]);
        }
      }
    }
  }
};

// fp32: one 32x32x2 product per 2 elements of the contraction; P stays fp32.
template <int D>
struct Path32 {
  static constexpr int kElemsPerChunk = 4;
  static constexpr int kChunks = D / 4;
  static constexpr int kGroups = D / 8;  // groups of 4 k-steps = 8 dims
  struct QRegs {
    f32x4 f[kGroups];
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
            k_tile + r * D + ((ch ^ chunk_swizzle<kChunks>(r)) * kElemsPerChunk));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], q.f[g][e], s[nb], 0, 0, 0);
        }
      }
    }
  }

  // V rows are stored unswizzled; each lane reads single fp32 elements.
  __device__ static __forceinline__ int v_swizzle(int) { return 0; }

  // O^T += V^T P^T with one key per k-step: lane (i, h) supplies p[nb][r]
  // (key 32nb + 16h + r) and V[32nb + 16h + r][32db + i].
  template <int NB, int DB>
  __device__ static __forceinline__ void pv(const float* v_tile, const f32x16 (&p)[NB], int lane,
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
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vrow[db * 32], p[nb][r], acc[db], 0, 0, 0);
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
  constexpr int BM = NW * 32;
  constexpr int NT = NW * 64;
  constexpr int EPC = Path::kElemsPerChunk;
  constexpr int NCH = Path::kChunks;
  constexpr int TILE_CHUNKS = BN * NCH;
  static_assert(TILE_CHUNKS % NT == 0, "tile copy must split evenly over the workgroup");
  constexpr int CPT = TILE_CHUNKS / NT;
  constexpr int NB = BN / 32;
  constexpr int DB = D / 32;
  using chunk_t = f32x4;  // 16 bytes

  __shared__ __attribute__((aligned(16))) T k_lds[2][BN * D];
  __shared__ __attribute__((aligned(16))) T v_lds[2][BN * D];

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
  const T* kp = static_cast<const T*>(a.k) + sr.b * a.k_sb + h * a.k_sh +
                static_cast<int64_t>(sr.k_start) * a.k_ss;
  const T* vp = static_cast<const T*>(a.v) + sr.b * a.v_sb + h * a.v_sh +
                static_cast<int64_t>(sr.k_start) * a.v_ss;
  T* op = static_cast<T*>(a.o) + sr.b * a.o_sb + h * a.o_sh +
          static_cast<int64_t>(sr.q_start) * a.o_ss;
  float* lsep = a.lse + sr.b * a.lse_sb + h * a.lse_sh + sr.q_start;

  const int row0 = m0 + wave * 32;  // first query row of this wave
  const int qi = row0 + li;         // this lane's query row
  const bool row_ok = qi < sr.len_q;
  const bool wave_active = row0 < sr.len_q;
  const int wave_last_row = min(row0 + 31, sr.len_q - 1);

  typename Path::QRegs qr;
  Path::load_q(qp + static_cast<int64_t>(qi) * a.q_ss, row_ok, lh, qr);

  int kend = sr.len_k;
  if constexpr (CAUSAL) kend = min(kend, min(m0 + BM, sr.len_q));
  const int n_tiles = (kend + BN - 1) / BN;

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  float m_run = kNegInf;  // running max of scale*log2(e)*s, this row
  float l_run = 0.f;      // running sum of this half-wave's weights

  chunk_t k_stage[CPT], v_stage[CPT];
  auto global_load = [&](int j0) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int id = c * NT + tid;
      const int r = id / NCH;
      const int ch = id % NCH;
      const int key = j0 + r;
      if (key < sr.len_k) {
        k_stage[c] = *reinterpret_cast<const chunk_t*>(kp + static_cast<int64_t>(key) * a.k_ss + ch * EPC);
        v_stage[c] = *reinterpret_cast<const chunk_t*>(vp + static_cast<int64_t>(key) * a.v_ss + ch * EPC);
      } else {
        k_stage[c] = chunk_t{};
        v_stage[c] = chunk_t{};
      }
    }
  };
  auto lds_store = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int id = c * NT + tid;
      const int r = id / NCH;
      const int ch = id % NCH;
      *reinterpret_cast<chunk_t*>(&k_lds[buf][r * D + (ch ^ chunk_swizzle<NCH>(r)) * EPC]) = k_stage[c];
      *reinterpret_cast<chunk_t*>(&v_lds[buf][r * D + (ch ^ Path::v_swizzle(r)) * EPC]) = v_stage[c];
    }
  };

  if (n_tiles > 0) {
    global_load(0);
    lds_store(0);
  }
  __syncthreads();

  const float c2 = a.scale_log2;
  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    const int j0 = t * BN;
    if (t + 1 < n_tiles) global_load(j0 + BN);

    const bool skip = !wave_active || (CAUSAL && j0 > wave_last_row);
    if (!skip) {
      f32x16 s[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) s[nb] = f32x16{};
      Path::template qk<NB>(k_lds[buf], qr, li, lh, s);

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
        const float alpha = (m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] *= alpha;
        m_run = m_new;
      }
      const float m_sub = (m_run == kNegInf) ? 0.f : m_run;

#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(s[nb][r], c2, -m_sub));
          s[nb][r] = p;
          l_run += p;
        }
      }
      Path::template pv<NB, DB>(v_lds[buf], s, lane, acc);
    }

    if (t + 1 < n_tiles) lds_store(buf ^ 1);
    __syncthreads();
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
