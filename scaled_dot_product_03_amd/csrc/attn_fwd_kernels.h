// Flash-attention forward kernels for CDNA4 (gfx950): the kernel templates
// and their typed launchers, included by attn_fwd.hip (dispatch, split
// forward) and attn_fwd_{bf16,f16,f32}.hip (one element type each).
//
// One workgroup computes block_m = 32 * waves query rows of one
// (batch or sequence, head); each wavefront owns 32 rows.  The workgroup
// walks the key axis in tiles of block_n keys.  K and V tiles go from HBM
// straight into LDS with buffer loads (two or three LDS stages, no register
// staging, rows past the sequence read back as zeros).  Every wave keeps its
// Q rows in VGPRs for the whole loop, multiplies them against the K tile on
// the matrix cores, folds the tile into a running reference max and running
// sum (online softmax) and accumulates P.V on the matrix cores.  The score
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
// B operand directly.  Accumulator register r of lane l holds key
// 8*(r/4) + 4*(l/32) + r%4 of its 32-key block.
//
// LDS layout.  Tiles are row-major [key][dim] with padded rows, chosen for
// gfx950's 64 banks of 4 bytes: the 16 consecutive K rows that one 128-bit
// fragment read touches land in 16 distinct 16-byte bank groups, and the 4
// V rows of one transposing read land in 4 distinct 64-byte bank blocks.
// Padding (not an XOR swizzle) keeps every fragment address "one per-lane
// base + an immediate offset", which saves dozens of address registers.
//
// Software pipeline.  Step t turns the scores of tile t into probabilities
// (VALU) while the matrix cores compute the scores of tile t+1, then
// accumulates P(t).V(t) on the matrix cores.  Later tiles' K and V are in
// flight meanwhile.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_common.h"
#include "fwd_args.h"

namespace sdpa03 {

// Exponents are taken against a stale reference max as long as each lane's
// sum of a tile's weights stays at or below this bound (so no weight exceeds
// it); a larger sum (a wave-uniform decision) triggers an exact max and a
// rescale.
constexpr float kSumLimit = 4096.0f;

// LDS row strides (bytes) of K and V tiles for element size ES and head
// dim D.  K: 16 bytes of padding per row shifts consecutive rows by one
// 16-byte bank group.  V (16-bit): 64 bytes shift consecutive rows by a
// quarter of the 256-byte bank cycle.  V (fp32): 32 bytes put rows r and
// r+4, which one fp32 read pairs, in opposite halves of the banks.
template <int ES, int D>
constexpr int k_lds_row_bytes() { return D * ES + 16; }
template <int ES, int D>
constexpr int v_lds_row_bytes() { return ES == 2 ? D * ES + 64 : D * ES + 32; }

// bf16 / fp16: one 32x32x16 product per 16 elements of the contraction.
template <typename T, int D>
struct Path16 {
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

  static constexpr int kRowK = k_lds_row_bytes<2, D>();
  static constexpr int kRowV = v_lds_row_bytes<2, D>();

  // A operand of k-step ks: lane (rho, h) reads K[32nb + rho][16ks + 8h ..+8]
  // -- rho is the lane's li, so the address is a per-lane base plus an
  // immediate.
  template <int NB>
  __device__ static __forceinline__ void qk(const T* k_tile, const QRegs& q, int li, int lh,
                                            f32x16 (&s)[NB]) {
    const char* base = reinterpret_cast<const char*>(k_tile) + li * kRowK + lh * 16;
#pragma unroll
    for (int ks = 0; ks < kQFrags; ++ks) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const frag a = *reinterpret_cast<const frag*>(base + nb * 32 * kRowK + ks * 32);
        s[nb] = Mma16<T>::mma(a, q.f[ks], s[nb]);
      }
    }
  }

  // An empty asm statement that takes the P fragments as operands: the
  // compiler must have computed them at this point (it would otherwise sink
  // the softmax past the masking branch that follows, next to its use).
  template <int NB>
  __device__ static __forceinline__ void pin(PRegs<NB>& p) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) asm volatile("" : "+v"(p.f[nb][half]));
    }
  }

  // Scheduling requests for the two pipeline phases (sched_group_barrier
  // masks: 0x008 MFMA, 0x100 LDS read, 0x002 VALU).  Phase A: keep a few K
  // fragment reads ahead, then one MFMA, one read and a share of the softmax
  // VALU work.  Phase B: two transposing V reads and a little VALU per MFMA.
  template <int NB>
  __device__ static __forceinline__ void interleave_qk() {
    constexpr int n_mfma = NB * kQFrags;
    constexpr int valu_per = (NB * 16 * 3 + n_mfma - 1) / n_mfma;
    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
    for (int i = 0; i < n_mfma; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, valu_per, 0);
    }
  }
  template <int NB, int DB>
  __device__ static __forceinline__ void interleave_pv() {
    constexpr int n_mfma = NB * 2 * DB;
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < n_mfma; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  }

  // One C interval of the ping-pong schedule: the scores of the next tile
  // and P.V of the current one, both on the matrix cores; keep a few LDS
  // reads ahead of the products.
  template <int NB, int DB>
  __device__ static __forceinline__ void interleave_c() {
    constexpr int n_mfma = NB * kQFrags + NB * 2 * DB;
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < n_mfma; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  }

  // p = 2^(s*c2 - m) for every score, rounded to T for the second product;
  // returns this lane's fp32 sum of the unrounded p.  (A sum of the rounded
  // weights would be cheaper -- v_dot2_f32_bf16 against (1, 1) -- but for rows
  // that see only a few keys its rounding error reaches 2^-9 of l, which the
  // logsumexp output cannot afford.)
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

  // O^T += V^T P^T.  Register r of lane (i, h) holds the weight of key
  // 32nb + 8(r/4) + 4h + r%4, so k-step (nb, half) -- registers 8half..+8 --
  // covers keys 32nb + 16half + {4h..4h+3, 8+4h..8+4h+3}, and its A operand
  // needs V at those eight keys in the lane's column d = li: a transposed
  // access.  ds_read_b64_tr_b16 serves it: within each group of 16 lanes,
  // lane i receives element (i & 3) of the 64-bit words read by lanes
  // 4j + (i >> 2), j = 0..3.  If lane t of the group points at row
  // R0 + t/4, column C0 + 4(t & 3), lane i therefore receives V[R0 + j][C0 + i]
  // for j = 0..3: four consecutive keys of its own column.  Two such reads
  // (R0 = 32nb + 16half + 4h and R0 + 8) give the eight keys of one operand.
  template <int NB, int DB>
  __device__ static __forceinline__ void pv(const T* v_tile, const PRegs<NB>& p, int lane,
                                            f32x16 (&acc)[DB]) {
    using s16x4 = short __attribute__((ext_vector_type(4)));
    const int t = lane & 15;
    const int grp = lane >> 4;
    const int row_lane = (grp >> 1) * 4 + (t >> 2);
    const int col_lane = (grp & 1) * 16 + 4 * (t & 3);
    const char* base = reinterpret_cast<const char*>(v_tile) + row_lane * kRowV + col_lane * 2;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          s16x4 w[2];
#pragma unroll
          for (int sub = 0; sub < 2; ++sub) {
            const char* src = base + (nb * 32 + half * 16 + sub * 8) * kRowV + db * 64;
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

  static constexpr int kRowK = k_lds_row_bytes<4, D>();
  static constexpr int kRowV = v_lds_row_bytes<4, D>();

  template <int NB>
  __device__ static __forceinline__ void qk(const float* k_tile, const QRegs& q, int li, int lh,
                                            f32x16 (&s)[NB]) {
    const char* base = reinterpret_cast<const char*>(k_tile) + li * kRowK + lh * 16;
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(base + nb * 32 * kRowK + g * 32);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], q.f[g][e], s[nb], 0, 0, 0);
        }
      }
    }
  }

  template <int NB>
  __device__ static __forceinline__ void pin(PRegs<NB>&) {}

  // fp32 is a correctness path: no scheduling requests.
  template <int NB>
  __device__ static __forceinline__ void interleave_qk() {}
  template <int NB, int DB>
  __device__ static __forceinline__ void interleave_pv() {}

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
  // (key 32nb + 8(r/4) + 4h + r%4) and V at that key in column 32db + i.
  template <int NB, int DB>
  __device__ static __forceinline__ void pv(const float* v_tile, const PRegs<NB>& p, int lane,
                                            f32x16 (&acc)[DB]) {
    const int li = lane & 31;
    const int lh = lane >> 5;
    const char* base = reinterpret_cast<const char*>(v_tile) + lh * 4 * kRowV + li * 4;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const char* vrow = base + (nb * 32 + 8 * (r >> 2) + (r & 3)) * kRowV;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const float vv = *reinterpret_cast<const float*>(vrow + db * 128);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv, p.f[nb][r], acc[db], 0, 0, 0);
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

// The additive bias of one key tile for this lane's query row.  Element r of
// block nb is the bias of key j0 + 32 nb + 8 (r / 4) + 4 h + r % 4: the key
// whose score register r of the 32x32 accumulator holds, in both paths.  Each
// group of four registers covers four consecutive keys, so a whole tile
// takes 4 NB vector loads of 4 elements per lane.  The tile that crosses the
// end of the keys, and a row whose keys start off a 4-element boundary (a
// compact sequence at any token), load key by key, only keys < len_k.
template <typename T, int NB>
struct BiasTile {
  T b[NB][16];

  __device__ __forceinline__ void load(const T* row, int j0, int len_k, int lh, bool vec) {
    if (vec && j0 + NB * 32 <= len_k) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          __builtin_memcpy(&b[nb][4 * g],
                           __builtin_assume_aligned(row + j0 + nb * 32 + 8 * g + 4 * lh,
                                                    4 * sizeof(T)),
                           4 * sizeof(T));
        }
      }
    } else {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + nb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
          b[nb][r] = key < len_k ? row[key] : T(0.f);
        }
      }
    }
  }

  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) b[nb][r] = T(0.f);
    }
  }

  // s <- scale * s + bias: the biased scores in natural-log units.
  __device__ __forceinline__ void fold(f32x16 (&s)[NB], float scale) const {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[nb][r] = fmaf(s[nb][r], scale, static_cast<float>(b[nb][r]));
    }
  }
};

// ---------------------------------------------------------------------------
// Tile bookkeeping
// ---------------------------------------------------------------------------

// Workgroups are dealt round-robin to the 8 XCDs, in launch order.
//
// Without a causal mask every query tile costs the same: the launch index
// is remapped so each XCD runs a contiguous range of logical tiles (whole
// heads, sharing that XCD's L2).  In a split forward the splits of one head
// follow each other, so the workgroups that read one key range of a head
// share an XCD too.
//
// Under a causal mask query tile m costs m + 1 key tiles.  Heaviest-first
// within each head still leaves long tiles starting late (a model of 64
// workgroup slots puts the makespan at 1.5 times the average load); here the
// launch index runs over (batch, head[, split]) fastest and over query tiles
// from the last one down, so all the heaviest tiles start first.  Consecutive
// launch indices walk the heads and land on consecutive XCDs, so every XCD
// gets the same mix of tile costs, and with a multiple of 8 (batch, head)
// groups each head stays on one XCD.
template <bool CAUSAL, bool SPLIT>
__device__ __forceinline__ void decode_tile(int m_tiles, int num_heads, int num_z, int num_splits,
                                            int& z, int& h, int& m, int& split) {
  const uint32_t n = blockIdx.x;
  if constexpr (CAUSAL) {
    const uint32_t per_split = static_cast<uint32_t>(num_heads) * static_cast<uint32_t>(num_z);
    const uint32_t groups = SPLIT ? per_split * static_cast<uint32_t>(num_splits) : per_split;
    const uint32_t g = n % groups;
    m = m_tiles - 1 - static_cast<int>(n / groups);
    uint32_t rest = g;
    split = 0;
    if constexpr (SPLIT) {
      split = static_cast<int>(rest % static_cast<uint32_t>(num_splits));
      rest /= static_cast<uint32_t>(num_splits);
    }
    h = static_cast<int>(rest % static_cast<uint32_t>(num_heads));
    z = static_cast<int>(rest / static_cast<uint32_t>(num_heads));
    return;
  }
  const uint32_t per_xcd = gridDim.x >> 3;
  uint32_t logical = n;
  if (n < (per_xcd << 3)) logical = (n & 7u) * per_xcd + (n >> 3);
  const uint32_t mt = logical % static_cast<uint32_t>(m_tiles);
  uint32_t rest = logical / static_cast<uint32_t>(m_tiles);
  m = m_tiles - 1 - static_cast<int>(mt);
  split = 0;
  if constexpr (SPLIT) {
    split = static_cast<int>(rest % static_cast<uint32_t>(num_splits));
    rest /= static_cast<uint32_t>(num_splits);
  }
  h = static_cast<int>(rest % static_cast<uint32_t>(num_heads));
  z = static_cast<int>(rest / static_cast<uint32_t>(num_heads));
}

// Rows and keys of program z (the shared rule in attn_common.h).
template <int MODE>
__device__ __forceinline__ SeqRange seq_range(const FwdArgs& a, int z) {
  return seq_range_of<MODE>(a.cu_q, a.cu_k, a.total_q, a.total_k, a.seqlen_q, a.seqlen_k, z);
}

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------

// STAGES LDS buffers each for K and V tiles (2 or 3).  With 3, a tile load
// issued at step t is first needed at step t+2, so it has two steps of
// compute to hide its latency behind.
// SPLIT: key-parallel dense forward.  The workgroup covers the key tiles of
// its split only and writes a normalised fp32 partial output and its
// logsumexp to the workspace; a second kernel merges the splits.
// BIAS: an additive bias joins the scores.  Each step loads the next tile's
// bias into registers before it issues its tile copies and adds it after
// P.V, so the loads have the whole step to land; the scores then hold
// scale * q.k + bias (natural-log units) and the softmax multiplies by
// log2(e) alone.
template <typename T, int D, int NW, int BN, int STAGES, int MODE, bool CAUSAL, bool SPLIT,
          bool BIAS>
__device__ __forceinline__ void attn_fwd_body(const FwdArgs& a, T* k_lds0, T* k_lds1, T* k_lds2,
                                              T* v_lds0, T* v_lds1, T* v_lds2) {
  static_assert(STAGES == 2 || STAGES == 3, "two or three LDS stages");
  static_assert(!SPLIT || MODE == MODE_DENSE, "the split forward serves the dense mode");
  static_assert(!(SPLIT && BIAS), "the split forward has no bias");
  using Path = typename PathFor<T, D>::type;
  using KCopy = TileCopy<T, D, BN, NW, Path::kRowK>;
  using VCopy = TileCopy<T, D, BN, NW, Path::kRowV>;
  using PRegs = typename Path::template PRegs<BN / 32>;
  constexpr int BM = NW * 32;
  constexpr int NB = BN / 32;
  constexpr int DB = D / 32;
  // Loads one step issues per wave; with three stages they may still be in
  // flight when the step ends.
  constexpr int kLoadsPerStep = KCopy::kInstPerWave + VCopy::kInstPerWave;
  constexpr int kInFlightAtStepEnd = (STAGES - 2) * kLoadsPerStep;

  int z, h, m, split;
  decode_tile<CAUSAL, SPLIT>(a.m_tiles, a.num_heads, a.num_z, a.num_splits, z, h, m, split);
  const SeqRange sr = seq_range<MODE>(a, z);
  const int m0 = m * BM;
  if (m0 >= sr.len_q) return;  // uniform over the workgroup

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps tile-copy addresses scalar
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
  // Key tiles [tile0, tile0 + n_tiles): all of them, or this split's share
  // (possibly none: an empty split still writes its partial result).
  int tile0 = 0;
  int n_tiles = (kend + BN - 1) / BN;
  if constexpr (SPLIT) {
    tile0 = split * a.split_tiles;
    n_tiles = max(0, min(n_tiles - tile0, a.split_tiles));
  }

  const int64_t k_row_bytes = a.k_ss * static_cast<int64_t>(sizeof(T));
  const int64_t v_row_bytes = a.v_ss * static_cast<int64_t>(sizeof(T));
  KCopy kcopy;
  VCopy vcopy;
  kcopy.init(wave, lane, k_row_bytes);
  vcopy.init(wave, lane, v_row_bytes);
  // Tile t lives in buffer t % STAGES.  Every call below names its buffers
  // directly (the loop is unrolled by STAGES), so after inlining each LDS
  // access refers to a known array.  Rows at or past `end` are not fetched
  // (they read back as zeros); a load past the last tile fetches nothing.
  auto issue_k = [&](int t, T* buf, int end) {
    const int j0 = (tile0 + t) * BN;
    kcopy.issue(kp + j0 * k_row_bytes, end - j0, k_row_bytes, buf, wave);
  };
  auto issue_v = [&](int t, T* buf, int end) {
    const int j0 = (tile0 + t) * BN;
    vcopy.issue(vp + j0 * v_row_bytes, end - j0, v_row_bytes, buf, wave);
  };

  typename Path::QRegs qr;
  Path::load_q(qp + static_cast<int64_t>(qi) * a.q_ss, row_ok, lh, qr);

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  float m_run = kNegInf;  // reference (stale) max of scale*log2(e)*s, this row
  float l_run = 0.f;      // running sum of this half-wave's weights
  const float c2 = BIAS ? kLog2e : a.scale_log2;

  // This lane's bias row (the sequence's block of the bias view).  Vector
  // loads need the block to start on a 4-element boundary; the strides are
  // multiples of 4 elements, so only the key offset decides.
  using Bias = BiasTile<T, NB>;
  const T* bias_row = nullptr;
  bool bias_vec = false;
  if constexpr (BIAS) {
    bias_row = static_cast<const T*>(a.bias) + sr.b * a.bias_sb + h * a.bias_sh +
               (static_cast<int64_t>(sr.q_start) + qi) * a.bias_sq + sr.k_start;
    bias_vec = (sr.k_start & 3) == 0;
  }
  auto load_bias = [&](int t, Bias& bt) {
    if (row_ok) {
      bt.load(bias_row, (tile0 + t) * BN, sr.len_k, lh, bias_vec);
    } else {
      bt.zero();
    }
  };

  // Masks the scores of tile t where keys run past the sequence or, under
  // the causal mask, past the lane's row (only tail and diagonal tiles).
  auto mask_tile = [&](int t, f32x16 (&s)[NB]) {
    const int j0 = (tile0 + t) * BN;
    const bool need_mask = (j0 + BN > sr.len_k) || (CAUSAL && j0 + BN - 1 > row0);
    if (need_mask) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + nb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
          const bool ok = key < sr.len_k && (!CAUSAL || key <= qi);
          if (!ok) s[nb][r] = kNegInf;
        }
      }
    }
  };
  // Row max of a score tile in scaled log2 units (scale > 0, so the max
  // commutes with the scaling).
  auto tile_max = [&](const f32x16 (&s)[NB]) {
    float mx = kNegInf;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[nb][r]);
    }
    return max_across_halves(mx) * c2;
  };
  // Probabilities of score tile s against the running reference m_run,
  // into p; returns this lane's share of the tile's row sum.  The reference
  // only has to keep every p bounded, not to equal the row max: while a
  // tile's sums stay <= 2^12 (so every p <= 2^12) nothing else is done.
  // Otherwise -- and on the first tile a row sees -- the exact row max is
  // taken, acc and l are rescaled to it, and p is recomputed (p <= 1).  The
  // result is unchanged: O = acc / l and LSE = m + log2 l for any m.
  auto probabilities = [&](const f32x16 (&s)[NB], PRegs& p) {
    const float m_sub = (m_run == kNegInf) ? 0.f : m_run;
    float tile_sum = Path::template softmax_p<NB>(s, c2, m_sub, p);
    const bool redo = !(tile_sum <= kSumLimit) || m_run == kNegInf;
    if (__builtin_amdgcn_ballot_w64(redo) != 0) {
      const float m_new = fmaxf(m_run, tile_max(s));
      const float alpha = (m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
      m_run = m_new;
      tile_sum = Path::template softmax_p<NB>(s, c2, (m_run == kNegInf) ? 0.f : m_run, p);
    }
    return tile_sum;
  };

  f32x16 s[NB];
  Bias bias_next;
  if (n_tiles > 0) {
    if constexpr (BIAS) load_bias(0, bias_next);
    issue_k(0, k_lds0, kend);
    issue_k(1, k_lds1, 1 < n_tiles ? kend : 0);
    issue_v(0, v_lds0, kend);
    if constexpr (STAGES > 2) {
      issue_k(2, k_lds2, 2 < n_tiles ? kend : 0);
      issue_v(1, v_lds1, 1 < n_tiles ? kend : 0);
    }
    wait_vmem();
    barrier_lds();
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) s[nb] = f32x16{};
    Path::template qk<NB>(k_lds0, qr, li, lh, s);
    if constexpr (BIAS) bias_next.fold(s, a.scale);
    mask_tile(0, s);
    barrier_lds();  // every wave is done with K(0) before K(STAGES) replaces it
  }

  // Under the causal mask a wave whose rows all precede the first key of
  // tile t has nothing left to add: tile t and every later one are masked
  // for all its rows.  Such a wave still issues its share of the tile copies
  // and meets every barrier, but skips the products and the softmax (a
  // wave-uniform branch).  The result is unchanged: the skipped weights are
  // exactly 0 and a tile without weights never triggers a rescale.  With
  // 256-row workgroups this removes 12 of the 32 wave-tiles of each diagonal
  // block.
  auto wave_done = [&](int t) { return CAUSAL && (tile0 + t) * BN > row0 + 31; };

  // Pipeline step for tile t when tile t+1 exists.  k_cur holds K(t) (done
  // with; K(t+STAGES) is loaded into it), k_nxt holds K(t+1), v_cur holds V(t)
  // and v_pre receives V(t+STAGES-1).  Phase A is straight-line code, so the
  // scheduler can interleave the softmax VALU work with the next tile's
  // score MFMAs.
  auto step = [&](int t, T* k_cur, T* k_nxt, T* v_cur, T* v_pre) {
    // The next tile's bias goes out before the tile copies, so waiting for it
    // never waits for them (also when this wave skips the tile: a
    // conditional load would keep two copies of the bias registers alive).
    if constexpr (BIAS) load_bias(t + 1, bias_next);
    issue_k(t + STAGES, k_cur, t + STAGES < n_tiles ? kend : 0);
    issue_v(t + STAGES - 1, v_pre, t + STAGES - 1 < n_tiles ? kend : 0);
    if (!wave_done(t)) {

    // Phase A: probabilities of tile t (VALU) || scores of tile t+1 (MFMA).
    PRegs p;
    f32x16 s_next[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) s_next[nb] = f32x16{};
    const float m_sub = (m_run == kNegInf) ? 0.f : m_run;
    float tile_sum = Path::template softmax_p<NB>(s, c2, m_sub, p);
    Path::template qk<NB>(k_nxt, qr, li, lh, s_next);
    Path::pin(p);  // P is computed here, beside the MFMAs, not after the branch
    Path::template interleave_qk<NB>();
    const bool redo = !(tile_sum <= kSumLimit) || m_run == kNegInf;
    if (__builtin_amdgcn_ballot_w64(redo) != 0) {  // rare: see probabilities()
      const float m_new = fmaxf(m_run, tile_max(s));
      const float alpha = (m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
      m_run = m_new;
      tile_sum = Path::template softmax_p<NB>(s, c2, (m_run == kNegInf) ? 0.f : m_run, p);
    }
    l_run += tile_sum;
    if constexpr (!BIAS) mask_tile(t + 1, s_next);

    // Phase B: O += P(t) V(t) on the matrix cores.
    Path::template pv<NB, DB>(v_cur, p, lane, acc);
    Path::template interleave_pv<NB, DB>();
    if constexpr (BIAS) {
      bias_next.fold(s_next, a.scale);
      mask_tile(t + 1, s_next);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) s[nb] = s_next[nb];
    }  // !wave_done(t)

    // K(t+2) and V(t+1) -- issued one step earlier with three stages, in
    // this step with two -- must have landed before the next step.
    wait_vmem_allow<kInFlightAtStepEnd>();
    barrier_lds();
  };
  // The last tile: probabilities and P.V only.
  auto last_step = [&](const T* v_cur) {
    if (wave_done(n_tiles - 1)) return;
    PRegs p;
    l_run += probabilities(s, p);
    Path::template pv<NB, DB>(v_cur, p, lane, acc);
  };

  // Each step body exists once (unrolled by STAGES so that every step names
  // its buffers at compile time); the loop leaves as soon as the next tile
  // would be the last one, and the last tile's V buffer is picked at run time
  // (the last step issues no loads, so nothing can be in flight into it).
  if (n_tiles > 0) {
    for (int t = 0;; t += STAGES) {
      if (t + 1 >= n_tiles) break;
      step(t, k_lds0, k_lds1, v_lds0, STAGES == 2 ? v_lds1 : v_lds2);
      if (t + 2 >= n_tiles) break;
      if constexpr (STAGES == 2) {
        step(t + 1, k_lds1, k_lds0, v_lds1, v_lds0);
      } else {
        step(t + 1, k_lds1, k_lds2, v_lds1, v_lds0);
        if (t + 3 >= n_tiles) break;
        step(t + 2, k_lds2, k_lds0, v_lds2, v_lds1);
      }
    }
    const int last = (n_tiles - 1) % STAGES;
    last_step(last == 0 ? v_lds0 : (last == 1 ? v_lds1 : v_lds2));
  }

  // Epilogue: O = acc / l, LSE = (m + log2 l) * ln 2, valid rows only.
  const float l_tot = sum_across_halves(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if constexpr (SPLIT) {
    if (row_ok) {
      const int64_t row = (static_cast<int64_t>(split) * a.num_z + z) * a.num_heads * sr.len_q +
                          static_cast<int64_t>(h) * sr.len_q + qi;
      float* wrow = a.ws_o + row * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          *reinterpret_cast<f32x4*>(wrow + db * 32 + g * 8 + lh * 4) =
              f32x4{acc[db][4 * g] * inv, acc[db][4 * g + 1] * inv, acc[db][4 * g + 2] * inv,
                    acc[db][4 * g + 3] * inv};
        }
      }
      if (lh == 0) a.ws_lse[row] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : kNegInf;
    }
    return;
  }
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
// Ping-pong schedule (16-bit inputs)
// ---------------------------------------------------------------------------
// Eight waves in two groups of four: waves w and w + 4 run on the same SIMD,
// so every SIMD holds one wave of each group.  A wave alternates two kinds
// of interval: C(n) -- matrix-core work: scores of tile n+1 (K(n+1) Q^T) and
// O += P(n) V(n) -- and S(n) -- vector work: mask and probabilities of tile
// n.  Group 1 runs one interval behind group 0, and every interval ends at a
// workgroup barrier, so on each SIMD one wave's softmax always runs beside
// the other wave's matrix products.
//
// With global interval j (group 0 runs its local interval u at j = u, group
// 1 at j = u + 1; u = 0 is the first tile's scores, then S(n) at u = 2n+1
// and C(n) at u = 2n+2), K(n) is read at j = 2n and 2n+1, V(n) at j = 2n+2
// and 2n+3.  Tiles rotate through STAGES buffers (tile n in buffer
// n % STAGES).  At the start of C(n) each wave issues its share of K(n +
// STAGES) into K(n)'s buffer and of V(n + STAGES - 1) into V(n - 1)'s: the
// last readers of both finished by global interval 2n+1, and C(n) starts at
// j >= 2n+2.  At the end of C(n) each wave waits until only the loads it
// issued in the last STAGES - 2 C intervals are in flight, so a tile issued
// in C(n) has landed after C(n + STAGES - 2) -- before its first reader at
// j = 2(n + STAGES) (K) or 2(n + STAGES - 1) + 2 (V).
template <typename T, int D, int BN, int STAGES, int MODE, bool CAUSAL>
__device__ __forceinline__ void attn_fwd_pingpong_body(const FwdArgs& a, T* k_lds0, T* k_lds1,
                                                       T* k_lds2, T* v_lds0, T* v_lds1,
                                                       T* v_lds2) {
  static_assert(sizeof(T) == 2, "the ping-pong schedule serves 16-bit inputs");
  static_assert(STAGES == 2 || STAGES == 3, "two or three LDS stages");
  constexpr int NW = 8;
  using Path = Path16<T, D>;
  using KCopy = TileCopy<T, D, BN, NW, Path::kRowK>;
  using VCopy = TileCopy<T, D, BN, NW, Path::kRowV>;
  using PRegs = typename Path::template PRegs<BN / 32>;
  constexpr int BM = NW * 32;
  constexpr int NB = BN / 32;
  constexpr int DB = D / 32;
  constexpr int kLoadsPerTile = KCopy::kInstPerWave + VCopy::kInstPerWave;
  constexpr int kInFlight = (STAGES - 2) * kLoadsPerTile;

  int z, h, m, split;
  decode_tile<CAUSAL, false>(a.m_tiles, a.num_heads, a.num_z, 1, z, h, m, split);
  const SeqRange sr = seq_range<MODE>(a, z);
  const int m0 = m * BM;
  if (m0 >= sr.len_q) return;  // uniform over the workgroup

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2;
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

  const int row0 = m0 + wave * 32;
  const int qi = row0 + li;
  const bool row_ok = qi < sr.len_q;

  int kend = sr.len_k;
  if constexpr (CAUSAL) kend = min(kend, min(m0 + BM, sr.len_q));
  const int n_tiles = (kend + BN - 1) / BN;

  const int64_t k_row_bytes = a.k_ss * static_cast<int64_t>(sizeof(T));
  const int64_t v_row_bytes = a.v_ss * static_cast<int64_t>(sizeof(T));
  KCopy kcopy;
  VCopy vcopy;
  kcopy.init(wave, lane, k_row_bytes);
  vcopy.init(wave, lane, v_row_bytes);
  auto issue_k = [&](int t, T* buf) {
    const int j0 = t * BN;
    kcopy.issue_untracked(kp + j0 * k_row_bytes, t < n_tiles ? kend - j0 : 0, k_row_bytes, buf,
                          wave);
  };
  auto issue_v = [&](int t, T* buf) {
    const int j0 = t * BN;
    vcopy.issue_untracked(vp + j0 * v_row_bytes, t < n_tiles ? kend - j0 : 0, v_row_bytes, buf,
                          wave);
  };

  typename Path::QRegs qr;
  Path::load_q(qp + static_cast<int64_t>(qi) * a.q_ss, row_ok, lh, qr);

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  float m_run = kNegInf;
  float l_run = 0.f;
  const float c2 = a.scale_log2;

  // Same masking and lazy-reference softmax as the single-group schedule.
  auto mask_tile = [&](int t, f32x16 (&s)[NB]) {
    const int j0 = t * BN;
    const bool need_mask = (j0 + BN > sr.len_k) || (CAUSAL && j0 + BN - 1 > row0);
    if (need_mask) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + nb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
          const bool ok = key < sr.len_k && (!CAUSAL || key <= qi);
          if (!ok) s[nb][r] = kNegInf;
        }
      }
    }
  };
  auto tile_max = [&](const f32x16 (&s)[NB]) {
    float mx = kNegInf;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[nb][r]);
    }
    return max_across_halves(mx) * c2;
  };
  auto probabilities = [&](const f32x16 (&s)[NB], PRegs& p) {
    const float m_sub = (m_run == kNegInf) ? 0.f : m_run;
    float tile_sum = Path::template softmax_p<NB>(s, c2, m_sub, p);
    const bool redo = !(tile_sum <= kSumLimit) || m_run == kNegInf;
    if (__builtin_amdgcn_ballot_w64(redo) != 0) {
      const float m_new = fmaxf(m_run, tile_max(s));
      const float alpha = (m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= alpha;
      m_run = m_new;
      tile_sum = Path::template softmax_p<NB>(s, c2, (m_run == kNegInf) ? 0.f : m_run, p);
    }
    return tile_sum;
  };

  f32x16 s[NB];
  PRegs p;
  if (n_tiles > 0) {
    // Prologue: Q (loaded above) and K(0) land before the first barrier;
    // K(i) and V(i-1), i < STAGES, stay in flight behind the first scores.
    // (Q's loads are the compiler's: the full wait settles them before any
    // untracked tile load is issued.)
    issue_k(0, k_lds0);
    wait_vmem();
    barrier_lds();
    issue_k(1, k_lds1);
    issue_v(0, v_lds0);
    if constexpr (STAGES > 2) {
      issue_k(2, k_lds2);
      issue_v(1, v_lds1);
    }
    if (group == 1) barrier_lds();  // group 1 sits out global interval 0

    // u = 0: scores of tile 0.
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) s[nb] = f32x16{};
    Path::template qk<NB>(k_lds0, qr, li, lh, s);
    wait_vmem_allow<kInFlight>();  // K(1) and V(0) have landed
    barrier_lds();

    // S(n): vector work on tile n's scores.
    auto s_interval = [&](int n) {
      mask_tile(n, s);
      l_run += probabilities(s, p);
      barrier_lds();
    };
    // C(n) for n + 1 < n_tiles.  k_cur: K(n)'s buffer (receives K(n+STAGES));
    // k_nxt: K(n+1); v_cur: V(n); v_pre: receives V(n+STAGES-1).
    // The loads are issued unconditionally (tiles past the end fetch zero
    // rows into buffers nobody reads again): a branch around them would make
    // the compiler lose track of which buffer each load writes and wait for
    // all of them before the first fragment read.
    auto c_interval = [&](int n, T* k_cur, T* k_nxt, T* v_cur, T* v_pre) {
      issue_k(n + STAGES, k_cur);
      issue_v(n + STAGES - 1, v_pre);
      f32x16 s_next[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) s_next[nb] = f32x16{};
      Path::template qk<NB>(k_nxt, qr, li, lh, s_next);
      Path::template pv<NB, DB>(v_cur, p, lane, acc);
      Path::template interleave_c<NB, DB>();
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) s[nb] = s_next[nb];
      wait_vmem_allow<kInFlight>();
      barrier_lds();
    };

    for (int n = 0;; n += STAGES) {
      if (n + 1 >= n_tiles) break;
      s_interval(n);
      c_interval(n, k_lds0, k_lds1, v_lds0, STAGES == 2 ? v_lds1 : v_lds2);
      if (n + 2 >= n_tiles) break;
      s_interval(n + 1);
      if constexpr (STAGES == 2) {
        c_interval(n + 1, k_lds1, k_lds0, v_lds1, v_lds0);
      } else {
        c_interval(n + 1, k_lds1, k_lds2, v_lds1, v_lds0);
        if (n + 3 >= n_tiles) break;
        s_interval(n + 2);
        c_interval(n + 2, k_lds2, k_lds0, v_lds2, v_lds1);
      }
    }
    // Last tile: S(T-1), then C(T-1) = P.V only.  Group 1's last interval is
    // the workgroup's last, so it ends without a barrier (every wave passes
    // the same number of barriers).
    s_interval(n_tiles - 1);
    const int last = (n_tiles - 1) % STAGES;
    const T* v_last = last == 0 ? v_lds0 : (last == 1 ? v_lds1 : v_lds2);
    Path::template pv<NB, DB>(v_last, p, lane, acc);
    wait_vmem();
    if (group == 0) barrier_lds();
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
        uint2 packed;
        __builtin_memcpy(&packed, out4, 8);
        *reinterpret_cast<uint2*>(orow + db * 32 + g * 8 + lh * 4) = packed;
      }
    }
    if (lh == 0) {
      lsep[qi] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : kNegInf;
    }
  }
}

template <typename T, int D, int BN, int STAGES, int MODE, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void attn_fwd_pingpong_kernel(FwdArgs a) {
  using Path = Path16<T, D>;
  constexpr int kKElems = TileCopy<T, D, BN, 8, Path::kRowK>::kArrayBytes / 2;
  constexpr int kVElems = TileCopy<T, D, BN, 8, Path::kRowV>::kArrayBytes / 2;
  __shared__ __attribute__((aligned(1024))) T k_lds0[kKElems];
  __shared__ __attribute__((aligned(1024))) T k_lds1[kKElems];
  __shared__ __attribute__((aligned(1024))) T v_lds0[kVElems];
  __shared__ __attribute__((aligned(1024))) T v_lds1[kVElems];
  if constexpr (STAGES > 2) {
    __shared__ __attribute__((aligned(1024))) T k_lds2[kKElems];
    __shared__ __attribute__((aligned(1024))) T v_lds2[kVElems];
    attn_fwd_pingpong_body<T, D, BN, STAGES, MODE, CAUSAL>(a, k_lds0, k_lds1, k_lds2, v_lds0,
                                                           v_lds1, v_lds2);
  } else {
    attn_fwd_pingpong_body<T, D, BN, STAGES, MODE, CAUSAL>(a, k_lds0, k_lds1, k_lds0, v_lds0,
                                                           v_lds1, v_lds0);
  }
}

// The kernel: declares the LDS buffers its stage count needs and runs the
// body.  Separate LDS arrays per buffer (not one [STAGES][...] array): each
// gets its own alias scope, so the compiler can see that fragment reads of
// one buffer do not depend on the buffer loads still landing in another,
// and need not wait for them.
template <typename T, int D, int NW, int BN, int STAGES, int MODE, bool CAUSAL, bool SPLIT,
          bool BIAS>
__global__ __launch_bounds__(NW * 64, 2) void attn_fwd_kernel(FwdArgs a) {
  using Path = typename PathFor<T, D>::type;
  constexpr int kKElems = TileCopy<T, D, BN, NW, Path::kRowK>::kArrayBytes / static_cast<int>(sizeof(T));
  constexpr int kVElems = TileCopy<T, D, BN, NW, Path::kRowV>::kArrayBytes / static_cast<int>(sizeof(T));
  __shared__ __attribute__((aligned(1024))) T k_lds0[kKElems];
  __shared__ __attribute__((aligned(1024))) T k_lds1[kKElems];
  __shared__ __attribute__((aligned(1024))) T v_lds0[kVElems];
  __shared__ __attribute__((aligned(1024))) T v_lds1[kVElems];
  if constexpr (STAGES > 2) {
    __shared__ __attribute__((aligned(1024))) T k_lds2[kKElems];
    __shared__ __attribute__((aligned(1024))) T v_lds2[kVElems];
    attn_fwd_body<T, D, NW, BN, STAGES, MODE, CAUSAL, SPLIT, BIAS>(a, k_lds0, k_lds1, k_lds2,
                                                                   v_lds0, v_lds1, v_lds2);
  } else {
    attn_fwd_body<T, D, NW, BN, STAGES, MODE, CAUSAL, SPLIT, BIAS>(a, k_lds0, k_lds1, k_lds0,
                                                                   v_lds0, v_lds1, v_lds0);
  }
}

// ---------------------------------------------------------------------------
// Merge of a split forward
// ---------------------------------------------------------------------------
// Split s of a row holds O_s (normalised over its own keys) and LSE_s.  The
// row's result is LSE = log sum_s exp(LSE_s) and O = sum_s exp(LSE_s - LSE)
// O_s: each O_s is a softmax-weighted mean over its keys, and exp(LSE_s) is
// the total weight of those keys.  A split that saw no key has LSE_s = -inf
// and weight 0; a row with no key at all gets O = 0 and LSE = -inf.  One
// thread per (row, 4 consecutive dims); the work is a few bytes of traffic
// per output element, bounded by HBM.
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_fwd_merge_kernel(MergeArgs a) {
  constexpr int kChunks = D / 4;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t row = gid / kChunks;
  if (row >= a.ws_rows) return;
  const int c = static_cast<int>(gid % kChunks);
  float m = kNegInf;
  for (int sp = 0; sp < a.num_splits; ++sp) m = fmaxf(m, a.ws_lse[sp * a.ws_rows + row]);
  float w_sum = 0.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  if (m != kNegInf) {
    for (int sp = 0; sp < a.num_splits; ++sp) {
      const int64_t r = sp * a.ws_rows + row;
      const float w = expf(a.ws_lse[r] - m);
      const f32x4 part = *reinterpret_cast<const f32x4*>(a.ws_o + r * D + 4 * c);
      w_sum += w;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = fmaf(w, part[e], acc[e]);
    }
  }
  const float inv = w_sum > 0.f ? 1.f / w_sum : 0.f;
  const int64_t i = row % a.seqlen_q;
  const int64_t zh = row / a.seqlen_q;
  const int64_t h = zh % a.num_heads;
  const int64_t z = zh / a.num_heads;
  T* dst = static_cast<T*>(a.o) + z * a.o_sb + h * a.o_sh + i * a.o_ss + 4 * c;
  if constexpr (sizeof(T) == 4) {
    *reinterpret_cast<f32x4*>(dst) = f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
  } else {
    T out4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) out4[e] = static_cast<T>(acc[e] * inv);
    uint2 packed;
    __builtin_memcpy(&packed, out4, 8);
    *reinterpret_cast<uint2*>(dst) = packed;
  }
  if (c == 0) a.lse[z * a.lse_sb + h * a.lse_sh + i] = m == kNegInf ? kNegInf : m + logf(w_sum);
}

// ---------------------------------------------------------------------------
// Dispatch: the compiled-in table and the launcher
// ---------------------------------------------------------------------------

#include "dispatch_table.inc"

namespace {

template <typename T, int D, int MODE, bool CAUSAL, bool BIAS, int BUCKET>
int launch_bucket(const FwdArgs& a, hipStream_t stream) {
  constexpr TableEntry e = launch_entry<T, D, BUCKET, BIAS>();
  const uint32_t grid = static_cast<uint32_t>(a.m_tiles) * a.num_heads * a.num_z;
  if constexpr (e.pingpong != 0) {
    static_assert(e.waves == 8 && sizeof(T) == 2, "ping-pong: 8 waves, 16-bit inputs");
    hipLaunchKernelGGL((attn_fwd_pingpong_kernel<T, D, e.block_n, e.stages, MODE, CAUSAL>),
                       dim3(grid), dim3(512), 0, stream, a);
  } else {
    hipLaunchKernelGGL(
        (attn_fwd_kernel<T, D, e.waves, e.block_n, e.stages, MODE, CAUSAL, false, BIAS>),
        dim3(grid), dim3(e.waves * 64), 0, stream, a);
  }
  return static_cast<int>(hipGetLastError());
}

// The bucket of the dispatch key comes from the sequence extents the kernel
// arguments carry (the longest sequence in the varlen layouts).
template <typename T, int D, int MODE, bool CAUSAL, bool BIAS>
int launch_typed(const FwdArgs& a, hipStream_t s) {
  switch (seq_bucket(a.seqlen_q, a.seqlen_k)) {
    case 0: return launch_bucket<T, D, MODE, CAUSAL, BIAS, 0>(a, s);
    case 1: return launch_bucket<T, D, MODE, CAUSAL, BIAS, 1>(a, s);
    case 2: return launch_bucket<T, D, MODE, CAUSAL, BIAS, 2>(a, s);
    case 3: return launch_bucket<T, D, MODE, CAUSAL, BIAS, 3>(a, s);
    case 4: return launch_bucket<T, D, MODE, CAUSAL, BIAS, 4>(a, s);
    case 5: return launch_bucket<T, D, MODE, CAUSAL, BIAS, 5>(a, s);
    case 6: return launch_bucket<T, D, MODE, CAUSAL, BIAS, 6>(a, s);
    default: return launch_bucket<T, D, MODE, CAUSAL, BIAS, 7>(a, s);
  }
}

template <typename T, int D, bool CAUSAL, int BUCKET>
int launch_split_bucket(const FwdArgs& a, const MergeArgs& mg, hipStream_t stream) {
  constexpr TableEntry e = launch_entry<T, D, BUCKET, true>();
  const uint32_t grid =
      static_cast<uint32_t>(a.m_tiles) * a.num_heads * a.num_z * static_cast<uint32_t>(a.num_splits);
  hipLaunchKernelGGL((attn_fwd_kernel<T, D, e.waves, e.block_n, e.stages, MODE_DENSE, CAUSAL, true, false>),
                     dim3(grid), dim3(e.waves * 64), 0, stream, a);
  int err = static_cast<int>(hipGetLastError());
  if (err != 0) return err;
  const int64_t threads = mg.ws_rows * (D / 4);
  hipLaunchKernelGGL((attn_fwd_merge_kernel<T, D>), dim3(static_cast<uint32_t>((threads + 255) / 256)),
                     dim3(256), 0, stream, mg);
  return static_cast<int>(hipGetLastError());
}

template <typename T, int D, bool CAUSAL>
int launch_split_typed(const FwdArgs& a, const MergeArgs& mg, hipStream_t s) {
  switch (seq_bucket(a.seqlen_q, a.seqlen_k)) {
    case 0: return launch_split_bucket<T, D, CAUSAL, 0>(a, mg, s);
    case 1: return launch_split_bucket<T, D, CAUSAL, 1>(a, mg, s);
    case 2: return launch_split_bucket<T, D, CAUSAL, 2>(a, mg, s);
    case 3: return launch_split_bucket<T, D, CAUSAL, 3>(a, mg, s);
    case 4: return launch_split_bucket<T, D, CAUSAL, 4>(a, mg, s);
    case 5: return launch_split_bucket<T, D, CAUSAL, 5>(a, mg, s);
    case 6: return launch_split_bucket<T, D, CAUSAL, 6>(a, mg, s);
    default: return launch_split_bucket<T, D, CAUSAL, 7>(a, mg, s);
  }
}

// The table entry a launch will use, at run time (host side).
template <typename T, int D, bool SINGLE_GROUP>
TableEntry entry_for(int bucket) {
  switch (bucket) {
    case 0: return launch_entry<T, D, 0, SINGLE_GROUP>();
    case 1: return launch_entry<T, D, 1, SINGLE_GROUP>();
    case 2: return launch_entry<T, D, 2, SINGLE_GROUP>();
    case 3: return launch_entry<T, D, 3, SINGLE_GROUP>();
    case 4: return launch_entry<T, D, 4, SINGLE_GROUP>();
    case 5: return launch_entry<T, D, 5, SINGLE_GROUP>();
    case 6: return launch_entry<T, D, 6, SINGLE_GROUP>();
    default: return launch_entry<T, D, 7, SINGLE_GROUP>();
  }
}

template <typename T, int D, bool BIAS>
int launch_mode(const FwdArgs& a, int mode, bool causal, hipStream_t s) {
  switch (mode) {
    case MODE_DENSE:
      return causal ? launch_typed<T, D, MODE_DENSE, true, BIAS>(a, s)
                    : launch_typed<T, D, MODE_DENSE, false, BIAS>(a, s);
    case MODE_COMPACT:
      return causal ? launch_typed<T, D, MODE_COMPACT, true, BIAS>(a, s)
                    : launch_typed<T, D, MODE_COMPACT, false, BIAS>(a, s);
    default:
      return causal ? launch_typed<T, D, MODE_PADDED, true, BIAS>(a, s)
                    : launch_typed<T, D, MODE_PADDED, false, BIAS>(a, s);
  }
}

}  // namespace

// The launches of one element type, with or without a bias.  Each element
// type's kernels are instantiated in a translation unit of their own
// (attn_fwd_{bf16,f16,f32}.hip, explicit instantiations below) so that they
// compile in parallel; other units only call these.
template <typename T, bool BIAS>
int launch_fwd_dtype(const FwdArgs& a, int head_dim, int mode, bool causal, hipStream_t s) {
  return head_dim == 64 ? launch_mode<T, 64, BIAS>(a, mode, causal, s)
                        : launch_mode<T, 128, BIAS>(a, mode, causal, s);
}

extern template int launch_fwd_dtype<__bf16, false>(const FwdArgs&, int, int, bool, hipStream_t);
extern template int launch_fwd_dtype<__bf16, true>(const FwdArgs&, int, int, bool, hipStream_t);
extern template int launch_fwd_dtype<_Float16, false>(const FwdArgs&, int, int, bool, hipStream_t);
extern template int launch_fwd_dtype<_Float16, true>(const FwdArgs&, int, int, bool, hipStream_t);
extern template int launch_fwd_dtype<float, false>(const FwdArgs&, int, int, bool, hipStream_t);
extern template int launch_fwd_dtype<float, true>(const FwdArgs&, int, int, bool, hipStream_t);

}  // namespace sdpa03
