// Flash-attention forward kernels for CDNA4 (gfx950): the kernel templates
// and their typed launchers, included by attn_fwd.hip (dispatch, split
// forward) and attn_fwd_{bf16,f16,f32}.hip (one element type each).
//
// One workgroup computes block_m = 32 * waves * row_blocks query rows of one
// (batch or sequence, head); each wavefront owns 32 rows (one row block) or
// 64 (two).  The workgroup walks the key axis in tiles of block_n keys.  K
// and V tiles go from HBM straight into LDS with buffer loads (two to four
// LDS stages, no register staging, rows past the sequence read back as
// zeros).  Every wave keeps its
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
// LDS layout.  Tiles are row-major [key][dim].  16-bit tiles of head dim
// 128 are unpadded and XOR-swizzled: the 16-byte chunk c of row r sits at chunk
// c ^ swizzle_of<D>(r) (attn_common.h), which keeps both the 128-bit K reads
// (one chunk of 16 consecutive rows per pass) and the transposing V reads
// (a 64-byte block of 4 rows per pass) free of bank conflicts on gfx950's 64
// banks of 4 bytes, while a tile takes exactly BN * D * 2 bytes.  A lane's
// chunk offsets then differ by XOR, not by a constant, so each lane keeps
// its offset for every K k-step and V dim block in registers, and the stage
// array's base and the row offsets ride in the instructions' immediates.
// Head dim 64 and fp32 tiles use padded rows instead (k_lds_row_bytes
// below); at head dim 64 the swizzle measured no faster.
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

// LDS row strides (bytes) of padded K and V tiles for element size ES and
// head dim D.  K: 16 bytes of padding per row shifts consecutive rows by one
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

  // Head dim 128: swizzled, unpadded tiles (rows of D * 2 bytes).  Head dim
  // 64: padded rows (k_lds_row_bytes / v_lds_row_bytes), where every
  // fragment is one per-lane base plus an immediate.
  static constexpr bool kSwizzle = (D == 128);
  static constexpr int kRowK = kSwizzle ? D * 2 : k_lds_row_bytes<2, D>();
  static constexpr int kRowV = kSwizzle ? D * 2 : v_lds_row_bytes<2, D>();
  template <int BN, int NW>
  using KCopy = TileCopy<T, D, BN, NW, kRowK, kSwizzle>;
  template <int BN, int NW>
  using VCopy = TileCopy<T, D, BN, NW, kRowV, kSwizzle>;

  // Per-lane byte offsets into a K and a V tile.
  //  k[ks]: the K fragment of k-step ks for key block 0 -- lane (rho, h)
  //    reads chunk 2 ks + h of row rho (stored at (2 ks + h) ^ swizzle(rho)
  //    in a swizzled tile); key block nb adds nb * 32 rows (the swizzle
  //    repeats every 16 rows).
  //  v[sub][db]: transposing read `sub` of dim block db for k-step
  //    (nb, half) = (0, 0) -- see pv(); later k-steps add whole 16-row groups.
  // The row offsets are multiples of the row size, so the chunk bits join
  // them by XOR; a tile's base (1024-aligned) and the block's row offset
  // are added at the read and fold into the instruction's immediate.  In a
  // padded tile the entries differ by constants, which fold the same way.
  struct Lanes {
    uint32_t k[kQFrags];
    uint32_t v[2][D / 32];
  };
  __device__ static __forceinline__ Lanes lanes(int lane) {
    Lanes L;
    const int li = lane & 31;
    const int lh = lane >> 5;
    const int t = lane & 15;
    const int grp = lane >> 4;
    const int row_lane = (grp >> 1) * 4 + (t >> 2);
    const int col_bytes = (grp & 1) * 32 + 8 * (t & 3);
    if constexpr (kSwizzle) {
      const uint32_t kl = li * kRowK + ((lh ^ swizzle_of<D>(li)) << 4);
#pragma unroll
      for (int ks = 0; ks < kQFrags; ++ks) L.k[ks] = kl ^ static_cast<uint32_t>(ks << 5);
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        const int r = sub * 8 + row_lane;
        const uint32_t vl = r * kRowV + (col_bytes ^ (swizzle_of<D>(r) << 4));
#pragma unroll
        for (int db = 0; db < D / 32; ++db) L.v[sub][db] = vl ^ static_cast<uint32_t>(db << 6);
      }
    } else {
      const uint32_t kl = li * kRowK + lh * 16;
#pragma unroll
      for (int ks = 0; ks < kQFrags; ++ks) L.k[ks] = kl + ks * 32;
      const uint32_t vl = row_lane * kRowV + col_bytes;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) L.v[sub][db] = vl + sub * 8 * kRowV + db * 64;
      }
    }
    return L;
  }

  // S^T += K Q^T over the K tile at `k_tile`, for RB row blocks (each K
  // fragment read once, used RB times).  A operand of k-step ks: lane
  // (rho, h) holds K[32nb + rho][16ks + 8h ..+8].  The reads go through a
  // pointer into the tile's own LDS array, so the compiler can tell them
  // from tile copies into other arrays.
  template <int NB, int RB>
  __device__ static __forceinline__ void qk(const T* k_tile, const Lanes& L, const QRegs (&q)[RB],
                                            f32x16 (&s)[RB][NB]) {
    const char* base = reinterpret_cast<const char*>(k_tile);
#pragma unroll
    for (int ks = 0; ks < kQFrags; ++ks) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const frag a = *reinterpret_cast<const frag*>(base + L.k[ks] + nb * 32 * kRowK);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) s[rb][nb] = Mma16<T>::mma(a, q[rb].f[ks], s[rb][nb]);
      }
    }
  }
  template <int NB>
  __device__ static __forceinline__ void qk(const T* k_tile, const Lanes& L, const QRegs& q,
                                            f32x16 (&s)[NB]) {
    qk<NB, 1>(k_tile, L, reinterpret_cast<const QRegs(&)[1]>(q),
              reinterpret_cast<f32x16(&)[1][NB]>(s));
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
  // fragment reads ahead, then per MFMA a share of the softmax VALU work and
  // one read per RB MFMAs.  Phase B: two transposing V reads per RB MFMAs.
  template <int NB, int RB = 1>
  __device__ static __forceinline__ void interleave_qk() {
    constexpr int n_mfma = RB * NB * kQFrags;
    constexpr int valu_per = (RB * NB * 16 * 3 + n_mfma - 1) / n_mfma;
    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
    for (int i = 0; i < n_mfma; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i % RB == RB - 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, valu_per, 0);
    }
  }
  template <int NB, int DB, int RB = 1>
  __device__ static __forceinline__ void interleave_pv() {
    constexpr int n_mfma = RB * NB * 2 * DB;
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < n_mfma; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i % RB == RB - 1) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  }

  // The single phase of the lagged schedule: the next tile's scores and the
  // previous tile's P.V on the matrix cores, this tile's probabilities on
  // the VALU.  Keep a few LDS reads ahead; per product one or two reads (the
  // K reads of Q.K^T and the transposing V reads of P.V) and an even share
  // of the softmax VALU work.
  template <int NB, int DB>
  __device__ static __forceinline__ void interleave_lag() {
    constexpr int n_qk = NB * kQFrags;
    constexpr int n_pv = NB * 2 * DB;
    constexpr int n_mfma = n_qk + n_pv;
    constexpr int n_reads = n_qk + 2 * n_pv;
    constexpr int valu_per = (NB * 16 * 4 + n_mfma - 1) / n_mfma;
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < n_mfma; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      // reads after product i (the branches fold away once the loop unrolls)
      const int r = (n_reads * (i + 1)) / n_mfma - (n_reads * i) / n_mfma;
      if (r == 1) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      } else if (r == 2) {
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      } else if (r >= 3) {
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x002, valu_per, 0);
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
  template <int NB, int DB, int RB>
  __device__ static __forceinline__ void pv(const T* v_tile, const Lanes& L, const PRegs<NB> (&p)[RB],
                                            f32x16 (&acc)[RB][DB]) {
    using s16x4 = short __attribute__((ext_vector_type(4)));
    const char* base = reinterpret_cast<const char*>(v_tile);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          s16x4 w[2];
#pragma unroll
          for (int sub = 0; sub < 2; ++sub) {
            const char* src = base + L.v[sub][db] + (nb * 32 + half * 16) * kRowV;
            w[sub] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4*)(lds_void_ptr)(const_cast<char*>(src)));
          }
          frag vf;
          __builtin_memcpy(&vf, w, sizeof(vf));
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            acc[rb][db] = Mma16<T>::mma(vf, p[rb].f[nb][half], acc[rb][db]);
          }
        }
      }
    }
  }
  template <int NB, int DB>
  __device__ static __forceinline__ void pv(const T* v_tile, const Lanes& L, const PRegs<NB>& p,
                                            f32x16 (&acc)[DB]) {
    pv<NB, DB, 1>(v_tile, L, reinterpret_cast<const PRegs<NB>(&)[1]>(p),
                  reinterpret_cast<f32x16(&)[1][DB]>(acc));
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

  static constexpr bool kSwizzle = false;
  static constexpr int kRowK = k_lds_row_bytes<4, D>();
  static constexpr int kRowV = v_lds_row_bytes<4, D>();
  template <int BN, int NW>
  using KCopy = TileCopy<float, D, BN, NW, kRowK>;
  template <int BN, int NW>
  using VCopy = TileCopy<float, D, BN, NW, kRowV>;

  // Per-lane byte offsets into a tile: K row li at dims 4h.., V rows 4h..
  // at column li; every fragment is one of these plus an immediate.
  struct Lanes {
    uint32_t k;
    uint32_t v;
  };
  __device__ static __forceinline__ Lanes lanes(int lane) {
    const int li = lane & 31;
    const int lh = lane >> 5;
    return Lanes{static_cast<uint32_t>(li * kRowK + lh * 16),
                 static_cast<uint32_t>(lh * 4 * kRowV + li * 4)};
  }

  template <int NB, int RB>
  __device__ static __forceinline__ void qk(const float* k_tile, const Lanes& L,
                                            const QRegs (&q)[RB], f32x16 (&s)[RB][NB]) {
    const char* base = reinterpret_cast<const char*>(k_tile) + L.k;
#pragma unroll
    for (int g = 0; g < kGroups; ++g) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(base + nb * 32 * kRowK + g * 32);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            s[rb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], q[rb].f[g][e], s[rb][nb], 0, 0, 0);
          }
        }
      }
    }
  }

  template <int NB>
  __device__ static __forceinline__ void pin(PRegs<NB>&) {}

  // fp32 is a correctness path: no scheduling requests.
  template <int NB, int RB = 1>
  __device__ static __forceinline__ void interleave_qk() {}
  template <int NB, int DB, int RB = 1>
  __device__ static __forceinline__ void interleave_pv() {}
  template <int NB, int DB>
  __device__ static __forceinline__ void interleave_lag() {}

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
  template <int NB, int DB, int RB>
  __device__ static __forceinline__ void pv(const float* v_tile, const Lanes& L,
                                            const PRegs<NB> (&p)[RB], f32x16 (&acc)[RB][DB]) {
    const char* base = reinterpret_cast<const char*>(v_tile) + L.v;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const char* vrow = base + (nb * 32 + 8 * (r >> 2) + (r & 3)) * kRowV;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const float vv = *reinterpret_cast<const float*>(vrow + db * 128);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            acc[rb][db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv, p[rb].f[nb][r], acc[rb][db], 0, 0, 0);
          }
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

  // Loads of a whole tile come in two widths.  Wide (16-bit types, 16-byte
  // aligned rows): lane (i, h) loads keys 16 j + 8 h .. + 7 of its row for
  // j = 0, 1 -- its own four keys of one group and the four its partner lane
  // (i, 1 - h) needs of the other -- and the two swap those halves, so a
  // tile takes 2 NB loads of 16 bytes instead of 4 NB of 8.  Narrow: 4 NB
  // loads of 4 keys (8-byte aligned rows).  mode: 2 wide, 1 narrow, 0 key
  // by key.
  __device__ __forceinline__ void load(const T* row, int j0, int len_k, int lh, int mode) {
    if constexpr (sizeof(T) == 2) {
      if (mode == 2 && j0 + NB * 32 <= len_k) {
        using u32x4 = uint32_t __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            u32x4 v;
            __builtin_memcpy(&v,
                             __builtin_assume_aligned(row + j0 + nb * 32 + 16 * j + 8 * lh, 16), 16);
            // h = 0 holds keys 16j .. 16j+7 and keeps the first four (group
            // 2j); h = 1 holds 16j+8 .. 16j+15 and keeps the last four
            // (group 2j+1).  The halves trade h = 0's dwords 2, 3 for h = 1's
            // dwords 0, 1: v_permlane32_swap of (dwords 0, 1) with (dwords
            // 2, 3) swaps exactly those between the lane halves, leaving
            // group 2j in the first result and group 2j+1 in the second on
            // both halves (a VALU swap; a shuffle would go through LDS).
            const auto x0 = __builtin_amdgcn_permlane32_swap(v[0], v[2], false, false);
            const auto x1 = __builtin_amdgcn_permlane32_swap(v[1], v[3], false, false);
            const uint32_t lo[2] = {x0[0], x1[0]};  // group 2j
            const uint32_t hi[2] = {x0[1], x1[1]};  // group 2j+1
            __builtin_memcpy(&b[nb][8 * j], lo, 8);
            __builtin_memcpy(&b[nb][8 * j + 4], hi, 8);
          }
        }
        return;
      }
    }
    if (mode >= 1 && j0 + NB * 32 <= len_k) {
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
// Under a causal mask query tile m costs m + 1 key tiles, so the order runs
// over query tiles from the last one down (heaviest first).  Workgroup n goes
// to XCD n % 8 and is that XCD's (n / 8)-th; the (batch, head[, split])
// groups are dealt to the XCDs round-robin (group g to XCD g % 8), so each
// head stays on one XCD.  An XCD's groups are taken in parts of `span`
// groups, one part after the other, each part heaviest tile first with its
// groups fastest: a part finishes its long tiles before the next part's
// start, so fewer heads' keys and values are in flight in the XCD's L2 at a
// time, while a part of at least four times the waves an XCD holds (the
// launcher's choice of span) still balances its workgroups' unequal costs.
// span 0 (split launches, or a group count that is not a multiple of 8)
// runs over the groups fastest across the whole grid instead.
template <bool CAUSAL, bool SPLIT>
__device__ __forceinline__ void decode_tile(int m_tiles, int num_heads, int num_z, int num_splits,
                                            int span, int& z, int& h, int& m, int& split) {
  const uint32_t n = blockIdx.x;
  if constexpr (CAUSAL && !SPLIT) {
    if (span > 0) {
      const uint32_t xcd = n & 7u, i = n >> 3;
      const uint32_t per_part = static_cast<uint32_t>(span);
      const uint32_t part_wgs = per_part * static_cast<uint32_t>(m_tiles);
      const uint32_t part = i / part_wgs, r = i % part_wgs;
      m = m_tiles - 1 - static_cast<int>(r / per_part);
      const uint32_t g = xcd + 8u * (part * per_part + r % per_part);
      split = 0;
      h = static_cast<int>(g % static_cast<uint32_t>(num_heads));
      z = static_cast<int>(g / static_cast<uint32_t>(num_heads));
      return;
    }
  }
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

// A compile-time LDS stage index (the step bodies are unrolled by stage, so
// every stage offset is an instruction immediate).
template <int S>
struct Stage {
  static constexpr int value = S;
};

// A compile-time flag passed to the step bodies.
template <bool B>
struct Flag {
  static constexpr bool value = B;
};

// The LDS arrays of the K and V stages.  Separate arrays (not one
// [STAGES][...] array): each is its own alias scope, so the compiler can see
// that fragment reads of one stage do not depend on the tile copies still
// landing in another, and need not wait for them.  Entries past STAGES
// repeat earlier ones and are never used.
template <typename T>
struct StageArrays {
  T* k[4];
  T* v[4];
};
// Filled field by field: an initializer list of these addresses would be
// emitted as a constant in global memory, which cannot hold LDS addresses.
template <typename T>
__device__ __forceinline__ StageArrays<T> stage_arrays(T* k0, T* k1, T* k2, T* k3, T* v0, T* v1,
                                                       T* v2, T* v3) {
  StageArrays<T> st;
  st.k[0] = k0;
  st.k[1] = k1;
  st.k[2] = k2;
  st.k[3] = k3;
  st.v[0] = v0;
  st.v[1] = v1;
  st.v[2] = v2;
  st.v[3] = v3;
  return st;
}

// STAGES LDS stages each for K and V tiles (2 to 4), tile t in stage
// t % STAGES.  With S stages a tile load issued at step t is first needed at
// step t + S - 1, so it has S - 1 steps of compute to hide its latency
// behind.  Every stage index below is a compile-time constant (the step
// bodies are unrolled by stage), so every copy and read names its array.
// RB: row blocks of 32 query rows per wave (1 or 2).  With two, every K and V
// fragment read from LDS feeds two products, halving the LDS reads per
// matrix-core operation (the transposing V reads are the slow ones); the
// wave's registers double, so such a kernel runs one wave per SIMD.
// SPLIT: key-parallel dense forward.  The workgroup covers the key tiles of
// its split only and writes a normalised fp32 partial output and its
// logsumexp to the workspace; a second kernel merges the splits.
// BIAS: an additive bias joins the scores.  Each step loads the next tile's
// bias into registers before it issues its tile copies and adds it after
// P.V, so the loads have the whole step to land; the scores then hold
// scale * q.k + bias (natural-log units) and the softmax multiplies by
// log2(e) alone.
// KG: key groups.  With KG > 1 the workgroup's NW = 4 KG waves form KG
// groups of four that share the same 128 query rows: every step copies a
// tile of KG * BN keys, group g takes its keys [g * BN, (g + 1) * BN), and
// each group keeps its own running max, sum and O.  At the end groups 1 ..
// KG-1 hand their state to group 0 through LDS, which merges them and writes
// O and LSE.  A launch with few query tiles and long key ranges then runs
// KG waves per SIMD on one copy of each key tile, where one row group per
// workgroup ran one (dense or varlen scores without mask, bias or split;
// 16-bit inputs).
template <typename T, int D, int NW, int RB, int BN, int STAGES, int MODE, bool CAUSAL, bool SPLIT,
          bool BIAS, bool LAG = false, int KG = 1>
__device__ __forceinline__ void attn_fwd_body(const FwdArgs& a, const StageArrays<T>& st) {
  static_assert(STAGES >= 2 && STAGES <= 4, "two to four LDS stages");
  static_assert(KG == 1 || (NW == 4 * KG && RB == 1 && !CAUSAL && !SPLIT && !BIAS && !LAG &&
                            sizeof(T) == 2),
                "key groups: four waves each, 16-bit, scores without mask, bias or split");
  static_assert(!LAG || (RB == 1 && STAGES >= 3), "the lagged schedule: one row block, >= 3 stages");
  static_assert(RB == 1 || RB == 2, "one or two row blocks per wave");
  static_assert(!SPLIT || MODE == MODE_DENSE, "the split forward serves the dense mode");
  static_assert(!(SPLIT && BIAS), "the split forward has no bias");
  using Path = typename PathFor<T, D>::type;
  using KCopy = typename Path::template KCopy<KG * BN, NW>;
  using VCopy = typename Path::template VCopy<KG * BN, NW>;
  using PRegs = typename Path::template PRegs<BN / 32>;
  constexpr int NWR = NW / KG;  // waves per key group, one row block each
  constexpr int BM = NWR * 32 * RB;
  constexpr int TBN = KG * BN;  // keys copied per step
  constexpr int NB = BN / 32;
  constexpr int DB = D / 32;
  // Loads one step issues per wave; those of the last STAGES - 2 steps may
  // still be in flight when a step ends (the next step reads K(t+2) and
  // V(t+1), issued STAGES - 2 steps before this one ends).
  constexpr int kLoadsPerStep = KCopy::kInstPerWave + VCopy::kInstPerWave;
  constexpr int kInFlightAtStepEnd = (STAGES - 2) * kLoadsPerStep;

  int z, h, m, split;
  decode_tile<CAUSAL, SPLIT>(a.m_tiles, a.num_heads, a.num_z, a.num_splits, a.causal_span, z, h,
                             m, split);
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

  const int wr = KG == 1 ? wave : wave % NWR;  // row block of this wave
  const int kg = KG == 1 ? 0 : wave / NWR;     // key group of this wave
  const int row0 = m0 + wr * 32 * RB;          // first query row of this wave
  int qi[RB];                            // this lane's query row in each block
  bool row_ok[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    qi[rb] = row0 + 32 * rb + li;
    row_ok[rb] = qi[rb] < sr.len_q;
  }

  int kend = sr.len_k;
  if constexpr (CAUSAL) kend = min(kend, min(m0 + BM, sr.len_q));
  // Key tiles [tile0, tile0 + n_tiles): all of them, or this split's share
  // (possibly none: an empty split still writes its partial result).
  int tile0 = 0;
  int n_tiles = (kend + TBN - 1) / TBN;
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
  // Rows at or past `end` are not fetched (they read back as zeros); a load
  // past the last tile fetches nothing.
  auto issue_k = [&](int t, int stage, int end) {
    const int j0 = (tile0 + t) * TBN;
    kcopy.issue(kp + j0 * k_row_bytes, end - j0, k_row_bytes, st.k[stage], wave);
  };
  auto issue_v = [&](int t, int stage, int end) {
    const int j0 = (tile0 + t) * TBN;
    vcopy.issue(vp + j0 * v_row_bytes, end - j0, v_row_bytes, st.v[stage], wave);
  };
  const typename Path::Lanes lanes = Path::lanes(lane);
  // Element offsets of this wave's key group inside a K and a V tile.
  int k_grp = 0;
  int v_grp = 0;
  if constexpr (KG > 1) {
    k_grp = kg * BN * (Path::kRowK / static_cast<int>(sizeof(T)));
    v_grp = kg * BN * (Path::kRowV / static_cast<int>(sizeof(T)));
  }

  typename Path::QRegs qr[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    Path::load_q(qp + static_cast<int64_t>(qi[rb]) * a.q_ss, row_ok[rb], lh, qr[rb]);
  }

  f32x16 acc[RB][DB];
  float m_run[RB];  // reference (stale) max of scale*log2(e)*s, per row
  float l_run[RB];  // running sum of this half-wave's weights, per row
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[rb][db] = f32x16{};
    m_run[rb] = kNegInf;
    l_run[rb] = 0.f;
  }
  const float c2 = BIAS ? kLog2e : a.scale_log2;

  // This lane's bias rows (the sequence's block of the bias view).
  using Bias = BiasTile<T, NB>;
  const T* bias_row[RB] = {};
  int bias_mode = 0;
  if constexpr (BIAS) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      bias_row[rb] = static_cast<const T*>(a.bias) + sr.b * a.bias_sb + h * a.bias_sh +
                     (static_cast<int64_t>(sr.q_start) + qi[rb]) * a.bias_sq + sr.k_start;
    }
    // Narrow vector loads need the block to start on a 4-element boundary
    // (the strides are multiples of 4 elements); wide ones a 16-byte
    // aligned base and 8-element strides and start.
    const bool wide = (reinterpret_cast<uintptr_t>(a.bias) & 15) == 0 && (a.bias_sb & 7) == 0 &&
                      (a.bias_sh & 7) == 0 && (a.bias_sq & 7) == 0 && (sr.k_start & 7) == 0;
    bias_mode = wide ? 2 : ((sr.k_start & 3) == 0 ? 1 : 0);
  }
  auto load_bias = [&](int t, Bias (&bt)[RB]) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (row_ok[rb]) {
        bt[rb].load(bias_row[rb], (tile0 + t) * BN, sr.len_k, lh, bias_mode);
      } else {
        bt[rb].zero();
      }
    }
  };

  // Masks the scores of tile t where keys run past the sequence or, under
  // the causal mask, past the lane's row (only tail and diagonal tiles).
  auto mask_tile = [&](int t, f32x16 (&s)[RB][NB]) {
    const int j0 = (tile0 + t) * TBN + kg * BN;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const bool need_mask = (j0 + BN > sr.len_k) || (CAUSAL && j0 + BN - 1 > row0 + 32 * rb);
      if (need_mask) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = j0 + nb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
            const bool ok = key < sr.len_k && (!CAUSAL || key <= qi[rb]);
            if (!ok) s[rb][nb][r] = kNegInf;
          }
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
  // Probabilities of a score tile against the running reference, into p;
  // returns this lane's share of the tile's row sum.  The reference only has
  // to keep every p bounded, not to equal the row max: while a tile's sums
  // stay <= 2^12 (so every p <= 2^12) nothing else is done.  Otherwise -- and
  // on the first tile a row sees -- the exact row max is taken, acc and l are
  // rescaled to it, and p is recomputed (p <= 1).  The result is unchanged:
  // O = acc / l and LSE = m + log2 l for any m.  The check is wave-uniform
  // per row block.
  auto first_pass = [&](int rb, const f32x16 (&s)[NB], PRegs& p) {
    return Path::template softmax_p<NB>(s, c2, (m_run[rb] == kNegInf) ? 0.f : m_run[rb], p);
  };
  auto settle = [&](int rb, const f32x16 (&s)[NB], PRegs& p, float tile_sum) {
    const bool redo = !(tile_sum <= kSumLimit) || m_run[rb] == kNegInf;
    if (__builtin_amdgcn_ballot_w64(redo) != 0) {  // rare
      const float m_new = fmaxf(m_run[rb], tile_max(s));
      const float alpha = (m_new == kNegInf) ? 1.f : __builtin_amdgcn_exp2f(m_run[rb] - m_new);
      l_run[rb] *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[rb][db] *= alpha;
      m_run[rb] = m_new;
      tile_sum = first_pass(rb, s, p);
    }
    l_run[rb] += tile_sum;
  };

  f32x16 s[RB][NB];
  Bias bias_next[RB];
  if constexpr (LAG) {
    // Lagged schedule: step t turns tile t's scores into probabilities (VALU)
    // while the matrix cores compute tile t+1's scores AND P(t-1).V(t-1), all
    // in one interleaved phase, so a wave overlaps its own softmax with its
    // own products (one wave per SIMD has no other wave to overlap with).
    // V(t-1) is read one step after K(t-1), so tile t's V lands in stage
    // t % STAGES as K does but is loaded STAGES - 2 steps ahead instead of
    // STAGES: at step t, K(t+STAGES) goes into K(t)'s stage (read in step
    // t-1) and V(t+STAGES-2) into V(t-2)'s (read in step t-1).  Both tiles
    // a step reads were issued STAGES - 1 steps earlier.
    if (n_tiles > 0) {
      if constexpr (BIAS) load_bias(0, bias_next);
#pragma unroll
      for (int i = 0; i < STAGES; ++i) {
        issue_k(i, i, i < n_tiles ? kend : 0);
        if (i < STAGES - 2) issue_v(i, i, i < n_tiles ? kend : 0);
      }
      wait_vmem();
      barrier_lds();
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) s[0][nb] = f32x16{};
      Path::template qk<NB, 1>(st.k[0], lanes, qr, s);
      if constexpr (BIAS) bias_next[0].fold(s[0], a.scale);
      mask_tile(0, s);
      // The stages are not refilled before every wave has read K(0).
      barrier_lds();
    }
    PRegs p_prev[1];
    // Step t (tile t+1 exists): K(t+1) in stage (t+1) % STAGES, V(t-1) in
    // stage (t-1) % STAGES (absent at t = 0).
    auto lag_step = [&](int t, auto stage, auto with_pv) {
      constexpr int ST = decltype(stage)::value;
      constexpr bool PV = decltype(with_pv)::value;
      if constexpr (BIAS) load_bias(t + 1, bias_next);
      issue_k(t + STAGES, ST, t + STAGES < n_tiles ? kend : 0);
      issue_v(t + STAGES - 2, (ST + STAGES - 2) % STAGES, t + STAGES - 2 < n_tiles ? kend : 0);
      PRegs p_cur[1];
      f32x16 s_next[1][NB];
      using P1 = typename Path::template PRegs<1>;
      const float m_sub = (m_run[0] == kNegInf) ? 0.f : m_run[0];
      float tile_sum = 0.f;
      // One scheduling region per 32-key block: its probabilities, its
      // scores of the next tile and its share of P(t-1).V(t-1), so only one
      // block's operands are live at a time.
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        P1& pc = reinterpret_cast<P1&>(p_cur[0].f[nb]);
        f32x16(&sn)[1][1] = reinterpret_cast<f32x16(&)[1][1]>(s_next[0][nb]);
        sn[0][0] = f32x16{};
        tile_sum += Path::template softmax_p<1>(reinterpret_cast<const f32x16(&)[1]>(s[0][nb]),
                                                c2, m_sub, pc);
        Path::template qk<1, 1>(st.k[(ST + 1) % STAGES] + nb * 32 * (Path::kRowK / sizeof(T)),
                                lanes, qr, sn);
        if constexpr (PV) {
          Path::template pv<1, DB, 1>(st.v[(ST + STAGES - 1) % STAGES] +
                                          nb * 32 * (Path::kRowV / sizeof(T)),
                                      lanes, reinterpret_cast<const P1(&)[1]>(p_prev[0].f[nb]),
                                      acc);
          Path::pin(pc);
          Path::template interleave_lag<1, DB>();
        } else {
          Path::pin(pc);
          Path::template interleave_qk<1, 1>();
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // A rescale (rare) also rescales P(t-1).V(t-1), which used the old reference.
      settle(0, s[0], p_cur[0], tile_sum);
      if constexpr (BIAS) bias_next[0].fold(s_next[0], a.scale);
      mask_tile(t + 1, s_next);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) s[0][nb] = s_next[0][nb];
      p_prev[0] = p_cur[0];
      // K(t+2) and V(t), issued STAGES - 2 steps before this one ends, must
      // have landed before the next step.
      wait_vmem_allow<kInFlightAtStepEnd>();
      barrier_lds();
    };
    if (n_tiles > 1) {
      lag_step(0, Stage<0>{}, Flag<false>{});
      for (int t = 1;; t += STAGES) {
        if (t + 1 >= n_tiles) break;
        lag_step(t, Stage<1 % STAGES>{}, Flag<true>{});
        if (t + 2 >= n_tiles) break;
        lag_step(t + 1, Stage<2 % STAGES>{}, Flag<true>{});
        if (t + 3 >= n_tiles) break;
        lag_step(t + 2, Stage<3 % STAGES>{}, Flag<true>{});
        if constexpr (STAGES > 3) {
          if (t + 4 >= n_tiles) break;
          lag_step(t + 3, Stage<4 % STAGES>{}, Flag<true>{});
        }
      }
    }
    if (n_tiles > 0) {
      // The last tile: its probabilities beside P(n-2).V(n-2), then P(n-1).V(n-1)
      // once every wave's share of V(n-1) has landed.
      auto v_stage = [&](int t) {
        const int i = t % STAGES;
        return i == 0 ? st.v[0] : (i == 1 ? st.v[1] : (i == 2 ? st.v[2] : st.v[3]));
      };
      PRegs p_cur[1];
      const float tile_sum = first_pass(0, s[0], p_cur[0]);
      if (n_tiles > 1) Path::template pv<NB, DB, 1>(v_stage(n_tiles - 2), lanes, p_prev, acc);
      settle(0, s[0], p_cur[0], tile_sum);
      wait_vmem();
      barrier_lds();
      Path::template pv<NB, DB, 1>(v_stage(n_tiles - 1), lanes, p_cur, acc);
    }
  } else {
  if (n_tiles > 0) {
    // K(0), then K(i) and V(i-1) for i < STAGES: the order the step-end
    // waits count on.  (The full wait also settles Q's loads, which are the
    // compiler's.)
    if constexpr (BIAS) load_bias(0, bias_next);
    issue_k(0, 0, kend);
#pragma unroll
    for (int i = 1; i < STAGES; ++i) {
      issue_k(i, i, i < n_tiles ? kend : 0);
      issue_v(i - 1, i - 1, i - 1 < n_tiles ? kend : 0);
    }
    wait_vmem();
    barrier_lds();
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) s[rb][nb] = f32x16{};
    }
    Path::template qk<NB, RB>(st.k[0] + k_grp, lanes, qr, s);
    if constexpr (BIAS) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) bias_next[rb].fold(s[rb], a.scale);
    }
    mask_tile(0, s);
    barrier_lds();  // every wave is done with K(0) before K(STAGES) replaces it
  }

  // Under the causal mask a wave whose rows all precede the first key of
  // tile t has nothing left to add: tile t and every later one are masked
  // for all its rows.  Such a wave still issues its share of the tile copies
  // and meets every barrier, but skips the products and the softmax (a
  // wave-uniform branch).  The result is unchanged: the skipped weights are
  // exactly 0 and a tile without weights never triggers a rescale.  With
  // 256-row workgroups of 32-row waves this removes 12 of the 32 wave-tiles
  // of each diagonal block.
  auto wave_done = [&](int t) { return CAUSAL && (tile0 + t) * BN > row0 + 32 * RB - 1; };

  // Pipeline step for tile t (in stage ST = t % STAGES) when tile t+1 exists.
  // K(t)'s stage is done with and receives K(t+STAGES); K(t+1) is in the next
  // stage; V(t) is in stage ST and V(t-1)'s stage receives V(t+STAGES-1).
  // Phase A is straight-line code, so the scheduler can interleave the
  // softmax VALU work with the next tile's score MFMAs.
  auto step = [&](int t, auto stage) {
    constexpr int ST = decltype(stage)::value;
    const T* k_nxt = st.k[(ST + 1) % STAGES] + k_grp;
    const T* v_cur = st.v[ST] + v_grp;
    // The next tile's bias goes out before the tile copies, so waiting for it
    // never waits for them (also when this wave skips the tile: a
    // conditional load would keep two copies of the bias registers alive).
    if constexpr (BIAS) load_bias(t + 1, bias_next);
    // The tile copies into K(t)'s and V(t-1)'s stages (their last readers
    // passed the previous barrier).  They are the compiler's buffer-load
    // builtins: it interleaves them with the first fragment reads and the
    // products (inline assembly there would make it drop the interleave
    // that interleave_qk / interleave_pv request).
    issue_k(t + STAGES, ST, t + STAGES < n_tiles ? kend : 0);
    issue_v(t + STAGES - 1, (ST + STAGES - 1) % STAGES, t + STAGES - 1 < n_tiles ? kend : 0);
    if (!wave_done(t)) {

    // Phase A: probabilities of tile t (VALU) || scores of tile t+1 (MFMA).
    // At head dim 128, in the split forward and with key groups, the wave
    // raises its issue priority for this phase and drops it for phase B: a
    // SIMD's other wave, in its product-only phase B, then fills the matrix
    // cores between this wave's softmax instructions instead of the other way
    // round.  Measured on the bf16 D128 workloads: dense causal S2048 73.8
    // against 77.0 us, padded varlen 1808 against 1870 us, non-causal and THD
    // unchanged; split fp16 D64 Sq512 Sk8192 87 against 89-91 us, with two key
    // groups 85.3-86.0 against 86.6-86.7 us.  The single-group D64 kernel keeps
    // one priority: with the instructions in its loop (even skipped at run
    // time) it compiled to a schedule 16-22 % slower on that workload.
    constexpr bool kPhasePrio = D == 128 || SPLIT || KG > 1;
    if constexpr (kPhasePrio) __builtin_amdgcn_s_setprio(1);
    PRegs p[RB];
    f32x16 s_next[RB][NB];
    float tile_sum[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) s_next[rb][nb] = f32x16{};
      tile_sum[rb] = first_pass(rb, s[rb], p[rb]);
    }
    Path::template qk<NB, RB>(k_nxt, lanes, qr, s_next);
    // P is computed here, beside the MFMAs, not after the branches
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) Path::pin(p[rb]);
    Path::template interleave_qk<NB, RB>();
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) settle(rb, s[rb], p[rb], tile_sum[rb]);
    if constexpr (!BIAS) mask_tile(t + 1, s_next);

    // Phase B: O += P(t) V(t) on the matrix cores.
    if constexpr (kPhasePrio) __builtin_amdgcn_s_setprio(0);
    Path::template pv<NB, DB, RB>(v_cur, lanes, p, acc);
    Path::template interleave_pv<NB, DB, RB>();
    if constexpr (BIAS) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) bias_next[rb].fold(s_next[rb], a.scale);
      mask_tile(t + 1, s_next);
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) s[rb][nb] = s_next[rb][nb];
    }
    }  // !wave_done(t)

    // K(t+2) and V(t+1) -- issued STAGES - 2 steps before this one -- must
    // have landed before the next step.
    wait_vmem_allow<kInFlightAtStepEnd>();
    barrier_lds();
  };
  // The last tile: probabilities and P.V only.  It issues no loads, but
  // the zero-row copies of earlier steps may still be in flight: every
  // wave settles its own before leaving.
  auto last_step = [&](const T* v_cur) {
    if (!wave_done(n_tiles - 1)) {
      PRegs p[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) settle(rb, s[rb], p[rb], first_pass(rb, s[rb], p[rb]));
      Path::template pv<NB, DB, RB>(v_cur, lanes, p, acc);
    }
    wait_vmem();
  };

  // Each step body exists once per stage (unrolled by STAGES so that every
  // step's stage offsets are constants); the loop leaves as soon as the next
  // tile would be the last one, and the last tile's V stage is picked at run
  // time.
  if (n_tiles > 0) {
    for (int t = 0;; t += STAGES) {
      if (t + 1 >= n_tiles) break;
      step(t, Stage<0>{});
      if (t + 2 >= n_tiles) break;
      step(t + 1, Stage<1>{});
      if constexpr (STAGES > 2) {
        if (t + 3 >= n_tiles) break;
        step(t + 2, Stage<2>{});
      }
      if constexpr (STAGES > 3) {
        if (t + 4 >= n_tiles) break;
        step(t + 3, Stage<3>{});
      }
    }
    const int last = (n_tiles - 1) % STAGES;
    last_step((last == 0 ? st.v[0] : (last == 1 ? st.v[1] : (last == 2 ? st.v[2] : st.v[3]))) +
              v_grp);
  }
  }  // LAG

  if constexpr (KG > 1) {
    // Groups 1 .. KG-1 hand their running max, sum and O to group 0 through
    // LDS once every wave is done with the tiles: wave r of each group owns
    // rows [32 r, 32 r + 32), and lane (i, h) of every group holds the same
    // row and half of the sums, so the exchange is lane to lane.  Row block
    // r's buffers lie in one stage array (K0, K1, V0, V1 for r = 0..3),
    // group g's at float (g - 1) * kVals * 64, its value i of lane L at
    // float i * 64 + L after that.
    constexpr int kVals = DB * 16 + 2;
    barrier_lds();
    float* xbase = reinterpret_cast<float*>(
        wr == 0 ? st.k[0] : (wr == 1 ? st.k[1] : (wr == 2 ? st.v[0] : st.v[1])));
    if (kg > 0) {
      float* xbuf = xbase + (kg - 1) * kVals * 64;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int r = 0; r < 16; ++r) xbuf[(db * 16 + r) * 64 + lane] = acc[0][db][r];
      }
      xbuf[(kVals - 2) * 64 + lane] = m_run[0];
      xbuf[(kVals - 1) * 64 + lane] = l_run[0];
    }
    barrier_lds();
    if (kg > 0) return;
#pragma unroll
    for (int g = 1; g < KG; ++g) {
      const float* xbuf = xbase + (g - 1) * kVals * 64;
      const float m1 = xbuf[(kVals - 2) * 64 + lane];
      const float l1 = xbuf[(kVals - 1) * 64 + lane];
      const float m_new = fmaxf(m_run[0], m1);
      // A group that saw no key keeps m = -inf and l = 0: its factor is 0.
      const float f0 = m_run[0] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m_run[0] - m_new);
      const float f1 = m1 == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m1 - m_new);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          acc[0][db][r] = acc[0][db][r] * f0 + xbuf[(db * 16 + r) * 64 + lane] * f1;
        }
      }
      l_run[0] = l_run[0] * f0 + l1 * f1;
      m_run[0] = m_new;
    }
  }

  // Epilogue: O = acc / l, LSE = (m + log2 l) * ln 2, valid rows only.
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float l_tot = sum_across_halves(l_run[rb]);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float lse = l_tot > 0.f ? (m_run[rb] + log2f(l_tot)) * kLn2 : kNegInf;
    if (!row_ok[rb]) continue;
    if constexpr (SPLIT) {
      const int64_t row = (static_cast<int64_t>(split) * a.num_z + z) * a.num_heads * sr.len_q +
                          static_cast<int64_t>(h) * sr.len_q + qi[rb];
      float* wrow = a.ws_o + row * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16& o = acc[rb][db];
          *reinterpret_cast<f32x4*>(wrow + db * 32 + g * 8 + lh * 4) =
              f32x4{o[4 * g] * inv, o[4 * g + 1] * inv, o[4 * g + 2] * inv, o[4 * g + 3] * inv};
        }
      }
      if (lh == 0) a.ws_lse[row] = lse;
    } else {
      T* orow = op + static_cast<int64_t>(qi[rb]) * a.o_ss;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          T out4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) out4[e] = static_cast<T>(acc[rb][db][4 * g + e] * inv);
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
      if (lh == 0) lsep[qi[rb]] = lse;
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
// and 2n+3.  Tiles rotate through STAGES stages (tile n in stage
// n % STAGES).  At the start of C(n) each wave issues its share of K(n +
// STAGES) into K(n)'s stage and of V(n + STAGES - 1) into V(n - 1)'s: the
// last readers of both finished by global interval 2n+1, and C(n) starts at
// j >= 2n+2.  At the end of C(n) each wave waits until only the loads it
// issued in the last STAGES - 2 C intervals are in flight, so a tile issued
// in C(n) has landed after C(n + STAGES - 2) -- before its first reader at
// j = 2(n + STAGES) (K) or 2(n + STAGES - 1) + 2 (V).
template <typename T, int D, int BN, int STAGES, int MODE, bool CAUSAL>
__device__ __forceinline__ void attn_fwd_pingpong_body(const FwdArgs& a, T* k_lds, T* v_lds) {
  static_assert(sizeof(T) == 2, "the ping-pong schedule serves 16-bit inputs");
  static_assert(STAGES >= 2 && STAGES <= 4, "two to four LDS stages");
  constexpr int NW = 8;
  using Path = Path16<T, D>;
  using KCopy = typename Path::template KCopy<BN, NW>;
  using VCopy = typename Path::template VCopy<BN, NW>;
  constexpr int kKStage = KCopy::kArrayBytes;
  constexpr int kVStage = VCopy::kArrayBytes;
  using PRegs = typename Path::template PRegs<BN / 32>;
  constexpr int BM = NW * 32;
  constexpr int NB = BN / 32;
  constexpr int DB = D / 32;
  constexpr int kLoadsPerTile = KCopy::kInstPerWave + VCopy::kInstPerWave;
  constexpr int kInFlight = (STAGES - 2) * kLoadsPerTile;

  int z, h, m, split;
  decode_tile<CAUSAL, false>(a.m_tiles, a.num_heads, a.num_z, 1, a.causal_span, z, h, m, split);
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
  auto issue_k = [&](int t, int stage) {
    const int j0 = t * BN;
    kcopy.issue_untracked(kp + j0 * k_row_bytes, t < n_tiles ? kend - j0 : 0, k_row_bytes,
                          k_lds + stage * (kKStage / 2), wave);
  };
  auto issue_v = [&](int t, int stage) {
    const int j0 = t * BN;
    vcopy.issue_untracked(vp + j0 * v_row_bytes, t < n_tiles ? kend - j0 : 0, v_row_bytes,
                          v_lds + stage * (kVStage / 2), wave);
  };
  const typename Path::Lanes lanes = Path::lanes(lane);

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
    issue_k(0, 0);
    wait_vmem();
    barrier_lds();
#pragma unroll
    for (int i = 1; i < STAGES; ++i) {
      issue_k(i, i);
      issue_v(i - 1, i - 1);
    }
    if (group == 1) barrier_lds();  // group 1 sits out global interval 0

    // u = 0: scores of tile 0.
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) s[nb] = f32x16{};
    Path::template qk<NB>(k_lds, lanes, qr, s);
    wait_vmem_allow<kInFlight>();  // K(1) and V(0) have landed
    barrier_lds();

    // S(n): vector work on tile n's scores.
    auto s_interval = [&](int n) {
      mask_tile(n, s);
      l_run += probabilities(s, p);
      barrier_lds();
    };
    // C(n) for n + 1 < n_tiles, tile n in stage ST.  K(n)'s stage receives
    // K(n+STAGES), K(n+1) is in the next stage, V(n) in stage ST, and V(n-1)'s
    // stage receives V(n+STAGES-1).  The loads are issued unconditionally
    // (tiles past the end fetch zero rows into stages nobody reads again), so
    // every wave issues the same count the waits rely on.
    auto c_interval = [&](int n, auto stage) {
      constexpr int ST = decltype(stage)::value;
      issue_k(n + STAGES, ST);
      issue_v(n + STAGES - 1, (ST + STAGES - 1) % STAGES);
      __builtin_amdgcn_sched_barrier(0);  // keep the inline-asm copies out of the products' region
      f32x16 s_next[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) s_next[nb] = f32x16{};
      Path::template qk<NB>(k_lds + ((ST + 1) % STAGES) * (kKStage / 2), lanes, qr, s_next);
      Path::template pv<NB, DB>(v_lds + ST * (kVStage / 2), lanes, p, acc);
      Path::template interleave_c<NB, DB>();
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) s[nb] = s_next[nb];
      wait_vmem_allow<kInFlight>();
      barrier_lds();
    };

    for (int n = 0;; n += STAGES) {
      if (n + 1 >= n_tiles) break;
      s_interval(n);
      c_interval(n, Stage<0>{});
      if (n + 2 >= n_tiles) break;
      s_interval(n + 1);
      c_interval(n + 1, Stage<1>{});
      if constexpr (STAGES > 2) {
        if (n + 3 >= n_tiles) break;
        s_interval(n + 2);
        c_interval(n + 2, Stage<2>{});
      }
      if constexpr (STAGES > 3) {
        if (n + 4 >= n_tiles) break;
        s_interval(n + 3);
        c_interval(n + 3, Stage<3>{});
      }
    }
    // Last tile: S(T-1), then C(T-1) = P.V only.  Group 1's last interval is
    // the workgroup's last, so it ends without a barrier (every wave passes
    // the same number of barriers).
    s_interval(n_tiles - 1);
    Path::template pv<NB, DB>(v_lds + ((n_tiles - 1) % STAGES) * (kVStage / 2), lanes, p, acc);
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

// The kernels declare one LDS array per operand holding all STAGES stages.
template <typename T, int D, int BN, int STAGES, int MODE, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void attn_fwd_pingpong_kernel(FwdArgs a) {
  using Path = Path16<T, D>;
  constexpr int kKElems = STAGES * Path::template KCopy<BN, 8>::kArrayBytes / 2;
  constexpr int kVElems = STAGES * Path::template VCopy<BN, 8>::kArrayBytes / 2;
  __shared__ __attribute__((aligned(1024))) T k_lds[kKElems];
  __shared__ __attribute__((aligned(1024))) T v_lds[kVElems];
  attn_fwd_pingpong_body<T, D, BN, STAGES, MODE, CAUSAL>(a, k_lds, v_lds);
}

// Two waves per SIMD with one row block per wave (at most 256 registers
// each); one wave per SIMD with two (up to 512).
template <typename T, int D, int NW, int RB, int BN, int STAGES, int MODE, bool CAUSAL, bool SPLIT,
          bool BIAS>
__global__ __launch_bounds__(NW * 64, RB == 2 ? 1 : 2) void attn_fwd_kernel(FwdArgs a) {
  using Path = typename PathFor<T, D>::type;
  constexpr int kES = static_cast<int>(sizeof(T));
  constexpr int kKElems = Path::template KCopy<BN, NW>::kArrayBytes / kES;
  constexpr int kVElems = Path::template VCopy<BN, NW>::kArrayBytes / kES;
  __shared__ __attribute__((aligned(1024))) T k_lds0[kKElems];
  __shared__ __attribute__((aligned(1024))) T k_lds1[kKElems];
  __shared__ __attribute__((aligned(1024))) T v_lds0[kVElems];
  __shared__ __attribute__((aligned(1024))) T v_lds1[kVElems];
  if constexpr (STAGES == 2) {
    attn_fwd_body<T, D, NW, RB, BN, STAGES, MODE, CAUSAL, SPLIT, BIAS>(
        a, stage_arrays(k_lds0, k_lds1, k_lds0, k_lds1, v_lds0, v_lds1, v_lds0, v_lds1));
  } else if constexpr (STAGES == 3) {
    __shared__ __attribute__((aligned(1024))) T k_lds2[kKElems];
    __shared__ __attribute__((aligned(1024))) T v_lds2[kVElems];
    attn_fwd_body<T, D, NW, RB, BN, STAGES, MODE, CAUSAL, SPLIT, BIAS>(
        a, stage_arrays(k_lds0, k_lds1, k_lds2, k_lds0, v_lds0, v_lds1, v_lds2, v_lds0));
  } else {
    __shared__ __attribute__((aligned(1024))) T k_lds2[kKElems];
    __shared__ __attribute__((aligned(1024))) T v_lds2[kVElems];
    __shared__ __attribute__((aligned(1024))) T k_lds3[kKElems];
    __shared__ __attribute__((aligned(1024))) T v_lds3[kVElems];
    attn_fwd_body<T, D, NW, RB, BN, STAGES, MODE, CAUSAL, SPLIT, BIAS>(
        a, stage_arrays(k_lds0, k_lds1, k_lds2, k_lds3, v_lds0, v_lds1, v_lds2, v_lds3));
  }
}

// KG key groups of four waves (see attn_fwd_body): 4 KG waves, KG waves per
// SIMD, two or three stages of KG * BN-key tiles.
template <typename T, int D, int KG, int BN, int STAGES, int MODE>
__global__ __launch_bounds__(KG * 256, KG) void attn_fwd_kg_kernel(FwdArgs a) {
  static_assert(KG == 2 || KG == 3, "two or three key groups");
  using Path = typename PathFor<T, D>::type;
  constexpr int kES = static_cast<int>(sizeof(T));
  constexpr int kKElems = Path::template KCopy<KG * BN, 4 * KG>::kArrayBytes / kES;
  constexpr int kVElems = Path::template VCopy<KG * BN, 4 * KG>::kArrayBytes / kES;
  static_assert(kKElems * kES >= (KG - 1) * (D / 2 + 2) * 256 &&
                    kVElems * kES >= (KG - 1) * (D / 2 + 2) * 256,
                "each stage array holds one row block's exchange buffers");
  __shared__ __attribute__((aligned(1024))) T k_lds0[kKElems];
  __shared__ __attribute__((aligned(1024))) T k_lds1[kKElems];
  __shared__ __attribute__((aligned(1024))) T v_lds0[kVElems];
  __shared__ __attribute__((aligned(1024))) T v_lds1[kVElems];
  if constexpr (STAGES == 2) {
    attn_fwd_body<T, D, 4 * KG, 1, BN, 2, MODE, false, false, false, false, KG>(
        a, stage_arrays(k_lds0, k_lds1, k_lds0, k_lds1, v_lds0, v_lds1, v_lds0, v_lds1));
  } else {
    static_assert(STAGES == 3, "two or three stages");
    __shared__ __attribute__((aligned(1024))) T k_lds2[kKElems];
    __shared__ __attribute__((aligned(1024))) T v_lds2[kVElems];
    attn_fwd_body<T, D, 4 * KG, 1, BN, 3, MODE, false, false, false, false, KG>(
        a, stage_arrays(k_lds0, k_lds1, k_lds2, k_lds0, v_lds0, v_lds1, v_lds2, v_lds0));
  }
}

// The single-group kernel built for three waves per SIMD: the launch bound
// limits a wave to 168 registers, so three four-wave workgroups (or a
// mix) share a CU where the LDS stages allow it.
template <typename T, int D, int NW, int BN, int STAGES, int MODE, bool CAUSAL, bool SPLIT, bool BIAS>
__global__ __launch_bounds__(NW * 64, 3) void attn_fwd_3w_kernel(FwdArgs a) {
  using Path = typename PathFor<T, D>::type;
  constexpr int kES = static_cast<int>(sizeof(T));
  constexpr int kKElems = Path::template KCopy<BN, NW>::kArrayBytes / kES;
  constexpr int kVElems = Path::template VCopy<BN, NW>::kArrayBytes / kES;
  __shared__ __attribute__((aligned(1024))) T k_lds0[kKElems];
  __shared__ __attribute__((aligned(1024))) T k_lds1[kKElems];
  __shared__ __attribute__((aligned(1024))) T v_lds0[kVElems];
  __shared__ __attribute__((aligned(1024))) T v_lds1[kVElems];
  if constexpr (STAGES == 2) {
    attn_fwd_body<T, D, NW, 1, BN, 2, MODE, CAUSAL, SPLIT, BIAS>(
        a, stage_arrays(k_lds0, k_lds1, k_lds0, k_lds1, v_lds0, v_lds1, v_lds0, v_lds1));
  } else {
    static_assert(STAGES == 3, "two or three stages");
    __shared__ __attribute__((aligned(1024))) T k_lds2[kKElems];
    __shared__ __attribute__((aligned(1024))) T v_lds2[kVElems];
    attn_fwd_body<T, D, NW, 1, BN, 3, MODE, CAUSAL, SPLIT, BIAS>(
        a, stage_arrays(k_lds0, k_lds1, k_lds2, k_lds0, v_lds0, v_lds1, v_lds2, v_lds0));
  }
}

// The lagged schedule (one row block per wave, three or four LDS stages).
template <typename T, int D, int NW, int BN, int STAGES, int MODE, bool CAUSAL, bool SPLIT, bool BIAS>
__global__ __launch_bounds__(NW * 64, 2) void attn_fwd_lagged_kernel(FwdArgs a) {
  static_assert(STAGES == 3 || STAGES == 4, "the lagged schedule keeps three or four stages");
  using Path = typename PathFor<T, D>::type;
  constexpr int kES = static_cast<int>(sizeof(T));
  constexpr int kKElems = Path::template KCopy<BN, NW>::kArrayBytes / kES;
  constexpr int kVElems = Path::template VCopy<BN, NW>::kArrayBytes / kES;
  __shared__ __attribute__((aligned(1024))) T k_lds0[kKElems];
  __shared__ __attribute__((aligned(1024))) T k_lds1[kKElems];
  __shared__ __attribute__((aligned(1024))) T k_lds2[kKElems];
  __shared__ __attribute__((aligned(1024))) T v_lds0[kVElems];
  __shared__ __attribute__((aligned(1024))) T v_lds1[kVElems];
  __shared__ __attribute__((aligned(1024))) T v_lds2[kVElems];
  if constexpr (STAGES == 3) {
    attn_fwd_body<T, D, NW, 1, BN, 3, MODE, CAUSAL, SPLIT, BIAS, true>(
        a, stage_arrays(k_lds0, k_lds1, k_lds2, k_lds0, v_lds0, v_lds1, v_lds2, v_lds0));
  } else {
    __shared__ __attribute__((aligned(1024))) T k_lds3[kKElems];
    __shared__ __attribute__((aligned(1024))) T v_lds3[kVElems];
    attn_fwd_body<T, D, NW, 1, BN, 4, MODE, CAUSAL, SPLIT, BIAS, true>(
        a, stage_arrays(k_lds0, k_lds1, k_lds2, k_lds3, v_lds0, v_lds1, v_lds2, v_lds3));
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

// Launches the key-group kernel serves (16-bit, no mask, no bias) and the
// largest grid for which it replaces four-wave single-group workgroups (one
// workgroup per CU of the 256).  Measured with two key groups against the
// best single-group shape, on grids of 256 workgroups of 128 rows: fp16 D64
// B2 H32 Sq512 Sk8192 85.0 against 91.9 us, bf16 D128 of that shape 141.1
// against 148.5 us, bf16 D128 B16 H16 Sq128 Sk4096 100.0 against 106.5 us;
// on grids of 384 to 768 workgroups 8-18 % slower.
template <typename T, bool CAUSAL, bool BIAS>
constexpr bool kKeyGroupsServe = sizeof(T) == 2 && !CAUSAL && !BIAS;
constexpr uint32_t kKeyGroupMaxWorkgroups = 256;
// Whether a stage array of the two-key-group tile holds one row block's
// exchange buffer (D / 2 + 2 floats per lane; not so for D 128 with 32-key
// groups, whose K and V arrays are 16 KiB).
template <typename T, int D, int BN>
constexpr bool key_groups_fit() {
  using Path = typename PathFor<T, D>::type;
  return Path::template KCopy<2 * BN, 8>::kArrayBytes >= (D / 2 + 2) * 256 &&
         Path::template VCopy<2 * BN, 8>::kArrayBytes >= (D / 2 + 2) * 256;
}

template <typename T, int D, int MODE, bool CAUSAL, bool BIAS, int BUCKET>
int launch_bucket(const FwdArgs& args, hipStream_t stream) {
  constexpr TableEntry e = launch_entry<T, D, BUCKET, mask_variant(CAUSAL, MODE), BIAS>();
  FwdArgs a = args;
  a.causal_span = CAUSAL ? causal_span(static_cast<int64_t>(a.num_heads) * a.num_z, a.m_tiles, e.waves,
                                       MODE == MODE_COMPACT ? kCausalPartWavesCompact
                                                            : kCausalPartWaves)
                         : 0;
  const uint32_t grid = static_cast<uint32_t>(a.m_tiles) * a.num_heads * a.num_z;
  if constexpr (e.schedule == kSchedPingPong) {
    static_assert(e.waves == 8 && sizeof(T) == 2, "ping-pong: 8 waves, 16-bit inputs");
    hipLaunchKernelGGL((attn_fwd_pingpong_kernel<T, D, e.block_n, e.stages, MODE, CAUSAL>),
                       dim3(grid), dim3(512), 0, stream, a);
  } else if constexpr (e.schedule == kSchedLagged) {
    hipLaunchKernelGGL((attn_fwd_lagged_kernel<T, D, e.waves, e.block_n, e.stages, MODE, CAUSAL,
                                               false, BIAS>),
                       dim3(grid), dim3(e.waves * 64), 0, stream, a);
  } else if constexpr (e.schedule == kSchedThreeWaves) {
    hipLaunchKernelGGL((attn_fwd_3w_kernel<T, D, e.waves, e.block_n, e.stages, MODE, CAUSAL, false,
                                           BIAS>),
                       dim3(grid), dim3(e.waves * 64), 0, stream, a);
  } else {
    // A launch of four-wave workgroups that holds at most one workgroup per
    // CU would run one wave per SIMD: two key groups of the same 128-row
    // tiles give each SIMD two waves instead (same m-tiles, same work).
    if constexpr (kKeyGroupsServe<T, CAUSAL, BIAS> && e.schedule == kSchedSingle &&
                  e.waves == 4 && key_groups_fit<T, D, e.block_n>()) {
      if (grid <= kKeyGroupMaxWorkgroups) {
        constexpr int kStages = D == 128 ? 2 : e.stages;
        hipLaunchKernelGGL((attn_fwd_kg_kernel<T, D, 2, e.block_n, kStages, MODE>), dim3(grid),
                           dim3(512), 0, stream, a);
        return static_cast<int>(hipGetLastError());
      }
    }
    hipLaunchKernelGGL((attn_fwd_kernel<T, D, e.waves, row_blocks(e), e.block_n, e.stages, MODE,
                                        CAUSAL, false, BIAS>),
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
  constexpr TableEntry e = launch_entry<T, D, BUCKET, 0, true>();
  const uint32_t grid =
      static_cast<uint32_t>(a.m_tiles) * a.num_heads * a.num_z * static_cast<uint32_t>(a.num_splits);
  if constexpr (e.schedule == kSchedLagged) {
    hipLaunchKernelGGL((attn_fwd_lagged_kernel<T, D, e.waves, e.block_n, e.stages, MODE_DENSE,
                                               CAUSAL, true, false>),
                       dim3(grid), dim3(e.waves * 64), 0, stream, a);
  } else if constexpr (e.schedule == kSchedThreeWaves) {
    hipLaunchKernelGGL((attn_fwd_3w_kernel<T, D, e.waves, e.block_n, e.stages, MODE_DENSE, CAUSAL,
                                           true, false>),
                       dim3(grid), dim3(e.waves * 64), 0, stream, a);
  } else {
    hipLaunchKernelGGL((attn_fwd_kernel<T, D, e.waves, row_blocks(e), e.block_n, e.stages,
                                        MODE_DENSE, CAUSAL, true, false>),
                       dim3(grid), dim3(e.waves * 64), 0, stream, a);
  }
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
template <typename T, int D, bool SINGLE_GROUP, int BUCKET>
TableEntry entry_for_bucket(int variant) {
  switch (variant) {
    case 0: return launch_entry<T, D, BUCKET, 0, SINGLE_GROUP>();
    case 1: return launch_entry<T, D, BUCKET, 1, SINGLE_GROUP>();
    case 2: return launch_entry<T, D, BUCKET, 2, SINGLE_GROUP>();
    default: return launch_entry<T, D, BUCKET, 3, SINGLE_GROUP>();
  }
}

template <typename T, int D, bool SINGLE_GROUP>
TableEntry entry_for(int bucket, int variant) {
  switch (bucket) {
    case 0: return entry_for_bucket<T, D, SINGLE_GROUP, 0>(variant);
    case 1: return entry_for_bucket<T, D, SINGLE_GROUP, 1>(variant);
    case 2: return entry_for_bucket<T, D, SINGLE_GROUP, 2>(variant);
    case 3: return entry_for_bucket<T, D, SINGLE_GROUP, 3>(variant);
    case 4: return entry_for_bucket<T, D, SINGLE_GROUP, 4>(variant);
    case 5: return entry_for_bucket<T, D, SINGLE_GROUP, 5>(variant);
    case 6: return entry_for_bucket<T, D, SINGLE_GROUP, 6>(variant);
    default: return entry_for_bucket<T, D, SINGLE_GROUP, 7>(variant);
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
