// Flash-attention backward kernels for CDNA4 (gfx950), bf16 and fp16 inputs.
//
// The backward of O = softmax(scale * Q K^T) V recomputes the softmax weights
// from the per-row logsumexp that the forward returns -- the one number per
// row that nvFuser issue #2278 "Investigate a new SDPA IR node" leaves the
// forward to stash for its SdpaOpBwd node -- and never writes the score
// matrix to memory.  With c = scale:
//
//   delta_i = sum_d dO_id O_id                          (dQ kernel)
//   P_ij    = exp(c q_i . k_j - LSE_i), 0 where masked
//   dP_ij   = dO_i . v_j
//   dS_ij   = P_ij (dP_ij - delta_i)
//   dQ_i    = c sum_j dS_ij k_j                          (dQ kernel)
//   dK_j    = c sum_i dS_ij q_i,   dV_j = sum_i P_ij dO_i (dK/dV kernel)
//
// P and dS are recomputed twice, once per query tile (dQ, a lane owns a query
// row) and once per key tile (dK and dV, a lane owns a key), so every
// gradient row is summed inside one workgroup: no atomics, deterministic.
//
// Register layout, as in the forward: in a 32x32 MFMA accumulator lane l
// holds column l % 32 and register r holds row 8 (r / 4) + 4 (l / 32) + r % 4.
//  - dQ kernel: S^T = K Q^T and dP^T = V dO^T (K and V tiles in LDS as A
//    operands, the wave's Q and dO rows in registers as B operands) put one
//    query row per lane; dQ^T += K^T dS^T reads K transposed.
//  - dK/dV kernel: S = Q K^T and dP = dO V^T (Q and dO tiles in LDS, the
//    wave's K and V rows in registers) put one key per lane;
//    dV^T += dO^T P and dK^T += Q^T dS read dO and Q transposed.
// In both, the rounded P or dS accumulator is directly the B operand of the
// transposed product, exactly as P is in the forward's P V.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_common.h"
#include "bwd_args.h"

namespace sdpa03 {
namespace {

// LDS tiles are unpadded (rows of exactly D * 2 bytes) and chunk-swizzled
// (swizzle_of<D>): conflict-free both for 16-row MFMA operand reads and for
// transposing reads, which no row padding achieves (D * 2 + 80, say, keeps
// the plain reads clean but makes every transposing pass of 4 rows overlap
// itself in the bank cycle).  Unpadded rows also make a tile a power of two
// in size, which the XOR-addressed stages need.
template <int D>
constexpr int swizzled_row_bytes() { return D * 2; }

template <typename T>
using frag_t = typename Mma16<T>::frag;

// A compile-time choice passed to a generic lambda: the masked and the
// unmasked forms of a step are separate code, so the steps of the tiles no
// mask reaches carry no compares or selects (the dQ kernel).
template <bool B>
struct MaskedStep {
  static constexpr bool value = B;
};

// Scheduling requests for one block of N_MFMA products fed by N_READ LDS
// fragment reads (sched_group_barrier masks: 0x008 MFMA, 0x100 LDS read):
// a few reads ahead, then one product and its share of reads.  Without them
// the compiler issues every read of the block first and runs out of
// registers.
template <int N_MFMA, int N_READ>
__device__ __forceinline__ void interleave_reads() {
  constexpr int per = (N_READ + N_MFMA - 1) / N_MFMA;
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * per, 0);
#pragma unroll
  for (int i = 0; i < N_MFMA; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, per, 0);
  }
}

// The two products on an LDS tile (swizzled, rows of ROW = D * 2 bytes),
// addressed by LDS byte address.  The tile's stage base is aligned to twice
// the stage size, so the lane's chunk bits join its base by XOR and the row
// offsets stay immediates.
//
// addr_rows_x_regs: c[nb] += A B for nb < NB.  A: rows 32 nb .. 32 nb + 31
// of the tile, 16 dims per k-step (lane (rho, h) reads the 16 bytes at dims
// 16 ks + 8 h -- chunk 2 ks + h, stored at (2 ks + h) ^ swizzle_of<D>(rho));
// lane_addr is the lane's address for ks = 0.  B: the wave's own rows, one
// fragment per k-step, in registers.
//
// addr_tr_x_frags: acc[db] += X^T W.  X: the tile's NB * 32 rows read
// transposed; W: the rounded fragments of NB 32-row accumulators over those
// rows, register r of lane (i, h) holding row 8 (r / 4) + 4 h + r % 4, so
// k-step (nb, half) -- registers 8 half .. 8 half + 7 -- covers rows
// 32 nb + 16 half + {4 h .. 4 h + 3, 8 + 4 h .. 8 + 4 h + 3}.  Within each
// group of 16 lanes, ds_read_b64_tr_b16 gives lane i element (i & 3) of the
// 64-bit words read by lanes 4 j + (i >> 2); with lane t pointing at row
// R0 + t / 4, column C0 + 4 (t & 3), lane i receives X[R0 + j][C0 + i] for
// j = 0..3.  Two reads (sub = 0, 1: R0 = 32 nb + 16 half + 4 h and R0 + 8)
// give the eight rows of one operand.  lane_addr[sub] is the address of the
// lane's row and column (its chunk bits XORed with the swizzle of the row,
// which modulo 16 depends only on sub and the lane) for nb = half = db = 0.
// An LDS byte address as a typed LDS pointer (through uintptr_t, so that the
// host pass, where such pointers are 64-bit, sees no widening cast).
template <typename P>
__device__ __forceinline__ __attribute__((address_space(3))) P* lds_ptr(uint32_t addr) {
  return (__attribute__((address_space(3))) P*)(static_cast<uintptr_t>(addr));
}

template <typename T>
__device__ __forceinline__ frag_t<T> lds_frag(uint32_t addr) {
  return *lds_ptr<const frag_t<T>>(addr);
}

template <typename T, int D, int ROW, int NB>
__device__ __forceinline__ void addr_rows_x_regs(uint32_t lane_addr, const frag_t<T> (&b)[D / 16],
                                                 f32x16 (&c)[NB]) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const uint32_t a0 = lane_addr ^ static_cast<uint32_t>(ks * 32);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      c[nb] = Mma16<T>::mma(lds_frag<T>(a0 + nb * 32 * ROW), b[ks], c[nb]);
    }
  }
}

template <typename T, int ROW, int NB, int DB>
__device__ __forceinline__ void addr_tr_x_frags(const uint32_t (&lane_addr)[2],
                                                const frag_t<T> (&w)[NB][2], f32x16 (&acc)[DB]) {
  using s16x4 = short __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        s16x4 x[2];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
          const uint32_t src = (lane_addr[sub] ^ static_cast<uint32_t>(db * 64)) +
                               (nb * 32 + half * 16 + sub * 8) * ROW;
          x[sub] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr<s16x4>(src));
        }
        frag_t<T> xf;
        __builtin_memcpy(&xf, x, sizeof(xf));
        acc[db] = Mma16<T>::mma(xf, w[nb][half], acc[db]);
      }
    }
  }
}

// The wave's own 32 rows as MFMA B-operand fragments: lane (i, h) holds the
// 8 elements at dims 16 ks + 8 h of row i (zeros for rows past the end).
template <typename T, int D>
__device__ __forceinline__ void load_row_frags(const T* row, bool ok, int lh,
                                               frag_t<T> (&f)[D / 16]) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    f[ks] = ok ? *reinterpret_cast<const frag_t<T>*>(row + 16 * ks + 8 * lh) : frag_t<T>{};
  }
}

// Stores a 32 x D accumulator whose lane owns one output row (register r of
// block db holds dims 32 db + 8 (r / 4) + 4 h + r % 4), times `mul`.
template <typename T, int DB>
__device__ __forceinline__ void store_row(T* row, const f32x16 (&acc)[DB], float mul, int lh) {
#pragma unroll
  for (int db = 0; db < DB; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      T out4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) out4[e] = static_cast<T>(acc[db][4 * g + e] * mul);
      uint2 packed;
      __builtin_memcpy(&packed, out4, 8);
      *reinterpret_cast<uint2*>(row + db * 32 + g * 8 + lh * 4) = packed;
    }
  }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per 256 query rows of one (batch, head); 8 waves of 32
// rows; key tiles of 64 stream through two LDS stages.
// ---------------------------------------------------------------------------
template <typename T, int D, int MODE, bool CAUSAL>
__global__ __launch_bounds__(512, 1) void attn_bwd_dq_kernel(BwdArgs a) {
  constexpr int NW = kBwdDqRows / 32;
  constexpr int BM = kBwdDqRows;
  constexpr int BN = 64;
  constexpr int NB = BN / 32;
  constexpr int DB = D / 32;
  // K (read plainly and transposed) and V (read plainly) tiles, both
  // unpadded and swizzled; two stages of each in one array, a power-of-two
  // stage apart (XOR-addressed stages, one loop body, untracked copies: as
  // in the dK/dV kernel).
  constexpr int kRow = swizzled_row_bytes<D>();
  using KCopy = TileCopy<T, D, BN, NW, kRow, true>;
  using frag = frag_t<T>;
  constexpr int kStage = KCopy::kArrayBytes;
  static_assert(kStage == BN * kRow && (kStage & (kStage - 1)) == 0, "power-of-two stages");
  __shared__ __attribute__((aligned(2 * kStage))) T k_lds[kStage];  // 2 stages of kStage bytes
  __shared__ __attribute__((aligned(2 * kStage))) T v_lds[kStage];

  // Under the causal mask the last query tiles cost the most: they go first.
  const uint32_t groups = static_cast<uint32_t>(a.num_heads) * static_cast<uint32_t>(a.num_z);
  uint32_t g, rank;
  bwd_launch_order(CAUSAL, static_cast<uint32_t>(a.q_tiles), groups, a.span_q, g, rank);
  const int m = CAUSAL ? a.q_tiles - 1 - static_cast<int>(rank) : static_cast<int>(rank);
  const int h = static_cast<int>(g % static_cast<uint32_t>(a.num_heads));
  const int z = static_cast<int>(g / static_cast<uint32_t>(a.num_heads));
  const SeqRange sr =
      seq_range_of<MODE>(a.cu_q, a.cu_k, a.total_q, a.total_k, a.seqlen_q, a.seqlen_k, z);
  const int m0 = m * BM;
  if (m0 >= sr.len_q) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31;
  const int lh = lane >> 5;
  const int row0 = m0 + wave * 32;
  const int qi = row0 + li;                       // local query row
  const bool row_ok = qi < sr.len_q;
  const int64_t token = static_cast<int64_t>(sr.q_start) + qi;  // row of the rank-4 view

  const T* qrow = static_cast<const T*>(a.q) + sr.b * a.q_sb + h * a.q_sh + token * a.q_ss;
  const T* drow = static_cast<const T*>(a.dout) + sr.b * a.do_sb + h * a.do_sh + token * a.do_ss;
  const char* kp = reinterpret_cast<const char*>(
      static_cast<const T*>(a.k) + sr.b * a.k_sb + h * a.k_sh +
      static_cast<int64_t>(sr.k_start) * a.k_ss);
  const char* vp = reinterpret_cast<const char*>(
      static_cast<const T*>(a.v) + sr.b * a.v_sb + h * a.v_sh +
      static_cast<int64_t>(sr.k_start) * a.v_ss);
  const int64_t k_row_bytes = a.k_ss * static_cast<int64_t>(sizeof(T));
  const int64_t v_row_bytes = a.v_ss * static_cast<int64_t>(sizeof(T));

  frag qf[D / 16];
  frag df[D / 16];
  load_row_frags<T, D>(qrow, row_ok, lh, qf);
  load_row_frags<T, D>(drow, row_ok, lh, df);
  // The row's delta = rowsum(dO * O) (lanes l and l + 32 hold half the row
  // each) and LSE * log2(e), kept here and written to the workspace for the
  // dK/dV kernel.  Rows of the tile that belong to no sequence -- past the
  // end (dense, padded) or past the last sequence (compact; rows past any
  // other sequence are the next one's) -- get delta = 0 and +inf, so any
  // weight computed from them is exactly 0: the dK/dV kernel reads whole
  // 64-row tiles, which end inside this 256-row tile.
  float delta = 0.f;
  float lse2 = __builtin_huge_valf();
  {
    const T* orow = static_cast<const T*>(a.o) + sr.b * a.o_sb + h * a.o_sh + token * a.o_ss;
    frag of[D / 16];
    load_row_frags<T, D>(orow, row_ok, lh, of);
    float part = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        part = fmaf(static_cast<float>(of[ks][e]), static_cast<float>(df[ks][e]), part);
      }
    }
    const float row_delta = sum_across_halves(part);
    if (row_ok) {
      delta = row_delta;
      lse2 = a.lse[sr.b * a.lse_sb + h * a.lse_sh + token] * kLog2e;
    }
    bool owned = row_ok;
    if constexpr (MODE == MODE_COMPACT) {
      const int real_rows = min(max(a.cu_q[a.num_z], 0), a.total_q);
      owned = owned || token >= real_rows;
    } else {
      owned = true;
    }
    if (lh == 0 && owned && token < a.ws_rows_pad) {
      const int64_t wrow = (static_cast<int64_t>(sr.b) * a.num_heads + h) * a.ws_rows_pad + token;
      a.ws_delta[wrow] = delta;
      a.ws_lse2[wrow] = lse2;
    }
  }
  if (!row_ok) lse2 = 0.f;
  const float c2 = a.scale_log2;

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  int kend = sr.len_k;
  if constexpr (CAUSAL) kend = min(kend, min(m0 + BM, sr.len_q));
  const int n_tiles = (kend + BN - 1) / BN;

  KCopy kcopy;
  KCopy vcopy;
  kcopy.init(wave, lane, k_row_bytes);
  vcopy.init(wave, lane, v_row_bytes);
  auto issue = [&](int t, int st) {
    const int j0 = t * BN;
    kcopy.issue_untracked(kp + j0 * k_row_bytes, kend - j0, k_row_bytes, k_lds + st * (kStage / 2),
                          wave);
    vcopy.issue_untracked(vp + j0 * v_row_bytes, kend - j0, v_row_bytes, v_lds + st * (kStage / 2),
                          wave);
  };

  // Per-lane LDS addresses in stage 0 (see the dK/dV kernel).
  const uint32_t k_base = (uint32_t)(uintptr_t)(lds_void_ptr)(k_lds);
  const uint32_t v_base = (uint32_t)(uintptr_t)(lds_void_ptr)(v_lds);
  const uint32_t plain_off = li * kRow + ((lh ^ swizzle_of<D>(li)) << 4);
  uint32_t tr_off[2];
  {
    const int tt = lane & 15;
    const int grp = lane >> 4;
    const int row_lane = (grp >> 1) * 4 + (tt >> 2);
    const int col_lane = (grp & 1) * 16 + 4 * (tt & 3);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      tr_off[sub] = row_lane * kRow + ((col_lane * 2) ^ (swizzle_of<D>(sub * 8 + row_lane) << 4));
    }
  }

  // Tile t, one 32-key block at a time (it keeps the live softmax state to
  // one block): scores, weights, dP, dS, then dQ^T += K^T dS^T.
  auto compute = [&](auto masked, int t, int st) {
    const uint32_t so = static_cast<uint32_t>(st * kStage);
    const uint32_t k_plain = (k_base + plain_off) ^ so;
    const uint32_t v_plain = (v_base + plain_off) ^ so;
    const uint32_t k_tr[2] = {(k_base + tr_off[0]) ^ so, (k_base + tr_off[1]) ^ so};
#pragma nounroll
    for (int nb = 0; nb < NB; ++nb) {
      const int j0 = t * BN + nb * 32;
      // Under the causal mask a block whose first key follows the wave's
      // last row adds nothing (every weight is 0): skipped, wave-uniform.
      if (CAUSAL && decltype(masked)::value && j0 > row0 + 31) continue;
      const uint32_t row_off = static_cast<uint32_t>(nb * 32 * kRow);
      f32x16 st_[1] = {f32x16{}};
      addr_rows_x_regs<T, D, kRow, 1>(k_plain + row_off, qf, st_);
      f32x16 dpt[1] = {f32x16{}};
      addr_rows_x_regs<T, D, kRow, 1>(v_plain + row_off, df, dpt);
      const bool need_mask =
          decltype(masked)::value && ((j0 + 32 > sr.len_k) || (CAUSAL && j0 + 31 > row0));
      frag w[1][2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = __builtin_amdgcn_exp2f(fmaf(st_[0][r], c2, -lse2));
        if (need_mask) {
          const int key = j0 + 8 * (r >> 2) + 4 * lh + (r & 3);
          if (!(key < sr.len_k && (!CAUSAL || key <= qi))) p = 0.f;
        }
        w[0][r >> 3][r & 7] = static_cast<T>(p * (dpt[0][r] - delta));
      }
      const uint32_t ktr[2] = {k_tr[0] + row_off, k_tr[1] + row_off};
      addr_tr_x_frags<T, kRow, 1, DB>(ktr, w, acc);
      // S^T and dP^T: 2 * D/16 products over as many reads; dQ: 2 * DB
      // products over 4 * DB transposing reads.
      interleave_reads<2 * (D / 16) + 2 * DB, 2 * (D / 16) + 4 * DB>();
    }
  };

  if (n_tiles > 0) {
    issue(0, 0);
    wait_vmem();
    barrier_lds();
    // Step t computes tile t from one stage while tile t + 1 loads into the
    // other (free: its last readers passed the barrier ending step t - 1).
    // Only the last key tile (ragged) and, under the causal mask, the tiles
    // from the workgroup's first row on can hold a masked key.
    const int first_masked = CAUSAL ? min(m0 / BN, (sr.len_k - 1) / BN) : (sr.len_k - 1) / BN;
    auto step = [&](auto masked, int t) {
      const int st = t & 1;
      if (t + 1 < n_tiles) issue(t + 1, st ^ 1);
      compute(masked, t, st);
      wait_vmem();
      barrier_lds();
    };
    const int split = max(0, min(first_masked, n_tiles));
    for (int t = 0; t < split; ++t) step(MaskedStep<false>{}, t);
    for (int t = split; t < n_tiles; ++t) step(MaskedStep<true>{}, t);
  }

  if (row_ok) {
    T* dqrow = static_cast<T*>(a.dq) + sr.b * a.q_sb + h * a.q_sh + token * a.q_ss;
    store_row<T, DB>(dqrow, acc, a.scale, lh);
  }
}

// ---------------------------------------------------------------------------
// dK and dV: one workgroup per 128 keys of one (batch, head); 4 waves of 32
// keys; query tiles of 64 rows (Q and dO) stream through two LDS stages.
// Two waves per SIMD: at D = 128 the wave's K and V rows and both
// accumulators take most of its 256 registers (the causal and compact
// kernels spill a few; still faster than one wave per SIMD).
// ---------------------------------------------------------------------------
template <typename T, int D, int MODE, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void attn_bwd_dkdv_kernel(BwdArgs a) {
  constexpr int NW = kBwdDkvKeys / 32;
  constexpr int BQ = 64;
  constexpr int NB = BQ / 32;
  constexpr int DB = D / 32;
  constexpr int kRow = swizzled_row_bytes<D>();
  using QCopy = TileCopy<T, D, BQ, NW, kRow, true>;
  // A tile's BQ workspace values (LSE * log2(e), delta) as one row of BQ
  // floats: one buffer load into a 1 KiB LDS block, issued by one wave.
  using WCopy = TileCopy<float, BQ, 1, 1, BQ * 4>;
  static_assert(WCopy::kArrayBytes == 1024, "one block per workspace vector");
  using frag = frag_t<T>;
  // Two stages of each tile kind in one array, kStage bytes (a power of two)
  // apart, the array aligned to 2 kStage: stage 1's addresses are stage 0's
  // XOR kStage.  One loop body then serves both stages (two unrolled bodies
  // made the compiler copy the dK and dV accumulators between them every
  // step).  The workspace vectors: per stage 1 KiB of LSE * log2(e), then
  // 1 KiB of delta.
  constexpr int kStage = QCopy::kArrayBytes;
  static_assert(kStage == BQ * kRow && (kStage & (kStage - 1)) == 0, "power-of-two stages");
  constexpr int kWStage = 2 * WCopy::kArrayBytes;
  __shared__ __attribute__((aligned(2 * kStage))) T q_lds[kStage];  // 2 stages of kStage bytes
  __shared__ __attribute__((aligned(2 * kStage))) T d_lds[kStage];
  __shared__ __attribute__((aligned(2 * kWStage))) float w_lds[kWStage / 2];

  // Under the causal mask the first key tiles cost the most: they go first.
  const uint32_t groups = static_cast<uint32_t>(a.num_heads) * static_cast<uint32_t>(a.num_z);
  uint32_t g, rank;
  bwd_launch_order(CAUSAL, static_cast<uint32_t>(a.k_tiles), groups, a.span_k, g, rank);
  const int kt = static_cast<int>(rank);
  const int h = static_cast<int>(g % static_cast<uint32_t>(a.num_heads));
  const int z = static_cast<int>(g / static_cast<uint32_t>(a.num_heads));
  const SeqRange sr =
      seq_range_of<MODE>(a.cu_q, a.cu_k, a.total_q, a.total_k, a.seqlen_q, a.seqlen_k, z);
  const int n0 = kt * kBwdDkvKeys;
  if (n0 >= sr.len_k) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31;
  const int lh = lane >> 5;
  const int key0 = n0 + wave * 32;  // first key of this wave
  const int kj = key0 + li;         // this lane's key (local)
  const bool key_ok = kj < sr.len_k;
  const int64_t ktoken = static_cast<int64_t>(sr.k_start) + kj;  // row of the rank-4 view

  const T* krow = static_cast<const T*>(a.k) + sr.b * a.k_sb + h * a.k_sh + ktoken * a.k_ss;
  const T* vrow = static_cast<const T*>(a.v) + sr.b * a.v_sb + h * a.v_sh + ktoken * a.v_ss;
  const char* qp = reinterpret_cast<const char*>(
      static_cast<const T*>(a.q) + sr.b * a.q_sb + h * a.q_sh +
      static_cast<int64_t>(sr.q_start) * a.q_ss);
  const char* dp = reinterpret_cast<const char*>(
      static_cast<const T*>(a.dout) + sr.b * a.do_sb + h * a.do_sh +
      static_cast<int64_t>(sr.q_start) * a.do_ss);
  const int64_t q_row_bytes = a.q_ss * static_cast<int64_t>(sizeof(T));
  const int64_t d_row_bytes = a.do_ss * static_cast<int64_t>(sizeof(T));
  // Workspace rows of this sequence's query rows (local row q at [q]).
  const int64_t wbase = (static_cast<int64_t>(sr.b) * a.num_heads + h) * a.ws_rows_pad + sr.q_start;
  const float* lse2p = a.ws_lse2 + wbase;
  const float* deltap = a.ws_delta + wbase;

  frag kf[D / 16];
  frag vf[D / 16];
  load_row_frags<T, D>(krow, key_ok, lh, kf);
  load_row_frags<T, D>(vrow, key_ok, lh, vf);
  const float c2 = a.scale_log2;

  f32x16 dk[DB];
  f32x16 dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  // Query rows before the workgroup's first key see none of its keys.
  const int qbeg = CAUSAL ? (n0 / BQ) * BQ : 0;
  const int n_tiles = sr.len_q > qbeg ? (sr.len_q - qbeg + BQ - 1) / BQ : 0;

  QCopy qcopy;
  QCopy dcopy;
  WCopy wcopy;
  qcopy.init(wave, lane, q_row_bytes);
  dcopy.init(wave, lane, d_row_bytes);
  wcopy.init(0, lane, BQ * 4);
  // The tile's workspace values travel with its Q and dO rows (waves 0 and 1
  // issue them): read from global memory inside the block loop, their waits
  // would also drain the next tile's copies, issued earlier, every block.
  // The workspace rows of a whole tile lie inside its padding.  The copies
  // are issued as inline assembly the compiler does not track (it could not
  // tell the stage being filled from the one being read); every wave waits
  // for its own copies at the end of the step, before the barrier.
  auto issue = [&](int t, int st) {
    const int q0 = qbeg + t * BQ;
    const int rows = sr.len_q - q0;
    qcopy.issue_untracked(qp + q0 * q_row_bytes, rows, q_row_bytes, q_lds + st * (kStage / 2),
                          wave);
    dcopy.issue_untracked(dp + q0 * d_row_bytes, rows, d_row_bytes, d_lds + st * (kStage / 2),
                          wave);
    if (wave == 0) {
      wcopy.issue_untracked(reinterpret_cast<const char*>(lse2p + q0), 1, BQ * 4,
                            w_lds + st * (kWStage / 4), 0);
    } else if (wave == 1) {
      wcopy.issue_untracked(reinterpret_cast<const char*>(deltap + q0), 1, BQ * 4,
                            w_lds + st * (kWStage / 4) + 256, 0);
    }
  };

  // Per-lane LDS addresses in stage 0: the plain reads' row li, chunk
  // lh ^ swizzle; the transposing reads' row and column of each sub-pass.
  const uint32_t q_base = (uint32_t)(uintptr_t)(lds_void_ptr)(q_lds);
  const uint32_t d_base = (uint32_t)(uintptr_t)(lds_void_ptr)(d_lds);
  const uint32_t w_base = (uint32_t)(uintptr_t)(lds_void_ptr)(w_lds);
  const uint32_t plain_off = li * kRow + ((lh ^ swizzle_of<D>(li)) << 4);
  uint32_t tr_off[2];
  {
    const int tt = lane & 15;
    const int grp = lane >> 4;
    const int row_lane = (grp >> 1) * 4 + (tt >> 2);
    const int col_lane = (grp & 1) * 16 + 4 * (tt & 3);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      tr_off[sub] = row_lane * kRow + ((col_lane * 2) ^ (swizzle_of<D>(sub * 8 + row_lane) << 4));
    }
  }

  // Query tile t, one 32-row block at a time: S = Q K^T, P,
  // dV^T += dO^T P, dP = dO V^T, dS, dK^T += Q^T dS.  Register r belongs to
  // query row q0 + 32 nb + 8 (r / 4) + 4 h + r % 4.
  auto compute = [&](int t, int st) {
    const uint32_t so = static_cast<uint32_t>(st * kStage);  // stage offset, an XOR
    const uint32_t q_plain = (q_base + plain_off) ^ so;
    const uint32_t d_plain = (d_base + plain_off) ^ so;
    const uint32_t q_tr[2] = {(q_base + tr_off[0]) ^ so, (q_base + tr_off[1]) ^ so};
    const uint32_t d_tr[2] = {(d_base + tr_off[0]) ^ so, (d_base + tr_off[1]) ^ so};
    const uint32_t w_st = w_base + static_cast<uint32_t>(st * kWStage);
#pragma nounroll
    for (int nb = 0; nb < NB; ++nb) {
      const int q0 = qbeg + t * BQ + nb * 32;
      // Under the causal mask a block whose last row precedes the wave's
      // first key adds nothing to its dK and dV: skipped, wave-uniform.
      if (CAUSAL && q0 + 31 < key0) continue;
      const uint32_t row_off = static_cast<uint32_t>(nb * 32 * kRow);
      const uint32_t qtr[2] = {q_tr[0] + row_off, q_tr[1] + row_off};
      const uint32_t dtr[2] = {d_tr[0] + row_off, d_tr[1] + row_off};
      const uint32_t lb = w_st + static_cast<uint32_t>(nb * 32 * 4);
      const uint32_t eb = lb + 1024;
      f32x16 s[1] = {f32x16{}};
      addr_rows_x_regs<T, D, kRow, 1>(q_plain + row_off, kf, s);
      // Dense and padded rows past the sequence carry LSE * log2(e) = +inf
      // (and delta 0) in the workspace and zero Q and dO rows, so their
      // weights are exactly 0 unmasked; keys past it feed only the lane's own
      // dK and dV columns, which are not stored.  Compact rows past the
      // sequence belong to the next one (finite LSE): those are masked, as
      // are keys past the row under the causal mask.
      const bool need_mask =
          (MODE == MODE_COMPACT && q0 + 32 > sr.len_q) || (CAUSAL && q0 < key0 + 31);
      float pr[16];
      frag w[1][2];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int qr = q0 + 8 * g4 + 4 * lh;
        const f32x4 l4 = *lds_ptr<const f32x4>(lb + static_cast<uint32_t>((8 * g4 + 4 * lh) * 4));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g4 + e;
          float p = __builtin_amdgcn_exp2f(fmaf(s[0][r], c2, -l4[e]));
          if (need_mask) {
            const int q = qr + e;
            if (!(q < sr.len_q && (!CAUSAL || kj <= q))) p = 0.f;
          }
          pr[r] = p;
          w[0][r >> 3][r & 7] = static_cast<T>(p);
        }
      }
      addr_tr_x_frags<T, kRow, 1, DB>(dtr, w, dv);
      f32x16 dpp[1] = {f32x16{}};
      addr_rows_x_regs<T, D, kRow, 1>(d_plain + row_off, vf, dpp);
      frag ws[1][2];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 d4 = *lds_ptr<const f32x4>(eb + static_cast<uint32_t>((8 * g4 + 4 * lh) * 4));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g4 + e;
          ws[0][r >> 3][r & 7] = static_cast<T>(pr[r] * (dpp[0][r] - d4[e]));
        }
      }
      addr_tr_x_frags<T, kRow, 1, DB>(qtr, ws, dk);
      interleave_reads<2 * (D / 16) + 4 * DB, 2 * (D / 16) + 8 * DB>();
    }
  };

  if (n_tiles > 0) {
    issue(0, 0);
    wait_vmem();
    barrier_lds();
    // One loop body for every tile: separate masked and unmasked loops
    // (as in the dQ kernel) measured 4 % slower here under the causal mask,
    // the extra body costing the dK and dV accumulators more spills.
    for (int t = 0; t < n_tiles; ++t) {
      const int st = t & 1;
      if (t + 1 < n_tiles) issue(t + 1, st ^ 1);
      compute(t, st);
      wait_vmem();
      barrier_lds();
    }
  }

  if (key_ok) {
    T* dkrow = static_cast<T*>(a.dk) + sr.b * a.k_sb + h * a.k_sh + ktoken * a.k_ss;
    T* dvrow = static_cast<T*>(a.dv) + sr.b * a.v_sb + h * a.v_sh + ktoken * a.v_ss;
    store_row<T, DB>(dkrow, dk, a.scale, lh);
    store_row<T, DB>(dvrow, dv, 1.f, lh);
  }
}

template <typename T, int D, int MODE, bool CAUSAL>
int launch_typed(const BwdArgs& args, hipStream_t s) {
  BwdArgs a = args;
  const uint32_t groups = static_cast<uint32_t>(a.num_heads) * static_cast<uint32_t>(a.num_z);
  a.span_q = CAUSAL ? causal_span(groups, a.q_tiles, kBwdDqRows * 2 / 64) : 0;
  a.span_k = CAUSAL ? causal_span(groups, a.k_tiles, kBwdDkvKeys * 2 / 64) : 0;
  if (a.q_tiles > 0) {
    hipLaunchKernelGGL((attn_bwd_dq_kernel<T, D, MODE, CAUSAL>),
                       dim3(static_cast<uint32_t>(a.q_tiles) * groups), dim3(kBwdDqRows * 2), 0, s, a);
    const int err = static_cast<int>(hipGetLastError());
    if (err != 0) return err;
  }
  if (a.k_tiles > 0) {
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, D, MODE, CAUSAL>),
                       dim3(static_cast<uint32_t>(a.k_tiles) * groups), dim3(kBwdDkvKeys * 2), 0, s, a);
    return static_cast<int>(hipGetLastError());
  }
  return 0;
}

template <typename T, int D>
int launch_mode(const BwdArgs& a, int mode, bool causal, hipStream_t s) {
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
int launch_dim(const BwdArgs& a, int head_dim, int mode, bool causal, hipStream_t s) {
  return head_dim == 64 ? launch_mode<T, 64>(a, mode, causal, s) : launch_mode<T, 128>(a, mode, causal, s);
}

}  // namespace

int launch_attn_bwd(const BwdArgs& a, int dtype, int head_dim, int mode, bool causal,
                    void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  return dtype == DT_F16 ? launch_dim<_Float16>(a, head_dim, mode, causal, s)
                         : launch_dim<__bf16>(a, head_dim, mode, causal, s);
}

}  // namespace sdpa03
