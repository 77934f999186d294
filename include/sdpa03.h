/*
 * sdpa03.h -- C ABI of libsdpa03.so: the flash-attention forward pass on
 * AMD Instinct MI355X (gfx950).
 *
 * Operation.  For one (batch or sequence, head) with Lq query rows and Lk
 * key rows, every entry point computes
 *
 *     S    = scale * Q K^T                      (fp32 accumulation)
 *     P    = softmax over the allowed keys of each row of S
 *     O    = P V                                 (stored in the input dtype)
 *     LSE  = per-row natural-log logsumexp of the allowed scaled scores (fp32)
 *
 * tile by tile with a running max and running sum, never writing S to
 * memory.  With causal != 0 query row i sees keys 0..i in indices local to
 * its sequence (top-left alignment; it equals bottom-right when Lq == Lk).
 * A row that sees no key (only when Lk == 0) gets O = 0 and LSE = -inf.
 * The operation is the scaled-dot-product attention that nvFuser issue
 * #2278 "Investigate a new SDPA IR node" wants as a forward node; LSE is the
 * per-row value that the issue's discussion of what to stash for the
 * backward pass calls for.
 *
 * Three entry points share one kernel family, as AOTriton PR #31 "Add
 * varlen support to AOTriton's Flash Attention" does for its forward
 * (opening comment): dense, compact variable-length and padded
 * variable-length.  Following the same PR's closing reply, a new layout
 * would get a new entry point rather than a flag on these.
 *
 * Conventions shared by all entry points
 * --------------------------------------
 *  - Tensors are rank-4 views (batch, head, seq, dim) given as a device
 *    pointer and four strides counted in ELEMENTS (the rank-4 view with
 *    pointer plus sizes plus strides that the PR's TensorView<4> names).
 *    stride[3] (dim) must be 1 and stride[2] (seq) at least head_dim (rows
 *    do not overlap); K and V row strides are at most 16 MiB (the kernels
 *    fetch K/V tiles with 32-bit buffer offsets).  Q, K, V and O share one dtype; K and V
 *    share their sizes; Q and O share their sizes; Q and K may differ only
 *    in sequence length (AOTriton issue #12, xinyazhang's reply on the
 *    attn_fwd constraints).
 *  - Base pointers must be 16-byte aligned and strides[0..2] times the
 *    element size must be multiples of 16 bytes (the kernels use 128-bit
 *    loads).  k and v may be NULL only when the key axis is empty
 *    (seqlen_k, total_k or seqlen_k_max is 0); every other pointer is
 *    required whenever there is a query row to produce.
 *  - lse is a contiguous fp32 array written for valid rows only.
 *  - Sequence-length arguments are int32, as the PR unifies them.
 *  - head_dim must be 64 or 128.  dtype is one of sdpa_dtype.
 *  - scale must be finite and > 0 (callers usually pass 1/sqrt(head_dim)).
 *  - Ownership: the caller allocates and owns every buffer.  The library
 *    allocates nothing, keeps no state between calls, never synchronises
 *    and may be called from several host threads at once.  Work is queued on
 *    hip_stream (a hipStream_t; NULL means the null stream) and completes
 *    asynchronously; outputs are valid once that stream has reached the
 *    launch.  Calls that share output buffers on different streams race.
 *  - Errors: every argument is checked on the host before anything is
 *    launched.  On any error nothing is launched and no output is touched;
 *    the status says what was wrong (sdpa_status_string).  A launch the HIP
 *    runtime rejects returns SDPA_ERR_HIP.  An empty problem (no query row
 *    to produce) returns SDPA_OK without launching.
 *  - Unsupported inputs are rejected, never silently mis-computed: Triton
 *    issue #2267 "[RFC] Goal for triton.ops.flash_attention" (opening
 *    comment) describes an attention op that gave wrong answers for inputs
 *    outside its assumptions, and nvFuser issue #2278 notes that flash
 *    attention does not cover every input.
 */
#ifndef SDPA03_H
#define SDPA03_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SDPA_F32 = 0,  /* float32 in and out; fp32 products (no 16-bit rounding) */
  SDPA_F16 = 1,  /* IEEE half in and out; fp32 accumulation */
  SDPA_BF16 = 2  /* bfloat16 in and out; fp32 accumulation */
} sdpa_dtype;

typedef enum {
  SDPA_OK = 0,
  SDPA_ERR_NULL = 1,      /* a required pointer is NULL */
  SDPA_ERR_DTYPE = 2,     /* dtype is not an sdpa_dtype value */
  SDPA_ERR_HEAD_DIM = 3,  /* head_dim is not 64 or 128 */
  SDPA_ERR_SHAPE = 4,     /* a size is negative, or the problem is too large to index */
  SDPA_ERR_STRIDE = 5,    /* stride[3] != 1, a negative stride, or offsets overflow */
  SDPA_ERR_ALIGN = 6,     /* a base pointer or stride breaks 16-byte alignment */
  SDPA_ERR_BATCH = 7,     /* compact varlen called with B != 1 */
  SDPA_ERR_SEQLEN = 8,    /* bad sequence-length arguments or cu_seqlens contents */
  SDPA_ERR_SCALE = 9,     /* scale is not finite and positive */
  SDPA_ERR_HIP = 10,      /* the HIP runtime rejected the launch */
  SDPA_ERR_WORKSPACE = 11, /* split forward: workspace NULL, misaligned or too small */
  SDPA_ERR_SCRATCH = 12    /* attn_fwd_splitk_noalloc: the plan needs more than the
                              library's static scratch (SDPA_NOALLOC_SCRATCH_BYTES) */
} sdpa_status;

/* Bytes of the library's static per-device scratch that
 * attn_fwd_splitk_noalloc uses in place of a caller's workspace. */
#define SDPA_NOALLOC_SCRATCH_BYTES (32u << 20)

/* Static text for a status code (never NULL). */
const char* sdpa_status_string(sdpa_status status);

/*
 * Dense forward.  Q: (B, H, seqlen_q, head_dim), K and V:
 * (B, H, seqlen_k, head_dim), O like Q, lse: (B, H, seqlen_q) fp32
 * contiguous.  seqlen_q != seqlen_k is allowed (Triton issue #2267 lists
 * differing query and key counts as a use case).  Sizes may be zero.
 */
sdpa_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     sdpa_dtype dtype, int32_t B, int32_t H, int32_t seqlen_q,
                     int32_t seqlen_k, int32_t head_dim,
                     const int64_t q_stride[4], const int64_t k_stride[4],
                     const int64_t v_stride[4], const int64_t o_stride[4],
                     float scale, int32_t causal, void* hip_stream);

/*
 * Compact variable-length forward (AOTriton PR #31, opening comment: rank-4
 * tensors whose batch size is exactly 1, over packed tokens).  Packed
 * (total, H, head_dim) token memory is passed as the (1, H, total, head_dim)
 * view with strides (total*H*D, D, H*D, 1); any view with dim stride 1 works.
 *
 * Sequence z owns query tokens [cu_seqlens_q[z], cu_seqlens_q[z+1]) and key
 * tokens [cu_seqlens_k[z], cu_seqlens_k[z+1]); no attention crosses
 * sequences and the causal mask uses indices local to the sequence.
 * cu_seqlens_q and cu_seqlens_k are DEVICE arrays of num_seqs + 1 int32
 * exclusive prefix sums; they are read only by the kernel.
 * lse: (1, H, total_q) fp32 contiguous.  Tokens past cu_seqlens_q[num_seqs]
 * are neither read nor written.
 *
 * B must be 1 (SDPA_ERR_BATCH otherwise: extra batches are refused rather
 * than ignored).  num_seqs >= 0; 0 <= max_seqlen_q <= total_q and
 * 0 <= max_seqlen_k <= total_k.
 *
 * Contract not checked on the device (the contents of device memory are not
 * read on the host): cu_seqlens_*[0] == 0, entries non-decreasing, the last
 * entry <= total_*, every length <= max_seqlen_*.  Host code that holds a
 * copy can check it with sdpa_check_cu_seqlens_host first.
 */
sdpa_status attn_fwd_compact_varlen(const void* q, const void* k, const void* v, void* o,
                                    float* lse, sdpa_dtype dtype, int32_t B, int32_t H,
                                    int32_t total_q, int32_t total_k, int32_t head_dim,
                                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                    int32_t num_seqs, int32_t max_seqlen_q,
                                    int32_t max_seqlen_k,
                                    const int64_t q_stride[4], const int64_t k_stride[4],
                                    const int64_t v_stride[4], const int64_t o_stride[4],
                                    float scale, int32_t causal, void* hip_stream);

/*
 * Padded variable-length forward.  Q: (B, H, seqlen_q_max, head_dim), K and
 * V: (B, H, seqlen_k_max, head_dim), O like Q, lse: (B, H, seqlen_q_max)
 * fp32 contiguous.  Batch b's true lengths are cu_seqlens_q[b+1] -
 * cu_seqlens_q[b] and cu_seqlens_k[b+1] - cu_seqlens_k[b] (DEVICE int32
 * arrays of B + 1 entries); its rows and keys start at offset 0 of its own
 * slab, as in the padded branch of the fwd_kernel.py excerpt that AOTriton
 * PR #31 quotes.  Rows and keys at or past a batch's true length are never
 * read; their O and lse entries are left untouched.
 *
 * Contract not checked on the device: entries non-decreasing and every
 * length <= seqlen_*_max.
 */
sdpa_status attn_fwd_padded_varlen(const void* q, const void* k, const void* v, void* o,
                                   float* lse, sdpa_dtype dtype, int32_t B, int32_t H,
                                   int32_t seqlen_q_max, int32_t seqlen_k_max,
                                   int32_t head_dim, const int32_t* cu_seqlens_q,
                                   const int32_t* cu_seqlens_k,
                                   const int64_t q_stride[4], const int64_t k_stride[4],
                                   const int64_t v_stride[4], const int64_t o_stride[4],
                                   float scale, int32_t causal, void* hip_stream);

/*
 * Forward with an additive bias, one entry point per layout.  AOTriton PR #31
 * (opening comment, note 1) keeps a rank-4 bias tensor input in its forward
 * calls (reserved there); the nvFuser issue #2278 points at PyTorch's
 * scaled_dot_product_attention, whose floating attn_mask is added to the
 * scaled scores.  Here the scores become
 *
 *     S = scale * q k^T + bias
 *
 * and everything else (mask, softmax, O, LSE) is as in the call without the
 * bias.  Arguments are those of attn_fwd, attn_fwd_compact_varlen and
 * attn_fwd_padded_varlen, plus:
 *  - bias: DEVICE memory of the same element type as q, read only, viewed
 *    as a rank-4 tensor indexed like the scores of the rank-4 views:
 *    (B, H, seqlen_q, seqlen_k) dense, (1, H, total_q, total_k) compact
 *    (sequence z reads the block at rows cu_seqlens_q[z].. and columns
 *    cu_seqlens_k[z]..), (B, H, seqlen_q_max, seqlen_k_max) padded (batch b
 *    reads from row and column 0).  Only entries of allowed (row, key) pairs
 *    are read.
 *  - bias_stride: element strides of that view.  The key stride must be 1;
 *    the others >= 0 (0 broadcasts, as PyTorch's expand does) and multiples
 *    of 4 elements; the base 16-byte aligned.
 * Entries must be finite or -inf.  A -inf entry hides the key from the row;
 * a row whose allowed scores are all -inf gets O = 0 and LSE = -inf, like a
 * row with no key.  Errors as the call without the bias, plus SDPA_ERR_NULL,
 * SDPA_ERR_STRIDE and SDPA_ERR_ALIGN for the bias.  The compact layout is
 * correct for any cu_seqlens_k, but a sequence whose keys start off a
 * multiple of 4 tokens loads its bias element by element (slower).
 */
sdpa_status attn_fwd_bias(const void* q, const void* k, const void* v, const void* bias,
                          void* o, float* lse, sdpa_dtype dtype, int32_t B, int32_t H,
                          int32_t seqlen_q, int32_t seqlen_k, int32_t head_dim,
                          const int64_t q_stride[4], const int64_t k_stride[4],
                          const int64_t v_stride[4], const int64_t bias_stride[4],
                          const int64_t o_stride[4], float scale, int32_t causal,
                          void* hip_stream);

sdpa_status attn_fwd_compact_varlen_bias(
    const void* q, const void* k, const void* v, const void* bias, void* o, float* lse,
    sdpa_dtype dtype, int32_t B, int32_t H, int32_t total_q, int32_t total_k, int32_t head_dim,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t num_seqs,
    int32_t max_seqlen_q, int32_t max_seqlen_k, const int64_t q_stride[4],
    const int64_t k_stride[4], const int64_t v_stride[4], const int64_t bias_stride[4],
    const int64_t o_stride[4], float scale, int32_t causal, void* hip_stream);

sdpa_status attn_fwd_padded_varlen_bias(
    const void* q, const void* k, const void* v, const void* bias, void* o, float* lse,
    sdpa_dtype dtype, int32_t B, int32_t H, int32_t seqlen_q_max, int32_t seqlen_k_max,
    int32_t head_dim, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
    const int64_t q_stride[4], const int64_t k_stride[4], const int64_t v_stride[4],
    const int64_t bias_stride[4], const int64_t o_stride[4], float scale, int32_t causal,
    void* hip_stream);

/*
 * Key-parallel ("split") dense forward for few query rows against many keys.
 * Triton issue #2267 (opening comment) counts differing numbers of queries
 * and keys among the use cases; with, say, 512 queries against 8192 keys a
 * grid of one workgroup per query tile leaves most of the 256 compute units
 * idle.  Here the key axis of every query tile is cut into num_splits
 * contiguous ranges of whole key tiles.  Each range is computed by its own
 * workgroup into a partial output normalised over the range's keys, kept in
 * fp32, plus the range's logsumexp; a second kernel then merges the ranges
 * row by row:
 *
 *     LSE = log sum_s exp(LSE_s),    O = sum_s exp(LSE_s - LSE) * O_s.
 *
 * The result is attn_fwd's O and LSE up to fp32 rounding order: the
 * logsumexp that the forward returns for the backward pass (nvFuser issue
 * #2278, on what to stash) is exactly what makes the ranges mergeable.
 *
 * Arguments as attn_fwd, plus:
 *  - num_splits: number of key ranges.  <= 0 lets the library choose (about
 *    two workgroups per compute unit of a 256-CU MI355X, and at least four
 *    key tiles per range); a request above the number of key tiles is cut
 *    to it.  sdpa_fwd_splitk_plan reports the value a call will use.
 *  - workspace: DEVICE memory of at least the workspace_bytes that
 *    sdpa_fwd_splitk_plan reports for the same dtype, sizes and num_splits,
 *    16-byte aligned and owned by the caller.  Its contents on entry do not
 *    matter; on return they are scratch.  Calls in flight at the same time
 *    must not share a workspace.
 * Returns SDPA_ERR_WORKSPACE for a NULL (when bytes are needed), misaligned
 * or too small workspace.  Empty problems return SDPA_OK without launching.
 */
sdpa_status attn_fwd_splitk(const void* q, const void* k, const void* v, void* o, float* lse,
                            sdpa_dtype dtype, int32_t B, int32_t H, int32_t seqlen_q,
                            int32_t seqlen_k, int32_t head_dim,
                            const int64_t q_stride[4], const int64_t k_stride[4],
                            const int64_t v_stride[4], const int64_t o_stride[4],
                            float scale, int32_t causal, int32_t num_splits, void* workspace,
                            uint64_t workspace_bytes, void* hip_stream);

/*
 * The split forward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops
 * and harnesses that forbid hipMalloc.  Same arguments and results as
 * attn_fwd_splitk, minus workspace and workspace_bytes: the partial outputs
 * and logsumexps go to a static buffer of SDPA_NOALLOC_SCRATCH_BYTES (32 MiB)
 * that the library holds on every GPU it runs on, from that GPU's first call
 * until the process ends.  The call allocates nothing (no hipMalloc, no
 * hipFree, no allocating library routine); its first call on a device looks
 * the buffer's address up once, with that device current.
 *
 *  - A problem whose plan (sdpa_fwd_splitk_plan with the same arguments)
 *    needs more than SDPA_NOALLOC_SCRATCH_BYTES is refused with
 *    SDPA_ERR_SCRATCH before anything is launched; e.g. 512 queries against
 *    8192 keys at head_dim 64 for B = 2, H = 32 in two splits need 17 MB.
 *  - Nothing in the buffer needs to start at zero: every partial result the
 *    merge reads is written earlier in the same call.  Each call leaves its
 *    own partial results behind.
 *  - Every call on a GPU shares that GPU's buffer: calls that overlap in time
 *    on one GPU (other streams, other host threads) race and may return
 *    garbage.  Serialise them, or use attn_fwd_splitk with a workspace each.
 *  - hip_stream must belong to the current device (SDPA_ERR_HIP otherwise).
 * Errors as attn_fwd_splitk (without the workspace ones), plus
 * SDPA_ERR_SCRATCH.
 */
sdpa_status attn_fwd_splitk_noalloc(const void* q, const void* k, const void* v, void* o,
                                    float* lse, sdpa_dtype dtype, int32_t B, int32_t H,
                                    int32_t seqlen_q, int32_t seqlen_k, int32_t head_dim,
                                    const int64_t q_stride[4], const int64_t k_stride[4],
                                    const int64_t v_stride[4], const int64_t o_stride[4],
                                    float scale, int32_t causal, int32_t num_splits,
                                    void* hip_stream);

/*
 * The split count attn_fwd_splitk will use for these sizes and request
 * (num_splits <= 0: the library's choice) and the workspace bytes it needs:
 * num_splits_used * B * H * seqlen_q * (head_dim + 1) * 4 plus alignment
 * padding.  Either output pointer may be NULL.  Errors: SDPA_ERR_DTYPE,
 * SDPA_ERR_HEAD_DIM, SDPA_ERR_SHAPE (negative or too large sizes).
 */
sdpa_status sdpa_fwd_splitk_plan(sdpa_dtype dtype, int32_t B, int32_t H, int32_t seqlen_q,
                                 int32_t seqlen_k, int32_t head_dim, int32_t num_splits,
                                 int32_t* num_splits_used, uint64_t* workspace_bytes);

/*
 * Dense backward (bf16 and fp16).  The nvFuser issue #2278 pairs the forward
 * SDPA node with an SdpaOpBwd node; AOTriton PR #31 pairs each forward API
 * with a backward one.  Given the forward's inputs q, k, v, its outputs o
 * and lse (as attn_fwd returns them, lse contiguous (B, H, seqlen_q) fp32)
 * and the gradient dout of o, it writes the gradients of
 * loss = sum(dout * o):
 *
 *     P = softmax over allowed keys of scale * q k^T   (rebuilt from lse)
 *     dv = P^T dout,   dS = P * (dout v^T - rowsum(dout * o)),
 *     dq = scale * dS k,   dk = scale * dS^T q.
 *
 * dq, dk and dv have the shapes and strides of q, k and v; dout has its own
 * strides.  Same mask convention as attn_fwd.  Every row of dq, dk and dv is
 * written (zeros where no allowed pair contributes); the results are
 * deterministic (no atomics).
 *
 * workspace: DEVICE memory of at least sdpa_bwd_workspace_bytes(B, H,
 * seqlen_q) bytes, 16-byte aligned, caller-owned scratch (it holds
 * rowsum(dout * o) and lse * log2(e) per query row).  Calls in flight at the
 * same time must not share it.
 * Errors as attn_fwd; SDPA_ERR_DTYPE for fp32 (not supported by the
 * backward); SDPA_ERR_WORKSPACE for a NULL, misaligned or small workspace.
 */
sdpa_status attn_bwd(const void* q, const void* k, const void* v, const void* o,
                     const void* dout, const float* lse, void* dq, void* dk, void* dv,
                     sdpa_dtype dtype, int32_t B, int32_t H, int32_t seqlen_q,
                     int32_t seqlen_k, int32_t head_dim,
                     const int64_t q_stride[4], const int64_t k_stride[4],
                     const int64_t v_stride[4], const int64_t o_stride[4],
                     const int64_t dout_stride[4], float scale, int32_t causal,
                     void* workspace, uint64_t workspace_bytes, void* hip_stream);

/*
 * Variable-length backward, compact (THD) layout: the gradients of
 * attn_fwd_compact_varlen with the same arguments.  Each sequence is an
 * independent problem, so its gradients are attn_bwd's on that sequence's
 * rows and keys alone (AOTriton PR #31 gives each varlen forward its
 * backward).  dout, o, dq have q's (1, H, total_q, head_dim) shape (dq with
 * q's strides), dk and dv k's and v's; lse is the forward's (1, H, total_q)
 * fp32 output.  Every row and key inside a sequence is written (zeros where
 * nothing contributes); tokens past cu_seqlens_*[num_seqs] are neither read
 * nor written.
 *
 * workspace: at least sdpa_bwd_workspace_bytes(1, H, total_q) bytes, as
 * for attn_bwd.  Same argument checks and device-side contract as
 * attn_fwd_compact_varlen; SDPA_ERR_DTYPE for fp32; SDPA_ERR_WORKSPACE as
 * attn_bwd.
 */
sdpa_status attn_bwd_compact_varlen(const void* q, const void* k, const void* v, const void* o,
                                    const void* dout, const float* lse, void* dq, void* dk,
                                    void* dv, sdpa_dtype dtype, int32_t B, int32_t H,
                                    int32_t total_q, int32_t total_k, int32_t head_dim,
                                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                    int32_t num_seqs, int32_t max_seqlen_q,
                                    int32_t max_seqlen_k,
                                    const int64_t q_stride[4], const int64_t k_stride[4],
                                    const int64_t v_stride[4], const int64_t o_stride[4],
                                    const int64_t dout_stride[4], float scale, int32_t causal,
                                    void* workspace, uint64_t workspace_bytes, void* hip_stream);

/*
 * Variable-length backward, padded layout: the gradients of
 * attn_fwd_padded_varlen with the same arguments (Q-side tensors
 * (B, H, seqlen_q_max, head_dim), key side (B, H, seqlen_k_max, head_dim),
 * lse (B, H, seqlen_q_max) fp32).  Rows and keys inside a batch's true
 * lengths are written (zeros where nothing contributes); those at or past
 * them are neither read nor written.
 *
 * workspace: at least sdpa_bwd_workspace_bytes(B, H, seqlen_q_max) bytes.
 * Same checks and device-side contract as attn_fwd_padded_varlen;
 * SDPA_ERR_DTYPE for fp32; SDPA_ERR_WORKSPACE as attn_bwd.
 */
sdpa_status attn_bwd_padded_varlen(const void* q, const void* k, const void* v, const void* o,
                                   const void* dout, const float* lse, void* dq, void* dk,
                                   void* dv, sdpa_dtype dtype, int32_t B, int32_t H,
                                   int32_t seqlen_q_max, int32_t seqlen_k_max,
                                   int32_t head_dim, const int32_t* cu_seqlens_q,
                                   const int32_t* cu_seqlens_k,
                                   const int64_t q_stride[4], const int64_t k_stride[4],
                                   const int64_t v_stride[4], const int64_t o_stride[4],
                                   const int64_t dout_stride[4], float scale, int32_t causal,
                                   void* workspace, uint64_t workspace_bytes, void* hip_stream);

/*
 * Workspace bytes the backward entry points need for B batches of H heads
 * with seqlen_q rows in the query view (total_q for the compact layout,
 * seqlen_q_max for the padded one): 2 * B * H * (roundup(seqlen_q, 64) + 64)
 * * 4.  SDPA_ERR_SHAPE for negative sizes.
 */
sdpa_status sdpa_bwd_workspace_bytes(int32_t B, int32_t H, int32_t seqlen_q,
                                     uint64_t* workspace_bytes);

/*
 * Host-side check of a HOST copy of a cu_seqlens array of n + 1 entries:
 * starts at 0, non-decreasing, last entry <= total, every length <=
 * max_len.  Returns SDPA_OK or SDPA_ERR_SEQLEN (SDPA_ERR_NULL for NULL).
 */
sdpa_status sdpa_check_cu_seqlens_host(const int32_t* cu, int32_t n, int32_t total,
                                       int32_t max_len);

/*
 * The compiled-in kernel choice of the forward for a problem: query rows
 * per workgroup (block_m), keys per tile (block_n) and wavefronts per
 * workgroup.  The dispatch key is the dtype, head_dim, the sequence extents,
 * the mask and the layout, as in the tuning database of AOTriton issue #12
 * (the maintainer's replies: an ahead-of-time autotune probing sequence
 * lengths, head dim and dtype that guides which kernel serves an input).
 * seqlen_q and seqlen_k are the dense lengths, the varlen calls'
 * max_seqlen_q / max_seqlen_k, or the padded calls' seqlen_*_max, in four
 * query buckets (<= 128, <= 512, <= 4096, longer) and two key buckets
 * (<= 512, longer); causal != 0 selects the causal entries and mode the
 * layout's (0 dense, 1 compact, 2 padded; the two variable-length layouts
 * share their entries).  single_group != 0 asks for the shape of the forward
 * with a bias (for its mask and layout) and of the split forward, which
 * uses the dense non-causal entry for both masks (query it with causal = 0,
 * mode = 0).  A 16-bit launch without the causal mask or a bias whose
 * entry has four waves, and which has at most 256 workgroups of block_m
 * rows, runs them as two key groups of four waves each (eight in all) over
 * the same block_m rows; block_m and block_n are unchanged, waves reports
 * the entry's four.  Any output pointer may be NULL.  Returns SDPA_ERR_DTYPE /
 * SDPA_ERR_HEAD_DIM for unsupported classes, SDPA_ERR_SHAPE for a bad mode
 * or negative length.
 */
sdpa_status sdpa_kernel_config(sdpa_dtype dtype, int32_t head_dim, int32_t causal,
                               int32_t mode, int32_t seqlen_q, int32_t seqlen_k,
                               int32_t single_group, int32_t* block_m, int32_t* block_n,
                               int32_t* waves);

#ifdef __cplusplus
}
#endif

#endif /* SDPA03_H */
