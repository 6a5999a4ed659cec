/*
 * attn.h -- C ABI of a fused, exact scaled-dot-product attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed (per batch b and head h, tensors of shape [B, H, N, d]):
 *
 *   S   = scale * Q K^T                     (N x N, never stored)
 *   P   = softmax(S) row-wise               (N x N, never stored)
 *   O   = P V
 *   LSE = per query row, m + ln(l), where m is the row max of S and l the sum
 *         of exp(S - m) over the row: the softmax statistics the backward
 *         pass recomputes P from, P_ij = exp(S_ij - LSE_i).
 *
 * The three-line definition is the one in "What Are We Computing?" of the page
 * "Paper Notes: FlashAttention"; the 1/sqrt(d) scale is the one of "build it
 * from scratch" on the "flash attention" page (here an explicit argument);
 * the tiled loop with a running max and running sum follows "Tiling:
 * Block-by-Block Softmax" (Paper Notes) and "Rescale and accumulate" (the
 * aicassindra.com FlashAttention page); saving only O and the per-row
 * statistics and recomputing S and P in the backward pass is "Background" /
 * "Key Ideas" (Paper Notes) and "The backward pass: recompute instead of
 * store" (aicassindra).  The causal mask ("Common pitfalls", aicassindra)
 * keeps key j for query i when j <= i.
 *
 * Conventions for every entry point:
 *   - Tensors are dense, row-major [B, H, N, d] (d innermost), in device
 *     memory, with the element type given by `dtype`; LSE and the softmax
 *     statistics are float32 [B, H, N].  Queries and keys have the same N.
 *   - Supported: d in {64, 128}; N >= 1; B, H >= 1; dtype ATTN_BF16 (bf16
 *     inputs and outputs, fp32 accumulation, outputs rounded to nearest-even)
 *     or ATTN_FP32 (fp32 throughout).  N * d must not exceed 2^30 and
 *     B * H * N must stay below 2^31.
 *   - Alignment: every [B, H, N, d] tensor pointer must be 16-byte aligned
 *     (the kernels move 16-byte vectors and fetch tiles by 16-byte
 *     buffer->LDS loads), every float32 [B, H, N] pointer (LSE, D) 4-byte
 *     aligned, workspaces 256-byte aligned; a block mask may have any
 *     alignment.  A misaligned pointer returns ATTN_E_ALIGN (a workspace,
 *     ATTN_E_WORKSPACE) before any HIP call.
 *   - The caller allocates and owns every buffer.  The library allocates no
 *     device memory; scratch memory the backward pass needs is passed in as
 *     `workspace`.
 *   - Arguments are validated on the host before any HIP call; an invalid
 *     argument returns a negative attn_status and launches nothing.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     null stream).  No call synchronises.  ATTN_E_HIP reports a launch
 *     failure.  NaN or Inf inputs propagate; they are not detected.
 *   - Output buffers must not alias inputs.  Calls on different streams with
 *     disjoint outputs may run concurrently; the library holds no state.
 */
#ifndef EXACT_IO_AWARE_ATTN_H
#define EXACT_IO_AWARE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_BF16 = 0, /* bfloat16 tensors */
  ATTN_FP32 = 1  /* float32 tensors */
} attn_dtype;

typedef enum {
  ATTN_OK = 0,
  ATTN_E_NULL = -1,        /* a required pointer is NULL */
  ATTN_E_SHAPE = -2,       /* B, H or N < 1, or a size limit exceeded */
  ATTN_E_UNSUPPORTED = -3, /* head dimension or dtype not supported */
  ATTN_E_SCALE = -4,       /* scale is NaN or infinite */
  ATTN_E_WORKSPACE = -5,   /* workspace missing or smaller than required */
  ATTN_E_HIP = -6,         /* a HIP launch failed */
  ATTN_E_DROPOUT = -7,     /* dropout probability outside [0, 1) or NaN */
  ATTN_E_ALIGN = -8,       /* a tensor pointer not 16-byte aligned, or an
                              LSE / D pointer not 4-byte aligned */
  ATTN_E_SCRATCH = -9      /* attn_bwd_noalloc: B * H * N * 4 bytes exceed
                              ATTN_NOALLOC_SCRATCH_BYTES */
} attn_status;

/*
 * Forward pass: O = softmax(scale * Q K^T [masked]) V and LSE.
 *
 *   q, k, v : inputs [B, H, N, d] of `dtype` (read only)
 *   o       : output [B, H, N, d] of `dtype` (written)
 *   lse     : output float32 [B, H, N], natural-log log-sum-exp of each
 *             scaled (and masked) score row (written)
 *   causal  : nonzero keeps only keys j <= i for query i
 *   scale   : multiplies Q K^T before the softmax (usually 1/sqrt(d)); any
 *             finite value
 *   stream  : hipStream_t to enqueue on
 *
 * Returns ATTN_OK or a negative attn_status.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int64_t B, int64_t H, int64_t N, int64_t d, int dtype, int causal,
             float scale, void* stream);

/*
 * Bytes of device workspace attn_bwd needs for this shape (0 on an invalid
 * shape).  The workspace holds the per-row statistic D_i = sum_k dO_ik O_ik
 * (float32 [B, H, N]).  Its content on entry does not matter; attn_bwd
 * overwrites it.
 */
size_t attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d,
                                int dtype);

/*
 * Backward pass by recomputation.  Given the forward inputs, its outputs O
 * and LSE (as produced by attn_fwd with the same causal and scale) and the
 * output gradient dO, computes
 *
 *   P  = exp(scale * Q K^T - LSE)            (recomputed tile by tile)
 *   dV = P^T dO,  dP = dO V^T,  D_i = sum_k dO_ik O_ik,
 *   dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
 *
 * The pages defer these formulas to a companion article; they are the
 * textbook chain rule of O = softmax(scale Q K^T) V.
 *
 *   q, k, v, o, dout : [B, H, N, d] of `dtype` (read only)
 *   lse              : float32 [B, H, N] from attn_fwd (read only)
 *   dq, dk, dv       : outputs [B, H, N, d] of `dtype` (written)
 *   causal, scale    : must equal the values given to attn_fwd
 *   workspace        : device memory of at least
 *                      attn_bwd_workspace_bytes(B, H, N, d, dtype) bytes,
 *                      256-byte aligned, not shared with a concurrent call
 *
 * The result is deterministic (no floating-point atomics).  Returns ATTN_OK
 * or a negative attn_status.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o,
             const void* dout, const float* lse, void* dq, void* dk, void* dv,
             int64_t B, int64_t H, int64_t N, int64_t d, int dtype, int causal,
             float scale, void* workspace, size_t workspace_bytes,
             void* stream);

/*
 * The backward pass with no allocation and no workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  Same arguments,
 * kernels and results as attn_bwd, bit for bit; its scratch (D, float32
 * [B, H, N]) lives in a fixed device array of ATTN_NOALLOC_SCRATCH_BYTES
 * that the library holds on every GPU it runs on until the process ends.
 *
 *   - B * H * N * 4 bytes above ATTN_NOALLOC_SCRATCH_BYTES (B * H * N above
 *     4194304) return ATTN_E_SCRATCH before any HIP call.
 *   - The current device must be the device of `stream` and of the tensors.
 *     The first call on a device looks the array's address up (no
 *     allocation); a failure there returns ATTN_E_HIP.
 *   - Every call on one GPU uses that GPU's one array: calls that overlap on
 *     a GPU (two streams, or two host threads) race and must be serialised by
 *     the caller.  The array's content on entry does not matter (D is fully
 *     written before it is read).
 *   - Calls no hipMalloc, hipFree or other allocating routine.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES (16u << 20)

int attn_bwd_noalloc(const void* q, const void* k, const void* v,
                     const void* o, const void* dout, const float* lse,
                     void* dq, void* dk, void* dv, int64_t B, int64_t H,
                     int64_t N, int64_t d, int dtype, int causal, float scale,
                     void* stream);

/*
 * The backward pass in its three phases.  They are exposed so that the two
 * gradient phases, which are independent once D is known, can run on two
 * streams, and so that each phase can be timed on its own (attn_bwd itself
 * runs attn_bwd_dq_dsum, below, then attn_bwd_dkdv for bf16).  Arguments mean what they mean for attn_bwd;
 * `dsum` is float32 [B, H, N] device memory (D_i = sum_k dO_ik O_ik), written
 * by attn_bwd_dsum and read by the other two.  Same validation and error
 * behaviour as attn_bwd (a NULL dsum is ATTN_E_NULL).
 */
int attn_bwd_dsum(const void* o, const void* dout, float* dsum, int64_t B,
                  int64_t H, int64_t N, int64_t d, int dtype, void* stream);

int attn_bwd_dkdv(const void* q, const void* k, const void* v,
                  const void* dout, const float* lse, const float* dsum,
                  void* dk, void* dv, int64_t B, int64_t H, int64_t N,
                  int64_t d, int dtype, int causal, float scale, void* stream);

int attn_bwd_dq(const void* q, const void* k, const void* v, const void* dout,
                const float* lse, const float* dsum, void* dq, int64_t B,
                int64_t H, int64_t N, int64_t d, int dtype, int causal,
                float scale, void* stream);

/*
 * The dQ phase with D formed inside it: reads O and dO, writes
 * dsum (D_i = sum_k dO_ik O_ik, float32 [B, H, N]) and dq.  attn_bwd runs
 * this, then attn_bwd_dkdv, for bf16 (one pass fewer over O and dO than
 * attn_bwd_dsum followed by attn_bwd_dq); for fp32 it runs attn_bwd_dsum and
 * attn_bwd_dq.  Same validation and error behaviour as attn_bwd_dq.
 */
int attn_bwd_dq_dsum(const void* q, const void* k, const void* v,
                     const void* o, const void* dout, const float* lse,
                     float* dsum, void* dq, int64_t B, int64_t H, int64_t N,
                     int64_t d, int dtype, int causal, float scale,
                     void* stream);

/*
 * Block-sparse attention: the block-sparse variant of the method that the
 * page "Paper Notes: FlashAttention" reports in "Experiments & Results"
 * (faster than dense FlashAttention in proportion to the sparsity).  The
 * pages give no further detail; here the score matrix of each head is cut
 * into ATTN_SPARSE_BLOCK x ATTN_SPARSE_BLOCK blocks (query block, key block)
 * and a caller-supplied mask says which blocks are computed.  Query i may
 * attend key j only when the block holding (i, j) is nonzero in the mask
 * (and, with `causal`, also j <= i); masked scores count as -inf, so the
 * result is the exact softmax over each row's allowed keys.  Masked blocks
 * are skipped, not computed.  A row with no allowed key gets O = 0,
 * LSE = -inf and dQ = 0, and contributes nothing to dK and dV.
 *
 *   block_mask       : device memory, uint8, [nb, nb] per head, row-major
 *                      (query block, key block), nb = ceil(N / 128);
 *                      nonzero = computed.  Read only; must not change
 *                      while the call runs.
 *   mask_head_stride : bytes between the masks of consecutive heads, in
 *                      b * H + h order; 0 = one mask for every head, else at
 *                      least nb * nb.
 *
 * Other arguments, layouts, ownership and errors as for attn_fwd / attn_bwd;
 * attn_bwd_blocksparse must get the mask and causal flag given to
 * attn_fwd_blocksparse, and the same workspace size as attn_bwd.  bf16 only
 * (ATTN_FP32 returns ATTN_E_UNSUPPORTED); N at most ATTN_SPARSE_MAX_N; a NULL
 * mask is ATTN_E_NULL, a stride out of range or a larger N ATTN_E_SHAPE.
 * Deterministic, like the dense calls.
 */
#define ATTN_SPARSE_BLOCK 128
#define ATTN_SPARSE_MAX_N 131072

int attn_fwd_blocksparse(const void* q, const void* k, const void* v, void* o,
                         float* lse, int64_t B, int64_t H, int64_t N,
                         int64_t d, int dtype, int causal, float scale,
                         const uint8_t* block_mask, int64_t mask_head_stride,
                         void* stream);

int attn_bwd_blocksparse(const void* q, const void* k, const void* v,
                         const void* o, const void* dout, const float* lse,
                         void* dq, void* dk, void* dv, int64_t B, int64_t H,
                         int64_t N, int64_t d, int dtype, int causal,
                         float scale, const uint8_t* block_mask,
                         int64_t mask_head_stride, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * Queries and keys of different lengths: q, o, dout, dq are [B, H, Nq, d],
 * k, v, dk, dv are [B, H, Nk, d], lse and the backward workspace's D are
 * [B, H, Nq].  The pages fix no causal alignment for unequal lengths; here it
 * is bottom-right, the alignment of Nq queries that follow Nk - Nq earlier
 * tokens (decoding, chunked prefill): query i sees key j when
 * j <= i + (Nk - Nq).  With Nq > Nk the first Nq - Nk rows see no key and get
 * O = 0, LSE = -inf, dQ = 0.  Nq == Nk is the square case of attn_fwd.
 *
 * Split-K/V (for few queries over many keys): the keys are cut into
 * num_splits chunks of whole 64-key tiles, each chunk's (normalised O, LSE)
 * per row goes to the workspace, and a second kernel merges them by the
 * two-block rule of "Tiling: Block-by-Block Softmax" (Paper Notes), in the
 * form LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s.
 * num_splits = 1: no split (no workspace); 2..64: at most that many chunks
 * (fewer if Nk has fewer tiles); 0: chosen by the library from the shape.
 * One to four query rows over at least as many keys (decoding) run a
 * vector-ALU kernel that streams K and V once (the matrix-core kernel's
 * 128-row tile would be mostly empty); its automatic split aims at about
 * 1024 workgroups with chunks of at least 128 keys (d = 128) or 256 (d = 64).
 * More rows: about 512 workgroups of 128 query rows, chunks of at least
 * 256 keys.
 *
 *   attn_fwd_qk_workspace_bytes : bytes attn_fwd_qk needs for this shape and
 *                                 num_splits (0 when no split is used, or on
 *                                 an invalid argument)
 *   attn_bwd_qk_workspace_bytes : bytes attn_bwd_qk needs: D ([B, H, Nq]
 *                                 fp32), then, when the shape has few query
 *                                 blocks for the chip (B * H * ceil(Nq / 256)
 *                                 at d = 128, ceil(Nq / 128) at d = 64, at
 *                                 most 128) and at least 8 key tiles, the dQ
 *                                 pass is split over chunks of whole 64-key
 *                                 tiles (about 256 workgroups, at least 4
 *                                 tiles a chunk, at most 64 chunks) and the
 *                                 workspace also holds one fp32 partial dQ
 *                                 [B, H, Nq, d] per chunk; the chunks are
 *                                 summed in a fixed order, so the result stays
 *                                 deterministic.
 *
 * Other arguments, ownership and errors as for attn_fwd / attn_bwd.  bf16 only
 * (ATTN_FP32 returns ATTN_E_UNSUPPORTED); num_splits outside 0..64 is
 * ATTN_E_SHAPE; a workspace that is NULL (when needed), too small or not
 * 256-byte aligned is ATTN_E_WORKSPACE.  Deterministic.
 */
size_t attn_fwd_qk_workspace_bytes(int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                                   int64_t d, int dtype, int num_splits);

int attn_fwd_qk(const void* q, const void* k, const void* v, void* o,
                float* lse, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                int64_t d, int dtype, int causal, float scale, int num_splits,
                void* workspace, size_t workspace_bytes, void* stream);

size_t attn_bwd_qk_workspace_bytes(int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                                   int64_t d, int dtype);

int attn_bwd_qk(const void* q, const void* k, const void* v, const void* o,
                const void* dout, const float* lse, void* dq, void* dk,
                void* dv, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                int64_t d, int dtype, int causal, float scale, void* workspace,
                size_t workspace_bytes, void* stream);

/*
 * Dropout on the probabilities.  The pages list dropout among the
 * element-wise operations kernel fusion folds into one kernel ("Background",
 * Paper Notes) and fix no formula; this is the usual attention dropout:
 *
 *   O = (P * Z) V / (1 - p_drop),  LSE as without dropout (the statistics of
 *   S; the backward pass recomputes P from it),
 *
 * with Z_ij in {0, 1}.  Z is drawn by Philox4x32-10 (Salmon, Moraes, Dror,
 * Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011), nothing is
 * stored: for head bh = b * H + h, query i and key j, the counter is
 * (j / 4, i, bh, offset mod 2^32) and the key (seed mod 2^32, seed / 2^32);
 * output word j % 4 is compared with t = min(floor(p_drop * 2^32), 2^32 - 1)
 * and the element is kept when the word is >= t (p_drop = 0 keeps every
 * element and gives attn_fwd's results bit for bit).  The backward pass
 * regenerates the same Z, so attn_bwd_dropout must get the p_drop, seed and
 * offset (and causal, scale) of the forward:
 *
 *   dV = (P * Z)^T dO / (1 - p),  dP = (dO V^T) * Z / (1 - p),
 *   dS = P * (dP - D) with D_i = sum_k dO_ik O_ik,  dQ = scale dS K,
 *   dK = scale dS^T Q.
 *
 * bf16 only (ATTN_FP32 returns ATTN_E_UNSUPPORTED); p_drop outside [0, 1)
 * or NaN returns ATTN_E_DROPOUT.  The backward workspace is that of attn_bwd
 * (attn_bwd_workspace_bytes).  Other arguments, ownership and errors as for
 * attn_fwd / attn_bwd.  Deterministic for given inputs, seed and offset.
 */
int attn_fwd_dropout(const void* q, const void* k, const void* v, void* o,
                     float* lse, int64_t B, int64_t H, int64_t N, int64_t d,
                     int dtype, int causal, float scale, float p_drop,
                     uint64_t seed, uint64_t offset, void* stream);

int attn_bwd_dropout(const void* q, const void* k, const void* v,
                     const void* o, const void* dout, const float* lse,
                     void* dq, void* dk, void* dv, int64_t B, int64_t H,
                     int64_t N, int64_t d, int dtype, int causal, float scale,
                     float p_drop, uint64_t seed, uint64_t offset,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Key padding: the mask half of the element-wise operations that kernel
 * fusion folds into the attention kernel ("Background", Paper Notes: mask
 * listed beside dropout), in its most common form, a per-sequence key
 * length.  For batch b, key j is masked (its score counts as -inf, as under
 * the causal mask) when j >= key_len[b], for every head and query:
 *
 *   S_ij = -inf for j >= key_len[b] (and, with causal, for j > i),
 *   P = softmax(S) per row, O = P V, LSE = log sum_j exp(S_ij),
 *
 * and the gradients are those of that masked softmax (textbook chain rule,
 * as in attn_bwd); the padded keys' dK and dV are zero.  A row that sees no
 * key (key_len[b] = 0) gets O = 0, LSE = -inf and dQ = 0.
 *
 * key_len: device int32 [B], read by the kernels (not validated on the
 * host); a value below 0 counts as 0, above N as N.  NULL returns
 * ATTN_E_NULL, a pointer not 4-byte aligned ATTN_E_ALIGN.  Square lengths,
 * dense (no block mask, no dropout); both dtypes.  The padded rows of K and
 * V must hold finite values (which ones does not change any result: they
 * enter only with weight zero).  Other arguments, layout, ownership,
 * workspace and errors as for attn_fwd / attn_bwd; the backward pass must be
 * given the key_len (and causal, scale) of the forward.
 */
int attn_fwd_kpad(const void* q, const void* k, const void* v, void* o,
                  float* lse, int64_t B, int64_t H, int64_t N, int64_t d,
                  int dtype, int causal, float scale, const int32_t* key_len,
                  void* stream);

int attn_bwd_kpad(const void* q, const void* k, const void* v, const void* o,
                  const void* dout, const float* lse, void* dq, void* dk,
                  void* dv, int64_t B, int64_t H, int64_t N, int64_t d,
                  int dtype, int causal, float scale, const int32_t* key_len,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Causal sliding window (local attention): a second mask of the same kind,
 * the causal mask restricted to the last `window` keys.  Query i attends
 * keys j with i - window < j <= i:
 *
 *   S_ij = -inf unless i - window < j <= i,  P = softmax(S) per row,
 *   O = P V, LSE = log sum_j exp(S_ij),
 *
 * with the gradients of that masked softmax (as in attn_bwd).  Every row sees
 * at least its own key.  Key tiles wholly outside a query block's window are
 * never visited, so the work grows as N * window rather than N^2 / 2.
 * window >= N gives attn_fwd / attn_bwd's causal results bit for bit (the
 * same kernels); window < 1 returns ATTN_E_SHAPE.  Square lengths, dense;
 * both dtypes.  Other arguments, layout, ownership, workspace and errors as
 * for attn_fwd / attn_bwd; the backward pass must be given the window (and
 * scale) of the forward.
 */
int attn_fwd_window(const void* q, const void* k, const void* v, void* o,
                    float* lse, int64_t B, int64_t H, int64_t N, int64_t d,
                    int dtype, int64_t window, float scale, void* stream);

int attn_bwd_window(const void* q, const void* k, const void* v,
                    const void* o, const void* dout, const float* lse,
                    void* dq, void* dk, void* dv, int64_t B, int64_t H,
                    int64_t N, int64_t d, int dtype, int64_t window,
                    float scale, void* workspace, size_t workspace_bytes,
                    void* stream);

/* Static, human-readable name of a status code (never NULL). */
const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_IO_AWARE_ATTN_H */
