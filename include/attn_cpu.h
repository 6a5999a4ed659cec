/*
 * attn_cpu.h -- C ABI of the cache-blocked multi-core CPU form of the same
 * fused, exact attention (forward and backward), float32.
 *
 * The aicassindra FlashAttention page ("Practical implications and the CPU /
 * small-model view") carries the method to a CPU: DRAM is the slow tier and
 * the caches the fast one, and the computation is blocked so that its tiles
 * stay resident in cache and no N x N matrix is ever written out.  This
 * library does exactly that: the tiled loop with a running max and running
 * sum ("Tiling: Block-by-Block Softmax", Paper Notes page) over 64-row query
 * blocks and 64-key tiles whose working set (a few tiles of 16-32 KiB) stays
 * in one core's L1/L2 cache, with one OpenMP thread per (batch * head, block)
 * work item.  The backward pass recomputes S and P from Q, K and the saved
 * LSE ("The backward pass: recompute instead of store", aicassindra) in two
 * passes: key-block-stationary for dK and dV, query-block-stationary for dQ.
 *
 * It is an alternative implementation for CPUs, not a fallback: the GPU entry
 * points of attn.h never call it.  It computes what attn.h computes:
 *
 *   S = scale * Q K^T, P = softmax(S) row-wise (causal: key j kept for query i
 *   when j <= i), O = P V, LSE_i = m_i + ln l_i;
 *   dV = P^T dO, dP = dO V^T, D_i = sum_k dO_ik O_ik, dS = P * (dP - D),
 *   dQ = scale * dS K, dK = scale * dS^T Q.
 *
 * Conventions:
 *   - Every tensor is host memory, float32, dense row-major [B, H, N, d] (d
 *     innermost); LSE is float32 [B, H, N].  Queries and keys have the same
 *     N.  The caller owns every buffer; the library allocates only per-thread
 *     tile scratch (a few hundred KiB per thread), released before returning.
 *   - Supported: 1 <= d <= 256, N >= 1, B, H >= 1, finite scale.
 *   - `threads` is the number of OpenMP threads (0: the OpenMP default).
 *   - Calls are synchronous and thread-safe (no global state).
 *   - Returns ATTN_CPU_OK (0) or a negative status, before touching any
 *     output: ATTN_CPU_E_NULL (-1) for a null pointer, ATTN_CPU_E_SHAPE (-2)
 *     for a size out of range, ATTN_CPU_E_UNSUPPORTED (-3) for d outside
 *     [1, 256], ATTN_CPU_E_SCALE (-4) for a non-finite scale (the same values
 *     as attn.h's statuses).
 *   - NaN or Inf inputs propagate; they are not detected.
 */
#ifndef ATTN_CPU_H
#define ATTN_CPU_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  ATTN_CPU_OK = 0,
  ATTN_CPU_E_NULL = -1,
  ATTN_CPU_E_SHAPE = -2,
  ATTN_CPU_E_UNSUPPORTED = -3,
  ATTN_CPU_E_SCALE = -4
};

/* Forward: o [B,H,N,d] and lse [B,H,N] from q, k, v [B,H,N,d]. */
int attn_cpu_fwd(const float* q, const float* k, const float* v, float* o, float* lse, int64_t B, int64_t H,
                 int64_t N, int64_t d, int causal, float scale, int threads);

/* Backward: dq, dk, dv [B,H,N,d] from q, k, v, the forward's o and lse, and
 * the output gradient dout.  causal and scale must equal the forward's. */
int attn_cpu_bwd(const float* q, const float* k, const float* v, const float* o, const float* dout,
                 const float* lse, float* dq, float* dk, float* dv, int64_t B, int64_t H, int64_t N, int64_t d,
                 int causal, float scale, int threads);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_CPU_H */
