// Cache-blocked multi-core CPU form of fused exact attention, float32.
//
// The blocking discipline of the method on a CPU (aicassindra,
// "Practical implications and the CPU / small-model view"): 64-row query
// blocks and 64-key tiles, the running max / running sum update of "Tiling:
// Block-by-Block Softmax" (Paper Notes) per tile, and the backward pass by
// recomputation ("The backward pass: recompute instead of store",
// aicassindra).  A work item (one batch * head and one block) keeps its
// tiles -- Q or K block, a transposed K or V tile, the 64 x 64 score tile and
// the accumulators, 16-32 KiB each at d = 128 -- in one core's L1/L2 cache;
// OpenMP spreads the work items over the cores.
//
// Every product has the form C[i][0:w] += sum_k a(i, k) B[k][0:w] with B and
// C rows contiguous (a tile transposed once where needed).  Four rows of C
// share each load of a B row segment: 4 x 16 columns in eight 8-float
// accumulators (AVX2), or 4 x 64 columns in sixteen 16-float accumulators
// (AVX-512, chosen at run time where the host has it; ATTN_CPU_ISA=avx2 forces
// the 8-float form).  Each element still adds its k terms in order, one fused
// multiply-add each, so both forms give the same results.
#include "attn_cpu.h"

#include <immintrin.h>
#include <omp.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <vector>

namespace {

constexpr int BQ = 64;  // query rows per block
constexpr int BK = 64;  // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef float v8f __attribute__((vector_size(32)));
typedef float v16f __attribute__((vector_size(64)));

// 2^x in float32 for the softmax: x = n + f with n = round(x), |f| <= 1/2;
// 2^f = exp(f ln 2) by its Taylor series to degree 7 (coefficients
// (ln 2)^k / k!; truncation error below 6e-9 relative), 2^n built in the
// exponent field.  x <= -127 (including -inf) gives 0 (results below 2^-126
// are flushed); x is at most 0 here (arguments are relative to a row max).
inline float exp2_sm(float x) {
  x = x < -127.f ? -127.f : x;
  x = x > 127.f ? 127.f : x;
  const float n = std::floor(x + 0.5f);
  const float f = x - n;
  float p = 1.5252733804059838e-05f;
  p = p * f + 1.5403530393381606e-04f;
  p = p * f + 1.3333558146428441e-03f;
  p = p * f + 9.6181291076284770e-03f;
  p = p * f + 5.5504108664821576e-02f;
  p = p * f + 2.4022650695910071e-01f;
  p = p * f + 6.9314718055994531e-01f;
  p = p * f + 1.0f;
  const int e = (int)n + 127;  // 0 for x = -127: the product below is 0
  float s;
  const uint32_t bits = (uint32_t)e << 23;
  std::memcpy(&s, &bits, 4);
  return p * s;
}

// exp2_sm on eight values at once: the same operations per element (clamps,
// rounding, polynomial, exponent field), so each lane equals exp2_sm of it.
inline v8f exp2_v8(v8f x) {
  const v8f lo = v8f{} - 127.f, hi = v8f{} + 127.f;
  x = x < lo ? lo : x;
  x = x > hi ? hi : x;
  const v8f n = (v8f)_mm256_floor_ps((__m256)(x + 0.5f));
  const v8f f = x - n;
  v8f p = v8f{} + 1.5252733804059838e-05f;
  p = p * f + 1.5403530393381606e-04f;
  p = p * f + 1.3333558146428441e-03f;
  p = p * f + 9.6181291076284770e-03f;
  p = p * f + 5.5504108664821576e-02f;
  p = p * f + 2.4022650695910071e-01f;
  p = p * f + 6.9314718055994531e-01f;
  p = p * f + 1.0f;
  const __m256i e = _mm256_add_epi32(_mm256_cvttps_epi32((__m256)n), _mm256_set1_epi32(127));
  const v8f sc = (v8f)_mm256_castsi256_ps(_mm256_slli_epi32(e, 23));
  return p * sc;
}

// Rows i0 .. i0 + RB - 1 of C, columns c0 .. c0 + NV * lanes(V) - 1:
// C[i][c] += sum_{k < kd} a(i, k) * B[k][c], a(i, k) = A[i * ai + k * ak].
// The accumulators stay in registers; every B row segment is loaded once for
// the RB rows.
template <typename V, int NV, int RB>
__attribute__((always_inline)) inline void axpy_block(int kd, const float* A, int ai, int ak, const float* B, int ldb,
                                                      float* C, int ldc, int i0, int c0) {
  constexpr int VW = (int)(sizeof(V) / sizeof(float));
  V acc[RB][NV];
#pragma GCC unroll 8
  for (int r = 0; r < RB; ++r)
#pragma GCC unroll 8
    for (int t = 0; t < NV; ++t) std::memcpy(&acc[r][t], C + (size_t)(i0 + r) * ldc + c0 + VW * t, sizeof(V));
  for (int k = 0; k < kd; ++k) {
    const float* b = B + (size_t)k * ldb + c0;
    V bv[NV];
#pragma GCC unroll 8
    for (int t = 0; t < NV; ++t) std::memcpy(&bv[t], b + VW * t, sizeof(V));
#pragma GCC unroll 8
    for (int r = 0; r < RB; ++r) {
      const V sv = V{} + A[(size_t)(i0 + r) * ai + (size_t)k * ak];
#pragma GCC unroll 8
      for (int t = 0; t < NV; ++t) acc[r][t] += sv * bv[t];
    }
  }
#pragma GCC unroll 8
  for (int r = 0; r < RB; ++r)
#pragma GCC unroll 8
    for (int t = 0; t < NV; ++t) std::memcpy(C + (size_t)(i0 + r) * ldc + c0 + VW * t, &acc[r][t], sizeof(V));
}

// C[i][0:w] += sum_{k < kd} a(i, k) * B[k][0:w] for i < m (w a multiple of
// 64; B, C row strides ldb, ldc): blocks of four rows, then single rows.
template <typename V, int NV>
__attribute__((always_inline)) inline void axpy_rows_v(int m, int kd, const float* A, int ai, int ak, const float* B,
                                                       int ldb, float* C, int ldc, int w) {
  constexpr int CW = NV * (int)(sizeof(V) / sizeof(float));
  for (int c0 = 0; c0 < w; c0 += CW) {
    int i = 0;
    for (; i + 4 <= m; i += 4) axpy_block<V, NV, 4>(kd, A, ai, ak, B, ldb, C, ldc, i, c0);
    for (; i < m; ++i) axpy_block<V, NV, 1>(kd, A, ai, ak, B, ldb, C, ldc, i, c0);
  }
}

void axpy_rows_avx2(int m, int kd, const float* A, int ai, int ak, const float* B, int ldb, float* C, int ldc,
                    int w) {
  axpy_rows_v<v8f, 2>(m, kd, A, ai, ak, B, ldb, C, ldc, w);
}

__attribute__((target("avx512f"))) void axpy_rows_avx512(int m, int kd, const float* A, int ai, int ak,
                                                          const float* B, int ldb, float* C, int ldc, int w) {
  axpy_rows_v<v16f, 4>(m, kd, A, ai, ak, B, ldb, C, ldc, w);
}

// The 16-float form where the host has AVX-512 (and ATTN_CPU_ISA does not
// ask for avx2).
bool use_avx512() {
  static const bool wide = [] {
    const char* isa = std::getenv("ATTN_CPU_ISA");
    if (isa != nullptr && std::strcmp(isa, "avx2") == 0) return false;
    __builtin_cpu_init();
    return __builtin_cpu_supports("avx512f") != 0;
  }();
  return wide;
}

inline void axpy_rows(int m, int kd, const float* A, int ai, int ak, const float* B, int ldb, float* C, int ldc,
                      int w) {
  if (use_avx512())
    axpy_rows_avx512(m, kd, A, ai, ak, B, ldb, C, ldc, w);
  else
    axpy_rows_avx2(m, kd, A, ai, ak, B, ldb, C, ldc, w);
}

// Rows [r0, r0 + rows) of a [n, d] matrix, transposed into T[dd][BK] (keys
// past the end and past `rows` are zero; dd = d padded to a multiple of 64
// only matters for the leading dimension, which is BK).
inline void load_t(const float* X, int n, int d, int r0, float* T) {
  for (int j = 0; j < BK; ++j) {
    const int r = r0 + j;
    if (r < n) {
      const float* x = X + (size_t)r * d;
      for (int k = 0; k < d; ++k) T[(size_t)k * BK + j] = x[k];
    } else {
      for (int k = 0; k < d; ++k) T[(size_t)k * BK + j] = 0.f;
    }
  }
}

// Rows [r0, r0 + BK) of a [n, d] matrix into R[BK][dp] (dp = d rounded up to
// 64; padding columns and rows past n are zero).
inline void load_rows(const float* X, int n, int d, int dp, int r0, float* R) {
  for (int j = 0; j < BK; ++j) {
    const int r = r0 + j;
    float* dst = R + (size_t)j * dp;
    if (r < n) {
      std::memcpy(dst, X + (size_t)r * d, sizeof(float) * d);
      std::fill(dst + d, dst + dp, 0.f);
    } else {
      std::fill(dst, dst + dp, 0.f);
    }
  }
}

int check(const void* const* ptrs, int np, int64_t B, int64_t H, int64_t N, int64_t d, float scale) {
  for (int i = 0; i < np; ++i)
    if (!ptrs[i]) return ATTN_CPU_E_NULL;
  if (B < 1 || H < 1 || N < 1 || B * H > (int64_t)1 << 31 || N > (int64_t)1 << 30 || N * d > (int64_t)1 << 31)
    return ATTN_CPU_E_SHAPE;
  if (d < 1 || d > 256) return ATTN_CPU_E_UNSUPPORTED;
  if (!std::isfinite(scale)) return ATTN_CPU_E_SCALE;
  return ATTN_CPU_OK;
}

int nthreads(int threads) { return threads > 0 ? threads : omp_get_max_threads(); }

}  // namespace

extern "C" int attn_cpu_fwd(const float* q, const float* k, const float* v, float* o, float* lse, int64_t B,
                            int64_t H, int64_t N, int64_t d, int causal, float scale, int threads) {
  const void* ptrs[] = {q, k, v, o, lse};
  if (int st = check(ptrs, 5, B, H, N, d, scale)) return st;
  const int n = (int)N, dd = (int)d, dp = (dd + 63) / 64 * 64;
  const int64_t bh = B * H;
  const int nqb = (n + BQ - 1) / BQ;
  const float c = scale * kLog2e;  // scores in log2 units
  const int64_t items = bh * nqb;

#pragma omp parallel num_threads(nthreads(threads))
  {
    std::vector<float> Qb((size_t)BQ * dp), Kt((size_t)dp * BK), Vb((size_t)BK * dp), S((size_t)BQ * BK),
        acc((size_t)BQ * dp);
    float m[BQ], l[BQ];
#pragma omp for schedule(dynamic, 1)
    for (int64_t it = 0; it < items; ++it) {
      // Causal: heavy (late) blocks first.
      const int64_t h = it / nqb;
      const int qb = causal ? nqb - 1 - (int)(it % nqb) : (int)(it % nqb);
      const int q0 = qb * BQ, rows = std::min(BQ, n - q0);
      const float* Qh = q + (size_t)h * n * dd;
      const float* Kh = k + (size_t)h * n * dd;
      const float* Vh = v + (size_t)h * n * dd;
      for (int i = 0; i < BQ; ++i) {
        float* dst = &Qb[(size_t)i * dp];
        if (i < rows) {
          std::memcpy(dst, Qh + (size_t)(q0 + i) * dd, sizeof(float) * dd);
          std::fill(dst + dd, dst + dp, 0.f);
        } else {
          std::fill(dst, dst + dp, 0.f);
        }
        m[i] = -INFINITY;
        l[i] = 0.f;
      }
      std::fill(acc.begin(), acc.end(), 0.f);
      const int kend = causal ? std::min(n, q0 + rows) : n;
      for (int j0 = 0; j0 < kend; j0 += BK) {
        load_t(Kh, n, dd, j0, Kt.data());
        load_rows(Vh, n, dd, dp, j0, Vb.data());
        std::fill(S.begin(), S.end(), 0.f);
        axpy_rows(rows, dd, Qb.data(), dp, 1, Kt.data(), BK, S.data(), BK, BK);
        for (int i = 0; i < rows; ++i) {
          float* s = &S[(size_t)i * BK];
          const int lim = causal ? std::min(kend, q0 + i + 1) : n;  // keys [j0, lim) are visible
          // Eight lanes at a time (BK = 64): scaled scores with the hidden
          // keys at -inf, their max, then the exponentials and their sum (as
          // eight partial sums).
          typedef int v8i __attribute__((vector_size(32)));
          const v8i lane = {0, 1, 2, 3, 4, 5, 6, 7};
          const v8f ninf = v8f{} - INFINITY;
          v8f mxv = v8f{} + m[i];
          for (int j = 0; j < BK; j += 8) {
            v8f x;
            std::memcpy(&x, s + j, 32);
            x = (lane + (j0 + j)) < lim ? x * c : ninf;
            std::memcpy(s + j, &x, 32);
            mxv = mxv > x ? mxv : x;
          }
          float mx = mxv[0];
          for (int t = 1; t < 8; ++t) mx = std::max(mx, mxv[t]);
          // Row i sees key j0 at least (square causal: j0 <= q0 <= i), so mx is finite.
          const float alpha = exp2_sm(m[i] - mx);
          v8f sv = v8f{};
          for (int j = 0; j < BK; j += 8) {
            v8f x;
            std::memcpy(&x, s + j, 32);
            x = exp2_v8(x - mx);
            std::memcpy(s + j, &x, 32);
            sv += x;
          }
          const float sum = ((sv[0] + sv[1]) + (sv[2] + sv[3])) + ((sv[4] + sv[5]) + (sv[6] + sv[7]));
          l[i] = l[i] * alpha + sum;
          m[i] = mx;
          float* a = &acc[(size_t)i * dp];
          for (int t = 0; t < dp; ++t) a[t] *= alpha;
        }
        axpy_rows(rows, BK, S.data(), BK, 1, Vb.data(), dp, acc.data(), dp, dp);
      }
      for (int i = 0; i < rows; ++i) {
        const float inv = 1.f / l[i];
        float* dst = o + ((size_t)h * n + q0 + i) * dd;
        const float* a = &acc[(size_t)i * dp];
        for (int t = 0; t < dd; ++t) dst[t] = a[t] * inv;
        lse[(size_t)h * n + q0 + i] = (m[i] + std::log2(l[i])) * kLn2;
      }
    }
  }
  return ATTN_CPU_OK;
}

extern "C" int attn_cpu_bwd(const float* q, const float* k, const float* v, const float* o, const float* dout,
                            const float* lse, float* dq, float* dk, float* dv, int64_t B, int64_t H, int64_t N,
                            int64_t d, int causal, float scale, int threads) {
  const void* ptrs[] = {q, k, v, o, dout, lse, dq, dk, dv};
  if (int st = check(ptrs, 9, B, H, N, d, scale)) return st;
  const int n = (int)N, dd = (int)d, dp = (dd + 63) / 64 * 64;
  const int64_t bh = B * H;
  const int nb = (n + BK - 1) / BK;  // blocks of 64 (BQ == BK)
  const float c = scale * kLog2e;
  const int nt = nthreads(threads);

  // D_i = sum_k dO_ik O_ik; LSE in log2 units.
  std::vector<float> Dv((size_t)bh * n), L2((size_t)bh * n);
#pragma omp parallel for num_threads(nt) schedule(static)
  for (int64_t r = 0; r < bh * n; ++r) {
    const float* a = o + (size_t)r * dd;
    const float* g = dout + (size_t)r * dd;
    float s = 0.f;
    for (int t = 0; t < dd; ++t) s += a[t] * g[t];
    Dv[r] = s;
    L2[r] = lse[r] * kLog2e;
  }

  // P and dS of one (query block at q0, key block at k0) pair into P, dS
  // ([BQ][BK]); Qb, Gb are the query block's Q and dO rows ([BQ][dp]), Kt, Vt
  // the key block's K and V transposed ([dp][BK]).
  auto tile_p_ds = [&](int64_t h, int q0, int k0, const float* Qb, const float* Gb, const float* Kt,
                       const float* Vt, float* P, float* dS, float* dP) {
    std::fill(P, P + BQ * BK, 0.f);
    std::fill(dP, dP + BQ * BK, 0.f);
    axpy_rows(BQ, dd, Qb, dp, 1, Kt, BK, P, BK, BK);
    axpy_rows(BQ, dd, Gb, dp, 1, Vt, BK, dP, BK, BK);
    for (int i = 0; i < BQ; ++i) {
      const int r = q0 + i;
      const bool live = r < n;
      const float l2 = live ? L2[(size_t)h * n + r] : 0.f;
      const float dr = live ? Dv[(size_t)h * n + r] : 0.f;
      const int lim = !live ? 0 : (causal ? std::min(n, r + 1) : n);
      typedef int v8i __attribute__((vector_size(32)));
      const v8i lane = {0, 1, 2, 3, 4, 5, 6, 7};
      for (int j = 0; j < BK; j += 8) {
        v8f pv, dpv;
        std::memcpy(&pv, P + i * BK + j, 32);
        std::memcpy(&dpv, dP + i * BK + j, 32);
        const v8f e = exp2_v8(pv * c - l2);
        const v8f pm = (lane + (k0 + j)) < lim ? e : v8f{};
        const v8f ds = pm * (dpv - dr);
        std::memcpy(P + i * BK + j, &pm, 32);
        std::memcpy(dS + i * BK + j, &ds, 32);
      }
    }
  };
  auto load_block = [&](const float* X, int r0, float* R) { load_rows(X, n, dd, dp, r0, R); };

  // Pass 1: dK, dV, key-block stationary.
#pragma omp parallel num_threads(nt)
  {
    std::vector<float> Kt((size_t)dp * BK), Vt((size_t)dp * BK), Qb((size_t)BQ * dp), Gb((size_t)BQ * dp),
        P((size_t)BQ * BK), dS((size_t)BQ * BK), dP((size_t)BQ * BK), dKa((size_t)BK * dp), dVa((size_t)BK * dp);
#pragma omp for schedule(dynamic, 1)
    for (int64_t it = 0; it < bh * nb; ++it) {
      const int64_t h = it / nb;
      const int kb = (int)(it % nb), k0 = kb * BK;
      const float* Qh = q + (size_t)h * n * dd;
      const float* Gh = dout + (size_t)h * n * dd;
      load_t(k + (size_t)h * n * dd, n, dd, k0, Kt.data());
      load_t(v + (size_t)h * n * dd, n, dd, k0, Vt.data());
      std::fill(dKa.begin(), dKa.end(), 0.f);
      std::fill(dVa.begin(), dVa.end(), 0.f);
      for (int qb = causal ? kb : 0; qb < nb; ++qb) {
        const int q0 = qb * BQ;
        load_block(Qh, q0, Qb.data());
        load_block(Gh, q0, Gb.data());
        tile_p_ds(h, q0, k0, Qb.data(), Gb.data(), Kt.data(), Vt.data(), P.data(), dS.data(), dP.data());
        // dV[j] += sum_i P[i][j] dO[i];  dK[j] += sum_i dS[i][j] Q[i]
        axpy_rows(BK, BQ, P.data(), 1, BK, Gb.data(), dp, dVa.data(), dp, dp);
        axpy_rows(BK, BQ, dS.data(), 1, BK, Qb.data(), dp, dKa.data(), dp, dp);
      }
      for (int j = 0; j < BK && k0 + j < n; ++j) {
        float* kd = dk + ((size_t)h * n + k0 + j) * dd;
        float* vd = dv + ((size_t)h * n + k0 + j) * dd;
        for (int t = 0; t < dd; ++t) {
          kd[t] = dKa[(size_t)j * dp + t] * scale;
          vd[t] = dVa[(size_t)j * dp + t];
        }
      }
    }
  }

  // Pass 2: dQ, query-block stationary.
#pragma omp parallel num_threads(nt)
  {
    std::vector<float> Kt((size_t)dp * BK), Vt((size_t)dp * BK), Kb((size_t)BK * dp), Qb((size_t)BQ * dp),
        Gb((size_t)BQ * dp), P((size_t)BQ * BK), dS((size_t)BQ * BK), dP((size_t)BQ * BK), dQa((size_t)BQ * dp);
#pragma omp for schedule(dynamic, 1)
    for (int64_t it = 0; it < bh * nb; ++it) {
      const int64_t h = it / nb;
      const int qb = causal ? nb - 1 - (int)(it % nb) : (int)(it % nb), q0 = qb * BQ;
      const float* Kh = k + (size_t)h * n * dd;
      const float* Vh = v + (size_t)h * n * dd;
      load_block(q + (size_t)h * n * dd, q0, Qb.data());
      load_block(dout + (size_t)h * n * dd, q0, Gb.data());
      std::fill(dQa.begin(), dQa.end(), 0.f);
      for (int kb = 0; kb <= (causal ? qb : nb - 1); ++kb) {
        const int k0 = kb * BK;
        load_t(Kh, n, dd, k0, Kt.data());
        load_t(Vh, n, dd, k0, Vt.data());
        load_block(Kh, k0, Kb.data());
        tile_p_ds(h, q0, k0, Qb.data(), Gb.data(), Kt.data(), Vt.data(), P.data(), dS.data(), dP.data());
        axpy_rows(BQ, BK, dS.data(), BK, 1, Kb.data(), dp, dQa.data(), dp, dp);  // dQ[i] += sum_j dS[i][j] K[j]
      }
      for (int i = 0; i < BQ && q0 + i < n; ++i) {
        float* qd = dq + ((size_t)h * n + q0 + i) * dd;
        for (int t = 0; t < dd; ++t) qd[t] = dQa[(size_t)i * dp + t] * scale;
      }
    }
  }
  return ATTN_CPU_OK;
}
