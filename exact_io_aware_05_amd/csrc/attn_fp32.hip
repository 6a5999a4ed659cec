// Float32 attention, forward and backward, on the vector ALUs (gfx950).
//
// The float32 path serves inputs that must be matched to ~1e-5: everything is
// fp32 end to end (products, sums, exponentials).  It keeps the method's
// structure -- K/V (or Q/dO) tiles staged in LDS, an online softmax with a
// running max and sum per query ("Tiling: Block-by-Block Softmax", Paper
// Notes page), and a backward pass that recomputes P from the saved LSE
// ("The backward pass: recompute instead of store", aicassindra page) -- but
// not the matrix cores: each query (or key) row is owned by 4 adjacent lanes
// that hold the features f with f % 4 == lane % 4, and dot products are
// finished with two butterfly shuffles.
//
// Backward: dK and dV are accumulated by a key-stationary kernel and dQ by a
// query-stationary kernel, so no floating-point atomics are needed and the
// result is deterministic.
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

namespace {

__device__ __forceinline__ float quad_sum(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  return x;
}

// Forward: a workgroup owns 16 queries of one head; each of its four waves
// holds all 16 (four lanes per query) and takes every fourth key of each
// 64-key tile, so a wave's running (m, l, O) covers a quarter of the keys.
// The four partial states are merged at the end with the two-block rule of
// "Tiling: Block-by-Block Softmax" (Paper Notes): m = max m_w, l = sum_w
// e^(m_w - m) l_w, O = sum_w e^(m_w - m) O_w / l.  Lane c of a query holds the
// features 4 (c + 4 i) .. 4 (c + 4 i) + 3 (i = 0 .. D / 16 - 1), so a key row
// is read from LDS with D / 16 16-byte reads whose four distinct addresses per
// wave fall in distinct banks.  The next tile's K and V rows are loaded into
// registers while the current tile is used.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                      const float* __restrict__ V, float* __restrict__ O,
                                                      float* __restrict__ LSE, int n, int nqb, float sl2e,
                                                      const int* __restrict__ klen, int heads, int wl) {
  constexpr int BQ = 16, BK = 64, NC = D / 16;  // NC: 4-float chunks per lane
  constexpr int PRE = BK * D / 4 / 256;         // 4-float chunks of a tile per thread (K, and V alike)
  __shared__ __attribute__((aligned(16))) float ks[BK * D];
  __shared__ __attribute__((aligned(16))) float vs[BK * D];
  const int tid = threadIdx.x, lane = tid & 63, c = lane & 3, ql = lane >> 2;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bh = blockIdx.x / nqb, qb = blockIdx.x % nqb;
  const int qrow = qb * BQ + ql;
  const size_t head = (size_t)bh * n * D;
  const float* Kh = K + head;
  const float* Vh = V + head;

  f32x4 qv[NC], acc[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    qv[i] = qrow < n ? *reinterpret_cast<const f32x4*>(Q + head + (size_t)qrow * D + 4 * (c + 4 * i)) : z;
    acc[i] = z;
  }
  float m = -INFINITY, l = 0.f;
  const int nkv = padded_keys(klen, heads, bh, n);  // keys from nkv on are masked
  const int kend = CAUSAL ? min(nkv, qb * BQ + BQ) : nkv;
  const int ntiles = (kend + BK - 1) / BK;
  // Sliding window (wl >= 0, with the causal mask): query i sees keys
  // i - wl .. i; tiles before the window of the first query are skipped.
  const bool win = wl >= 0;
  const int t0 = win ? max(0, qb * BQ - wl) / BK : 0;

  // Thread tid stages chunks tid + 256 r of a tile (row = chunk / (D / 4)).
  f32x4 kn[PRE], vn[PRE];
  auto load = [&](int j0) {
#pragma unroll
    for (int r = 0; r < PRE; ++r) {
      const int idx = tid + 256 * r, row = idx / (D / 4), c4 = idx % (D / 4), key = j0 + row;
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      kn[r] = key < n ? *reinterpret_cast<const f32x4*>(Kh + (size_t)key * D + 4 * c4) : z;
      vn[r] = key < n ? *reinterpret_cast<const f32x4*>(Vh + (size_t)key * D + 4 * c4) : z;
    }
  };
  if (ntiles > t0) load(t0 * BK);
  for (int t = t0; t < ntiles; ++t) {
    const int j0 = t * BK;
    __syncthreads();  // every wave is done with the previous tile
#pragma unroll
    for (int r = 0; r < PRE; ++r) {
      *reinterpret_cast<f32x4*>(&ks[4 * (tid + 256 * r)]) = kn[r];
      *reinterpret_cast<f32x4*>(&vs[4 * (tid + 256 * r)]) = vn[r];
    }
    __syncthreads();
    if (t + 1 < ntiles) load(j0 + BK);
    // This wave's keys of the tile: rows w, w + 4, ..., w + 60.
    float s[BK / 4];
    float mx = -INFINITY;
#pragma unroll
    for (int jj = 0; jj < BK / 4; ++jj) {
      const int row = 4 * jj + w;
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        const f32x4 kk = *reinterpret_cast<const f32x4*>(&ks[row * D + 4 * (c + 4 * i)]);
#pragma unroll
        for (int e = 0; e < 4; ++e) part = fmaf(qv[i][e], kk[e], part);
      }
      const float x = quad_sum(part) * sl2e;
      const int key = j0 + row;
      const bool dead = key >= nkv || (CAUSAL && key > qrow) || (win && key < qrow - wl);
      s[jj] = dead ? -INFINITY : x;
      mx = fmaxf(mx, s[jj]);
    }
    const float m_new = fmaxf(m, mx);
    // A wave may have seen no visible key of this query yet (causal): its
    // state stays (-inf, 0, 0).
    if (m_new != -INFINITY) {
      const float alpha = fast_exp2(m - m_new);  // 0 while m = -inf
      l *= alpha;
#pragma unroll
      for (int i = 0; i < NC; ++i) acc[i] *= alpha;
#pragma unroll
      for (int jj = 0; jj < BK / 4; ++jj) {
        const int row = 4 * jj + w;
        const float p = fast_exp2(s[jj] - m_new);
        l += p;
#pragma unroll
        for (int i = 0; i < NC; ++i) {
          const f32x4 vv = *reinterpret_cast<const f32x4*>(&vs[row * D + 4 * (c + 4 * i)]);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][e] = fmaf(p, vv[e], acc[i][e]);
        }
      }
      m = m_new;
    }
  }

  // Merge the four waves' states through LDS: wave w's unnormalised output
  // rows in the K tile area, (m, l) per query in the V tile area.
  __syncthreads();
  float* const ro = ks;  // [w][ql][D]
  float* const rm = vs;  // [w][ql][2]
  static_assert(4 * BQ * D <= BK * D && 4 * BQ * 2 <= BK * D, "merge areas fit the tiles");
#pragma unroll
  for (int i = 0; i < NC; ++i) *reinterpret_cast<f32x4*>(&ro[(w * BQ + ql) * D + 4 * (c + 4 * i)]) = acc[i];
  if (c == 0) {
    rm[(w * BQ + ql) * 2] = m;
    rm[(w * BQ + ql) * 2 + 1] = l;
  }
  __syncthreads();
  if (w != 0 || qrow >= n) return;
  float mw[4], lw[4];
  float mt = -INFINITY;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    mw[u] = rm[(u * BQ + ql) * 2];
    lw[u] = rm[(u * BQ + ql) * 2 + 1];
    mt = fmaxf(mt, mw[u]);
  }
  // Without key padding key 0 is visible to every query, so mt is finite; a
  // row that sees no key (every key padded) gets O = 0 and LSE = -inf.
  float wt[4], lt = 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    wt[u] = mw[u] == -INFINITY ? 0.f : fast_exp2(mw[u] - mt);
    lt += wt[u] * lw[u];
  }
  const bool empty = lt == 0.f;
  const float inv = empty ? 0.f : 1.0f / lt;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(&ro[(u * BQ + ql) * D + 4 * (c + 4 * i)]);
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = fmaf(wt[u], a[e], o[e]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] *= inv;
    *reinterpret_cast<f32x4*>(O + head + (size_t)qrow * D + 4 * (c + 4 * i)) = o;
  }
  if (c == 0) LSE[(size_t)bh * n + qrow] = empty ? -INFINITY : (mt + fast_log2(lt)) * kLn2;
}

// dK, dV for a block of 64 keys; streams query tiles of 32 rows.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_kv_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                         const float* __restrict__ V,
                                                         const float* __restrict__ dO,
                                                         const float* __restrict__ LSE,
                                                         const float* __restrict__ Dsum, float* __restrict__ dK,
                                                         float* __restrict__ dV, int n, int nkb, float scale,
                                                         float sl2e, const int* __restrict__ klen, int heads,
                                                         int wl) {
  constexpr int BKEY = 64, BQ = 32, DQ = D / 4;
  __shared__ __attribute__((aligned(16))) float qs[BQ * D];
  __shared__ __attribute__((aligned(16))) float dos[BQ * D];
  __shared__ float lse2[BQ];
  __shared__ float dsm[BQ];
  const int tid = threadIdx.x, c = tid & 3, kl = tid >> 2;
  const int bh = blockIdx.x / nkb, kb = blockIdx.x % nkb;
  const int key = kb * BKEY + kl;
  const size_t head = (size_t)bh * n * D;
  const float* Qh = Q + head;
  const float* dOh = dO + head;

  float kv[DQ], vv[DQ], dk[DQ], dv[DQ];
#pragma unroll
  for (int i = 0; i < DQ; ++i) {
    kv[i] = key < n ? K[head + (size_t)key * D + 4 * i + c] : 0.f;
    vv[i] = key < n ? V[head + (size_t)key * D + 4 * i + c] : 0.f;
    dk[i] = 0.f;
    dv[i] = 0.f;
  }
  const int nkv = padded_keys(klen, heads, bh, n);  // keys from nkv on: P = 0, so dK = dV = 0
  const int istart = CAUSAL ? (kb * BKEY / BQ) * BQ : 0;
  // Sliding window (wl >= 0): the block's keys are seen by queries up to
  // its last key + wl.
  const bool win = wl >= 0;
  const int iend = win ? min(n, kb * BKEY + BKEY + wl) : n;
  for (int i0 = istart; i0 < iend; i0 += BQ) {
    __syncthreads();
    for (int idx = tid; idx < BQ * D / 4; idx += 256) {
      const int row = idx / (D / 4), c4 = idx % (D / 4), qi = i0 + row;
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f32x4*>(&qs[row * D + 4 * c4]) =
          qi < n ? *reinterpret_cast<const f32x4*>(Qh + (size_t)qi * D + 4 * c4) : z;
      *reinterpret_cast<f32x4*>(&dos[row * D + 4 * c4]) =
          qi < n ? *reinterpret_cast<const f32x4*>(dOh + (size_t)qi * D + 4 * c4) : z;
    }
    if (tid < BQ) {
      const int qi = i0 + tid;
      lse2[tid] = qi < n ? LSE[(size_t)bh * n + qi] * kLog2e : 0.f;
      dsm[tid] = qi < n ? Dsum[(size_t)bh * n + qi] : 0.f;
    }
    __syncthreads();
    for (int ii = 0; ii < BQ; ++ii) {
      const int qi = i0 + ii;
      float sp = 0.f, dpp = 0.f;
#pragma unroll
      for (int i = 0; i < DQ; ++i) {
        sp = fmaf(qs[ii * D + 4 * i + c], kv[i], sp);
        dpp = fmaf(dos[ii * D + 4 * i + c], vv[i], dpp);
      }
      const float s = quad_sum(sp);
      const float dp = quad_sum(dpp);
      const bool live = key < nkv && qi < n && (!CAUSAL || key <= qi) && (!win || qi - key <= wl);
      const float p = live ? fast_exp2(s * sl2e - lse2[ii]) : 0.f;
      const float ds = p * (dp - dsm[ii]);
#pragma unroll
      for (int i = 0; i < DQ; ++i) {
        dv[i] = fmaf(p, dos[ii * D + 4 * i + c], dv[i]);
        dk[i] = fmaf(ds, qs[ii * D + 4 * i + c], dk[i]);
      }
    }
  }
  if (key < n) {
#pragma unroll
    for (int i = 0; i < DQ; ++i) {
      dK[head + (size_t)key * D + 4 * i + c] = dk[i] * scale;
      dV[head + (size_t)key * D + 4 * i + c] = dv[i];
    }
  }
}

// dQ for a block of 64 queries; streams key tiles of 32 rows.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_q_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                        const float* __restrict__ V,
                                                        const float* __restrict__ dO,
                                                        const float* __restrict__ LSE,
                                                        const float* __restrict__ Dsum, float* __restrict__ dQ,
                                                        int n, int nqb, float scale, float sl2e,
                                                        const int* __restrict__ klen, int heads, int wl) {
  constexpr int BQ = 64, BKEY = 32, DQ = D / 4;
  __shared__ __attribute__((aligned(16))) float ks[BKEY * D];
  __shared__ __attribute__((aligned(16))) float vs[BKEY * D];
  const int tid = threadIdx.x, c = tid & 3, ql = tid >> 2;
  const int bh = blockIdx.x / nqb, qb = blockIdx.x % nqb;
  const int qrow = qb * BQ + ql;
  const size_t head = (size_t)bh * n * D;
  const float* Kh = K + head;
  const float* Vh = V + head;

  float qv[DQ], dov[DQ], dq[DQ];
#pragma unroll
  for (int i = 0; i < DQ; ++i) {
    qv[i] = qrow < n ? Q[head + (size_t)qrow * D + 4 * i + c] : 0.f;
    dov[i] = qrow < n ? dO[head + (size_t)qrow * D + 4 * i + c] : 0.f;
    dq[i] = 0.f;
  }
  const float l2 = qrow < n ? LSE[(size_t)bh * n + qrow] * kLog2e : 0.f;
  const float dsq = qrow < n ? Dsum[(size_t)bh * n + qrow] : 0.f;
  const int nkv = padded_keys(klen, heads, bh, n);  // keys from nkv on are masked
  const int kend = CAUSAL ? min(nkv, qb * BQ + BQ) : nkv;
  // Sliding window (wl >= 0): keys from the window of the block's first query.
  const bool win = wl >= 0;
  const int jstart = win ? max(0, qb * BQ - wl) / BKEY * BKEY : 0;
  for (int j0 = jstart; j0 < kend; j0 += BKEY) {
    __syncthreads();
    for (int idx = tid; idx < BKEY * D / 4; idx += 256) {
      const int row = idx / (D / 4), c4 = idx % (D / 4), kj = j0 + row;
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f32x4*>(&ks[row * D + 4 * c4]) =
          kj < n ? *reinterpret_cast<const f32x4*>(Kh + (size_t)kj * D + 4 * c4) : z;
      *reinterpret_cast<f32x4*>(&vs[row * D + 4 * c4]) =
          kj < n ? *reinterpret_cast<const f32x4*>(Vh + (size_t)kj * D + 4 * c4) : z;
    }
    __syncthreads();
    for (int jj = 0; jj < BKEY; ++jj) {
      const int kj = j0 + jj;
      float sp = 0.f, dpp = 0.f;
#pragma unroll
      for (int i = 0; i < DQ; ++i) {
        sp = fmaf(qv[i], ks[jj * D + 4 * i + c], sp);
        dpp = fmaf(dov[i], vs[jj * D + 4 * i + c], dpp);
      }
      const float s = quad_sum(sp);
      const float dp = quad_sum(dpp);
      const bool live = kj < nkv && qrow < n && (!CAUSAL || kj <= qrow) && (!win || qrow - kj <= wl);
      const float p = live ? fast_exp2(s * sl2e - l2) : 0.f;
      const float ds = p * (dp - dsq);
#pragma unroll
      for (int i = 0; i < DQ; ++i) dq[i] = fmaf(ds, ks[jj * D + 4 * i + c], dq[i]);
    }
  }
  if (qrow < n) {
#pragma unroll
    for (int i = 0; i < DQ; ++i) dQ[head + (size_t)qrow * D + 4 * i + c] = dq[i] * scale;
  }
}

template <int D, bool CAUSAL>
hipError_t fwd_f32_t(const FwdArgs& a) {
  const int nqb = (int)((a.n + 15) / 16);
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)(a.bh * nqb)), dim3(256), 0, a.stream,
                     (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse, (int)a.n, nqb,
                     a.scale * kLog2e, a.klen, a.heads, a.window - 1);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t dkdv_f32_t(const BwdArgs& a) {
  const int nkb = (int)((a.n + 63) / 64);
  hipLaunchKernelGGL((bwd_kv_f32_kernel<D, CAUSAL>), dim3((unsigned)(a.bh * nkb)), dim3(256), 0, a.stream,
                     (const float*)a.q, (const float*)a.k, (const float*)a.v, (const float*)a.dout, a.lse,
                     (const float*)a.dsum, (float*)a.dk, (float*)a.dv, (int)a.n, nkb, a.scale,
                     a.scale * kLog2e, a.klen, a.heads, a.window - 1);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t dq_f32_t(const BwdArgs& a) {
  const int nqb = (int)((a.n + 63) / 64);
  hipLaunchKernelGGL((bwd_q_f32_kernel<D, CAUSAL>), dim3((unsigned)(a.bh * nqb)), dim3(256), 0, a.stream,
                     (const float*)a.q, (const float*)a.k, (const float*)a.v, (const float*)a.dout, a.lse,
                     (const float*)a.dsum, (float*)a.dq, (int)a.n, nqb, a.scale, a.scale * kLog2e, a.klen,
                     a.heads, a.window - 1);
  return hipGetLastError();
}

}  // namespace

hipError_t fwd_f32(const FwdArgs& a) {
  if (a.d == 64) return a.causal ? fwd_f32_t<64, true>(a) : fwd_f32_t<64, false>(a);
  return a.causal ? fwd_f32_t<128, true>(a) : fwd_f32_t<128, false>(a);
}

hipError_t bwd_f32_dkdv(const BwdArgs& a) {
  if (a.d == 64) return a.causal ? dkdv_f32_t<64, true>(a) : dkdv_f32_t<64, false>(a);
  return a.causal ? dkdv_f32_t<128, true>(a) : dkdv_f32_t<128, false>(a);
}

hipError_t bwd_f32_dq(const BwdArgs& a) {
  if (a.d == 64) return a.causal ? dq_f32_t<64, true>(a) : dq_f32_t<64, false>(a);
  return a.causal ? dq_f32_t<128, true>(a) : dq_f32_t<128, false>(a);
}

}  // namespace attn
