// Fused exact attention backward, bf16 in / bf16 out, fp32 accumulation, gfx950.
//
// The backward pass keeps only O and the per-row log-sum-exp from the forward
// pass and recomputes each score tile and its probabilities from Q, K and LSE
// ("Background" and "Key Ideas" on the Paper Notes page; "The backward pass:
// recompute instead of store" on the aicassindra page).  The gradient
// formulas, which the pages leave to a companion article, are the textbook
// chain rule:
//   P = exp(scale*Q K^T - LSE), dV = P^T dO, dP = dO V^T,
//   dS = P * (dP - D) with D_i = dO_i . O_i, dQ = scale dS K, dK = scale dS^T Q.
//
// Two kernels, neither uses atomics (deterministic results):
//  * bwd_kv: a workgroup owns 128 keys and keeps K, V and the dK, dV
//    accumulators in registers while query tiles of 64 rows stream through
//    LDS; two waves share each 32-key group (one for S, P and dV, one for
//    dP, dS and dK).  S and dP use the C[q][key] layout (lane = key,
//    registers run over queries), so P and dS feed dV^T += dO^T P and
//    dK^T += Q^T dS straight from registers as the B operand, each as a
//    hi + lo pair of bf16 values.  dO^T and Q^T are read from the row-major
//    tiles with transposing LDS reads.
//  * bwd_q: a workgroup owns a block of queries (32 per wave) with Q, dO,
//    LSE and D in registers and streams key tiles of 64 rows: S^T = K Q^T and
//    dP^T = V dO^T (lane = query), dS^T, then dQ^T += K^T dS^T, with K^T
//    read transposed from the row-major K tile.
// Tiles come from buffer->LDS DMA into two buffers (the next tile streams in
// while the current one is used; rows past the end of the head arrive as
// zeros).
#include "attn_device.h"
#include "attn_launch.h"
#include "attn_tile.h"

namespace attn {

namespace {

// ---------------------------------------------------------------------------
// dK, dV: key-stationary, with paired waves
//
// A workgroup of 8 waves owns 128 keys.  Waves w and w + 4 (which the
// hardware places on the same SIMD) share keys 32w .. 32w + 31 and split the
// work of each 64-query tile without duplicating any of it:
//  * the S wave computes S = Q K^T and P = exp(S - LSE), publishes P through
//    LDS, and accumulates dV^T += dO^T P;
//  * the dP wave computes dP = dO V^T, reads P, forms dS = P * (dP - D) and
//    accumulates dK^T += Q^T dS.
// Each wave keeps only its half of the state (K or V fragments, dV or dK
// accumulators), so two waves fit per SIMD and one's matrix work overlaps
// the other's vector work.
// ---------------------------------------------------------------------------
// Magnitude from which P and dS enter the dV and dK products as hi + lo bf16
// pairs (see bwd_kv_kernel).
constexpr float kSplitThreshold = 1.0f / 16.0f;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(512, 2) void bwd_kv_kernel(const uint16_t* __restrict__ Q,
                                                        const uint16_t* __restrict__ K,
                                                        const uint16_t* __restrict__ V,
                                                        const uint16_t* __restrict__ dO,
                                                        const float* __restrict__ LSE,
                                                        const float* __restrict__ Dsum,
                                                        uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
                                                        int n, int nkb, int total, float scale, float sl2e) {
  constexpr int NW = 8, BKV = 128, BQ = 64;

  __shared__ __attribute__((aligned(1024))) uint16_t q0s[BQ * D];
  __shared__ __attribute__((aligned(1024))) uint16_t g0s[BQ * D];
  __shared__ __attribute__((aligned(1024))) uint16_t q1s[BQ * D];
  __shared__ __attribute__((aligned(1024))) uint16_t g1s[BQ * D];
  // P of the current tile, per key group and half tile, lane-major:
  // [group][t][r / 4][lane][r % 4].
  __shared__ __attribute__((aligned(1024))) float pxs[4 * 2 * 4 * 64 * 4];
  __shared__ __attribute__((aligned(16))) float lse0s[BQ], dsm0s[BQ], lse1s[BQ], dsm1s[BQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int hh = lane >> 5, l32 = lane & 31;
  const TileReader<D> TR(lane);
  const int grp = w & 3;        // key group: keys 32*grp .. +31 of the block
  const bool s_role = w < 4;    // S wave (dV) or dP wave (dK)

  // Causal: low key blocks see the most queries; they come first.
  const int lid = xcd_remap(blockIdx.x, total);
  const int bh = lid / nkb, kb = lid % nkb;
  const int k0 = kb * BKV;
  const int kw0 = k0 + 32 * grp;
  const int key = kw0 + l32;

  const size_t head = (size_t)bh * (size_t)n * D;
  const uint32_t head_bytes = (uint32_t)n * D * 2u;
  const auto rq = make_rsrc(Q + head, head_bytes);
  const auto rdo = make_rsrc(dO + head, head_bytes);
  const auto rl = make_rsrc(LSE + (size_t)bh * n, (uint32_t)n * 4u);
  const auto rd = make_rsrc(Dsum + (size_t)bh * n, (uint32_t)n * 4u);

  // B operands of S (K rows) for the S wave, of dP (V rows) for the dP wave.
  bf16x8 bf[D / 16];
  {
    const auto rkv = make_rsrc((s_role ? K : V) + head, head_bytes);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) bf[s] = as_bf16x8(bload16(rkv, (uint32_t)key * (D * 2) + 32 * s + 16 * hh));
  }

  f32x16 acc[D / 32];  // dV^T (S wave) or dK^T (dP wave)
#pragma unroll
  for (int e = 0; e < D / 32; ++e)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[e][r] = 0.f;

  const int ntq = (n + BQ - 1) / BQ;
  const int it0 = CAUSAL ? (k0 / BQ) : 0;

  // Query rows past n load as zero (Q, dO, LSE, D), so they contribute
  // nothing: P = 1 is finite and multiplies dO = 0 and dS = 0.
  float lr = 0.f, dr = 0.f;
  auto issue = [&](uint16_t* qd, uint16_t* gd, int i0) ATTN_INLINE {
    dma_tile<D, NW>(rq, qd, i0, w, lane);
    dma_tile<D, NW>(rdo, gd, i0, w, lane);
    if (tid < BQ) {
      lr = bload4f(rl, (uint32_t)(i0 + tid) * 4u) * kLog2e;
      dr = bload4f(rd, (uint32_t)(i0 + tid) * 4u);
    }
  };
  auto publish = [&](float* ld, float* dd) ATTN_INLINE {
    if (tid < BQ) {
      ld[tid] = lr;
      dd[tid] = dr;
    }
    wait_vmem();
    __syncthreads();
  };

  float* px = pxs + grp * (2 * 4 * 64 * 4);

  // P or dS of one half tile into dV or dK: hi + lo bf16 pairs where the
  // half tile holds a magnitude >= 1/16 (a single bf16 rounding, relative
  // 2^-9, of a probability near 1 can move a column sum of magnitude > 4 by
  // more than the output's own rounding leaves), one bf16 term elsewhere
  // (long rows, away from the causal diagonal, lose nothing measurable).
  // The test is wave-uniform (ballot).
  auto accumulate = [&](const uint16_t* bs, const float* vt, int t) ATTN_INLINE {
    __builtin_amdgcn_sched_barrier(0);
    float vmax = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) vmax = fmaxf(vmax, fabsf(vt[r]));
    if (__builtin_amdgcn_ballot_w64(vmax >= kSplitThreshold) != 0) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        bf16x8 hi, lo;
        split_bf16x8(vt + 8 * u, hi, lo);
#pragma unroll
        for (int e = 0; e < D / 32; ++e) {
          const bf16x8 a = TR.cols(bs, 32 * t + 16 * u, e);
          acc[e] = mfma32(a, hi, acc[e]);
          acc[e] = mfma32(a, lo, acc[e]);
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8 hi = pack_bf16x8(vt + 8 * u);
#pragma unroll
        for (int e = 0; e < D / 32; ++e) acc[e] = mfma32(TR.cols(bs, 32 * t + 16 * u, e), hi, acc[e]);
      }
    }
  };

  // S wave: S = Q K^T for both half tiles (two independent MFMA chains
  // sharing each K fragment), P = exp(S - LSE) published through LDS, then
  // dV^T += dO^T P.
  auto compute_s = [&](const uint16_t* qs, const uint16_t* gs, const float* lse2s, int i0, bool active,
                       bool need_mask) ATTN_INLINE {
    float v[2][16];
    if (active) {
      f32x16 c0, c1;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        c0[r] = 0.f;
        c1[r] = 0.f;
      }
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        c0 = mfma32(TR.rows(qs, 0, s), bf[s], c0);
        c1 = mfma32(TR.rows(qs, 32, s), bf[s], c1);
      }
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lse2s[32 * t + 8 * g + 4 * hh]);
          f32x4 o;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float pv = fast_exp2(fmaf(t == 0 ? c0[4 * g + i] : c1[4 * g + i], sl2e, -l4[i]));
            if (need_mask) {
              const int q = i0 + 32 * t + 8 * g + 4 * hh + i;
              pv = key > q ? 0.f : pv;
            }
            v[t][4 * g + i] = pv;
            o[i] = pv;
          }
          *reinterpret_cast<f32x4*>(&px[((t * 4 + g) * 64 + lane) * 4]) = o;
        }
    }
    __syncthreads();  // P of this tile is visible to the dP waves
    if (active) {
      accumulate(gs, v[0], 0);
      accumulate(gs, v[1], 1);
    }
  };

  // dP wave: dP = dO V^T accumulated onto -D (registers run over queries),
  // so it ends with dP - D; after P arrives, dS = P * (dP - D), then
  // dK^T += Q^T dS.
  auto compute_dp = [&](const uint16_t* qs, const uint16_t* gs, const float* dsms, bool active) ATTN_INLINE {
    float v[2][16];
    if (active) {
      f32x16 c0, c1;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(&dsms[8 * g + 4 * hh]);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(&dsms[32 + 8 * g + 4 * hh]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          c0[4 * g + i] = -d0[i];
          c1[4 * g + i] = -d1[i];
        }
      }
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        c0 = mfma32(TR.rows(gs, 0, s), bf[s], c0);
        c1 = mfma32(TR.rows(gs, 32, s), bf[s], c1);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        v[0][r] = c0[r];
        v[1][r] = c1[r];
      }
    }
    __syncthreads();  // P of this tile is ready
    if (active) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 p4 = *reinterpret_cast<const f32x4*>(&px[((t * 4 + g) * 64 + lane) * 4]);
#pragma unroll
          for (int i = 0; i < 4; ++i) v[t][4 * g + i] *= p4[i];
        }
        accumulate(qs, v[t], t);
      }
    }
  };

  // The tile loop, once per role: each role's loop is its own region for the
  // register allocator (the two roles together would not fit), and both run
  // the same sequence of barriers.  A tile whose queries all precede this key
  // group is skipped (causal); both waves of a pair decide alike, and every
  // wave reaches the mid-tile barrier inside compute_s / compute_dp.
  auto run = [&](auto&& compute) ATTN_INLINE {
    issue(q0s, g0s, it0 * BQ);
    publish(lse0s, dsm0s);
    for (int it = it0; it < ntq; it += 2) {
      if (it + 1 < ntq) issue(q1s, g1s, (it + 1) * BQ);
      compute(q0s, g0s, lse0s, dsm0s, it * BQ);
      publish(lse1s, dsm1s);
      if (it + 1 >= ntq) break;
      if (it + 2 < ntq) issue(q0s, g0s, (it + 2) * BQ);
      compute(q1s, g1s, lse1s, dsm1s, (it + 1) * BQ);
      publish(lse0s, dsm0s);
    }
  };
  if (s_role) {
    run([&](const uint16_t* qs, const uint16_t* gs, const float* lse2s, const float*, int i0) ATTN_INLINE {
      compute_s(qs, gs, lse2s, i0, !CAUSAL || (i0 + BQ - 1 >= kw0), CAUSAL && (i0 < kw0 + 31));
    });
  } else {
    run([&](const uint16_t* qs, const uint16_t* gs, const float*, const float* dsms, int i0) ATTN_INLINE {
      compute_dp(qs, gs, dsms, !CAUSAL || (i0 + BQ - 1 >= kw0));
    });
  }

  if (key < n) {
    uint16_t* row = (s_role ? dV : dK) + head + (size_t)key * D;
    const float f = s_role ? 1.0f : scale;
#pragma unroll
    for (int e = 0; e < D / 32; ++e)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 o2;
        o2[0] = pack_bf16x2(acc[e][4 * g + 0] * f, acc[e][4 * g + 1] * f);
        o2[1] = pack_bf16x2(acc[e][4 * g + 2] * f, acc[e][4 * g + 3] * f);
        *reinterpret_cast<u32x2*>(row + 32 * e + 8 * g + 4 * hh) = o2;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ: query-stationary
// ---------------------------------------------------------------------------
template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 2) void bwd_q_kernel(const uint16_t* __restrict__ Q,
                                                           const uint16_t* __restrict__ K,
                                                           const uint16_t* __restrict__ V,
                                                           const uint16_t* __restrict__ dO,
                                                           const float* __restrict__ LSE,
                                                           const float* __restrict__ Dsum,
                                                           uint16_t* __restrict__ dQ, int n, int nqb, int total,
                                                           float scale, float sl2e) {
  constexpr int BR = NW * 32, BC = 64;

  __shared__ __attribute__((aligned(1024))) uint16_t k0s[BC * D];
  __shared__ __attribute__((aligned(1024))) uint16_t v0s[BC * D];
  __shared__ __attribute__((aligned(1024))) uint16_t k1s[BC * D];
  __shared__ __attribute__((aligned(1024))) uint16_t v1s[BC * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int l32 = lane & 31, hh = lane >> 5;
  const TileReader<D> TR(lane);

  const int lid = xcd_remap(blockIdx.x, total);
  const int bh = lid / nqb;
  const int qb = CAUSAL ? (nqb - 1 - lid % nqb) : (lid % nqb);
  const int q0 = qb * BR;
  const int wq0 = q0 + 32 * w;
  const int qrow = wq0 + l32;

  const size_t head = (size_t)bh * (size_t)n * D;
  const uint32_t head_bytes = (uint32_t)n * D * 2u;
  const auto rq = make_rsrc(Q + head, head_bytes);
  const auto rdo = make_rsrc(dO + head, head_bytes);
  const auto rk = make_rsrc(K + head, head_bytes);
  const auto rv = make_rsrc(V + head, head_bytes);

  bf16x8 qf[D / 16], gf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    qf[s] = as_bf16x8(bload16(rq, (uint32_t)qrow * (D * 2) + 32 * s + 16 * hh));
    gf[s] = as_bf16x8(bload16(rdo, (uint32_t)qrow * (D * 2) + 32 * s + 16 * hh));
  }
  const float l2 = qrow < n ? LSE[(size_t)bh * n + qrow] * kLog2e : 0.f;
  const float dq_d = qrow < n ? Dsum[(size_t)bh * n + qrow] : 0.f;

  f32x16 dqa[D / 32];
#pragma unroll
  for (int e = 0; e < D / 32; ++e)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqa[e][r] = 0.f;

  const int kend = CAUSAL ? min(n, q0 + BR) : n;
  const int ntiles = (kend + BC - 1) / BC;

  auto compute = [&](const uint16_t* ks, const uint16_t* vs, int j0) {
    const bool active = !CAUSAL || (j0 <= wq0 + 31);
    if (!active) return;
    const bool need_mask = (j0 + BC > n) || (CAUSAL && j0 + BC - 1 > wq0);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      // One half tile at a time: interleaving the halves costs more
      // registers than the file holds at two waves per SIMD.
      __builtin_amdgcn_sched_barrier(0);
      f32x16 sacc, pacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sacc[r] = 0.f;
        pacc[r] = 0.f;
      }
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        sacc = mfma32(TR.rows(ks, 32 * t, s), qf[s], sacc);
        pacc = mfma32(TR.rows(vs, 32 * t, s), gf[s], pacc);
      }

      float ds[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float pv = fast_exp2(fmaf(sacc[r], sl2e, -l2));
        if (need_mask) {
          const int kj = j0 + 32 * t + crow(r, hh);
          pv = (kj >= n || (CAUSAL && kj > qrow)) ? 0.f : pv;
        }
        ds[r] = pv * (pacc[r] - dq_d);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bf16x8 df = pack_bf16x8(ds + 8 * u);
#pragma unroll
        for (int e = 0; e < D / 32; ++e)
          dqa[e] = mfma32(TR.cols(ks, 32 * t + 16 * u, e), df, dqa[e]);
      }
    }
  };

  dma_tile<D, NW>(rk, k0s, 0, w, lane);
  dma_tile<D, NW>(rv, v0s, 0, w, lane);
  wait_vmem();
  __syncthreads();

  for (int jt = 0; jt < ntiles; jt += 2) {
    if (jt + 1 < ntiles) {
      dma_tile<D, NW>(rk, k1s, (jt + 1) * BC, w, lane);
      dma_tile<D, NW>(rv, v1s, (jt + 1) * BC, w, lane);
    }
    compute(k0s, v0s, jt * BC);
    wait_vmem();
    __syncthreads();
    if (jt + 1 >= ntiles) break;
    if (jt + 2 < ntiles) {
      dma_tile<D, NW>(rk, k0s, (jt + 2) * BC, w, lane);
      dma_tile<D, NW>(rv, v0s, (jt + 2) * BC, w, lane);
    }
    compute(k1s, v1s, (jt + 1) * BC);
    wait_vmem();
    __syncthreads();
  }

  if (qrow < n) {
    uint16_t* drow = dQ + head + (size_t)qrow * D;
#pragma unroll
    for (int e = 0; e < D / 32; ++e)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 o2;
        o2[0] = pack_bf16x2(dqa[e][4 * g + 0] * scale, dqa[e][4 * g + 1] * scale);
        o2[1] = pack_bf16x2(dqa[e][4 * g + 2] * scale, dqa[e][4 * g + 3] * scale);
        *reinterpret_cast<u32x2*>(drow + 32 * e + 8 * g + 4 * hh) = o2;
      }
  }
}

template <int D, bool CAUSAL>
hipError_t launch_dkdv(const BwdArgs& a) {
  const int n = (int)a.n;
  const int nkb = (n + 127) / 128;
  const int total = (int)(a.bh * nkb);
  hipLaunchKernelGGL((bwd_kv_kernel<D, CAUSAL>), dim3(total), dim3(512), 0, a.stream, (const uint16_t*)a.q,
                     (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dout, a.lse, a.dsum,
                     (uint16_t*)a.dk, (uint16_t*)a.dv, n, nkb, total, a.scale, a.scale * kLog2e);
  return hipGetLastError();
}

#ifndef ATTN_DQ_NW128
#define ATTN_DQ_NW128 8  // waves per dQ workgroup at d = 128 (tuning knob)
#endif

template <int D, bool CAUSAL>
hipError_t launch_dq(const BwdArgs& a) {
  constexpr int NW = D == 128 ? ATTN_DQ_NW128 : 4;
  const int n = (int)a.n;
  const int nqb = (n + NW * 32 - 1) / (NW * 32);
  const int total = (int)(a.bh * nqb);
  hipLaunchKernelGGL((bwd_q_kernel<D, NW, CAUSAL>), dim3(total), dim3(NW * 64), 0, a.stream, (const uint16_t*)a.q,
                     (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dout, a.lse, a.dsum,
                     (uint16_t*)a.dq, n, nqb, total, a.scale, a.scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t bwd_bf16_dkdv(const BwdArgs& a) {
  if (a.d == 64) return a.causal ? launch_dkdv<64, true>(a) : launch_dkdv<64, false>(a);
  return a.causal ? launch_dkdv<128, true>(a) : launch_dkdv<128, false>(a);
}

hipError_t bwd_bf16_dq(const BwdArgs& a) {
  if (a.d == 64) return a.causal ? launch_dq<64, true>(a) : launch_dq<64, false>(a);
  return a.causal ? launch_dq<128, true>(a) : launch_dq<128, false>(a);
}

}  // namespace attn
