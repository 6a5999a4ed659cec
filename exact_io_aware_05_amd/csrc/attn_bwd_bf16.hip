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
//  * bwd_kv: a workgroup owns 128 keys (32 per wave) and keeps K, V and the
//    dK, dV accumulators in registers while query tiles of 64 rows stream
//    through LDS.  Per 32-query half tile a wave computes S and dP (C[q][key]
//    layout, so lane = key and registers run over queries), then
//    dV^T += dO^T P and dK^T += Q^T dS with P and dS taken straight from
//    those registers as the B operand, each as a hi + lo pair of bf16 values
//    (see below).  Q and dO are staged in LDS twice: row-major (A operand of
//    S and dP) and transposed (A operand of dV^T and dK^T).
//  * bwd_q: a workgroup owns a block of queries (32 per wave) with Q, dO,
//    LSE and D in registers and streams key tiles of 64 rows: S^T = K Q^T and
//    dP^T = V dO^T (lane = query), dS^T, then dQ^T += K^T dS^T.  K is staged
//    row-major and transposed, V row-major.
// Row-major LDS tiles use an XOR swizzle of the 16-byte chunk index so that
// both the staging writes and the operand reads are free of bank conflicts;
// transposed tiles are padded by 16 bytes per row.  Tiles are read with
// buffer loads, which return zero past the end of the head (ragged tails).
// Working on one 32-row half tile at a time keeps the live registers of the
// key-stationary kernel within the register file.
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

namespace {

// 16-byte chunk swizzle for row-major tiles of 64 rows: the chunk index is
// XORed with a function of the row that is one-to-one on any 8 consecutive
// rows starting at a multiple of 8 (operand reads) and on the rows
// {KPT*a + r : a = 0..7} written together during staging.
template <int KPT>
__device__ __forceinline__ int swz(int row) {
  return (row ^ (row >> (KPT == 4 ? 2 : 3))) & 7;
}

// A 64-row tile of a [n, D] bf16 matrix, loaded so that each thread owns KPT
// consecutive rows x 8 features, then stored to LDS row-major (swizzled)
// and/or transposed (feature-major, rows in slot order).
template <int D, int NT>
struct Stage64 {
  static constexpr int ROWS = 64;
  static constexpr int CPR = D / 8;
  static constexpr int KPT = ROWS * CPR / NT;
  static constexpr int GROUPS = ROWS / KPT;
  static constexpr int TSTR = ROWS + 8;  // transposed pitch (bf16)
  static_assert(KPT == 2 || KPT == 4, "tile/thread ratio");
  static_assert(GROUPS * CPR == NT, "mapping");

  u32x4 r[KPT];

  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, int row0, int tid) {
    const int a = tid % GROUPS, b = tid / GROUPS;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int row = row0 + KPT * a + i;
      r[i] = bload16(rs, (uint32_t)row * (D * 2) + 16 * b);
    }
  }
  __device__ __forceinline__ void store_rowmajor(uint16_t* lds, int tid) const {
    const int a = tid % GROUPS, b = tid / GROUPS;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int row = KPT * a + i;
      *reinterpret_cast<u32x4*>(lds + row * D + 8 * (b ^ swz<KPT>(row))) = r[i];
    }
  }
  __device__ __forceinline__ void store_transposed(uint16_t* lds, int tid) const {
    const int a = tid % GROUPS, b = tid / GROUPS;
    const int pos = slot_pos(KPT * a);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint16_t* dst = lds + (8 * b + i) * TSTR + pos;
      const int w = i >> 1;
      if constexpr (KPT == 4) {
        u32x2 o2;
        o2[0] = (i & 1) ? pack_hi16(r[0][w], r[1][w]) : pack_lo16(r[0][w], r[1][w]);
        o2[1] = (i & 1) ? pack_hi16(r[2][w], r[3][w]) : pack_lo16(r[2][w], r[3][w]);
        *reinterpret_cast<u32x2*>(dst) = o2;
      } else {
        *reinterpret_cast<uint32_t*>(dst) = (i & 1) ? pack_hi16(r[0][w], r[1][w]) : pack_lo16(r[0][w], r[1][w]);
      }
    }
  }
};

// A operand fragment from a swizzled row-major 64-row tile: row `row`,
// features 16*s + 8*h .. +7.
template <int D, int KPT>
__device__ __forceinline__ bf16x8 frag_rowmajor(const uint16_t* lds, int row, int s, int h) {
  const int ch = (2 * s + h) ^ swz<KPT>(row);
  return *reinterpret_cast<const bf16x8*>(lds + row * D + 8 * ch);
}

// ---------------------------------------------------------------------------
// dK, dV: key-stationary
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void bwd_kv_kernel(const uint16_t* __restrict__ Q,
                                                        const uint16_t* __restrict__ K,
                                                        const uint16_t* __restrict__ V,
                                                        const uint16_t* __restrict__ dO,
                                                        const float* __restrict__ LSE,
                                                        const float* __restrict__ Dsum,
                                                        uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
                                                        int n, int nkb, int total, float scale, float sl2e) {
  constexpr int NT = 256, BKV = 128, BQ = 64;
  using ST = Stage64<D, NT>;
  constexpr int KPT = ST::KPT, TSTR = ST::TSTR;

  __shared__ __attribute__((aligned(16))) uint16_t qs[2][BQ * D];
  __shared__ __attribute__((aligned(16))) uint16_t dos[2][BQ * D];
  __shared__ __attribute__((aligned(16))) uint16_t qts[2][D * TSTR];
  __shared__ __attribute__((aligned(16))) uint16_t dots[2][D * TSTR];
  __shared__ __attribute__((aligned(16))) float lse2s[2][BQ];
  __shared__ __attribute__((aligned(16))) float dsms[2][BQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;

  // Causal: low key blocks see the most queries; they come first.
  const int lid = xcd_remap(blockIdx.x, total);
  const int bh = lid / nkb, kb = lid % nkb;
  const int k0 = kb * BKV;
  const int kw0 = k0 + 32 * w;
  const int key = kw0 + l32;

  const size_t head = (size_t)bh * (size_t)n * D;
  const uint32_t head_bytes = (uint32_t)n * D * 2u;
  const auto rq = make_rsrc(Q + head, head_bytes);
  const auto rdo = make_rsrc(dO + head, head_bytes);
  const auto rk = make_rsrc(K + head, head_bytes);
  const auto rv = make_rsrc(V + head, head_bytes);
  const auto rl = make_rsrc(LSE + (size_t)bh * n, (uint32_t)n * 4u);
  const auto rd = make_rsrc(Dsum + (size_t)bh * n, (uint32_t)n * 4u);

  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    kf[s] = as_bf16x8(bload16(rk, (uint32_t)key * (D * 2) + 32 * s + 16 * hh));
    vf[s] = as_bf16x8(bload16(rv, (uint32_t)key * (D * 2) + 32 * s + 16 * hh));
  }

  f32x16 dva[D / 32], dka[D / 32];
#pragma unroll
  for (int e = 0; e < D / 32; ++e)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dva[e][r] = 0.f;
      dka[e][r] = 0.f;
    }

  const int ntq = (n + BQ - 1) / BQ;
  const int it0 = CAUSAL ? (k0 / BQ) : 0;

  // Query rows past n load as zero (Q, dO, LSE, D), so they contribute
  // nothing: P = 1 is finite and multiplies dO = 0 and dS = 0.
  ST sq, sd;
  float lr = 0.f, dr = 0.f;
  auto gload = [&](int i0) {
    sq.load(rq, i0, tid);
    sd.load(rdo, i0, tid);
    if (tid < BQ) {
      lr = bload4f(rl, (uint32_t)(i0 + tid) * 4u) * kLog2e;
      dr = bload4f(rd, (uint32_t)(i0 + tid) * 4u);
    }
  };
  auto lstore = [&](int buf) {
    sq.store_rowmajor(qs[buf], tid);
    sq.store_transposed(qts[buf], tid);
    sd.store_rowmajor(dos[buf], tid);
    sd.store_transposed(dots[buf], tid);
    if (tid < BQ) {
      lse2s[buf][tid] = lr;
      dsms[buf][tid] = dr;
    }
  };

  gload(it0 * BQ);
  lstore(0);
  __syncthreads();

  for (int it = it0; it < ntq; ++it) {
    const int buf = (it - it0) & 1;
    const int i0 = it * BQ;
    if (it + 1 < ntq) gload(i0 + BQ);

    // Skip a tile whose queries all precede this wave's keys (causal).
    const bool active = !CAUSAL || (i0 + BQ - 1 >= kw0);
    if (active) {
      const bool need_mask = CAUSAL && (i0 < kw0 + 31);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        f32x16 sacc, pacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sacc[r] = 0.f;
          pacc[r] = 0.f;
        }
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
          const bf16x8 aq = frag_rowmajor<D, KPT>(qs[buf], 32 * t + l32, s, hh);
          const bf16x8 ad = frag_rowmajor<D, KPT>(dos[buf], 32 * t + l32, s, hh);
          sacc = mfma32(aq, kf[s], sacc);
          pacc = mfma32(ad, vf[s], pacc);
        }

        float p[16], ds[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lse2s[buf][32 * t + 8 * g + 4 * hh]);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(&dsms[buf][32 * t + 8 * g + 4 * hh]);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * g + i;
            float pv = fast_exp2(fmaf(sacc[r], sl2e, -l4[i]));
            if (need_mask) {
              const int q = i0 + 32 * t + 8 * g + 4 * hh + i;
              pv = key > q ? 0.f : pv;
            }
            p[r] = pv;
            ds[r] = pv * (pacc[r] - d4[i]);
          }
        }

        // P and dS enter dV and dK as hi + lo bf16 pairs: a single bf16
        // rounding (relative 2^-9) of a probability near 1 can move a column
        // sum of magnitude > 4 by more than the output's own rounding leaves.
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          bf16x8 ph, pl, dh, dl;
          split_bf16x8(p + 8 * u, ph, pl);
          split_bf16x8(ds + 8 * u, dh, dl);
#pragma unroll
          for (int e = 0; e < D / 32; ++e) {
            const int off = (32 * e + l32) * TSTR + 32 * t + 16 * u + 8 * hh;
            const bf16x8 adt = *reinterpret_cast<const bf16x8*>(&dots[buf][off]);
            const bf16x8 aqt = *reinterpret_cast<const bf16x8*>(&qts[buf][off]);
            dva[e] = mfma32(adt, ph, dva[e]);
            dka[e] = mfma32(aqt, dh, dka[e]);
            dva[e] = mfma32(adt, pl, dva[e]);
            dka[e] = mfma32(aqt, dl, dka[e]);
          }
        }
      }
    }

    if (it + 1 < ntq) lstore(buf ^ 1);
    __syncthreads();
  }

  if (key < n) {
    uint16_t* dvrow = dV + head + (size_t)key * D;
    uint16_t* dkrow = dK + head + (size_t)key * D;
#pragma unroll
    for (int e = 0; e < D / 32; ++e)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 v2, k2;
        v2[0] = pack_bf16x2(dva[e][4 * g + 0], dva[e][4 * g + 1]);
        v2[1] = pack_bf16x2(dva[e][4 * g + 2], dva[e][4 * g + 3]);
        k2[0] = pack_bf16x2(dka[e][4 * g + 0] * scale, dka[e][4 * g + 1] * scale);
        k2[1] = pack_bf16x2(dka[e][4 * g + 2] * scale, dka[e][4 * g + 3] * scale);
        *reinterpret_cast<u32x2*>(dvrow + 32 * e + 8 * g + 4 * hh) = v2;
        *reinterpret_cast<u32x2*>(dkrow + 32 * e + 8 * g + 4 * hh) = k2;
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
  constexpr int NT = NW * 64, BR = NW * 32, BC = 64;
  using ST = Stage64<D, NT>;
  constexpr int KPT = ST::KPT, TSTR = ST::TSTR;

  __shared__ __attribute__((aligned(16))) uint16_t ks[2][BC * D];
  __shared__ __attribute__((aligned(16))) uint16_t vs[2][BC * D];
  __shared__ __attribute__((aligned(16))) uint16_t kts[2][D * TSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;

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

  ST sk, sv;
  auto gload = [&](int j0) {
    sk.load(rk, j0, tid);
    sv.load(rv, j0, tid);
  };
  auto lstore = [&](int buf) {
    sk.store_rowmajor(ks[buf], tid);
    sk.store_transposed(kts[buf], tid);
    sv.store_rowmajor(vs[buf], tid);
  };

  gload(0);
  lstore(0);
  __syncthreads();

  for (int jt = 0; jt < ntiles; ++jt) {
    const int buf = jt & 1;
    const int j0 = jt * BC;
    if (jt + 1 < ntiles) gload(j0 + BC);

    const bool active = !CAUSAL || (j0 <= wq0 + 31);
    if (active) {
      const bool need_mask = (j0 + BC > n) || (CAUSAL && j0 + BC - 1 > wq0);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        f32x16 sacc, pacc;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sacc[r] = 0.f;
          pacc[r] = 0.f;
        }
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
          const bf16x8 ak = frag_rowmajor<D, KPT>(ks[buf], 32 * t + l32, s, hh);
          const bf16x8 av = frag_rowmajor<D, KPT>(vs[buf], 32 * t + l32, s, hh);
          sacc = mfma32(ak, qf[s], sacc);
          pacc = mfma32(av, gf[s], pacc);
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
          for (int e = 0; e < D / 32; ++e) {
            const bf16x8 akt =
                *reinterpret_cast<const bf16x8*>(&kts[buf][(32 * e + l32) * TSTR + 32 * t + 16 * u + 8 * hh]);
            dqa[e] = mfma32(akt, df, dqa[e]);
          }
        }
      }
    }

    if (jt + 1 < ntiles) lstore(buf ^ 1);
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
  hipLaunchKernelGGL((bwd_kv_kernel<D, CAUSAL>), dim3(total), dim3(256), 0, a.stream, (const uint16_t*)a.q,
                     (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dout, a.lse, a.dsum,
                     (uint16_t*)a.dk, (uint16_t*)a.dv, n, nkb, total, a.scale, a.scale * kLog2e);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_dq(const BwdArgs& a) {
  constexpr int NW = D == 128 ? 8 : 4;
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
