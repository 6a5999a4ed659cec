// Fused exact attention forward, bf16 in / bf16 out, fp32 accumulation, gfx950.
//
// One workgroup owns a block of BR = 32 * NW query rows of one (batch, head)
// and streams the head's keys and values past it in tiles of BC = 64 rows,
// keeping the running row max m, running sum l and the unnormalised output in
// registers ("Tiling: Block-by-Block Softmax" on the Paper Notes page; the
// loop of "build it from scratch" on the "flash attention" page and of
// "Rescale and accumulate" on the aicassindra page).  The N x N score matrix
// exists only one 64 x 32 tile at a time, per wave, in registers.
//
// Layout choices (MI355X-specific):
//  * Each wave owns 32 query rows.  It computes the transposed score tile
//    S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so lane l holds all scores of
//    one query (l % 32) for 16 keys per 32-key sub-tile; the row max and row
//    sum are in-lane, plus one v_permlane32_swap between the wave halves.
//  * The transposed output O^T = V^T P^T takes P^T straight from the score
//    registers as the B operand (no LDS round trip for P).  V^T is staged in
//    LDS transposed, with keys in the slot order of the result layout so each
//    operand fragment is one 16-byte LDS read.
//  * K and V tiles are double-buffered in LDS: the global loads of tile j+1
//    are in flight while tile j is computed; one barrier per tile.
//  * The scale is folded with log2(e) so softmax uses v_exp_f32 (2^x).
//  * Causal: key tiles beyond the workgroup's last query are never visited;
//    a wave skips tiles that lie wholly above its own rows; masking code runs
//    only on diagonal and ragged-tail tiles.
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 2) void fwd_bf16_kernel(const uint16_t* __restrict__ Q,
                                                              const uint16_t* __restrict__ K,
                                                              const uint16_t* __restrict__ V,
                                                              uint16_t* __restrict__ O,
                                                              float* __restrict__ LSE, int n, int nqb,
                                                              int total, float sl2e) {
  constexpr int BC = 64;                // keys per tile
  constexpr int NT = NW * 64;           // threads
  constexpr int BR = NW * 32;           // query rows per workgroup
  constexpr int KSTR = D + 8;           // LDS row pitch of K (bf16), 16 B pad
  constexpr int VSTR = BC + 8;          // LDS row pitch of V^T (bf16), 16 B pad
  constexpr int CPR = D / 8;            // 16-byte chunks per row
  constexpr int LPT = BC * CPR / NT;    // 16-byte loads per thread per tensor
  constexpr int KPT = LPT;              // keys per thread in the V transpose
  constexpr int KGROUPS = BC / KPT;
  static_assert(LPT == 2 || LPT == 4, "tile/thread ratio");
  static_assert(KGROUPS * (D / 8) == NT, "V transpose mapping");

  __shared__ __attribute__((aligned(16))) uint16_t ks[2][BC * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t vts[2][D * VSTR];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;

  // Logical tile: contiguous per XCD; heavy (late) query blocks first.
  const int lid = xcd_remap(blockIdx.x, total);
  const int bh = lid / nqb;
  const int qb = CAUSAL ? (nqb - 1 - lid % nqb) : (lid % nqb);
  const int q0 = qb * BR;

  const size_t head = (size_t)bh * (size_t)n * D;
  const uint16_t* Qh = Q + head;
  const uint16_t* Kh = K + head;
  const uint16_t* Vh = V + head;

  // Q^T fragments (B operand of S^T = K Q^T): lane holds its query's 8
  // consecutive features per 16-feature step.
  const int qrow = q0 + 32 * w + l32;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    qf[s] = as_bf16x8(load16_or_zero(Qh + (size_t)qrow * D + 16 * s + 8 * hh, qrow < n));

  // Key range visited by this workgroup.
  const int kend = CAUSAL ? min(n, q0 + BR) : n;
  const int ntiles = (kend + BC - 1) / BC;

  // Staging registers for one K tile and one V tile.
  u32x4 kr[LPT], vr[KPT];
  const int va = tid % KGROUPS;  // key group of this thread in the V transpose
  const int vb = tid / KGROUPS;  // 8-feature chunk of this thread

  auto gload = [&](int j0) {
#pragma unroll
    for (int r = 0; r < LPT; ++r) {
      const int c = tid + NT * r;
      const int row = c / CPR, ch = c % CPR;
      kr[r] = load16_or_zero(Kh + (size_t)(j0 + row) * D + 8 * ch, j0 + row < n);
    }
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const int key = j0 + KPT * va + r;
      vr[r] = load16_or_zero(Vh + (size_t)key * D + 8 * vb, key < n);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int r = 0; r < LPT; ++r) {
      const int c = tid + NT * r;
      const int row = c / CPR, ch = c % CPR;
      *reinterpret_cast<u32x4*>(&ks[buf][row * KSTR + 8 * ch]) = kr[r];
    }
    // Transpose: feature 8*vb + i of keys KPT*va .. KPT*va + KPT-1 become
    // KPT consecutive bf16 in V^T row (8*vb + i) at slot position of KPT*va.
    const int pos = slot_pos(KPT * va);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint16_t* dst = &vts[buf][(8 * vb + i) * VSTR + pos];
      if constexpr (KPT == 4) {
        u32x2 o2;
        o2[0] = (i & 1) ? pack_hi16(vr[0][i >> 1], vr[1][i >> 1]) : pack_lo16(vr[0][i >> 1], vr[1][i >> 1]);
        o2[1] = (i & 1) ? pack_hi16(vr[2][i >> 1], vr[3][i >> 1]) : pack_lo16(vr[2][i >> 1], vr[3][i >> 1]);
        *reinterpret_cast<u32x2*>(dst) = o2;
      } else {
        const uint32_t o1 =
            (i & 1) ? pack_hi16(vr[0][i >> 1], vr[1][i >> 1]) : pack_lo16(vr[0][i >> 1], vr[1][i >> 1]);
        *reinterpret_cast<uint32_t*>(dst) = o1;
      }
    }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int e = 0; e < D / 32; ++e)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[e][r] = 0.f;
  float m = -INFINITY;  // running max, log2 units
  float lsum = 0.f;     // this lane's share of the running sum

  const int wq0 = q0 + 32 * w;  // first query of this wave

  gload(0);
  lstore(0);
  __syncthreads();

  for (int jt = 0; jt < ntiles; ++jt) {
    const int buf = jt & 1;
    const int j0 = jt * BC;
    if (jt + 1 < ntiles) gload(j0 + BC);

    const bool active = !CAUSAL || (j0 <= wq0 + 31);
    if (active) {
      const uint16_t* kb = ks[buf];
      const uint16_t* vb2 = vts[buf];
      f32x16 sacc[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[t][r] = 0.f;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(kb + l32 * KSTR + 16 * s + 8 * hh);
        const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(kb + (32 + l32) * KSTR + 16 * s + 8 * hh);
        sacc[0] = mfma32(a0, qf[s], sacc[0]);
        sacc[1] = mfma32(a1, qf[s], sacc[1]);
      }

      // Scale into log2 units, mask, and take this query's tile max.
      const bool need_mask = (j0 + BC > n) || (CAUSAL && j0 + BC - 1 > wq0);
      float mx = -INFINITY;
      if (need_mask) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = j0 + 32 * t + crow(r, hh);
            float x = sacc[t][r] * sl2e;
            const bool dead = (key >= n) || (CAUSAL && key > qrow);
            x = dead ? -INFINITY : x;
            sacc[t][r] = x;
            mx = fmaxf(mx, x);
          }
      } else {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float x = sacc[t][r] * sl2e;
            sacc[t][r] = x;
            mx = fmaxf(mx, x);
          }
      }
      mx = half_max(mx);
      // Tile 0 always holds key 0, which every query may see, so m_new is
      // finite from the first tile on and exp2(m - m_new) is well defined.
      const float m_new = fmaxf(m, mx);
      const float alpha = fast_exp2(m - m_new);
      m = m_new;
      lsum *= alpha;
#pragma unroll
      for (int e = 0; e < D / 32; ++e)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[e][r] *= alpha;

      bf16x8 pf[2][2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          float p[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            p[i] = fast_exp2(sacc[t][8 * u + i] - m_new);
            lsum += p[i];
          }
          pf[t][u] = pack_bf16x8(p);
        }

      // O^T += V^T P^T over the 64 keys of the tile.
#pragma unroll
      for (int e = 0; e < D / 32; ++e)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const bf16x8 va2 =
                *reinterpret_cast<const bf16x8*>(vb2 + (32 * e + l32) * VSTR + 32 * t + 16 * u + 8 * hh);
            oacc[e] = mfma32(va2, pf[t][u], oacc[e]);
          }
    }

    if (jt + 1 < ntiles) lstore(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: O = acc / l (bf16, nearest-even), LSE = (m + log2 l) * ln 2.
  const float ltot = half_sum(lsum);
  const float inv = 1.0f / ltot;
  if (qrow < n) {
    uint16_t* orow = O + head + (size_t)qrow * D;
#pragma unroll
    for (int e = 0; e < D / 32; ++e)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 o2;
        o2[0] = pack_bf16x2(oacc[e][4 * g + 0] * inv, oacc[e][4 * g + 1] * inv);
        o2[1] = pack_bf16x2(oacc[e][4 * g + 2] * inv, oacc[e][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + 32 * e + 8 * g + 4 * hh) = o2;
      }
    if (hh == 0) LSE[(size_t)bh * n + qrow] = (m + fast_log2(ltot)) * kLn2;
  }
}

template <int D, int NW, bool CAUSAL>
static hipError_t launch_fwd(const FwdArgs& a) {
  constexpr int BR = NW * 32;
  const int nqb = (int)((a.n + BR - 1) / BR);
  const int total = (int)(a.bh * nqb);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, CAUSAL>), dim3(total), dim3(NW * 64), 0, a.stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o, a.lse,
                     (int)a.n, nqb, total, a.scale * kLog2e);
  return hipGetLastError();
}

hipError_t fwd_bf16(const FwdArgs& a) {
  if (a.d == 64) return a.causal ? launch_fwd<64, 4, true>(a) : launch_fwd<64, 4, false>(a);
  return a.causal ? launch_fwd<128, 4, true>(a) : launch_fwd<128, 4, false>(a);
}

}  // namespace attn
