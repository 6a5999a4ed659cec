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
//    registers as the B operand (no LDS round trip for P).  The V^T operand
//    comes from the row-major V tile through transposing LDS reads.
//  * K and V tiles are fetched by buffer->LDS DMA into two buffers: the DMA
//    of tile j+1 is in flight while tile j is computed (no staging
//    registers, no staging instructions); one barrier per tile.  Rows past
//    the end of the head arrive as zeros, so ragged tails need no branches.
//  * Softmax in base 2: the exponent argument is one FMA, x * c - m * c with
//    c = |scale| log2(e); a negative scale is folded into Q by flipping the
//    sign bits of its bf16 values (exact).  The row sum adds the fp32
//    probabilities, so LSE (which the backward pass recomputes P from) keeps
//    fp32 accuracy.
//  * Lazy rescaling: the reference max used for exp2 is raised only when some
//    row's max grows by more than 2^8 over it (a wave-uniform decision), so
//    the output accumulator is rarely rescaled.  l and O always share the
//    same reference, so the result is the same exact softmax; probabilities
//    stay below 2^8 before normalisation.
//  * Causal: key tiles beyond the workgroup's last query are never visited;
//    a wave skips tiles that lie wholly above its own rows; masking code runs
//    only on diagonal and ragged-tail tiles.
#include "attn_device.h"
#include "attn_launch.h"
#include "attn_tile.h"

namespace attn {

template <int D, int NW, bool CAUSAL, bool SPARSE, bool QK>
__global__ __launch_bounds__(NW * 64, 2) void fwd_bf16_kernel(const uint16_t* __restrict__ Q,
                                                              const uint16_t* __restrict__ K,
                                                              const uint16_t* __restrict__ V,
                                                              uint16_t* __restrict__ O,
                                                              float* __restrict__ LSE, int n, int nqb,
                                                              int total, float c, uint32_t qsign,
                                                              const uint8_t* __restrict__ bmask,
                                                              long long mask_stride, int nb, QkKernelArgs qa) {
  constexpr int BC = 64;                // keys per tile
  constexpr int BR = NW * 32;           // query rows per workgroup
  constexpr float kTau = 8.0f;          // lazy-rescale threshold, log2 units

  __shared__ __attribute__((aligned(1024))) uint16_t k0s[BC * D];
  __shared__ __attribute__((aligned(1024))) uint16_t v0s[BC * D];
  __shared__ __attribute__((aligned(1024))) uint16_t k1s[BC * D];
  __shared__ __attribute__((aligned(1024))) uint16_t v1s[BC * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int l32 = lane & 31, hh = lane >> 5;
  const TileReader<D> TR(lane);

  // Logical tile: contiguous per XCD; heavy (late) query blocks first.
  // Unequal lengths (QK): n is the query length, nk the key length; with
  // split-K/V a workgroup owns one query block and one chunk of keys.
  const int nsplit = QK ? qa.nsplit : 1;
  const int lid = xcd_remap(blockIdx.x, total);
  const int per_head = nqb * nsplit;
  const int bh = lid / per_head;
  const int rem = lid % per_head;
  const int qi = QK ? rem / nsplit : rem;
  const int sp = QK ? rem % nsplit : 0;
  const int qb = CAUSAL ? (nqb - 1 - qi) : qi;
  const int q0 = qb * BR;
  const int nk = QK ? qa.nk : n;

  const size_t head = (size_t)bh * (size_t)n * D;
  const size_t khead = (size_t)bh * (size_t)nk * D;
  const uint32_t head_bytes = (uint32_t)n * D * 2u;
  const uint32_t khead_bytes = (uint32_t)nk * D * 2u;
  const auto rq = make_rsrc(Q + head, head_bytes);
  const auto rk = make_rsrc(K + khead, khead_bytes);
  const auto rv = make_rsrc(V + khead, khead_bytes);

  // Q^T fragments (B operand of S^T = K Q^T): lane holds its query's 8
  // consecutive features per 16-feature step.  Rows past n read as zero.
  const int qrow = q0 + 32 * w + l32;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    u32x4 u = bload16(rq, (uint32_t)qrow * (D * 2) + 32 * s + 16 * hh);
    u ^= qsign;
    qf[s] = as_bf16x8(u);
  }

  // Keys of this workgroup: [klo, khi) (its split; all keys when square),
  // keys >= khi masked; causal (bottom-right when lengths differ: query i
  // sees key j when j <= i + coff) visits only up to kend.  Tiles jlo ..
  // ntiles - 1.
  const int coff = (QK && CAUSAL) ? qa.coff : 0;
  const int klo = QK ? sp * qa.kchunk : 0;
  const int khi = QK ? min(nk, klo + qa.kchunk) : n;
  const int kend = CAUSAL ? min(khi, q0 + BR + coff) : khi;
  const int jlo = klo / BC;
  const int ntiles = kend > klo ? (kend + BC - 1) / BC : jlo;

  f32x16 oacc[D / 32];
#pragma unroll
  for (int e = 0; e < D / 32; ++e)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[e][r] = 0.f;
  float mref = -INFINITY;  // reference max (raw score units) used by exp2
  float lsum = 0.f;        // this lane's share of the running sum
  const float tau_raw = kTau / c;
  const int wq0 = q0 + 32 * w;  // first query of this wave

  auto compute = [&](const uint16_t* kb, const uint16_t* vb, int j0) {
    const bool active = !CAUSAL || (j0 <= wq0 + 31 + coff);
    if (!active) return;
    f32x16 sacc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[t][r] = 0.f;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      sacc[0] = mfma32(TR.rows(kb, 0, s), qf[s], sacc[0]);
      sacc[1] = mfma32(TR.rows(kb, 32, s), qf[s], sacc[1]);
    }

    // Mask (diagonal and ragged tiles only) and take this query's tile max.
    const bool need_mask = (j0 + BC > khi) || (CAUSAL && j0 + BC - 1 > wq0 + coff);
    if (need_mask) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + 32 * t + crow(r, hh);
          const bool dead = (key >= khi) || (CAUSAL && key > qrow + coff);
          sacc[t][r] = dead ? -INFINITY : sacc[t][r];
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[t][r]);
    mx = half_max(mx);

    // Raise the reference max only when some row outgrew it by > 2^tau.
    // Square: tile 0 always holds key 0, which every query may see, so the
    // reference is finite from the first tile on.  Unequal lengths: a row
    // may see no key of its first tiles, so its reference can stay -inf;
    // then nothing is rescaled and its probabilities are 0.
    if (__builtin_amdgcn_ballot_w64(mx > mref + tau_raw) != 0) {
      const float m_new = fmaxf(mref, mx);
      const float alpha = (QK && m_new == -INFINITY) ? 1.f : fast_exp2((mref - m_new) * c);
      mref = m_new;
      lsum *= alpha;
#pragma unroll
      for (int e = 0; e < D / 32; ++e)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[e][r] *= alpha;
    }
    const float mc = (QK && mref == -INFINITY) ? 0.f : mref * c;

    bf16x8 pf[2][2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          p[i] = fast_exp2(fmaf(sacc[t][8 * u + i], c, -mc));
          lsum += p[i];
        }
        pf[t][u] = pack_bf16x8(p);
      }

    // O^T += V^T P^T over the 64 keys of the tile.
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < D / 32; ++e)
          oacc[e] = mfma32(TR.cols(vb, 32 * t + 16 * u, e), pf[t][u], oacc[e]);
  };

  if constexpr (SPARSE) {
    // Block-sparse: only the key tiles of the blocks this query block may
    // attend are fetched and computed (a workgroup's 128 rows are exactly one
    // mask block row; a 64-key tile is half of a mask block).  Their indices
    // are listed in LDS first, then walked like the dense sequence.
    static_assert(BR == kSparseBlock, "one workgroup per mask block row");
    __shared__ uint32_t tlist[kMaxSparseTiles];
    __shared__ int tcount;
    const uint8_t* mrow = bmask + (size_t)bh * mask_stride + (size_t)qb * nb;
    const int cnt = build_tile_list([&](int j) ATTN_INLINE { return mrow[j >> 1] != 0; }, 0, ntiles, tlist, &tcount,
                                    w, lane);
    auto tile = [&](int p) ATTN_INLINE { return __builtin_amdgcn_readfirstlane((int)tlist[p]); };
    if (cnt > 0) {
      dma_tile<D, NW>(rk, k0s, tile(0) * BC, w, lane);
      dma_tile<D, NW>(rv, v0s, tile(0) * BC, w, lane);
      wait_vmem();
      __syncthreads();
    }
    for (int p = 0; p < cnt; p += 2) {
      if (p + 1 < cnt) {
        dma_tile<D, NW>(rk, k1s, tile(p + 1) * BC, w, lane);
        dma_tile<D, NW>(rv, v1s, tile(p + 1) * BC, w, lane);
      }
      compute(k0s, v0s, tile(p) * BC);
      wait_vmem();
      __syncthreads();
      if (p + 1 >= cnt) break;
      if (p + 2 < cnt) {
        dma_tile<D, NW>(rk, k0s, tile(p + 2) * BC, w, lane);
        dma_tile<D, NW>(rv, v0s, tile(p + 2) * BC, w, lane);
      }
      compute(k1s, v1s, tile(p + 1) * BC);
      wait_vmem();
      __syncthreads();
    }
  } else {
  if (!QK || jlo < ntiles) {
    dma_tile<D, NW>(rk, k0s, jlo * BC, w, lane);
    dma_tile<D, NW>(rv, v0s, jlo * BC, w, lane);
    wait_vmem();
    __syncthreads();
  }

  for (int jt = jlo; jt < ntiles; jt += 2) {
    // Even tile from buffer 0; tile jt+1 streams into buffer 1.
    if (jt + 1 < ntiles) {
      dma_tile<D, NW>(rk, k1s, (jt + 1) * BC, w, lane);
      dma_tile<D, NW>(rv, v1s, (jt + 1) * BC, w, lane);
    }
    compute(k0s, v0s, jt * BC);
    wait_vmem();
    __syncthreads();
    if (jt + 1 >= ntiles) break;
    // Odd tile from buffer 1; tile jt+2 streams into buffer 0.
    if (jt + 2 < ntiles) {
      dma_tile<D, NW>(rk, k0s, (jt + 2) * BC, w, lane);
      dma_tile<D, NW>(rv, v0s, (jt + 2) * BC, w, lane);
    }
    compute(k1s, v1s, (jt + 1) * BC);
    wait_vmem();
    __syncthreads();
  }
  }

  // Epilogue: O = acc / l (bf16, nearest-even), LSE = (m c + log2 l) ln 2.
  // Rows that may attend no key (block-sparse, unequal lengths, or a split
  // with none of the row's keys) have l = 0: O = 0 and LSE = -inf.
  const float ltot = half_sum(lsum);
  const bool empty = (SPARSE || QK) && ltot == 0.f;
  const float inv = empty ? 0.f : 1.0f / ltot;
  const float lse_v = empty ? -INFINITY : (mref * c + fast_log2(ltot)) * kLn2;
  if (QK && nsplit > 1) {
    // Split-K/V: this chunk's normalised output and LSE, in fp32.
    if (qrow < n) {
      const size_t prow = ((size_t)bh * nsplit + sp) * (size_t)n + qrow;
      float* orow = qa.opart + prow * D;
#pragma unroll
      for (int e = 0; e < D / 32; ++e)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 o4;
#pragma unroll
          for (int i = 0; i < 4; ++i) o4[i] = oacc[e][4 * g + i] * inv;
          *reinterpret_cast<f32x4*>(orow + 32 * e + 8 * g + 4 * hh) = o4;
        }
      if (hh == 0) qa.lpart[prow] = lse_v;
    }
    return;
  }
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
    if (hh == 0) LSE[(size_t)bh * n + qrow] = lse_v;
  }
}

template <int D, int NW, bool CAUSAL, bool SPARSE, bool QK>
static hipError_t launch_fwd(const FwdArgs& a) {
  constexpr int BR = NW * 32;
  const int nqb = (int)((a.n + BR - 1) / BR);
  const int nsplit = QK ? a.nsplit : 1;
  const int total = (int)(a.bh * nqb * nsplit);
  // |scale| below ~7e-31 (including 0) is raised to a normal float: the
  // exponent arguments then differ from the exact ones by < 1e-28 and the
  // lazy-rescale threshold tau / c stays finite.
  float c = fabsf(a.scale) * kLog2e;
  if (c < 1e-30f) c = 1e-30f;
  const uint32_t qsign = a.scale < 0.f ? 0x80008000u : 0u;
  const int nb = (int)((a.n + kSparseBlock - 1) / kSparseBlock);
  QkKernelArgs qa{};
  if (QK) {
    qa.nk = (int)a.nk;
    qa.coff = (int)(a.nk - a.n);
    qa.kchunk = nsplit > 1 ? a.kchunk : (int)((a.nk + 63) / 64 * 64);
    qa.nsplit = nsplit;
    qa.opart = a.opart;
    qa.lpart = a.lpart;
  }
  hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, CAUSAL, SPARSE, QK>), dim3(total), dim3(NW * 64), 0, a.stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o, a.lse,
                     (int)a.n, nqb, total, c, qsign, a.bmask, (long long)a.mask_stride, nb, qa);
  return hipGetLastError();
}

template <bool SPARSE, bool QK>
static hipError_t fwd_bf16_t(const FwdArgs& a) {
  if (a.d == 64)
    return a.causal ? launch_fwd<64, 4, true, SPARSE, QK>(a) : launch_fwd<64, 4, false, SPARSE, QK>(a);
  return a.causal ? launch_fwd<128, 4, true, SPARSE, QK>(a) : launch_fwd<128, 4, false, SPARSE, QK>(a);
}

hipError_t fwd_bf16(const FwdArgs& a) {
  if (a.bmask) return fwd_bf16_t<true, false>(a);
  if (a.nk >= 0) return fwd_bf16_t<false, true>(a);
  return fwd_bf16_t<false, false>(a);
}

// ---------------------------------------------------------------------------
// Split-K/V merge: WPR waves per query row, 4 waves per workgroup.  With the
// chunks' LSE values l_s and normalised outputs o_s, LSE = log sum_s
// exp(l_s) and O = sum_s exp(l_s - LSE) o_s -- the two-block rule of "Tiling:
// Block-by-Block Softmax" (Paper Notes) applied to all chunks at once, in
// the (LSE, normalised O) form.  With WPR = 4 (few rows, as in decoding) wave
// w sums chunks w, w + 4, ... and the partial sums meet in LDS; with WPR = 1
// (many rows) each wave sums one row's chunks.  A row that no chunk saw gets
// O = 0 and LSE = -inf.  At most 64 chunks.
// ---------------------------------------------------------------------------
template <int D, int WPR>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ opart,
                                                      const float* __restrict__ lpart, uint16_t* __restrict__ O,
                                                      float* __restrict__ LSE, int n, int nsplit, long long rows) {
  constexpr int F = D / 64;  // features per lane
  __shared__ float red[WPR > 1 ? WPR - 1 : 1][D];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int w = wave % WPR;  // this wave's share of the row's chunks
  const long long row = (long long)blockIdx.x * (4 / WPR) + wave / WPR;  // bh * n + i
  if (row >= rows) return;
  const long long bh = row / n, i = row % n;
  const float ls = lane < nsplit ? lpart[(bh * nsplit + lane) * n + i] : -INFINITY;
  float mx = ls;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  float acc[F];
#pragma unroll
  for (int f = 0; f < F; ++f) acc[f] = 0.f;
  float lse = -INFINITY;
  if (mx != -INFINITY) {
    const float wl = lane < nsplit ? expf(ls - mx) : 0.f;
    float sum = wl;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
    lse = mx + logf(sum);
    const float inv = 1.0f / sum;
    // Every chunk wrote finite partials (zeros where it saw nothing), so the
    // loads are unconditional and independent.
#pragma unroll 4
    for (int s = w; s < nsplit; s += WPR) {
      const float ws = __shfl(wl, s) * inv;
      const float* src = opart + ((bh * nsplit + s) * n + i) * D;
#pragma unroll
      for (int f = 0; f < F; ++f) acc[f] += ws * src[lane + 64 * f];
    }
  }
  if constexpr (WPR > 1) {
    if (w > 0) {
#pragma unroll
      for (int f = 0; f < F; ++f) red[w - 1][lane + 64 * f] = acc[f];
    }
    __syncthreads();
    if (w != 0) return;
#pragma unroll
    for (int f = 0; f < F; ++f)
#pragma unroll
      for (int r = 0; r < WPR - 1; ++r) acc[f] += red[r][lane + 64 * f];
  }
  uint16_t* dst = O + row * D;
#pragma unroll
  for (int f = 0; f < F; ++f) dst[lane + 64 * f] = (uint16_t)(pack_bf16x2(acc[f], 0.f) & 0xFFFFu);
  if (lane == 0) LSE[row] = lse;
}

template <int D, int WPR>
static void launch_combine(const FwdArgs& a, long long rows) {
  const dim3 grid((unsigned)((rows + (4 / WPR) - 1) / (4 / WPR)));
  hipLaunchKernelGGL((combine_kernel<D, WPR>), grid, dim3(256), 0, a.stream, a.opart, a.lpart, (uint16_t*)a.o,
                     a.lse, (int)a.n, a.nsplit, rows);
}

hipError_t fwd_combine(const FwdArgs& a) {
  // Below about four rows per CU, spread each row over a workgroup.
  const long long rows = (long long)(a.bh * a.n);
  const bool few = rows < 1024;
  if (a.d == 64)
    few ? launch_combine<64, 4>(a, rows) : launch_combine<64, 1>(a, rows);
  else
    few ? launch_combine<128, 4>(a, rows) : launch_combine<128, 1>(a, rows);
  return hipGetLastError();
}

}  // namespace attn
