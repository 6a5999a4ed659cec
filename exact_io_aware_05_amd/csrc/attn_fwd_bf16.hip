// Fused exact attention forward, bf16 in / bf16 out, fp32 accumulation, gfx950.
//
// One workgroup owns a block of BR = 32 * NW query rows of one (batch, head)
// and streams the head's keys and values past it, keeping the running row
// max m, running sum l and the unnormalised output in registers ("Tiling:
// Block-by-Block Softmax" on the Paper Notes page; the loop of "build it from
// scratch" on the "flash attention" page and of "Rescale and accumulate" on
// the aicassindra page).  The N x N score matrix exists only one 32 x 32
// block at a time, per wave, in registers.
//
// Layout choices (MI355X-specific):
//  * Each wave owns 32 query rows.  It computes transposed score blocks
//    S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so lane l holds the scores of
//    one query (l % 32) for 16 of the block's 32 keys; the row sums are
//    in-lane, plus one v_permlane32_swap between the wave halves at the end.
//  * The transposed output O^T = V^T P^T takes P^T straight from the score
//    registers as the B operand (no LDS round trip for P).  The V^T operand
//    comes from the row-major V tile through transposing LDS reads.
//  * Software pipeline over units of 32 keys: step u issues the score
//    products of unit u + 1 and the output products of unit u - 1, and
//    between them the exponentials of unit u, so every wave always has
//    vector work to overlap with its own matrix products.
//  * K and V tiles (64 keys) are fetched by buffer->LDS DMA into two rings of
//    R tiles (no staging registers); V is consumed one tile after K, so the
//    fetch of tile t + R - 1 (K) and t + R - 2 (V) is issued at the barrier
//    that opens tile t.  Rows past the end of the head arrive as zeros.
//  * Softmax in base 2: the exponent argument is one FMA, x * c - m * c with
//    c = |scale| log2(e); a negative scale is folded into Q by flipping the
//    sign bits of its bf16 values (exact).  The row sum adds the fp32
//    probabilities, so LSE (which the backward pass recomputes P from) keeps
//    fp32 accuracy.
//  * Lazy rescaling without a per-block max: the probabilities of a unit are
//    computed against the current reference max m, and only if some lane's
//    sum over the unit exceeds 2^8 (so possibly one probability does) is the
//    unit's max taken, m raised, the output and sum rescaled and the unit
//    recomputed.  l and O always share m, so the result is the same exact
//    softmax; probabilities stay at most 2^8 before normalisation, and a row
//    whose m is still -inf (nothing seen yet) always takes that path.
//  * Causal: key tiles beyond the workgroup's last query are never visited;
//    units wholly above a wave's rows are skipped by that wave; masking code
//    runs only on diagonal and ragged-tail units, which come last.  The
//    heavy query blocks are scheduled first, longest first within each XCD
//    (heavy_first in attn_device.h).
#include "attn_device.h"
#include "attn_launch.h"
#include "attn_tile.h"

namespace attn {

template <int D, int NW, bool CAUSAL, bool SPARSE, bool QK, bool DROP, bool WIN = false>
__global__ __launch_bounds__(NW * 64, 2) void fwd_bf16_kernel(const uint16_t* __restrict__ Q,
                                                                   const uint16_t* __restrict__ K,
                                                                   const uint16_t* __restrict__ V,
                                                                   uint16_t* __restrict__ O,
                                                                   float* __restrict__ LSE, int n, int nqb,
                                                                   int total, float c, uint32_t qsign,
                                                                   const uint8_t* __restrict__ bmask,
                                                                   long long mask_stride, int nb, QkKernelArgs qa,
                                                                   DropArgs dr, const int* __restrict__ klen,
                                                                   int heads, int wl, int hf_pass, int hf_fill) {
  constexpr int BC = 64;               // keys per K/V tile
  constexpr int BU = 32;               // keys per pipeline unit (half a tile)
  constexpr int BR = NW * 32;          // query rows per workgroup
  constexpr int R = NW == 8 ? 3 : 2;   // tiles per ring
  constexpr int TB = BC * D;           // elements per tile
  constexpr int IPW = (D / 8) / NW;    // DMA loads per wave per tile
  constexpr float kGate = 256.0f;      // 2^8
  // Ring slots are separate LDS arrays, always addressed at compile-time
  // slots: the compiler can then tell a DMA into one slot from reads of
  // another, and waits for the DMA only where its slot is read.
  __shared__ __attribute__((aligned(1024))) uint16_t k0s[TB], k1s[TB], k2s[R > 2 ? TB : 1];
  __shared__ __attribute__((aligned(1024))) uint16_t v0s[TB], v1s[TB], v2s[R > 2 ? TB : 1];
  auto kslot = [&](auto ic) ATTN_INLINE -> uint16_t* {
    constexpr int i = decltype(ic)::value % R;
    if constexpr (i == 0) return k0s;
    else if constexpr (i == 1) return k1s;
    else return k2s;
  };
  auto vslot = [&](auto ic) ATTN_INLINE -> uint16_t* {
    constexpr int i = decltype(ic)::value % R;
    if constexpr (i == 0) return v0s;
    else if constexpr (i == 1) return v1s;
    else return v2s;
  };
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int l32 = lane & 31, hh = lane >> 5;
  const TileReader<D> TRK(lane);
  const TileReader<D> TRV(lane);

  // Logical tile: contiguous per XCD; under the causal mask heavy (late)
  // query blocks first, longest first within each XCD.  Unequal lengths
  // (QK): n is the query length, nk the key length; with split-K/V a
  // workgroup owns one query block and one chunk of keys.
  const int nsplit = QK ? qa.nsplit : 1;
  int bh, qi, sp = 0;
  if (CAUSAL && nsplit == 1) {
    heavy_first(blockIdx.x, total / nqb, nqb, bh, qi, hf_pass, hf_fill);
  } else {
    const int lid = xcd_remap(blockIdx.x, total);
    const int per_head = nqb * nsplit;
    bh = lid / per_head;
    const int rem = lid % per_head;
    qi = QK ? rem / nsplit : rem;
    sp = QK ? rem % nsplit : 0;
  }
  const int qb = CAUSAL ? (nqb - 1 - qi) : qi;
  const int q0 = qb * BR;
  const int nk = QK ? qa.nk : n;

  const size_t head = (size_t)bh * (size_t)n * D;
  const size_t khead = (size_t)bh * (size_t)nk * D;
  const uint32_t head_bytes = (uint32_t)n * D * 2u;
  const uint32_t khead_bytes = (uint32_t)nk * D * 2u;
  const auto rq = make_rsrc(Q + head, head_bytes);
  const RsrcWords rk = rsrc_words(K + khead, khead_bytes);
  const RsrcWords rv = rsrc_words(V + khead, khead_bytes);

  // Q^T fragments (B operand of S^T = K Q^T): lane holds its query's 8
  // consecutive features per 16-feature step.  Rows past n read as zero.
  const int wq0 = q0 + 32 * w;  // first query of this wave
  const int qrow = wq0 + l32;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    u32x4 u = bload16(rq, (uint32_t)qrow * (D * 2) + 32 * s + 16 * hh);
    u ^= qsign;
    qf[s] = as_bf16x8(u);
  }

  // Keys of this workgroup: [klo, khi) (its split; all keys when square,
  // or those below the padding), keys >= khi masked; causal (bottom-right when lengths differ: query i
  // sees key j when j <= i + coff) visits only up to kend.  Tiles jlo ..
  // ntiles - 1.
  // Key padding (square lengths): keys from padded_keys(..) on are masked
  // like keys past the end.
  // Sliding window (WIN, with the causal mask): query i sees keys i - wl ..
  // i, so the workgroup starts at key q0 - wl.
  const int coff = (QK && CAUSAL) ? qa.coff : 0;
  const int klo = QK ? sp * qa.kchunk : (WIN ? max(0, q0 - wl) : 0);
  const int khi = QK ? min(nk, klo + qa.kchunk) : padded_keys(klen, heads, bh, n);
  const int kend = CAUSAL ? min(khi, q0 + BR + coff) : khi;
  const int jlo = klo / BC;
  const int ntiles = kend > klo ? (kend + BC - 1) / BC : jlo;

  // Visited tiles by position p = 0 .. P - 1, and units u = 0 .. U - 1
  // (unit u is half u % 2 of the tile at position u / 2).
  int P, U;
  __shared__ uint32_t tlist[SPARSE ? kMaxSparseTiles + 1 : 1];
  if constexpr (SPARSE) {
    // Block-sparse: only the key tiles of the blocks this query block may
    // attend (a workgroup's 128 rows are exactly one mask block row; a
    // 64-key tile is half of a mask block), listed in LDS first.
    static_assert(BR == kSparseBlock, "one workgroup per mask block row");
    int* const tcount = reinterpret_cast<int*>(tlist + kMaxSparseTiles);
    const uint8_t* mrow = bmask + (size_t)bh * mask_stride + (size_t)qb * nb;
    P = build_tile_list([&](int j) ATTN_INLINE { return mrow[j >> 1] != 0; }, 0, ntiles, tlist, tcount, w, lane);
    U = 2 * P;
  } else {
    P = ntiles - jlo;
    U = P > 0 ? (kend - jlo * BC + BU - 1) / BU : 0;
  }
  auto tile = [&](int p) ATTN_INLINE {
    if constexpr (SPARSE)
      return __builtin_amdgcn_readfirstlane((int)tlist[p]);
    else
      return jlo + p;
  };
  auto ju = [&](int u) ATTN_INLINE { return tile(u >> 1) * BC + BU * (u & 1); };  // first key of unit u
  auto active = [&](int j0) ATTN_INLINE { return !CAUSAL || j0 <= wq0 + 31 + coff; };
  auto need_mask = [&](int j0) ATTN_INLINE {
    return j0 + BU > khi || (CAUSAL && j0 + BU - 1 > wq0 + coff) || (WIN && j0 < wq0 + 31 - wl);
  };

  // K of position p lives in ring slot p % R, V likewise.  Slots are
  // compile-time constants: SLOT = p mod R.
  auto issue_k = [&](auto slot, int p) ATTN_INLINE {
    if (p < P) dma_tile_asm<D, NW>(rk, kslot(slot), tile(p) * BC, w, lane);
  };
  auto issue_v = [&](auto slot, int p) ATTN_INLINE {
    if (p >= 0 && p < P) dma_tile_asm<D, NW>(rv, vslot(slot), tile(p) * BC, w, lane);
  };
  // Fetches issued when tile t opens (t modulo R = TM): K(t + R - 1), V(t + R - 2).
  auto issue = [&](auto tm, int t) ATTN_INLINE {
    constexpr int T = decltype(tm)::value;
    issue_k(std::integral_constant<int, (T + R - 1) % R>{}, t + R - 1);
    issue_v(std::integral_constant<int, (T + 2 * R - 2) % R>{}, t + R - 2);
  };
  // Opening tile t (before step 2t - 1, the first to read K of tile t and V
  // of tile t - 1): their fetches are complete, every wave is done with the
  // slots of K(t - 1) and V(t - 2), which the next fetches overwrite.
  auto handover = [&](auto tm, int t) ATTN_INLINE {
    if constexpr (R > 2) {
      if (t + R - 2 < P)
        wait_vmem_upto<(R - 2) * 2 * IPW>();  // the later batches stay in flight
      else
        wait_vmem();
    } else {
      wait_vmem();
    }
    __syncthreads();
    issue(tm, t);
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int e = 0; e < D / 32; ++e)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[e][r] = 0.f;
  float mref = -INFINITY;  // reference max (raw score units) used by exp2
  float mc = 0.f;          // mref * c (0 while mref = -inf)
  float gate = -1.f;       // a unit sum above this takes the slow path
  float lsum = 0.f;        // this lane's share of the running sum
  f32x16 s0, s1;           // scores of even / odd units
  bf16x8 p0[2], p1[2];     // probabilities of even / odd units
  // Sliding window: a wave's first needed unit holds key wq0 - wl; the steps
  // before the one that computes its scores are skipped by this wave (its
  // probability registers start at zero, so the first step it runs adds
  // nothing for the unit before).
  int u_need = 0;
  if constexpr (WIN) {
    u_need = (max(0, wq0 - wl) - jlo * BC) / BU;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      p0[h] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
      p1[h] = p0[h];
    }
  }

  // One pipeline step: scores of the next unit (tile rows at kb) into sn;
  // probabilities of this unit (sc -> pn; returns this lane's sum); output
  // products of the previous unit (po, tile rows at vb).  Straight-line code:
  // a unit that must not contribute is masked to -inf (probabilities 0, so
  // its output products add zeros to finite V rows), and the matrix and
  // vector work can be interleaved freely.
  // Dropout: keep bit r of a unit starting at key j0 for this lane's query;
  // the four words of one generator call cover keys j0 + 8g + 4hh + 0..3,
  // which are exactly registers 4g .. 4g + 3.
  auto keep_bits = [&](int j0) ATTN_INLINE -> uint32_t {
    uint32_t bits = 0;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const u32x4 wd = philox4x32_10((uint32_t)(j0 + 8 * g + 4 * hh) >> 2, (uint32_t)qrow, (uint32_t)bh, dr.offset,
                                     dr.seed_lo, dr.seed_hi);
#pragma unroll
      for (int i = 0; i < 4; ++i) bits |= (wd[i] >= dr.thr ? 1u : 0u) << (4 * g + i);
    }
    return bits;
  };
  // Probabilities as they enter the output products: dropped ones are 0,
  // kept ones scaled by 1 / (1 - p) (the row sum keeps all of them).
  auto pack_p = [&](const float* p, uint32_t keep, bf16x8(&pn)[2]) ATTN_INLINE {
    if constexpr (DROP) {
      float pd[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) pd[r] = (keep >> r) & 1u ? p[r] * dr.keep_scale : 0.f;
      pn[0] = pack_bf16x8(pd);
      pn[1] = pack_bf16x8(pd + 8);
    } else {
      pn[0] = pack_bf16x8(p);
      pn[1] = pack_bf16x8(p + 8);
    }
  };

  auto step = [&](auto has_pv, f32x16& sc, f32x16& sn, bf16x8(&pn)[2], const bf16x8(&po)[2], const uint16_t* kb,
                  const uint16_t* vb, int j0, uint32_t& keep) ATTN_INLINE -> float {
#pragma unroll
    for (int r = 0; r < 16; ++r) sn[r] = 0.f;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) sn = mfma32(TRK.rows(kb, 0, s), qf[s], sn);
    // (Step 0 has no previous unit; its V slot holds no data yet.)
    if constexpr (decltype(has_pv)::value) {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < D / 32; ++e) oacc[e] = mfma32(TRV.cols(vb, 16 * h, e), po[h], oacc[e]);
    }
    float p[16], a[4];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = fast_exp2(fmaf(sc[r], c, -mc));
      a[r & 3] = r < 4 ? p[r] : a[r & 3] + p[r];
    }
    if constexpr (DROP) keep = keep_bits(j0);
    pack_p(p, keep, pn);
    // Keep the conversions here, so the 16 probabilities die in this step.
    asm volatile("" ::"v"(pn[0]), "v"(pn[1]));
    // Interleave: each matrix product is preceded by LDS reads for a later
    // one and followed by a share of the exponential work (masks: 0x100 LDS
    // read, 0x008 MFMA, 0x402 VALU).
    constexpr int NP = D / 16;
    constexpr int NV = DROP ? 56 + 200 : 56;  // vector instructions per step, about
    constexpr int VPM = (NV + 2 * NP - 1) / (2 * NP);
    __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, VPM, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x402, VPM, 0);
    }
    return (a[0] + a[1]) + (a[2] + a[3]);
  };

  // After a step: if some lane's unit sum exceeds the gate, raise the
  // reference to the unit's max, rescale, and recompute the unit.
  auto settle = [&](f32x16& sc, bf16x8(&pn)[2], float ps, uint32_t keep) ATTN_INLINE {
    if (__builtin_amdgcn_ballot_w64(ps > gate) != 0) {
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[r]);
      mx = half_max(mx);
      const float m_new = fmaxf(mref, mx);
      const float alpha = m_new == -INFINITY ? 1.f : fast_exp2((mref - m_new) * c);
      mref = m_new;
      mc = m_new == -INFINITY ? 0.f : m_new * c;
      gate = m_new == -INFINITY ? -1.f : kGate;
      lsum *= alpha;
#pragma unroll
      for (int e = 0; e < D / 32; ++e)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[e][r] *= alpha;
      float p[16];
      ps = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p[r] = fast_exp2(fmaf(sc[r], c, -mc));
        ps += p[r];
      }
      pack_p(p, keep, pn);
    }
    lsum += ps;
  };

  // Step u (u = 0 .. U; step U only ends the output products of unit U - 1),
  // with k = u modulo 2R so that every ring slot is a compile-time offset.
  // Units that need a mask (diagonal, ragged, past the end) are masked in
  // place first; a causal step whose units all lie above this wave's rows is
  // skipped.
  auto run_step = [&](auto kc, int u) ATTN_INLINE {
    constexpr int k = decltype(kc)::value;
    constexpr bool ODD = k & 1;
    constexpr int half = ((k + 1) & 1) * BU * D;                           // of units u + 1 and u - 1
    const uint16_t* kb = kslot(std::integral_constant<int, ((k + 1) >> 1)>{}) + half;           // unit u + 1
    const uint16_t* vb = vslot(std::integral_constant<int, ((k + 2 * R - 1) >> 1)>{}) + half;  // unit u - 1
    auto go = [&](f32x16& sc, f32x16& sn, bf16x8(&pn)[2], const bf16x8(&po)[2]) ATTN_INLINE {
      const int j0 = u < U ? ju(u) : khi;
      if (CAUSAL && u >= 1 && !active(ju(u - 1))) return;
      if (WIN && u + 1 < u_need) return;  // every key of units u - 1 .. u + 1 precedes this wave's window
      if (need_mask(j0)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + crow(r, hh);
          const bool dead = (key >= khi) || (CAUSAL && key > qrow + coff) || (WIN && key < qrow - wl);
          sc[r] = dead ? -INFINITY : sc[r];
        }
      }
      uint32_t keep = 0xFFFFu;
      const float ps = step(std::bool_constant<(k > 0)>{}, sc, sn, pn, po, kb, vb, j0, keep);
      settle(sc, pn, ps, keep);
    };
    if constexpr (ODD)
      go(s1, s0, p1, p0);
    else
      go(s0, s1, p0, p1);
  };

  if (P > 0) {
    issue_k(std::integral_constant<int, 0>{}, 0);
    if constexpr (R > 2) issue(std::integral_constant<int, R - 1>{}, -1);
    issue(std::integral_constant<int, 0>{}, 0);
    if constexpr (R > 1) {
      if (R - 1 < P)
        wait_vmem_upto<(R - 1) * 2 * IPW>();  // K of tile 0 has arrived
      else
        wait_vmem();
    }
    __syncthreads();
  }

  if (U > 0) {
    // Scores of unit 0, then the steps; step u > 0 ends the output products
    // of unit u - 1, so the last one is step U.
#pragma unroll
    for (int r = 0; r < 16; ++r) s0[r] = 0.f;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) s0 = mfma32(TRK.rows(k0s, 0, s), qf[s], s0);
    run_step(std::integral_constant<int, 0>{}, 0);
    int u = 1;
    bool run = true;
    while (run) {
      auto body = [&](auto kc) ATTN_INLINE {
        constexpr int k = decltype(kc)::value;
        if (!run || u > U) {
          run = false;
          return;
        }
        if constexpr (k & 1) handover(std::integral_constant<int, (((k + 1) >> 1) % R)>{}, (u + 1) >> 1);
        run_step(kc, u);
        ++u;
      };
      body(std::integral_constant<int, 1>{});
      body(std::integral_constant<int, 2>{});
      body(std::integral_constant<int, 3>{});
      body(std::integral_constant<int, 4>{});
      if constexpr (R > 2) {
        body(std::integral_constant<int, 5>{});
        body(std::integral_constant<int, 6>{});
      }
    }
  }

  // Epilogue: O = acc / l (bf16, nearest-even), LSE = (m c + log2 l) ln 2.
  // Rows that may attend no key (block-sparse, unequal lengths, or a split
  // with none of the row's keys) have l = 0: O = 0 and LSE = -inf.
  const float ltot = half_sum(lsum);
  const bool empty = ltot == 0.f;
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
  // O leaves through LDS so that every store writes whole 128-byte row
  // segments: each wave stages its 32 rows, 64 features at a time, in a
  // region of the ring (rows 144 bytes apart; three regions per slot at
  // d = 128, one at d = 64), and reads them back 16 bytes per lane, eight
  // rows per instruction.  The ring is free once every wave has passed this
  // barrier.
  __syncthreads();
  constexpr int RS = 72;                           // row stride in bf16 elements (144 bytes)
  constexpr int PER = TB >= 3 * 32 * RS ? 3 : 1;  // regions per ring slot
  static_assert(NW <= PER * (R > 2 ? 3 : 4), "the staging regions fit the ring");
  static_assert(TB >= 32 * RS, "a staging region fits a ring slot");
  const int ra = w / PER;
  uint16_t* const base = R > 2 ? (ra == 0 ? k0s : ra == 1 ? k1s : k2s)
                               : (ra == 0 ? k0s : ra == 1 ? k1s : ra == 2 ? v0s : v1s);
  uint16_t* const stage = base + (w % PER) * (32 * RS);
#pragma unroll
  for (int p = 0; p < D / 64; ++p) {
#pragma unroll
    for (int e2 = 0; e2 < 2; ++e2)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int e = 2 * p + e2;
        u32x2 o2;
        o2[0] = pack_bf16x2(oacc[e][4 * g + 0] * inv, oacc[e][4 * g + 1] * inv);
        o2[1] = pack_bf16x2(oacc[e][4 * g + 2] * inv, oacc[e][4 * g + 3] * inv);
        *reinterpret_cast<u32x2*>(stage + l32 * RS + 32 * e2 + 8 * g + 4 * hh) = o2;
      }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int r = 8 * k + (lane >> 3), c = lane & 7;
      const u32x4 v4 = *reinterpret_cast<const u32x4*>(stage + r * RS + 8 * c);
      if (wq0 + r < n) *reinterpret_cast<u32x4*>(O + head + (size_t)(wq0 + r) * D + 64 * p + 8 * c) = v4;
    }
  }
  if (qrow < n && hh == 0) LSE[(size_t)bh * n + qrow] = lse_v;
}

template <int D, int NW, bool CAUSAL, bool SPARSE, bool QK, bool DROP = false, bool WIN = false>
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
  static int hf_pass = -1, hf_fill = 0;  // start-up placement of the causal order
  if (hf_pass < 0) start_fill(fwd_bf16_kernel<D, NW, CAUSAL, SPARSE, QK, DROP, WIN>, NW * 64, hf_pass, hf_fill);
  // The forward takes the start-up placement only while most of its
  // workgroups start at once (at most three start-up fills per XCD): with
  // more, the rank-major order over all of an XCD's heads keeps too many keys
  // and values in flight and the grouped order is faster (B=8 H=32 N=2048
  // d=64 causal: 6%).
  const bool place = (long long)total <= 3LL * 8 * hf_fill;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, CAUSAL, SPARSE, QK, DROP, WIN>), dim3(total), dim3(NW * 64), 0, a.stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o, a.lse,
                     (int)a.n, nqb, total, c, qsign, a.bmask, (long long)a.mask_stride, nb, qa, a.drop, a.klen,
                     a.heads, a.window - 1, place ? hf_pass : 0, place ? hf_fill : 0);
  return hipGetLastError();
}

template <bool SPARSE, bool QK>
static hipError_t fwd_bf16_t(const FwdArgs& a) {
  if (a.d == 64)
    return a.causal ? launch_fwd<64, 4, true, SPARSE, QK>(a) : launch_fwd<64, 4, false, SPARSE, QK>(a);
  // d = 128, dense: eight waves (256 query rows) share each K/V tile, which
  // halves the fetch's LDS writes per query (3.3% faster at N = 4096; at
  // d = 64 eight waves are 6% slower).  Up to N = 2048 four-wave workgroups,
  // two per CU, overlap one another's start-up and epilogue, which weigh
  // more against short key loops (N = 1024 causal 8%, N = 2048 causal 2%
  // faster; from N = 4096 on eight waves are 1.5-2% faster).  Block-sparse
  // workgroups stay one 128-row mask block; unequal lengths keep four waves.
  if constexpr (!SPARSE && !QK) {
    if (a.n <= 2048)
      return a.causal ? launch_fwd<128, 4, true, false, false>(a) : launch_fwd<128, 4, false, false, false>(a);
    return a.causal ? launch_fwd<128, 8, true, false, false>(a) : launch_fwd<128, 8, false, false, false>(a);
  } else
    return a.causal ? launch_fwd<128, 4, true, SPARSE, QK>(a) : launch_fwd<128, 4, false, SPARSE, QK>(a);
}

hipError_t fwd_bf16(const FwdArgs& a) {
  if (a.window > 0) {  // causal sliding window, dense, square lengths
    if (a.d == 64) return launch_fwd<64, 4, true, false, false, false, true>(a);
    // A workgroup visits the union of its rows' windows (window + rows - 1
    // keys): up to 2048-key windows, 128-row workgroups waste less of it
    // than the 256-row ones save on fetches (N = 4096 and 16384: 20-27%
    // faster at windows of 128-512, equal to 9% faster at 1024-2048).
    if (a.window <= 2048) return launch_fwd<128, 4, true, false, false, false, true>(a);
    return launch_fwd<128, 8, true, false, false, false, true>(a);
  }
  if (a.dropout) {
    // Dense, square lengths only (checked by the caller).
    if (a.d == 64)
      return a.causal ? launch_fwd<64, 4, true, false, false, true>(a) : launch_fwd<64, 4, false, false, false, true>(a);
    return a.causal ? launch_fwd<128, 4, true, false, false, true>(a) : launch_fwd<128, 4, false, false, false, true>(a);
  }
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
