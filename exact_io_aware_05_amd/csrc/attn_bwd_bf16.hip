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
// Two kernels (plus a merge for the split dQ), none uses atomics
// (deterministic results):
//  * bwd_kv: a workgroup owns 128 keys and keeps K, V and the dK, dV
//    accumulators in registers while query tiles of 64 rows stream through
//    LDS; two waves share each 32-key group (one for S, P and dV, one for
//    dP, dS and dK).  S and dP use the C[q][key] layout (lane = key,
//    registers run over queries), so P and dS feed dV^T += dO^T P and
//    dK^T += Q^T dS straight from registers as the B operand, as bf16
//    values (hi + lo pairs on half tiles where a term's weight reaches
//    1/16).  dO^T and Q^T are read from the row-major tiles with transposing
//    LDS reads.
//  * bwd_q: a workgroup owns a block of queries (32 per wave) with Q, dO,
//    LSE and D in registers and streams key tiles of 64 rows: S^T = K Q^T and
//    dP^T = V dO^T (lane = query), dS^T, then dQ^T += K^T dS^T, with K^T
//    read transposed from the row-major K tile.  With unequal lengths and
//    few query blocks, the keys are split into chunks: each chunk's
//    workgroups write fp32 partial dQ, and dq_merge adds the chunks in a
//    fixed order (still deterministic).
// Tiles come from buffer->LDS DMA, into three buffers in bwd_kv (the tile
// after next streams in while the current one is used) and two in bwd_q;
// rows past the end of the head arrive as zeros.
#include <algorithm>
#include <type_traits>

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
//
// Per tile there are two barriers: one after P is published (mid-tile), one
// at the hand-over to the next tile.  Between them the S wave has its
// exponentials (before the mid-tile barrier) and the dP wave its dS products
// (after it); to keep the matrix cores busy through both, the dP wave defers
// the dK products of each tile to the first half of the next tile, where
// they run beside the S wave's exponentials.  That keeps a tile's Q one tile
// longer in LDS: Q and dO tiles are triple-buffered, and the DMA of tile
// i + 2 is issued once the mid-tile barrier of tile i has retired the reads
// of tile i - 1.
// ---------------------------------------------------------------------------
// Magnitude of a product term's weight from which P (in dV) and scale * dS
// (in dK) enter the products as hi + lo bf16 pairs (see bwd_kv_kernel).
constexpr float kSplitThreshold = 1.0f / 16.0f;

// Schedule hint for a block of M operand reads feeding M MFMAs: issue half of
// the reads up front, then alternate MFMA and read, so each read is in flight
// for several MFMAs before its result is needed.
template <int M>
__device__ __forceinline__ void pipeline_reads() {
  constexpr int AHEAD = M / 2;
  __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);
#pragma unroll
  for (int i = 0; i < M - AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
}

// Same, for MFMAs whose operand takes two reads; AHEAD MFMAs' operands are
// read before the first MFMA.
template <int M, int AHEAD = M / 2>
__device__ __forceinline__ void pipeline_reads2() {
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * AHEAD, 0);
#pragma unroll
  for (int i = 0; i < M - AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
}

template <int N>
using int_c = std::integral_constant<int, N>;

template <int D, bool CAUSAL, bool SPARSE, bool QK, bool DROP, bool WIN = false>
__global__ __launch_bounds__(512, 2) void bwd_kv_kernel(const uint16_t* __restrict__ Q,
                                                        const uint16_t* __restrict__ K,
                                                        const uint16_t* __restrict__ V,
                                                        const uint16_t* __restrict__ dO,
                                                        const float* __restrict__ LSE,
                                                        const float* __restrict__ Dsum,
                                                        uint16_t* __restrict__ dK, uint16_t* __restrict__ dV,
                                                        int n, int nkb, int total, float scale, float sl2e,
                                                        const uint8_t* __restrict__ bmask, long long mask_stride,
                                                        int nk_arg, int coff_arg, DropArgs dr,
                                                        const int* __restrict__ klen, int heads, int wl) {
  constexpr int NW = 8, BKV = 128, BQ = 64;
  constexpr int TB = BQ * D * 2;  // bytes per 64-row tile
  constexpr int IPW = (D / 8) / NW;  // DMA loads per wave per tile

  // LDS, carved by hand:
  //   [0, 2 KiB)     LSE (x log2 e) and D of up to three query tiles,
  //   Q tiles 0-2, then dO tiles 0-2 (64 rows x D bf16 each),
  //   P exchange     per key group and half tile, lane-major:
  //                  [group][t][r / 4][lane][r % 4] fp32,
  //   (block-sparse only) the list of query tiles to visit and its length.
  // Reads of the dO tiles go through readers shifted by 3 tiles, so that
  // every tile read uses an immediate offset below 64 KiB.
  constexpr int SMALL = 2048, GSHIFT = 3 * TB;
  constexpr int PXB = 4 * 2 * 4 * 64 * 4 * 4;  // P exchange bytes
  constexpr int LISTB = SPARSE ? kMaxSparseTiles * 4 + 16 : 0;  // block-sparse tile list
  __shared__ __attribute__((aligned(1024))) char smem[SMALL + 6 * TB + PXB + LISTB];
  auto lse_at = [&](auto b) ATTN_INLINE { return reinterpret_cast<float*>(smem + 512 * decltype(b)::value); };
  auto dsm_at = [&](auto b) ATTN_INLINE { return reinterpret_cast<float*>(smem + 512 * decltype(b)::value + 256); };
  auto q_at = [&](auto b) ATTN_INLINE {
    return reinterpret_cast<uint16_t*>(smem + SMALL + TB * decltype(b)::value);
  };
  auto g_at = [&](auto b) ATTN_INLINE {
    return reinterpret_cast<uint16_t*>(smem + SMALL + TB * (3 + decltype(b)::value));
  };
  float* const pxs = reinterpret_cast<float*>(smem + SMALL + 6 * TB);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int hh = lane >> 5, l32 = lane & 31;
  const int grp = w & 3;        // key group: keys 32*grp .. +31 of the block
  const bool s_role = w < 4;    // S wave (dV) or dP wave (dK)

  // Key blocks: under the causal mask (square lengths, no block mask or
  // dropout) a workgroup takes key block j and then its mirror nkb - 1 - j,
  // so every workgroup visits the same number of query tiles (block kb
  // visits ntq - 2 kb of them) and there are half as many workgroup
  // hand-overs; otherwise one block, low key blocks (the most queries under
  // the causal mask) first.
  constexpr bool PAIRED = CAUSAL && !SPARSE && !QK && !DROP && !WIN;
  const int lid = xcd_remap(blockIdx.x, total);
  const int nper = PAIRED ? (nkb + 1) / 2 : nkb;
  const int bh = lid / nper, kj = lid % nper;
#pragma unroll
  for (int rep = 0; rep < (PAIRED ? 2 : 1); ++rep) {
    const int kb = rep == 0 ? kj : nkb - 1 - kj;
    if (rep == 1) {
      if (kb == kj) break;
      // Every read of the first block's tiles and P exchange is done before
      // the second block's fetches refill the buffers.
      __syncthreads();
    }
    const int k0 = kb * BKV;
    const int kw0 = k0 + 32 * grp;
    const int key = kw0 + l32;
    // Unequal lengths (QK): n is the query length, nk the key length, and
    // query i sees key j when j <= i + coff (causal, bottom-right).
    const int nk = QK ? nk_arg : n;
    const int coff = (QK && CAUSAL) ? coff_arg : 0;

    const size_t head = (size_t)bh * (size_t)n * D;
    const size_t khead = (size_t)bh * (size_t)nk * D;
    // Key padding (square lengths): keys from nkv on are masked for every
    // query, so their dK and dV are zero; a block of padded keys only writes
    // those zeros.
    const int nkv = QK ? nk : padded_keys(klen, heads, bh, n);
    if (k0 >= nkv) {
      if (key < nk) {
        uint16_t* row = (s_role ? dV : dK) + khead + (size_t)key * D;
        const u32x2 z = {0u, 0u};
#pragma unroll
        for (int e = 0; e < D / 32; ++e)
#pragma unroll
          for (int g = 0; g < 4; ++g) *reinterpret_cast<u32x2*>(row + 32 * e + 8 * g + 4 * hh) = z;
      }
      continue;
    }
    const uint32_t head_bytes = (uint32_t)n * D * 2u;
    // Q and dO tiles are fetched through inline asm (dma_tile_asm): the
    // compiler would otherwise make LDS accesses of one buffer wait for the
    // fetch in flight into another; the waits it needs are explicit here.
    const RsrcWords rq = rsrc_words(Q + head, head_bytes);
    const RsrcWords rdo = rsrc_words(dO + head, head_bytes);
    const RsrcWords rl = rsrc_words(LSE + (size_t)bh * n, (uint32_t)n * 4u);
    const RsrcWords rd = rsrc_words(Dsum + (size_t)bh * n, (uint32_t)n * 4u);

    // B operands of S (K rows) for the S wave, of dP (V rows) for the dP wave.
    bf16x8 bf[D / 16];
    {
      const auto rkv = make_rsrc((s_role ? K : V) + khead, (uint32_t)nk * D * 2u);
#pragma unroll
      for (int s = 0; s < D / 16; ++s) bf[s] = as_bf16x8(bload16(rkv, (uint32_t)key * (D * 2) + 32 * s + 16 * hh));
      // Complete before any tile fetch is issued: a wait for these registers
      // inside the tile loop would also wait for the fetches in flight.
      wait_vmem();
    }

    f32x16 acc[D / 32];  // dV^T (S wave) or dK^T (dP wave)
#pragma unroll
    for (int e = 0; e < D / 32; ++e)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[e][r] = 0.f;

    // Query tiles it0 .. ntq - 1; under the sliding window (WIN: query i
    // sees keys i - wl .. i) they end with the window of the block's last key.
    const int ntq = WIN ? min((n + BQ - 1) / BQ, (k0 + BKV - 1 + wl) / BQ + 1) : (n + BQ - 1) / BQ;
    const int it0 = CAUSAL ? max(0, k0 - coff) / BQ : 0;
    // A tile whose queries all precede this key group, or (WIN) all lie past
    // its window, is skipped; both waves of a pair decide alike.
    auto active = [&](int i) ATTN_INLINE {
      return (!CAUSAL || (i * BQ + BQ - 1 >= kw0 - coff)) && (!WIN || i * BQ <= kw0 + 31 + wl);
    };

    // Block-sparse: the query tiles whose mask block (a 64-row tile is half of
    // a 128-row block) may attend this key block (a workgroup's 128 keys are
    // one mask block column), listed in LDS in increasing order.
    uint32_t* const tlist = reinterpret_cast<uint32_t*>(smem + SMALL + 6 * TB + PXB);
    int* const tcount = reinterpret_cast<int*>(tlist + kMaxSparseTiles);
    int tcnt = 0;
    if constexpr (SPARSE) {
      const uint8_t* mcol = bmask + (size_t)bh * mask_stride + kb;
      const int nbq = (n + kSparseBlock - 1) / kSparseBlock;
      tcnt = build_tile_list([&](int i) ATTN_INLINE { return mcol[(size_t)(i >> 1) * nbq] != 0; }, it0, ntq, tlist,
                             tcount, w, lane);
    }

    // Query rows past n load as zero (Q, dO, LSE, D), so they contribute
    // nothing: P = 1 is finite and multiplies dO = 0 and dS = 0.
    // A tile's batch of fetches: LSE and D rows (wave 0, one load each), then
    // the Q and dO tiles (2 * IPW loads per wave).  Every tile issues the same
    // batch (past the last tile: copies of the last one, never read), so the
    // counts below hold on every path.
    constexpr int SMALLN = 2;  // LSE and D loads of wave 0
    auto dma = [&](int i, auto b) ATTN_INLINE {
      if (w == 0) {
        const uint32_t off = __builtin_amdgcn_readfirstlane((uint32_t)i * (BQ * 4));
        const uint32_t sbase = (uint32_t)(uintptr_t)(ATTN_LDS char*)smem;
        dma_row64_asm(rl, sbase + 512u * decltype(b)::value, off, lane);
        dma_row64_asm(rd, sbase + 512u * decltype(b)::value + 256u, off, lane);
      }
      dma_tile_asm<D, NW>(rq, q_at(b), i * BQ, w, lane);
      dma_tile_asm<D, NW>(rdo, g_at(b), i * BQ, w, lane);
    };
    // Wave 0 scales the landed LSE row of buffer b to base 2 and negates the
    // D row, in place; the tiles fetched after them (LATER loads) may still be
    // in flight.
    auto fix_small = [&](auto b, auto later) ATTN_INLINE {
      if (w == 0) {
        wait_vmem_upto<decltype(later)::value>();
        asm volatile("" ::: "memory");
        lse_at(b)[lane] *= kLog2e;
        dsm_at(b)[lane] = -dsm_at(b)[lane];
      }
    };
    // End of a tile: the batch of the next tile must have landed; the batch
    // of the tile after it (issued last) stays in flight.
    auto handover = [&]() ATTN_INLINE {
      if (w == 0)
        wait_vmem_upto<SMALLN + 2 * IPW>();
      else
        wait_vmem_upto<2 * IPW>();
      barrier_lds();
    };

    float* px = pxs + grp * (2 * 4 * 64 * 4);

    // Dropout keep bits of this lane's key for queries qbase + 0..3 (bit k).
    // One generator call covers four consecutive keys of one query, so the
    // four lanes of a quad (keys 4a .. 4a + 3) call it for the four queries
    // and exchange words by a 4 x 4 transpose within the quad (DPP rotations).
    auto quad_keep = [&](int qbase) ATTN_INLINE -> uint32_t {
      const int tq = lane & 3;
      const u32x4 wd = philox4x32_10((uint32_t)(kw0 + (l32 & ~3)) >> 2, (uint32_t)(qbase + tq), (uint32_t)bh,
                                     dr.offset, dr.seed_lo, dr.seed_hi);
      // y[k] = word tq of quad lane k: query qbase + k, this lane's key.
      uint32_t y[4];
      auto pick = [&](int idx) ATTN_INLINE {
        return idx == 0 ? wd[0] : idx == 1 ? wd[1] : idx == 2 ? wd[2] : wd[3];
      };
#pragma unroll
      for (int k = 0; k < 4; ++k) y[k] = 0u;
      y[0] = tq == 0 ? wd[0] : y[0];
      y[1] = tq == 1 ? wd[1] : y[1];
      y[2] = tq == 2 ? wd[2] : y[2];
      y[3] = tq == 3 ? wd[3] : y[3];
      auto rot = [&](auto rc) ATTN_INLINE {
        constexpr int RT = decltype(rc)::value;
        // Lane s sends its word (s - RT) mod 4; lane r receives from lane
        // (r + RT) mod 4 its word r.
        const uint32_t x = pick((tq - RT) & 3);
        constexpr int ctrl = ((0 + RT) & 3) | (((1 + RT) & 3) << 2) | (((2 + RT) & 3) << 4) | (((3 + RT) & 3) << 6);
        const uint32_t r = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, ctrl, 0xF, 0xF, false);
        const int src = (tq + RT) & 3;
        y[0] = src == 0 ? r : y[0];
        y[1] = src == 1 ? r : y[1];
        y[2] = src == 2 ? r : y[2];
        y[3] = src == 3 ? r : y[3];
      };
      rot(int_c<1>{});
      rot(int_c<2>{});
      rot(int_c<3>{});
      uint32_t bits = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) bits |= (y[k] >= dr.thr ? 1u : 0u) << k;
      return bits;
    };

    // Products of P or dS for one half tile into dV or dK.  Where the half
    // tile holds a weight (P, or scale * dS) >= 1/16 the values enter as hi +
    // lo bf16 pairs (a
    // single bf16 rounding, relative 2^-9, of a probability near 1 can move a
    // column sum of magnitude > 4 by more than the output's own rounding
    // leaves); each term is one call, with packed operands h[u].
    auto acc_plain = [&](auto& tr, const uint16_t* bs, const bf16x8* h, int t) ATTN_INLINE {
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 a[2][D / 32];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < D / 32; ++e) a[u][e] = tr.cols(bs, 32 * t + 16 * u, e);
#pragma unroll
      for (int e = 0; e < D / 32; ++e) acc[e] = mfma32(a[0][e], h[0], acc[e]);
#pragma unroll
      for (int e = 0; e < D / 32; ++e) acc[e] = mfma32(a[1][e], h[1], acc[e]);
      pipeline_reads2<D / 16>();
      __builtin_amdgcn_sched_barrier(0);
    };
    // The products of both half tiles (operands h0 for queries 0-31, h1 for
    // 32-63) as one stream of 4 D / 16 MFMAs, so that operand reads run ahead
    // across the two halves instead of stalling at the start of each.
    auto acc_pair = [&](auto& tr, const uint16_t* bs, const bf16x8* h0, const bf16x8* h1) ATTN_INLINE {
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 a[4][D / 32];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int e = 0; e < D / 32; ++e) a[q][e] = tr.cols(bs, 16 * q, e);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x8& hq = q < 2 ? h0[q & 1] : h1[q & 1];
#pragma unroll
        for (int e = 0; e < D / 32; ++e) acc[e] = mfma32(a[q][e], hq, acc[e]);
      }
      pipeline_reads2<D / 8, 4>();
      __builtin_amdgcn_sched_barrier(0);
    };
    // Wave-uniform test for the split.  P enters dV as it is; dS enters dK
    // unscaled (the scale is applied to the accumulator at the end), so its
    // threshold is divided by |scale|: a term's rounding error in the output
    // is then bounded alike in both products.
    const float tau = s_role ? kSplitThreshold : kSplitThreshold / fabsf(scale);
    auto needs_split = [&](const float* vt) ATTN_INLINE {
      float vmax = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) vmax = fmaxf(vmax, fabsf(vt[r]));
      return __builtin_amdgcn_ballot_w64(vmax >= tau) != 0;
    };
    // Two independent MFMA chains (queries 0-31 and 32-63 of the tile) over
    // the row-major tile `src`, with this wave's key-side fragments.
    auto chains = [&](auto& tr, const uint16_t* src, f32x16& c0, f32x16& c1) ATTN_INLINE {
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 a0[D / 16], a1[D / 16];
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        a0[s] = tr.rows(src, 0, s);
        a1[s] = tr.rows(src, 32, s);
      }
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        c0 = mfma32(a0[s], bf[s], c0);
        c1 = mfma32(a1[s], bf[s], c1);
      }
      pipeline_reads<D / 8>();
      __builtin_amdgcn_sched_barrier(0);
    };

    // Tile loop skeleton shared by both roles (same barriers in both): tile i
    // lives in buffer b = (i - it0) mod 3.  body(b, i, mid) does the role's
    // work on tile i and calls mid() exactly once, between its two halves.
    auto run_dense = [&](auto&& body) ATTN_INLINE {
      auto step = [&](auto b, int i) ATTN_INLINE {
        constexpr int B = decltype(b)::value;
        body(b, i, [&]() ATTN_INLINE {
          fix_small(int_c<(B + 1) % 3>{}, int_c<2 * IPW>{});  // LSE of tile i + 1
          barrier_lds();  // P of tile i is published; reads of tile i - 1 are done
          dma(min(i + 2, ntq - 1), int_c<(B + 2) % 3>{});
        });
        handover();
      };
      dma(it0, int_c<0>{});
      dma(min(it0 + 1, ntq - 1), int_c<1>{});
      fix_small(int_c<0>{}, int_c<SMALLN + 4 * IPW>{});
      handover();
      for (int it = it0; it < ntq; it += 3) {
        step(int_c<0>{}, it);
        if (it + 1 >= ntq) break;
        step(int_c<1>{}, it + 1);
        if (it + 2 >= ntq) break;
        step(int_c<2>{}, it + 2);
      }
    };
    // The same sequence over the listed tiles: position p holds tile T(p) in
    // buffer p mod 3.
    auto run_list = [&](auto&& body) ATTN_INLINE {
      auto T = [&](int p) ATTN_INLINE { return __builtin_amdgcn_readfirstlane((int)tlist[p]); };
      auto step = [&](auto b, int p) ATTN_INLINE {
        constexpr int B = decltype(b)::value;
        body(b, T(p), [&]() ATTN_INLINE {
          fix_small(int_c<(B + 1) % 3>{}, int_c<2 * IPW>{});  // LSE of the next tile
          barrier_lds();  // P of this tile is published; reads of the previous one are done
          dma(T(min(p + 2, tcnt - 1)), int_c<(B + 2) % 3>{});
        });
        handover();
      };
      if (tcnt == 0) return;
      dma(T(0), int_c<0>{});
      dma(T(min(1, tcnt - 1)), int_c<1>{});
      fix_small(int_c<0>{}, int_c<SMALLN + 4 * IPW>{});
      handover();
      for (int p = 0; p < tcnt; p += 3) {
        step(int_c<0>{}, p);
        if (p + 1 >= tcnt) break;
        step(int_c<1>{}, p + 1);
        if (p + 2 >= tcnt) break;
        step(int_c<2>{}, p + 2);
      }
    };
    auto run = [&](auto&& body) ATTN_INLINE {
      if constexpr (SPARSE)
        run_list(body);
      else
        run_dense(body);
      wait_vmem();  // no fetch outlives the loop
    };

    if (s_role) {
      // S wave: S = Q K^T, P = exp(S - LSE) published through LDS, then
      // dV^T += dO^T P.
      const TileReader<D, 0, GSHIFT> TR(lane);
      run([&](auto b, int i, auto&& mid) ATTN_INLINE {
        const bool act = active(i);
        float v[2][16];
        if (act) {
          const float* lse2s = lse_at(b);
          f32x16 c0, c1;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            c0[r] = 0.f;
            c1[r] = 0.f;
          }
          chains(TR, q_at(b), c0, c1);
          // Exponent arguments; on the diagonal tiles only (a wave-uniform
          // branch), entries whose key follows the query become -inf, whose
          // exp2 is 0.  Written as selects inside the exponential loop, the
          // mask ran on every tile.
          float x[2][16];
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lse2s[32 * t + 8 * g + 4 * hh]);
#pragma unroll
              for (int k = 0; k < 4; ++k) x[t][4 * g + k] = fmaf(t == 0 ? c0[4 * g + k] : c1[4 * g + k], sl2e, -l4[k]);
            }
          if (CAUSAL && i * BQ < kw0 + 31 - coff) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int q = i * BQ + 32 * t + crow(r, hh);
                x[t][r] = key > q + coff ? -INFINITY : x[t][r];
              }
          }
          if (WIN && i * BQ + BQ - 1 > kw0 + wl) {  // the window's far edge crosses the tile
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int q = i * BQ + 32 * t + crow(r, hh);
                x[t][r] = q > key + wl ? -INFINITY : x[t][r];
              }
          }
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int qbase = i * BQ + 32 * t + 8 * g + 4 * hh;  // queries qbase + k of registers 4g + k
              uint32_t keep = 0xFu;
              if constexpr (DROP) keep = quad_keep(qbase);
              f32x4 o;
#pragma unroll
              for (int k = 0; k < 4; ++k) {
                const float pv = fast_exp2(x[t][4 * g + k]);
                if constexpr (DROP) {
                  // dV takes the dropped, rescaled probability; the dP wave
                  // gets P with the keep bit in the sign (P >= 0).
                  const bool kept = (keep >> k) & 1u;
                  v[t][4 * g + k] = kept ? pv * dr.keep_scale : 0.f;
                  o[k] = kept ? pv : -pv;
                } else {
                  v[t][4 * g + k] = pv;
                  o[k] = pv;
                }
              }
              *reinterpret_cast<f32x4*>(&px[((t * 4 + g) * 64 + lane) * 4]) = o;
            }
        }
        mid();
        if (act) {
          // hi terms always (both halves as one stream), lo terms only where
          // the half tile needs them: the accumulators are only ever updated in
          // place (no alternative paths that the register allocator would join
          // with copies).
          const bf16x8 h0[2] = {pack_bf16x8(v[0]), pack_bf16x8(v[0] + 8)};
          const bf16x8 h1[2] = {pack_bf16x8(v[1]), pack_bf16x8(v[1] + 8)};
          const bool sp0 = needs_split(v[0]), sp1 = needs_split(v[1]);
          acc_pair(TR, g_at(b), h0, h1);
          if (sp0) {
            const bf16x8 l[2] = {split_lo_bf16x8(v[0], h0[0]), split_lo_bf16x8(v[0] + 8, h0[1])};
            acc_plain(TR, g_at(b), l, 0);
          }
          if (sp1) {
            const bf16x8 l[2] = {split_lo_bf16x8(v[1], h1[0]), split_lo_bf16x8(v[1] + 8, h1[1])};
            acc_plain(TR, g_at(b), l, 1);
          }
        }
      });
    } else {
      // dP wave: dP = dO V^T accumulated onto -D (registers run over queries),
      // so it ends with dP - D; after P arrives, dS = P * (dP - D).  The dK^T
      // += Q^T dS products of each half tile are deferred to the next tile's
      // first half, with dS kept packed in registers (hi and, where the half
      // tile needs the split, lo bf16 terms).
      const TileReader<D, GSHIFT, 0> TR(lane);
      bf16x8 dhi[2][2], dlo[2][2];
      bool pend = false, spl0 = false, spl1 = false;
      auto deferred = [&](const uint16_t* qs) ATTN_INLINE {
        acc_pair(TR, qs, dhi[0], dhi[1]);
        if (spl0) acc_plain(TR, qs, dlo[0], 0);
        if (spl1) acc_plain(TR, qs, dlo[1], 1);
      };
      run([&](auto b, int i, auto&& mid) ATTN_INLINE {
        constexpr int BP = (decltype(b)::value + 2) % 3;  // buffer of the previous tile
        const bool act = active(i);
        // The accumulators start from -D (with dropout from 0: dP is needed
        // alone, dS = P (Z dP / (1 - p) - D)).  The -D rows are read before
        // the deferred products, which hide the LDS latency; read just before
        // the chains, the first product waited for them.
        f32x16 c0, c1;
        {
          const float* dsms = dsm_at(b);
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 d0 = *reinterpret_cast<const f32x4*>(&dsms[8 * g + 4 * hh]);
            const f32x4 d1 = *reinterpret_cast<const f32x4*>(&dsms[32 + 8 * g + 4 * hh]);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              c0[4 * g + k] = DROP ? 0.f : d0[k];
              c1[4 * g + k] = DROP ? 0.f : d1[k];
            }
          }
        }
        if (pend) deferred(q_at(int_c<BP>{}));
        if (act) chains(TR, g_at(b), c0, c1);
        mid();
        pend = act;
        if (act) {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            float v[16];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const f32x4 p4 = *reinterpret_cast<const f32x4*>(&px[((t * 4 + g) * 64 + lane) * 4]);
              if constexpr (DROP) {
                const f32x4 d4 = *reinterpret_cast<const f32x4*>(&dsm_at(b)[32 * t + 8 * g + 4 * hh]);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                  const float dpv = t == 0 ? c0[4 * g + k] : c1[4 * g + k];
                  const bool kept = (__float_as_uint(p4[k]) >> 31) == 0u;
                  v[4 * g + k] = fabsf(p4[k]) * ((kept ? dpv * dr.keep_scale : 0.f) + d4[k]);  // d4 = -D
                }
              } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) v[4 * g + k] = (t == 0 ? c0[4 * g + k] : c1[4 * g + k]) * p4[k];
              }
            }
            const bool sp = needs_split(v);
            (t == 0 ? spl0 : spl1) = sp;
            dhi[t][0] = pack_bf16x8(v);
            dhi[t][1] = pack_bf16x8(v + 8);
            if (sp) {
              dlo[t][0] = split_lo_bf16x8(v, dhi[t][0]);
              dlo[t][1] = split_lo_bf16x8(v + 8, dhi[t][1]);
            }
          }
        }
      });
      // Deferred products of the last tile (no DMA is in flight any more).
      if (pend) {
        const int bl = (SPARSE ? tcnt - 1 : ntq - 1 - it0) % 3;
        deferred(bl == 0 ? q_at(int_c<0>{}) : bl == 1 ? q_at(int_c<1>{}) : q_at(int_c<2>{}));
      }
    }

    const float f = s_role ? 1.0f : scale;
    const bool live = key < nkv;  // a padded key of a partly padded block: zero
    uint16_t* const out = s_role ? dV : dK;
    if constexpr (D == 128) {
      // dK and dV leave through LDS so that every store writes whole 128-byte
      // row segments: each wave stages its 32 keys, 64 features at a time, in
      // its own 4.5 KiB of the Q tile buffers (rows 144 bytes apart), once
      // every wave is done with the tiles.
      __syncthreads();
      constexpr int RS = 72;  // row stride in bf16 elements
      uint16_t* const stage = reinterpret_cast<uint16_t*>(smem + SMALL) + w * (32 * RS);
#pragma unroll
      for (int p = 0; p < 2; ++p) {
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int e = 2 * p + e2;
            u32x2 o2;
            o2[0] = pack_bf16x2(acc[e][4 * g + 0] * f, acc[e][4 * g + 1] * f);
            o2[1] = pack_bf16x2(acc[e][4 * g + 2] * f, acc[e][4 * g + 3] * f);
            if (!live) o2[0] = o2[1] = 0u;
            *reinterpret_cast<u32x2*>(stage + l32 * RS + 32 * e2 + 8 * g + 4 * hh) = o2;
          }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int r = 8 * k + (lane >> 3), c = lane & 7;
          const u32x4 v4 = *reinterpret_cast<const u32x4*>(stage + r * RS + 8 * c);
          if (kw0 + r < nk) *reinterpret_cast<u32x4*>(out + khead + (size_t)(kw0 + r) * D + 64 * p + 8 * c) = v4;
        }
      }
    } else if (key < nk) {
      uint16_t* row = out + khead + (size_t)key * D;
#pragma unroll
      for (int e = 0; e < D / 32; ++e)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 o2;
          o2[0] = pack_bf16x2(acc[e][4 * g + 0] * f, acc[e][4 * g + 1] * f);
          o2[1] = pack_bf16x2(acc[e][4 * g + 2] * f, acc[e][4 * g + 3] * f);
          if (!live) o2[0] = o2[1] = 0u;
          *reinterpret_cast<u32x2*>(row + 32 * e + 8 * g + 4 * hh) = o2;
        }
    }
  }
}

// ---------------------------------------------------------------------------
// dQ: query-stationary
// ---------------------------------------------------------------------------
template <int D, int NW, bool CAUSAL, bool SPARSE, bool QK, bool DROP, bool WIN = false>
__global__ __launch_bounds__(NW * 64, 2) void bwd_q_kernel(const uint16_t* __restrict__ Q,
                                                           const uint16_t* __restrict__ K,
                                                           const uint16_t* __restrict__ V,
                                                           const uint16_t* __restrict__ dO,
                                                           const float* __restrict__ LSE,
                                                           const float* __restrict__ Dsum,
                                                           uint16_t* __restrict__ dQ, int n, int nqb, int total,
                                                           float scale, float sl2e,
                                                           const uint8_t* __restrict__ bmask, long long mask_stride,
                                                           int nb, int nk_arg, int coff_arg, DropArgs dr,
                                                           int kchunk, float* __restrict__ dqpart,
                                                           const uint16_t* __restrict__ Osrc,
                                                           float* __restrict__ Dout,
                                                           const int* __restrict__ klen, int heads, int wl,
                                                           int hf_pass, int hf_fill) {
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

  // Unequal lengths, split over keys: the grid holds one copy of the
  // (head, query block) items per chunk of kchunk keys.
  const bool split = QK && dqpart != nullptr;
  int bid = blockIdx.x, ks = 0;
  if (split) {
    ks = bid / total;
    bid -= ks * total;
  }
  // Under the causal mask heavy (late) query blocks first, longest first
  // within each XCD.
  int bh, qi;
  if (CAUSAL) {
    heavy_first(bid, total / nqb, nqb, bh, qi, hf_pass, hf_fill);
  } else {
    const int lid = xcd_remap(bid, total);
    bh = lid / nqb;
    qi = lid % nqb;
  }
  const int qb = CAUSAL ? (nqb - 1 - qi) : qi;
  const int q0 = qb * BR;
  const int wq0 = q0 + 32 * w;
  const int qrow = wq0 + l32;

  // Unequal lengths (QK): n is the query length, nk the key length, and
  // query i sees key j when j <= i + coff (causal, bottom-right).  A chunk
  // of the split is the same problem on keys kb .. kb + nk - 1: K and V start
  // kb rows later and the causal offset drops by kb (rows that see no key of
  // the chunk get a zero partial).
  // Key padding (square lengths): keys from padded_keys(..) on are masked
  // like keys past the end.
  const int kb = split ? ks * kchunk : 0;
  const int nk = QK ? (split ? min(kchunk, nk_arg - kb) : nk_arg) : padded_keys(klen, heads, bh, n);
  const int coff = (QK && CAUSAL) ? coff_arg - kb : 0;
  const size_t head = (size_t)bh * (size_t)n * D;
  const size_t khead = (size_t)bh * (size_t)(QK ? nk_arg : n) * D + (size_t)kb * D;
  const uint32_t head_bytes = (uint32_t)n * D * 2u;
  const auto rq = make_rsrc(Q + head, head_bytes);
  const auto rdo = make_rsrc(dO + head, head_bytes);
  const auto rk = make_rsrc(K + khead, (uint32_t)nk * D * 2u);
  const auto rv = make_rsrc(V + khead, (uint32_t)nk * D * 2u);

  bf16x8 qf[D / 16], gf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    qf[s] = as_bf16x8(bload16(rq, (uint32_t)qrow * (D * 2) + 32 * s + 16 * hh));
    gf[s] = as_bf16x8(bload16(rdo, (uint32_t)qrow * (D * 2) + 32 * s + 16 * hh));
  }
  const float l2 = qrow < n ? LSE[(size_t)bh * n + qrow] * kLog2e : 0.f;
  // D_i = dO_i . O_i: read from Dsum, or (Osrc given) formed here from the
  // row's O, whose fragments are loaded like dO's (this lane: half hh of the
  // row's features), summed over the two lane halves, and written to Dout
  // for the key-stationary pass, which then runs after this one.  Rows past
  // n load as zero.
  float dq_d;
  if (Osrc != nullptr) {
    const auto ro = make_rsrc(Osrc + head, head_bytes);
    float part = 0.f;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const u32x4 ov = bload16(ro, (uint32_t)qrow * (D * 2) + 32 * s + 16 * hh);
      const u32x4 gv = __builtin_bit_cast(u32x4, gf[s]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        part = fmaf(__uint_as_float(ov[i] << 16), __uint_as_float(gv[i] << 16), part);
        part = fmaf(__uint_as_float(ov[i] & 0xFFFF0000u), __uint_as_float(gv[i] & 0xFFFF0000u), part);
      }
    }
    dq_d = half_sum(part);
    if (hh == 0 && qrow < n) Dout[(size_t)bh * n + qrow] = dq_d;
  } else {
    dq_d = qrow < n ? Dsum[(size_t)bh * n + qrow] : 0.f;
  }

  f32x16 dqa[D / 32];
#pragma unroll
  for (int e = 0; e < D / 32; ++e)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqa[e][r] = 0.f;

  const int kend = CAUSAL ? min(nk, q0 + BR + coff) : nk;
  const int ntiles = kend > 0 ? (kend + BC - 1) / BC : 0;

  // TAIL: the tile may need masking (keys past nk, or under causal keys
  // after some row of the wave) or be skipped by some wave; calls without it
  // are for tiles every key of which every row of the workgroup sees.
  auto compute = [&](const uint16_t* ks, const uint16_t* vs, int j0, auto tail) ATTN_INLINE {
    constexpr bool TAIL = decltype(tail)::value;
    // (WIN: sliding window, query i sees keys i - wl .. i.)
    const bool active = !TAIL || ((!CAUSAL || j0 <= wq0 + 31 + coff) && (!WIN || j0 + BC - 1 >= wq0 - wl));
    if (!active) return;
    const bool need_mask =
        TAIL && ((j0 + BC > nk) || (CAUSAL && j0 + BC - 1 > wq0 + coff) || (WIN && j0 < wq0 + 31 - wl));
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      // One half tile at a time: interleaving the halves costs more
      // registers than the file holds at two waves per SIMD.
      __builtin_amdgcn_sched_barrier(0);
      // Dropout: bit r kept (keys j0 + 32t + 8g + 4hh + 0..3 are one call).
      uint32_t keep = 0xFFFFu;
      if constexpr (DROP) {
        keep = 0u;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x4 wd = philox4x32_10((uint32_t)(j0 + 32 * t + 8 * g + 4 * hh) >> 2, (uint32_t)qrow, (uint32_t)bh,
                                         dr.offset, dr.seed_lo, dr.seed_hi);
#pragma unroll
          for (int i = 0; i < 4; ++i) keep |= (wd[i] >= dr.thr ? 1u : 0u) << (4 * g + i);
        }
      }
      // dP accumulates onto -D (it ends as dP - D), except with dropout,
      // where dP itself is needed (dS = P (Z dP / (1 - p) - D)).
      f32x16 sacc, pacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sacc[r] = 0.f;
        pacc[r] = DROP ? 0.f : -dq_d;
      }
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        sacc = mfma32(TR.rows(ks, 32 * t, s), qf[s], sacc);
        pacc = mfma32(TR.rows(vs, 32 * t, s), gf[s], pacc);
      }

      // dP - D of register r.
      auto dpd_of = [&](int r) ATTN_INLINE {
        if constexpr (DROP)
          return ((keep >> r) & 1u ? pacc[r] * dr.keep_scale : 0.f) - dq_d;
        else
          return pacc[r];
      };
      float ds[16];
      if constexpr (CAUSAL || DROP) {
        // Exponent arguments; masked entries (diagonal and ragged tiles
        // only, a wave-uniform branch) become -inf, whose exp2 is 0.  Keys
        // past n lie above the diagonal of every row that is written.
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = fmaf(sacc[r], sl2e, -l2);
        if (need_mask) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kj = j0 + 32 * t + crow(r, hh);
            x[r] = (kj >= nk || (CAUSAL && kj > qrow + coff) || (WIN && kj < qrow - wl)) ? -INFINITY : x[r];
          }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) ds[r] = fast_exp2(x[r]) * dpd_of(r);
      } else {
        // Full mask: only keys past nk (in the last tile) are masked, as
        // selects, in the calls that may hold them.
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pv = fast_exp2(fmaf(sacc[r], sl2e, -l2));
          if (need_mask) pv = (j0 + 32 * t + crow(r, hh) >= nk) ? 0.f : pv;
          ds[r] = pv * dpd_of(r);
        }
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

  if constexpr (SPARSE) {
    // Key tiles that some query block of this workgroup may attend (BR / 128
    // mask block rows; a 64-key tile is half of a mask block), listed in LDS
    // in increasing order as (tile << 2) | (bit r: block row r wants it).  A
    // wave computes a listed tile only if its own block row wants it (its 32
    // rows lie in one block row).
    constexpr int QBLK = BR / kSparseBlock;
    static_assert(QBLK * kSparseBlock == BR && QBLK <= 2, "workgroups cover one or two mask block rows");
    __shared__ uint32_t tlist[kMaxSparseTiles];
    __shared__ int tcount;
    const uint8_t* mrow = bmask + (size_t)bh * mask_stride + (size_t)(q0 / kSparseBlock) * nb;
    const int nrows = min(QBLK, nb - q0 / kSparseBlock);
    const int qsub = (wq0 - q0) / kSparseBlock;
    // Tile indices here are below 2^11 (the list's capacity), so the row
    // bits fit below them.
    const int cnt = build_tile_list(
        [&](int j) ATTN_INLINE {
          bool any = false;
          for (int r = 0; r < nrows; ++r) any = any || mrow[(size_t)r * nb + (j >> 1)] != 0;
          return any;
        },
        0, ntiles, tlist, &tcount, w, lane);
    if (w == 0) {
      for (int p = lane; p < cnt; p += 64) {
        const uint32_t j = tlist[p];
        uint32_t bits = 0;
        for (int r = 0; r < nrows; ++r) bits |= (mrow[(size_t)r * nb + (j >> 1)] != 0 ? 1u : 0u) << r;
        tlist[p] = (j << 2) | bits;
      }
    }
    __syncthreads();
    auto tile = [&](int p) ATTN_INLINE { return __builtin_amdgcn_readfirstlane((int)tlist[p]); };
    auto run_tile = [&](const uint16_t* ks, const uint16_t* vs, int e) ATTN_INLINE {
      if ((e >> qsub) & 1) compute(ks, vs, (e >> 2) * BC, std::true_type{});
    };
    if (cnt > 0) {
      dma_tile<D, NW>(rk, k0s, (tile(0) >> 2) * BC, w, lane);
      dma_tile<D, NW>(rv, v0s, (tile(0) >> 2) * BC, w, lane);
      wait_vmem();
      __syncthreads();
    }
    for (int p = 0; p < cnt; p += 2) {
      if (p + 1 < cnt) {
        dma_tile<D, NW>(rk, k1s, (tile(p + 1) >> 2) * BC, w, lane);
        dma_tile<D, NW>(rv, v1s, (tile(p + 1) >> 2) * BC, w, lane);
      }
      run_tile(k0s, v0s, tile(p));
      wait_vmem();
      __syncthreads();
      if (p + 1 >= cnt) break;
      if (p + 2 < cnt) {
        dma_tile<D, NW>(rk, k0s, (tile(p + 2) >> 2) * BC, w, lane);
        dma_tile<D, NW>(rv, v0s, (tile(p + 2) >> 2) * BC, w, lane);
      }
      run_tile(k1s, v1s, tile(p + 1));
      wait_vmem();
      __syncthreads();
    }
  } else if (ntiles > 0) {
    // Tiles 0 .. nfree - 1 need no mask and no skip (full mask: all but the
    // last tile, the only one that can hold keys past nk; causal: the tiles
    // whose keys all precede the workgroup's first row).  They run in pairs
    // (buffer 0, buffer 1), each pair fetching the next two, with no exit
    // inside the pair: a loop that could leave between its two halves made
    // the register allocator copy the dQ accumulators on every tile.  The
    // remaining tiles (the last one, or the diagonal ones) follow in a loop
    // with the checks.
    // (Under key padding a causal tile before the first row can still hold
    // padded keys: free tiles also lie wholly below nk.)
    // Under the sliding window the tiles start at the window of the first
    // row, jlo, and every tile takes the checked path.
    const int jlo = WIN ? max(0, q0 - wl) / BC : 0;
    const int nfree =
        WIN ? jlo : (CAUSAL ? min(min(ntiles, nk / BC), max(0, (q0 + coff + 1) / BC)) : ntiles - 1);
    auto fetch = [&](uint16_t* ks, uint16_t* vs, int jt) ATTN_INLINE {
      dma_tile<D, NW>(rk, ks, jt * BC, w, lane);
      dma_tile<D, NW>(rv, vs, jt * BC, w, lane);
    };
    auto settle = [&]() ATTN_INLINE {
      wait_vmem();
      __syncthreads();
    };
    fetch(k0s, v0s, jlo);
    settle();
    int jt = jlo;
    for (; jt + 1 < nfree && jt + 2 < ntiles; jt += 2) {
      fetch(k1s, v1s, jt + 1);
      compute(k0s, v0s, jt * BC, std::false_type{});
      settle();
      fetch(k0s, v0s, jt + 2);
      compute(k1s, v1s, (jt + 1) * BC, std::false_type{});
      settle();
    }
    // Tile jt is in buffer 0.
    if constexpr (CAUSAL) {
      for (; jt < ntiles; jt += 2) {
        if (jt + 1 < ntiles) fetch(k1s, v1s, jt + 1);
        compute(k0s, v0s, jt * BC, std::true_type{});
        if (jt + 1 >= ntiles) break;
        settle();
        if (jt + 2 < ntiles) fetch(k0s, v0s, jt + 2);
        compute(k1s, v1s, (jt + 1) * BC, std::true_type{});
        settle();
      }
    } else if (jt + 1 < ntiles) {  // tiles last - 1 (buffer 0) and last
      fetch(k1s, v1s, jt + 1);
      compute(k0s, v0s, jt * BC, std::false_type{});
      settle();
      compute(k1s, v1s, (jt + 1) * BC, std::true_type{});
    } else {  // the last tile, in buffer 0
      compute(k0s, v0s, jt * BC, std::true_type{});
    }
  }

  if (split && qrow < n) {
    float* prow = dqpart + ((size_t)ks * (size_t)(total / nqb) * (size_t)n * D) + head + (size_t)qrow * D;
#pragma unroll
    for (int e = 0; e < D / 32; ++e)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 o4;
#pragma unroll
        for (int i = 0; i < 4; ++i) o4[i] = dqa[e][4 * g + i] * scale;
        *reinterpret_cast<f32x4*>(prow + 32 * e + 8 * g + 4 * hh) = o4;
      }
  } else if (!split) {
    // dQ leaves through LDS so that every store writes whole 128-byte row
    // segments (as the forward's O): each wave stages its 32 rows, 64
    // features at a time, in a region of the tile buffers (rows 144 bytes
    // apart; three regions per buffer at d = 128, one at d = 64), once every
    // wave is done with the tiles.
    __syncthreads();
    constexpr int RS = 72;                                // row stride in bf16 elements
    constexpr int PER = BC * D >= 3 * 32 * RS ? 3 : 1;  // regions per tile buffer
    static_assert(NW <= 4 * PER, "the staging regions fit the tile buffers");
    static_assert(BC * D >= 32 * RS, "a staging region fits a tile buffer");
    const int ra = w / PER;
    uint16_t* const stage = (ra == 0 ? k0s : ra == 1 ? v0s : ra == 2 ? k1s : v1s) + (w % PER) * (32 * RS);
#pragma unroll
    for (int p = 0; p < D / 64; ++p) {
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int e = 2 * p + e2;
          u32x2 o2;
          o2[0] = pack_bf16x2(dqa[e][4 * g + 0] * scale, dqa[e][4 * g + 1] * scale);
          o2[1] = pack_bf16x2(dqa[e][4 * g + 2] * scale, dqa[e][4 * g + 3] * scale);
          *reinterpret_cast<u32x2*>(stage + l32 * RS + 32 * e2 + 8 * g + 4 * hh) = o2;
        }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int r = 8 * k + (lane >> 3), c = lane & 7;
        const u32x4 v4 = *reinterpret_cast<const u32x4*>(stage + r * RS + 8 * c);
        if (wq0 + r < n) *reinterpret_cast<u32x4*>(dQ + head + (size_t)(wq0 + r) * D + 64 * p + 8 * c) = v4;
      }
    }
  } else if (qrow < n) {
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

// Sum of the split dQ partials, chunk 0 first (a fixed order: the result does
// not depend on scheduling), rounded once to bf16 (nearest-even).  Four
// consecutive features per thread; the partials of chunk s start s * n4
// vectors after those of chunk 0.
__global__ __launch_bounds__(256) void dq_merge_kernel(const f32x4* __restrict__ part, uint16_t* __restrict__ dq,
                                                       long long n4, int nsplit) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n4; i += (long long)gridDim.x * 256) {
    f32x4 acc = part[i];
    for (int s = 1; s < nsplit; ++s) {
      const f32x4 v = part[i + (long long)s * n4];
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] += v[c];
    }
    u32x2 o2;
    o2[0] = pack_bf16x2(acc[0], acc[1]);
    o2[1] = pack_bf16x2(acc[2], acc[3]);
    *reinterpret_cast<u32x2*>(dq + 4 * i) = o2;
  }
}

template <int D, bool CAUSAL, bool SPARSE, bool QK, bool DROP = false, bool WIN = false>
hipError_t launch_dkdv(const BwdArgs& a) {
  const int n = (int)a.n;
  const int nk = QK ? (int)a.nk : n;
  const int nkb = (nk + 127) / 128;
  // Causal, square, dense, no dropout: one workgroup per pair of mirrored
  // key blocks (see bwd_kv_kernel).
  constexpr bool PAIRED = CAUSAL && !SPARSE && !QK && !DROP && !WIN;
  const int total = (int)(a.bh * (PAIRED ? (nkb + 1) / 2 : nkb));
  hipLaunchKernelGGL((bwd_kv_kernel<D, CAUSAL, SPARSE, QK, DROP, WIN>), dim3(total), dim3(512), 0, a.stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dout,
                     a.lse, a.dsum, (uint16_t*)a.dk, (uint16_t*)a.dv, n, nkb, total, a.scale, a.scale * kLog2e,
                     a.bmask, (long long)a.mask_stride, nk, nk - n, a.drop, a.klen, a.heads, a.window - 1);
  return hipGetLastError();
}

#ifndef ATTN_DQ_NW128
#define ATTN_DQ_NW128 8  // waves per dQ workgroup at d = 128 (tuning knob)
#endif

template <int D, int NW, bool CAUSAL, bool SPARSE, bool QK, bool DROP = false, bool WIN = false>
hipError_t launch_dq_nw(const BwdArgs& a) {
  const int n = (int)a.n;
  const int nqb = (n + NW * 32 - 1) / (NW * 32);
  const int total = (int)(a.bh * nqb);
  const int nb = (n + kSparseBlock - 1) / kSparseBlock;
  const int nk = QK ? (int)a.nk : n;
  const bool split = QK && a.nsplit > 1;
  const bool form_d = a.dq_forms_dsum && !split;
  static int hf_pass = -1, hf_fill = 0;  // start-up placement of the causal order
  if (hf_pass < 0) start_fill(bwd_q_kernel<D, NW, CAUSAL, SPARSE, QK, DROP, WIN>, NW * 64, hf_pass, hf_fill);
  hipLaunchKernelGGL((bwd_q_kernel<D, NW, CAUSAL, SPARSE, QK, DROP, WIN>), dim3(total * (split ? a.nsplit : 1)),
                     dim3(NW * 64), 0, a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (const uint16_t*)a.dout, a.lse, form_d ? nullptr : a.dsum, (uint16_t*)a.dq, n, nqb, total,
                     a.scale,
                     a.scale * kLog2e, a.bmask, (long long)a.mask_stride, nb, nk, nk - n, a.drop,
                     split ? a.kchunk : 0, split ? a.dqpart : nullptr,
                     form_d ? (const uint16_t*)a.o : nullptr, form_d ? a.dsum : nullptr, a.klen, a.heads,
                     a.window - 1, split ? 0 : hf_pass, split ? 0 : hf_fill);
  if (!split) return hipGetLastError();
  const long long n4 = a.bh * a.n * (long long)D / 4;
  const long long blocks = std::min<long long>((n4 + 255) / 256, 4096);
  hipLaunchKernelGGL(dq_merge_kernel, dim3((unsigned)blocks), dim3(256), 0, a.stream, (const f32x4*)a.dqpart,
                     (uint16_t*)a.dq, n4, a.nsplit);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool SPARSE, bool QK, bool DROP = false, bool WIN = false>
hipError_t launch_dq(const BwdArgs& a) {
  // Block-sparse: one mask block row per workgroup (4 waves), so that every
  // wave of a workgroup wants every tile the workgroup fetches.  Sliding
  // window: 4 waves too (the workgroup visits the union of its rows'
  // windows; at N = 16384, windows of 128-2048 keys, the backward runs 2-7%
  // faster than with 8).
  constexpr int NW = (D == 128 && !SPARSE && !WIN) ? ATTN_DQ_NW128 : 4;
  // Square lengths up to N = 2048 at d = 128: four waves, two workgroups per
  // CU overlapping one another's start-up and epilogue against short key
  // loops (N = 1024: 3-5% faster at full mask, 10-12% causal; N = 2048:
  // 2-4%); from N = 8192 on eight waves are 2-3% faster.  The arithmetic of
  // a row does not depend on the wave count.  (Dropout keeps eight: its
  // four-wave form would spill registers.)
  if constexpr (NW == 8 && !QK && !DROP) {
    if (a.n <= 2048) return launch_dq_nw<D, 4, CAUSAL, SPARSE, QK, DROP, WIN>(a);
  }
  return launch_dq_nw<D, NW, CAUSAL, SPARSE, QK, DROP, WIN>(a);
}

template <bool SPARSE, bool QK>
hipError_t dkdv_t(const BwdArgs& a) {
  if (a.d == 64) return a.causal ? launch_dkdv<64, true, SPARSE, QK>(a) : launch_dkdv<64, false, SPARSE, QK>(a);
  return a.causal ? launch_dkdv<128, true, SPARSE, QK>(a) : launch_dkdv<128, false, SPARSE, QK>(a);
}

template <bool SPARSE, bool QK>
hipError_t dq_t(const BwdArgs& a) {
  if (a.d == 64) return a.causal ? launch_dq<64, true, SPARSE, QK>(a) : launch_dq<64, false, SPARSE, QK>(a);
  return a.causal ? launch_dq<128, true, SPARSE, QK>(a) : launch_dq<128, false, SPARSE, QK>(a);
}

}  // namespace

hipError_t bwd_bf16_dkdv(const BwdArgs& a) {
  if (a.window > 0)  // causal sliding window, dense, square lengths
    return a.d == 64 ? bwd_bf16_dkdv64(a) : launch_dkdv<128, true, false, false, false, true>(a);
  if (a.dropout) {  // dense, square lengths only (checked by the caller)
    if (a.d == 64) return a.causal ? launch_dkdv<64, true, false, false, true>(a) : launch_dkdv<64, false, false, false, true>(a);
    return a.causal ? launch_dkdv<128, true, false, false, true>(a) : launch_dkdv<128, false, false, false, true>(a);
  }
  if (a.bmask) return dkdv_t<true, false>(a);
  if (a.nk >= 0) return dkdv_t<false, true>(a);
  if (a.d == 64) return bwd_bf16_dkdv64(a);
  return dkdv_t<false, false>(a);
}

int bwd_dq_rows(int64_t d) { return d == 128 ? 32 * ATTN_DQ_NW128 : 128; }

hipError_t bwd_bf16_dq(const BwdArgs& a) {
  if (a.window > 0)  // causal sliding window, dense, square lengths
    return a.d == 64 ? launch_dq<64, true, false, false, false, true>(a) : launch_dq<128, true, false, false, false, true>(a);
  if (a.dropout) {
    if (a.d == 64) return a.causal ? launch_dq<64, true, false, false, true>(a) : launch_dq<64, false, false, false, true>(a);
    return a.causal ? launch_dq<128, true, false, false, true>(a) : launch_dq<128, false, false, false, true>(a);
  }
  if (a.bmask) return dq_t<true, false>(a);
  if (a.nk >= 0) return dq_t<false, true>(a);
  return dq_t<false, false>(a);
}

}  // namespace attn
