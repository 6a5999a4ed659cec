// dK and dV at head dimension 64, bf16 in / bf16 out, fp32 accumulation,
// gfx950: the key-stationary half of the backward pass by recomputation
// ("Background" and "Key Ideas" on the Paper Notes page; "The backward
// pass: recompute instead of store" on the aicassindra page), with the
// textbook gradients P = exp(scale Q K^T - LSE), dV = P^T dO,
// dP = dO V^T, dS = P * (dP - D), dK = scale dS^T Q.
//
// At d = 64 one wave can hold everything a 32-key group needs: the K and V
// rows of its keys (B operands of S = Q K^T and dP = dO V^T, 8 registers
// each per 32 features) and both accumulators dV^T and dK^T (32 registers
// each), about 96 registers.  So each wave does both halves of the work for
// its own keys -- no P exchange between waves and one barrier per query
// tile -- and a workgroup of four waves (128 keys) leaves room for two
// workgroups per CU, whose independent instruction streams fill each
// other's matrix and vector gaps.  (At d = 128 the same state is twice as
// large, and bwd_kv_kernel in attn_bwd_bf16.hip splits it over a pair of
// waves instead.)
//
// Per 32-query unit of a 64-row query tile, a wave computes
//   S and dP (C[query][key] layout: lane = key, registers run over queries),
//   P = exp2(S scale log2 e - LSE log2 e), dS = P (dP - D) (dP accumulated
//   onto -D), both packed to bf16,
//   dV^T += dO^T P and dK^T += Q^T dS with P and dS straight from registers
//   as the B operand and dO^T, Q^T read from the row-major LDS tiles with
//   transposing reads.
// Where a 32 x 32 block holds a term of weight >= 1/16 (P itself for dV,
// scale |dS| for dK) the term enters as a hi + lo bf16 pair, as in
// bwd_kv_kernel (single bf16 rounding of a probability near 1 can move a
// column sum by more than the output's own rounding).
// Query tiles are fetched by buffer->LDS DMA into three buffers: the tile
// after next streams in while the current one is used; rows past the end of
// the head arrive as zeros (and contribute nothing: dO = 0, dS = 0).
#include <type_traits>

#include "attn_device.h"
#include "attn_launch.h"
#include "attn_tile.h"

namespace attn {

namespace {

template <int N>
using ic = std::integral_constant<int, N>;

// Buffer->LDS DMA of this wave's share of a 64 x D tile (rows row0 ..
// row0 + 63 of the buffer `rs`) into LDS at byte address `lds` (wave-uniform,
// a scalar), issued through inline assembly like dma_tile_asm
// (attn_tile.h), but with the LDS address and the lane's swizzled offset
// `boff` (tile_off(lane / (D / 8), lane % (D / 8))) computed once by the
// caller: under register pressure the compiler otherwise kept the LDS base in
// a vector register, spilled it, and the reload's wait for vector memory
// also waited for every tile fetch in flight.
template <int D, int NW>
__device__ __forceinline__ void dma_tile_at(const RsrcWords& rs, uint32_t lds, uint32_t boff, int row0, int w) {
  constexpr int IPW = (D / 8) / NW;
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)row0 * (D * 2));
#pragma unroll
  for (int r = 0; r < IPW; ++r) {
    const int k = w * IPW + r;
    const uint32_t xk = D == 128 ? 16u * (k & 3) : 32u * (k & 1);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(lds + 1024u * k), "v"(base + 1024u * k + (boff ^ xk)), "s"(rs.w)
        : "memory");
  }
}

#ifndef ATTN_KV64_WAVES
#define ATTN_KV64_WAVES 3  // waves per SIMD the register budget is sized for (tuning knob)
#endif

template <bool CAUSAL, bool WIN = false>
__global__ __launch_bounds__(256, ATTN_KV64_WAVES) void bwd_kv64_kernel(const uint16_t* __restrict__ Q,
                                                          const uint16_t* __restrict__ K,
                                                          const uint16_t* __restrict__ V,
                                                          const uint16_t* __restrict__ dO,
                                                          const float* __restrict__ LSE,
                                                          const float* __restrict__ Dsum, uint16_t* __restrict__ dK,
                                                          uint16_t* __restrict__ dV, int n, int nkb, int total,
                                                          float scale, float sl2e, float tau_ds,
                                                          const int* __restrict__ klen, int heads, int wl,
                                                          int hf_pass, int hf_fill) {
  constexpr int D = 64, NW = 4, BKV = 32 * NW, BQ = 64;
  constexpr int TB = BQ * D * 2;     // bytes per 64-row tile
  constexpr int IPW = (D / 8) / NW;  // DMA loads per wave per tile
  constexpr float kTau = 1.0f / 16.0f;

  // LDS: [0, 1536) LSE (x log2 e) and -D rows of three tiles (512 B each:
  // 64 LSE values, then 64 -D values), then Q tiles 0-2, then dO tiles 0-2.
  constexpr int SMALL = 1536;
  __shared__ __attribute__((aligned(1024))) char smem[SMALL + 6 * TB];
  auto lse_at = [&](auto b) ATTN_INLINE { return reinterpret_cast<float*>(smem + 512 * decltype(b)::value); };
  auto dsm_at = [&](auto b) ATTN_INLINE { return reinterpret_cast<float*>(smem + 512 * decltype(b)::value + 256); };
  auto q_at = [&](auto b) ATTN_INLINE {
    return reinterpret_cast<uint16_t*>(smem + SMALL + TB * decltype(b)::value);
  };
  auto g_at = [&](auto b) ATTN_INLINE {
    return reinterpret_cast<uint16_t*>(smem + SMALL + TB * (3 + decltype(b)::value));
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, l32 = lane & 31;

  // Causal: low key blocks see the most queries; they come first, longest
  // first within each XCD (heavy_first, with the start-up placement).
  int bh, kb;
  if (CAUSAL) {
    heavy_first(blockIdx.x, total / nkb, nkb, bh, kb, hf_pass, hf_fill);
  } else {
    const int lid = xcd_remap(blockIdx.x, total);
    bh = lid / nkb;
    kb = lid % nkb;
  }
  const int k0 = kb * BKV;
  const int kw0 = k0 + 32 * w;
  const int key = kw0 + l32;

  const size_t head = (size_t)bh * (size_t)n * D;
  // Key padding: keys from nkv on are masked for every query, so their dK
  // and dV are zero; a block of padded keys only writes those zeros.
  const int nkv = padded_keys(klen, heads, bh, n);
  if (k0 >= nkv) {
    if (key < n) {
      const u32x2 z = {0u, 0u};
#pragma unroll
      for (int e = 0; e < D / 32; ++e)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          *reinterpret_cast<u32x2*>(dV + head + (size_t)key * D + 32 * e + 8 * g + 4 * hh) = z;
          *reinterpret_cast<u32x2*>(dK + head + (size_t)key * D + 32 * e + 8 * g + 4 * hh) = z;
        }
    }
    return;
  }
  const uint32_t head_bytes = (uint32_t)n * D * 2u;
  const RsrcWords rq = rsrc_words(Q + head, head_bytes);
  const RsrcWords rdo = rsrc_words(dO + head, head_bytes);
  const RsrcWords rl = rsrc_words(LSE + (size_t)bh * n, (uint32_t)n * 4u);
  const RsrcWords rd = rsrc_words(Dsum + (size_t)bh * n, (uint32_t)n * 4u);

  // This lane's key row of K and V: B operands of S and dP (8 features per
  // 16-feature step).  Keys past n read as zero.
  bf16x8 kf[D / 16], vf[D / 16];
  {
    const auto rk = make_rsrc(K + head, head_bytes);
    const auto rv = make_rsrc(V + head, head_bytes);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      kf[s] = as_bf16x8(bload16(rk, (uint32_t)key * (D * 2) + 32 * s + 16 * hh));
      vf[s] = as_bf16x8(bload16(rv, (uint32_t)key * (D * 2) + 32 * s + 16 * hh));
    }
    // Complete before any tile fetch: a wait for these registers inside the
    // tile loop would also wait for the fetches in flight.
    wait_vmem();
  }

  f32x16 dva[D / 32], dka[D / 32];  // dV^T and dK^T: rows = features, columns = keys
#pragma unroll
  for (int e = 0; e < D / 32; ++e)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dva[e][r] = 0.f;
      dka[e][r] = 0.f;
    }

  // Query tiles it0 .. ntq - 1; under the sliding window (WIN: query i sees
  // keys i - wl .. i) they end with the window of the block's last key.
  const int ntq = WIN ? min((n + BQ - 1) / BQ, (k0 + BKV - 1 + wl) / BQ + 1) : (n + BQ - 1) / BQ;
  const int it0 = CAUSAL ? k0 / BQ : 0;
  const TileReader<D> TR(lane);

  // A tile's batch of fetches: wave 0 the LSE and D rows (one load each),
  // every wave its share of the Q and dO tiles.  Every tile issues the same
  // batch (past the last tile: copies of the last one, never read), so the
  // wait counts below hold on every path.
  constexpr int SMALLN = 2;
  const uint32_t sbase = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(ATTN_LDS char*)smem);
  uint32_t boff = tile_off<D>(lane / (D / 8), lane % (D / 8));
  asm volatile("" : "+v"(boff));
  auto dma = [&](int i, auto b) ATTN_INLINE {
    constexpr uint32_t B = decltype(b)::value;
    if (w == 0) {
      const uint32_t off = __builtin_amdgcn_readfirstlane((uint32_t)i * (BQ * 4));
      dma_row64_asm(rl, sbase + 512u * B, off, lane);
      dma_row64_asm(rd, sbase + 512u * B + 256u, off, lane);
    }
    dma_tile_at<D, NW>(rq, sbase + SMALL + TB * B, boff, i * BQ, w);
    dma_tile_at<D, NW>(rdo, sbase + SMALL + TB * (3 + B), boff, i * BQ, w);
  };
  // Before the barrier that opens a tile: that tile's batch has landed (the
  // next batch, issued last, stays in flight); wave 0 scales the LSE row to
  // base 2 and negates the D row in place.
  auto open = [&](auto b) ATTN_INLINE {
    if (w == 0) {
      wait_vmem_upto<SMALLN + 2 * IPW>();
      asm volatile("" ::: "memory");
      lse_at(b)[lane] *= kLog2e;
      dsm_at(b)[lane] = -dsm_at(b)[lane];
    } else {
      wait_vmem_upto<2 * IPW>();
    }
    barrier_lds();
  };

  // Wave-uniform: does some |x| of the 16 values reach t?
  auto any_reaches = [&](const float* x, float t) ATTN_INLINE {
    float m0 = fmaxf(fabsf(x[0]), fabsf(x[1])), m1 = fmaxf(fabsf(x[2]), fabsf(x[3]));
#pragma unroll
    for (int r = 4; r < 16; r += 2) {
      m0 = fmaxf(m0, fabsf(x[r]));
      m1 = fmaxf(m1, fabsf(x[r + 1]));
    }
    return __builtin_amdgcn_ballot_w64(fmaxf(m0, m1) >= t) != 0;
  };

  // One 32-query unit t of the tile in buffer b (tile i).
  auto unit = [&](auto b, int i, int t) ATTN_INLINE {
    const uint16_t* qs = q_at(b);
    const uint16_t* gs = g_at(b);
    const float* ls = lse_at(b);
    const float* dsr = dsm_at(b);
    const int q0 = i * BQ + 32 * t;
    if (CAUSAL && q0 + 31 < kw0) return;  // every query of the unit precedes every key of the wave
    if (WIN && q0 > kw0 + 31 + wl) return;  // every query of the unit is past every key's window
    // dP starts from -D (its rows' values, in the registers' query order),
    // S from zero; both chains read their A operand rows from LDS.
    f32x16 cs, cp;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(&dsr[32 * t + 8 * g + 4 * hh]);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        cs[4 * g + k] = 0.f;
        cp[4 * g + k] = d4[k];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      cs = mfma32(TR.rows(qs, 32 * t, s), kf[s], cs);
      cp = mfma32(TR.rows(gs, 32 * t, s), vf[s], cp);
    }
    __builtin_amdgcn_sched_barrier(0);
    // P = exp2(S scale log2 e - LSE log2 e); on a unit that crosses the
    // diagonal (a wave-uniform branch) entries whose key follows the query
    // become -inf first.
    float p[16], ds[16];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(&ls[32 * t + 8 * g + 4 * hh]);
#pragma unroll
      for (int k = 0; k < 4; ++k) p[4 * g + k] = fmaf(cs[4 * g + k], sl2e, -l4[k]);
    }
    if (CAUSAL && q0 < kw0 + 31) {
      // key > query  <=>  l32 - 4 hh > (q0 - kw0) + crow(r, 0): one lane value,
      // derived here from the lane id (not kept live through the loop).
      int lrel = threadIdx.x & 63;
      asm volatile("" : "+v"(lrel));
      lrel = (lrel & 31) - 4 * (lrel >> 5);
      const int dq = q0 - kw0;
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = lrel > dq + crow(r, 0) ? -INFINITY : p[r];
    }
    if (WIN && q0 + 31 > kw0 + wl) {
      // query > key + wl  <=>  (q0 - kw0 - wl) + crow(r, 0) > l32 - 4 hh.
      int lrel = threadIdx.x & 63;
      asm volatile("" : "+v"(lrel));
      lrel = (lrel & 31) - 4 * (lrel >> 5);
      const int dw = q0 - kw0 - wl;
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = dw + crow(r, 0) > lrel ? -INFINITY : p[r];
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = fast_exp2(p[r]);
      ds[r] = p[r] * cp[r];
    }
    const bf16x8 ph[2] = {pack_bf16x8(p), pack_bf16x8(p + 8)};
    const bf16x8 dh[2] = {pack_bf16x8(ds), pack_bf16x8(ds + 8)};
    // The lo terms first, only where a block needs them (the fp32 values die
    // here, before the operand reads of the main products).  The empty asm
    // statements keep the lo computation inside its branch: hoisted out, it
    // ran on every unit.
    if (any_reaches(p, kTau)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) asm volatile("" : "+v"(p[r]));
      const bf16x8 pl[2] = {split_lo_bf16x8(p, ph[0]), split_lo_bf16x8(p + 8, ph[1])};
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < D / 32; ++e) dva[e] = mfma32(TR.cols(gs, 32 * t + 16 * u, e), pl[u], dva[e]);
    }
    if (any_reaches(ds, tau_ds)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) asm volatile("" : "+v"(ds[r]));
      const bf16x8 dl[2] = {split_lo_bf16x8(ds, dh[0]), split_lo_bf16x8(ds + 8, dh[1])};
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < D / 32; ++e) dka[e] = mfma32(TR.cols(qs, 32 * t + 16 * u, e), dl[u], dka[e]);
    }
    // dV^T += dO^T P and dK^T += Q^T dS over the unit's 32 queries (two
    // 16-query slices, slot order of the result layout).
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < D / 32; ++e) {
        dva[e] = mfma32(TR.cols(gs, 32 * t + 16 * u, e), ph[u], dva[e]);
        dka[e] = mfma32(TR.cols(qs, 32 * t + 16 * u, e), dh[u], dka[e]);
      }
    __builtin_amdgcn_sched_barrier(0);
  };

  if (it0 < ntq) {
    // Tile i lives in buffer (i - it0) mod 3; the batch of tile i + 2 is
    // issued once the barrier opening tile i has retired every read of tile
    // i - 1, whose buffer it reuses.
    auto step = [&](auto b, int i) ATTN_INLINE {
      constexpr int B = decltype(b)::value;
      dma(min(i + 2, ntq - 1), ic<(B + 2) % 3>{});
      unit(b, i, 0);
      unit(b, i, 1);
      open(ic<(B + 1) % 3>{});
    };
    dma(it0, ic<0>{});
    dma(min(it0 + 1, ntq - 1), ic<1>{});
    open(ic<0>{});
    for (int it = it0; it < ntq; it += 3) {
      step(ic<0>{}, it);
      if (it + 1 >= ntq) break;
      step(ic<1>{}, it + 1);
      if (it + 2 >= ntq) break;
      step(ic<2>{}, it + 2);
    }
    wait_vmem();  // no fetch outlives the loop
  }

  // The lane's key and row addresses are derived again here (kept live
  // through the loop, they were spilled under the loop's register pressure).
  int le = threadIdx.x & 63;
  asm volatile("" : "+v"(le));
  const int keye = kw0 + (le & 31), hhe = le >> 5;
  const bool live = keye < nkv;  // a padded key of a partly padded block: zero
  // dV and dK leave through LDS so that every store writes whole 128-byte
  // rows: each wave stages its 32 keys of both (rows 144 bytes apart) in its
  // own 9 KiB of the tile buffers, once every wave is done with the tiles,
  // and reads them back 16 bytes per lane, eight rows per instruction.
  __syncthreads();
  constexpr int RS = 72;  // row stride in bf16 elements
  uint16_t* const sv = reinterpret_cast<uint16_t*>(smem + SMALL) + w * (2 * 32 * RS);
  uint16_t* const sk = sv + 32 * RS;
  const int le32 = le & 31;
#pragma unroll
  for (int e = 0; e < D / 32; ++e)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 v2, k2;
      v2[0] = pack_bf16x2(dva[e][4 * g + 0], dva[e][4 * g + 1]);
      v2[1] = pack_bf16x2(dva[e][4 * g + 2], dva[e][4 * g + 3]);
      k2[0] = pack_bf16x2(dka[e][4 * g + 0] * scale, dka[e][4 * g + 1] * scale);
      k2[1] = pack_bf16x2(dka[e][4 * g + 2] * scale, dka[e][4 * g + 3] * scale);
      if (!live) v2[0] = v2[1] = k2[0] = k2[1] = 0u;
      *reinterpret_cast<u32x2*>(sv + le32 * RS + 32 * e + 8 * g + 4 * hhe) = v2;
      *reinterpret_cast<u32x2*>(sk + le32 * RS + 32 * e + 8 * g + 4 * hhe) = k2;
    }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = 8 * k + (le >> 3), c = le & 7;
    const u32x4 v4 = *reinterpret_cast<const u32x4*>(sv + r * RS + 8 * c);
    const u32x4 k4 = *reinterpret_cast<const u32x4*>(sk + r * RS + 8 * c);
    if (kw0 + r < n) {
      *reinterpret_cast<u32x4*>(dV + head + (size_t)(kw0 + r) * D + 8 * c) = v4;
      *reinterpret_cast<u32x4*>(dK + head + (size_t)(kw0 + r) * D + 8 * c) = k4;
    }
  }
}

}  // namespace

// dK, dV at d = 64 for dense, square-length problems without dropout.
hipError_t bwd_bf16_dkdv64(const BwdArgs& a) {
  const int n = (int)a.n;
  const int nkb = (n + 127) / 128;
  const int total = (int)(a.bh * nkb);
  // Split threshold of dS, which enters the products unscaled (the scale
  // multiplies dK at the end): a term's weight scale |dS| reaches 1/16.
  const float tau_ds = (1.0f / 16.0f) / fabsf(a.scale);
  static int hp[2] = {-1, -1}, hf[2] = {0, 0};  // start-up placement of the causal order
  if (hp[0] < 0) start_fill(bwd_kv64_kernel<true, false>, 256, hp[0], hf[0]);
  if (hp[1] < 0) start_fill(bwd_kv64_kernel<true, true>, 256, hp[1], hf[1]);
  const int w = a.window > 0 ? 1 : 0;
  if (a.window > 0)
    hipLaunchKernelGGL((bwd_kv64_kernel<true, true>), dim3(total), dim3(256), 0, a.stream, (const uint16_t*)a.q,
                       (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dout, a.lse, a.dsum,
                       (uint16_t*)a.dk, (uint16_t*)a.dv, n, nkb, total, a.scale, a.scale * kLog2e, tau_ds,
                       a.klen, a.heads, a.window - 1, hp[w], hf[w]);
  else if (a.causal)
    hipLaunchKernelGGL(bwd_kv64_kernel<true>, dim3(total), dim3(256), 0, a.stream, (const uint16_t*)a.q,
                       (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dout, a.lse, a.dsum,
                       (uint16_t*)a.dk, (uint16_t*)a.dv, n, nkb, total, a.scale, a.scale * kLog2e, tau_ds,
                       a.klen, a.heads, a.window - 1, hp[w], hf[w]);
  else
    hipLaunchKernelGGL(bwd_kv64_kernel<false>, dim3(total), dim3(256), 0, a.stream, (const uint16_t*)a.q,
                       (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dout, a.lse, a.dsum,
                       (uint16_t*)a.dk, (uint16_t*)a.dv, n, nkb, total, a.scale, a.scale * kLog2e, tau_ds,
                       a.klen, a.heads, a.window - 1, hp[w], hf[w]);
  return hipGetLastError();
}

}  // namespace attn
