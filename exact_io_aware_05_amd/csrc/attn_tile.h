// LDS tiles of 64 rows x D bf16 features, shared by the gfx950 kernels.
//
// Layout: row-major, no padding, with the 16-byte chunk index c of each row
// replaced by c XOR tile_swz<D>(row).  The gfx950 LDS serves 256 bytes per
// clock (64 banks of 4 bytes); a 16-byte read is resolved 16 lanes at a time
// and an 8-byte transposing read 32 lanes at a time.  The swizzle makes both
// ways the kernels read a tile conflict-free:
//  * row reads: 16 consecutive lanes read the same chunk of 16 consecutive
//    rows -- the swizzle is one-to-one on any 16 consecutive rows (counting
//    the two half-lines of a 256-byte line separately when D = 64);
//  * transposed reads: 32 lanes read chunks 4e .. 4e+3 of 4 consecutive rows
//    (starting at a multiple of 4) -- the swizzle sends the 4 rows' groups of
//    4 chunks to disjoint bank ranges.
// D = 128 (256-byte rows): tile_swz = 4 * (row % 4) + (row / 4) % 4.
// D = 64 (128-byte rows): tile_swz = 4 * ((row / 2) % 2) + (row / 4) % 4.
// TileReader below gives the two read patterns.
// Tiles are filled by 16-byte buffer->LDS DMA: lane i of a wave's load lands
// at LDS byte 16*i after the wave's base, so each lane fetches the global
// chunk that belongs at that position.  Rows past the end of the head read
// as zero (buffer range check), in LDS as well.
#pragma once

#include "attn_device.h"

namespace attn {

typedef short s16x4 __attribute__((ext_vector_type(4)));
#define ATTN_LDS __attribute__((address_space(3)))

template <int D>
__device__ __forceinline__ constexpr int tile_swz(int row) {
  static_assert(D == 64 || D == 128, "head dimension");
  return D == 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : (((row & 2) << 1) | ((row >> 2) & 3));
}

// Byte offset of (row, 16-byte chunk c) in a tile with D features per row.
template <int D>
__device__ __forceinline__ constexpr uint32_t tile_off(int row, int c) {
  return (uint32_t)(row * (D * 2) + 16 * (c ^ tile_swz<D>(row)));
}

// Wait for this wave's outstanding vector-memory operations (LDS DMA
// included); lgkm and export counters are left unconstrained.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait until at most N of this wave's vector-memory operations are
// outstanding (they complete in issue order), lgkm and export unconstrained.
template <int N>
__device__ __forceinline__ void wait_vmem_upto() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier for LDS hand-overs that leaves vector-memory operations
// (tile fetches into LDS among them) in flight: this wave's LDS reads and
// writes are complete (lgkmcnt 0), then s_barrier.  __syncthreads() would
// also wait for every outstanding fetch (its release fence waits vmcnt 0),
// which defeats fetching a tile more than one tile ahead.  Callers wait for
// the fetches they need (wait_vmem_upto) before the barrier; the empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt unconstrained
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// DMA rows [row0, row0 + 64) of a [n, D] bf16 matrix (buffer `rs`) into the
// LDS tile at `lds`.  The NW waves of the workgroup split the 64 rows.
// Load k (k = 0 .. D/8 - 1) fills LDS bytes 1024k .. 1024k + 1023, lane i the
// 16 bytes at 1024k + 16i, so each lane fetches the global chunk that belongs
// there.  Its byte offset within the tile is 1024k + (b ^ x(k)): b is load
// 0's offset for the lane and x(k) the part of the swizzle that varies with k
// (16 (k % 4) at D = 128, 32 (k % 2) at D = 64).
template <int D, int NW>
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t rs, uint16_t* lds, int row0, int w, int lane) {
  constexpr int CPR = D / 8;      // 16-byte chunks per row
  constexpr int IPW = CPR / NW;   // 1 KiB loads per wave
  static_assert(IPW >= 1 && IPW * NW == CPR, "waves must split the tile evenly");
  // One long-lived register per lane; the copy is opaque, so the per-load
  // offsets are formed here rather than kept in registers across loops.
  uint32_t b = tile_off<D>(lane / CPR, lane % CPR);
  asm volatile("" : "+v"(b));
  // The tile's byte offset goes through readfirstlane: opaque to loop
  // strength reduction, which would otherwise keep one address vector per
  // load and buffer alive across the tile loop.
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)row0 * (D * 2));
#pragma unroll
  for (int r = 0; r < IPW; ++r) {
    const int k = w * IPW + r;
    const uint32_t xk = D == 128 ? 16u * (k & 3) : 32u * (k & 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (ATTN_LDS void*)(lds + 512 * k), 16, base + 1024u * k + (b ^ xk),
                                             0, 0, 0);
  }
}

// The same fetch issued through inline assembly, invisible to the compiler's
// LDS-DMA tracking.  The compiler cannot always tell an LDS read of one tile
// from a fetch in flight into another (it then waits for every fetch before
// the read, which serialises a software pipeline); kernels using this form
// wait for their fetches themselves (wait_vmem* before the barrier that
// hands a tile over).  `words` is the buffer descriptor of make_rsrc as four
// 32-bit words, so it can live in scalar registers of the asm operand.
struct RsrcWords {
  u32x4 w;
};
__device__ __forceinline__ RsrcWords rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  RsrcWords r;
  r.w[0] = (uint32_t)a;
  r.w[1] = (uint32_t)(a >> 32) & 0xFFFFu;  // stride 0
  r.w[2] = bytes;
  r.w[3] = 0x00020000u;
  return r;
}

template <int D, int NW>
__device__ __forceinline__ void dma_tile_asm(const RsrcWords& rs, uint16_t* lds, int row0, int w, int lane) {
  constexpr int CPR = D / 8;
  constexpr int IPW = CPR / NW;
  static_assert(IPW >= 1 && IPW * NW == CPR, "waves must split the tile evenly");
  uint32_t b = tile_off<D>(lane / CPR, lane % CPR);
  asm volatile("" : "+v"(b));
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)row0 * (D * 2));
  const uint32_t l0 = (uint32_t)(uintptr_t)(ATTN_LDS uint16_t*)lds;
#pragma unroll
  for (int r = 0; r < IPW; ++r) {
    const int k = w * IPW + r;
    const uint32_t xk = D == 128 ? 16u * (k & 3) : 32u * (k & 1);
    const uint32_t m0 = __builtin_amdgcn_readfirstlane(l0 + 1024u * k);
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %1\n\t"
        "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "s"(m0), "v"(base + 1024u * k + (b ^ xk)), "s"(rs.w)
        : "memory");
  }
}

// 64 consecutive fp32 values (one per lane: bytes 4 * lane) into LDS at
// byte address `lds_addr`, through the same invisible path.  (M0, which
// addresses the LDS side of these loads, is restored after each one.)
__device__ __forceinline__ void dma_row64_asm(const RsrcWords& rs, uint32_t lds_addr, uint32_t byte_off, int lane) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0), "v"(byte_off + 4u * (uint32_t)lane), "s"(rs.w)
      : "memory");
}

// Per-lane LDS byte offsets for reading MFMA operand fragments from tiles in
// this layout.  Every fragment a kernel reads starts at a row that is a
// multiple of 16, so the swizzle term depends only on the lane and the
// offsets are a few per-lane bases plus compile-time immediates:
//  * rows(lds, rbase, s): lane l gets 8 consecutive features 16*s + 8*(l/32)
//    .. +7 of row rbase + l % 32 (operand whose contraction index is the
//    feature).
//  * cols(lds, rbase, e): lane l (half h = l / 32) gets feature
//    32*e + l % 32 of the 8 rows rbase + {4h .. 4h+3, 8+4h .. 8+4h+3}, in that
//    order -- rows in the slot order of the 32x32 result layout, so the
//    fragment pairs with result registers 8u..8u+7 when rbase = 32t + 16u
//    (operand whose contraction index is the row, i.e. the transposed tile).
//    Two ds_read_b64_tr_b16: within each 16-lane group the hardware hands lane
//    i element i % 4 of the 8-byte piece addressed by lane 4s + i/4, so lane
//    j = 4s + c addresses row (4h + s) and features 4c .. 4c+3 of its group's
//    16-feature slice.
// An LDS read reaches at most 64 KiB past its address register.  A kernel
// whose tiles extend beyond that gives the reader byte shifts RS (row reads)
// and CS (transposed reads): the shift moves into the per-lane bases (hidden
// from the compiler, so it is not folded back) and out of the immediate.
template <int D, int RS = 0, int CS = 0>
struct TileReader {
  static constexpr int NS = D / 16;  // row fragments per row
  static constexpr int NE = D / 32;  // transposed fragments per 32 features
  uint32_t row_base[NS];
  uint32_t col_base[NE][2];

  __device__ __forceinline__ explicit TileReader(int lane) {
    const int l32 = lane & 31, h = lane >> 5;
    const int w = tile_swz<D>(l32);
#pragma unroll
    for (int s = 0; s < NS; ++s) row_base[s] = (uint32_t)(l32 * (D * 2) + 16 * ((2 * s + h) ^ w));
    const int g = lane >> 4, i16 = lane & 15;
    const int r0 = 4 * h + (i16 >> 2);
    const int z = 2 * (g & 1) + ((i16 & 3) >> 1);
#pragma unroll
    for (int e = 0; e < NE; ++e)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int r = r0 + 8 * k;
        col_base[e][k] = (uint32_t)(r * (D * 2) + 16 * ((4 * e + z) ^ tile_swz<D>(r)) + 8 * (i16 & 1));
      }
    if constexpr (RS != 0) {
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        row_base[s] += RS;
        asm("" : "+v"(row_base[s]));
      }
    }
    if constexpr (CS != 0) {
#pragma unroll
      for (int e = 0; e < NE; ++e)
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          col_base[e][k] += CS;
          asm("" : "+v"(col_base[e][k]));
        }
    }
  }

  __device__ __forceinline__ bf16x8 rows(const uint16_t* lds, int rbase, int s) const {
    const char* p = reinterpret_cast<const char*>(lds) + (rbase * (D * 2) - RS) + row_base[s];
    return *reinterpret_cast<const bf16x8*>(p);
  }

  __device__ __forceinline__ bf16x8 cols(const uint16_t* lds, int rbase, int e) const {
    const char* p = reinterpret_cast<const char*>(lds) + (rbase * (D * 2) - CS);
    const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS s16x4*)(p + col_base[e][0]));
    const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS s16x4*)(p + col_base[e][1]));
    u32x4 u;
    u[0] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(a, a, 0, 1));
    u[1] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(a, a, 2, 3));
    u[2] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(b, b, 0, 1));
    u[3] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(b, b, 2, 3));
    return as_bf16x8(u);
  }
};

// Block-sparse tile list.  Wave 0 of the workgroup writes, in increasing
// order, the tile indices j in [j0, j1) with want(j) true into `list` (LDS,
// at most kMaxSparseTiles entries) and the count into *count; every thread
// returns the count after the barrier.  want(j) is evaluated by one lane per
// tile (64 tiles per round: ballot, then each wanted lane writes its slot).
constexpr int kMaxSparseTiles = 2048;

template <typename F>
__device__ __forceinline__ int build_tile_list(F want, int j0, int j1, uint32_t* list, int* count, int w, int lane) {
  if (w == 0) {
    int cnt = 0;
    for (int c = j0; c < j1; c += 64) {
      const int j = c + lane;
      const bool f = j < j1 && want(j);
      const uint64_t bal = __builtin_amdgcn_ballot_w64(f);
      const int pre = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
      if (f) list[cnt + pre] = (uint32_t)j;
      cnt += __builtin_popcountll(bal);
    }
    if (lane == 0) *count = cnt;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*count);
}

}  // namespace attn
