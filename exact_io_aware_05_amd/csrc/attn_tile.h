// LDS tiles of 64 rows x D bf16 features, shared by the gfx950 kernels.
//
// Layout: row-major, no padding, with the 16-byte chunk index of each row
// XORed with swz(row) = 2*(row & 3) + ((row >> 2) & 1).  That permutation is
// one-to-one on any 8 consecutive rows starting at a multiple of 8 and, on
// any 4 consecutive rows starting at a multiple of 4, maps the chunk pairs
// {2k, 2k+1} to 4 distinct pairs.  So both ways the kernels read a tile are
// free of LDS bank conflicts:
//  * frag_rows: 16 bytes = 8 consecutive features of one row per lane, rows
//    l % 32 -- the MFMA operand whose contraction index is the feature;
//  * frag_cols: two ds_read_b64_tr_b16 per lane, which return one feature of
//    8 rows (in the slot order of the 32x32 result layout) -- the operand
//    whose contraction index is the row, i.e. the transposed tile.
// Tiles are filled by 16-byte buffer->LDS DMA: lane i of a wave's load lands
// at LDS byte 16*i after the wave's base, so each lane fetches the global
// chunk that belongs at that position.  Rows past the end of the head read
// as zero (buffer range check), in LDS as well.
#pragma once

#include "attn_device.h"

namespace attn {

typedef short s16x4 __attribute__((ext_vector_type(4)));
#define ATTN_LDS __attribute__((address_space(3)))

__device__ __forceinline__ constexpr int tile_swz(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }

// Byte offset of (row, 16-byte chunk c) in a tile with D features per row.
template <int D>
__device__ __forceinline__ constexpr uint32_t tile_off(int row, int c) {
  return (uint32_t)(row * (D * 2) + 16 * (c ^ tile_swz(row)));
}

// Wait for this wave's outstanding vector-memory operations (LDS DMA
// included); lgkm and export counters are left unconstrained.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// DMA rows [row0, row0 + 64) of a [n, D] bf16 matrix (buffer `rs`) into the
// LDS tile at `lds`.  The NW waves of the workgroup split the 64 rows.
template <int D, int NW>
__device__ __forceinline__ void dma_tile(__amdgpu_buffer_rsrc_t rs, uint16_t* lds, int row0, int w, int lane) {
  constexpr int CPR = D / 8;      // 16-byte chunks per row
  constexpr int IPW = CPR / NW;   // 1 KiB loads per wave
  static_assert(IPW >= 1 && IPW * NW == CPR, "waves must split the tile evenly");
#pragma unroll
  for (int r = 0; r < IPW; ++r) {
    const int k = w * IPW + r;
    const int p = 64 * k + lane;          // LDS chunk this lane fills
    const int row = p / CPR, cp = p % CPR;
    const int c = cp ^ tile_swz(row);     // global chunk that belongs there
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (ATTN_LDS void*)(lds + 512 * k), 16,
                                             (uint32_t)(row0 + row) * (D * 2) + 16 * c, 0, 0, 0);
  }
}

// Operand fragment of row `row` (features 16*s + 8*h .. +7).
template <int D>
__device__ __forceinline__ bf16x8 frag_rows(const uint16_t* lds, int row, int s, int h) {
  return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(lds) + tile_off<D>(row, 2 * s + h));
}

// Transposed operand fragment: lane l (half h = l / 32) receives feature
// f = 32 * e + l % 32 of the 8 rows rbase + {4h .. 4h+3, 8+4h .. 8+4h+3},
// in that order -- rows in the slot order of the 32x32 result layout, so
// the fragment pairs with result registers 8u..8u+7 when rbase = 32t + 16u.
// Within each 16-lane group the hardware hands lane i element i % 4 of the
// 8-byte piece addressed by lane 4s + i/4, for s = 0..3.
template <int D>
__device__ __forceinline__ bf16x8 frag_cols(const uint16_t* lds, int rbase, int e, int lane) {
  const int g = lane >> 4, i16 = lane & 15;
  const int h = g >> 1;
  const int col = 32 * e + 16 * (g & 1) + 4 * (i16 & 3);  // first of 4 features this lane addresses
  const int r0 = rbase + 4 * h + (i16 >> 2);
  const char* base = reinterpret_cast<const char*>(lds);
  const uint32_t o0 = tile_off<D>(r0, col >> 3) + 2 * (col & 7);
  const uint32_t o1 = tile_off<D>(r0 + 8, col >> 3) + 2 * (col & 7);
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS s16x4*)(base + o0));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS s16x4*)(base + o1));
  u32x4 u;
  u[0] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(a, a, 0, 1));
  u[1] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(a, a, 2, 3));
  u[2] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(b, b, 0, 1));
  u[3] = __builtin_bit_cast(uint32_t, __builtin_shufflevector(b, b, 2, 3));
  return as_bf16x8(u);
}

}  // namespace attn
