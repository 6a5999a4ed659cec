// Device-side building blocks shared by the attention kernels (gfx950 only).
//
// Matrix-core conventions used throughout (CDNA 32x32 MFMA):
//   v_mfma_f32_32x32x16_bf16 D = A(32x16) * B(16x32) + C(32x32).
//   Lane l supplies row (l % 32) of A and column (l % 32) of B, each as 8
//   bf16 values of the contraction index; both operands use the same
//   lane/slot -> contraction-index map, so any consistent assignment of the
//   contraction index to (lane half, slot) gives the same product.
//   The 32x32 fp32 result lives in 16 registers per lane:
//   register r of lane l holds row 8*(r/4) + 4*(l/32) + (r%4), column l%32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Lambdas that capture a kernel's register arrays by reference must be
// inlined, or the arrays are placed in scratch memory.
#define ATTN_INLINE __attribute__((always_inline))

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row index (within a 32x32 result tile) held by register r in lane half h.
__device__ __forceinline__ constexpr int crow(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Position of index x (within a block of 32) in the "slot order" of the 32x32
// result layout: the 8 rows that one lane half holds in registers 8u..8u+7
// (rows 16u + {4h..4h+3, 8+4h..8+4h+3}) become 8 consecutive positions
// 16u + 8h + 0..7.  It swaps bits 2 and 3 of x and is its own inverse.
__device__ __forceinline__ constexpr int slot_pos(int x) {
  return (x & ~0xC) | ((x & 4) << 1) | ((x & 8) >> 1);
}

// Symmetric combination of the two 32-lane halves of a wave: every lane gets
// op(x[l % 32], x[l % 32 + 32]).  v_permlane32_swap exchanges one half of its
// two operands, so passing x twice yields both halves in one instruction.
__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Round two floats to bf16 (nearest, ties to even) and pack them, low first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 b = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ bf16x8 pack_bf16x8(const float* x) {
  u32x4 u;
  u[0] = pack_bf16x2(x[0], x[1]);
  u[1] = pack_bf16x2(x[2], x[3]);
  u[2] = pack_bf16x2(x[4], x[5]);
  u[3] = pack_bf16x2(x[6], x[7]);
  return __builtin_bit_cast(bf16x8, u);
}

// x = hi + lo with hi = bf16(x) and lo = bf16(x - hi): the pair carries about
// 16 significant bits, so a product accumulated as hi*b + lo*b has the
// rounding error of fp32-class operands while both MFMA inputs stay bf16
// (and so keep bf16's full exponent range).
__device__ __forceinline__ void split_bf16x8(const float* x, bf16x8& hi, bf16x8& lo) {
  u32x4 h, l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
    const float r0 = x[2 * i] - __uint_as_float(h[i] << 16);
    const float r1 = x[2 * i + 1] - __uint_as_float(h[i] & 0xFFFF0000u);
    l[i] = pack_bf16x2(r0, r1);
  }
  hi = __builtin_bit_cast(bf16x8, h);
  lo = __builtin_bit_cast(bf16x8, l);
}

// The lo term of split_bf16x8 for a given hi = pack_bf16x8(x).
__device__ __forceinline__ bf16x8 split_lo_bf16x8(const float* x, bf16x8 hi) {
  const u32x4 h = __builtin_bit_cast(u32x4, hi);
  u32x4 l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float r0 = x[2 * i] - __uint_as_float(h[i] << 16);
    const float r1 = x[2 * i + 1] - __uint_as_float(h[i] & 0xFFFF0000u);
    l[i] = pack_bf16x2(r0, r1);
  }
  return __builtin_bit_cast(bf16x8, l);
}

// Low 16 bits of a and b packed (a low), and high 16 bits of a and b packed.
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& u) { return __builtin_bit_cast(bf16x8, u); }

// Buffer resource over `bytes` bytes at `base`: raw buffer loads through it
// return zero for any offset at or past `bytes`, so ragged tiles need no
// branches.  Word 3 is the gfx9 raw-buffer format (no swizzle, 32-bit data).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ float bload4f(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

// 16-byte global load with a predicate (zero when off).
__device__ __forceinline__ u32x4 load16_or_zero(const uint16_t* p, bool ok) {
  u32x4 z = {0u, 0u, 0u, 0u};
  return ok ? *reinterpret_cast<const u32x4*>(p) : z;
}

// Philox4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC 2011): counter (c0, c1, c2, c3), key
// (k0, k1); each round takes the full 64-bit products c0 * 0xD2511F53 and
// c2 * 0xCD9E8D57 and sets (c0, c1, c2, c3) to (hi(c2 M1) ^ c1 ^ k0,
// lo(c2 M1), hi(c0 M0) ^ c3 ^ k1, lo(c0 M0)); the key gains (0x9E3779B9,
// 0xBB67AE85) before every round but the first.  The key is wave-uniform
// here, so its schedule is scalar work.
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                               uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)c0 * 0xD2511F53u;
    const uint64_t p1 = (uint64_t)c2 * 0xCD9E8D57u;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
  }
  u32x4 w;
  w[0] = c0;
  w[1] = c1;
  w[2] = c2;
  w[3] = c3;
  return w;
}

// Workgroup order.  Workgroups are handed to the 8 XCDs of the chip round
// robin (id % 8).  This maps the hardware id to a logical id so that each
// XCD receives a contiguous range of logical ids (tiles of the same head
// share one L2).  Bijective for any total.
__device__ __forceinline__ int xcd_remap(int pid, int total) {
  const int q = total >> 3, r = total & 7;
  const int x = pid & 7, k = pid >> 3;
  return x * q + (x < r ? x : r) + k;
}

// Causal workgroup order: longest first within each XCD.  Under the causal
// mask the work of a query block grows with its index, and a workgroup
// order that walks one head's blocks heavy to light, head after head,
// leaves an XCD's last CUs with heavy blocks at the end.  When the head
// count is a multiple of 8, XCD x (hardware id % 8) owns heads x * hx ..
// x * hx + hx - 1 (hx = heads / 8, so a head's blocks share one L2) and
// takes them in groups of up to four heads, each group rank-major: rank 0
// (the heaviest block) of its heads, then rank 1, and so on (a last group
// may be smaller).  All hx heads rank-major at once kept every head's keys
// and values in flight and fetched 3x the minimum from HBM (B=4 H=16 N=4096
// forward); groups of four fetch 1.5x and run as fast; groups of two fetch
// the minimum but run 2-3% slower.
// Every XCD receives exactly hx * nblk ids, so the map is a bijection of
// [0, heads * nblk).  Otherwise the xcd_remap order (head-major) is kept.
//
// Several workgroups per CU (`fill` > `pass`): the first `fill` workgroups of
// an XCD are placed at once, one slot of every CU per pass of `pass` (its CU
// count), the k-th on CU k mod pass; so the blocks sharing a CU from the
// start are those `pass` apart.  Then the XCD's heads are taken rank-major
// (longest first over all of them) and, within the first fill, every odd
// pass is reversed, so that a CU that starts with one of the heaviest blocks
// of a pass also gets one of the lightest of the next (workgroups dispatched
// later, into freed slots, keep the longest-first order).
__device__ __forceinline__ void heavy_first(int pid, int heads, int nblk, int& bh, int& rank, int pass = 0,
                                            int fill = 0) {
  if ((heads & 7) == 0 && pass > 0 && fill > pass) {
    const int hx = heads >> 3;
    const int x = pid & 7, s = pid >> 3;
    const int f = min(fill, hx * nblk);
    int i = s;  // position in the XCD's longest-first list
    if (s < f) {
      const int p = s / pass, j = s - p * pass;
      const int q = min(pass, f - p * pass);  // blocks in this pass
      if (p & 1) i = p * pass + (q - 1 - j);
    }
    rank = i / hx;
    bh = x * hx + (i - rank * hx);
    return;
  }
  if ((heads & 7) == 0) {
    const int hx = heads >> 3;
    const int x = pid & 7, s = pid >> 3;
    const int g = hx >= 4 ? 4 : hx;  // heads per group
    const int full = hx / g;         // groups of g heads
    const int span = g * nblk;       // ids per full group
    int grp, sub, gl;
    if (s < full * span) {
      grp = s / span;
      sub = s - grp * span;
      gl = g;
    } else {
      grp = full;
      sub = s - full * span;
      gl = hx - full * g;
    }
    rank = sub / gl;
    bh = x * hx + grp * g + (sub - rank * gl);
  } else {
    const int lid = xcd_remap(pid, heads * nblk);
    bh = lid / nblk;
    rank = lid % nblk;
  }
}

}  // namespace attn
