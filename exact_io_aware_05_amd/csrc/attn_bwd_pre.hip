// Backward-pass preprocessing: D_i = sum_k dO_ik * O_ik per query row.
//
// D_i equals sum_j P_ij dP_ij (the row term of the softmax gradient,
// dS = P * (dP - D)), computed from O instead of P so the N x N matrix is
// never needed.  The pages defer the gradient formulas to a companion
// article; this is the textbook identity sum_j P_ij (dO_i . V_j) = dO_i . O_i.
// Memory bound: one pass over O and dO.
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

namespace {

__device__ __forceinline__ void load8(const uint16_t* p, float* x) {
  const u32x4 u = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(u[i] << 16);
    x[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float* x) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = a[i];
    x[4 + i] = b[i];
  }
}

template <int D, typename T>
__global__ __launch_bounds__(256) void dsum_kernel(const T* __restrict__ O, const T* __restrict__ dO,
                                                   float* __restrict__ Dsum, int rows) {
  constexpr int CPR = D / 8;       // lanes per row, 8 features each
  constexpr int RPB = 256 / CPR;   // rows per workgroup
  const int tid = threadIdx.x;
  const int row = blockIdx.x * RPB + tid / CPR;
  const int ch = tid % CPR;
  float s = 0.f;
  if (row < rows) {
    float o[8], g[8];
    load8(O + (size_t)row * D + 8 * ch, o);
    load8(dO + (size_t)row * D + 8 * ch, g);
#pragma unroll
    for (int i = 0; i < 8; ++i) s = fmaf(o[i], g[i], s);
  }
#pragma unroll
  for (int off = CPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (ch == 0 && row < rows) Dsum[row] = s;
}

template <int D, typename T>
hipError_t dsum_t(const BwdArgs& a) {
  constexpr int RPB = 256 / (D / 8);
  const int rows = (int)(a.bh * a.n);
  const int blocks = (rows + RPB - 1) / RPB;
  hipLaunchKernelGGL((dsum_kernel<D, T>), dim3(blocks), dim3(256), 0, a.stream, (const T*)a.o, (const T*)a.dout,
                     a.dsum, rows);
  return hipGetLastError();
}

}  // namespace

hipError_t bwd_dsum(const BwdArgs& a, bool bf16) {
  if (bf16) return a.d == 64 ? dsum_t<64, uint16_t>(a) : dsum_t<128, uint16_t>(a);
  return a.d == 64 ? dsum_t<64, float>(a) : dsum_t<128, float>(a);
}

}  // namespace attn
