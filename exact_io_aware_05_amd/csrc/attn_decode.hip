// Attention for a few query rows over many keys (decoding), bf16 in / bf16
// out, fp32 arithmetic, gfx950.
//
// With one query row per head the work per key is a d-long dot product and a
// d-long scaled add, so the pass is bound by reading K and V from HBM; a
// 128-row matrix-core tile would leave 127 of its rows empty.  This kernel
// streams K and V with plain vector loads and computes in fp32 on the
// vector ALUs:
//  * A group of d / 8 lanes holds one key row, 16 bytes (8 bf16) per lane, so
//    one load instruction of a wave fetches 64 / (d / 8) consecutive key rows,
//    1 KiB of contiguous memory.  A wave takes 8 such loads of K and 8 of V
//    per batch (32 keys at d = 128, 64 at d = 64; 4 of each with four rows).
//  * The score q . k_j is four v_dot2 (bf16 pairs into fp32) per lane, then a
//    sum over the group's lanes by DPP adds (quad swaps and row mirrors).
//  * Every lane group keeps its own softmax state for the keys it holds --
//    running max m, running sum l, unnormalised output (8 features per lane)
//    -- rescaled once per batch: the block-by-block rule of "Tiling:
//    Block-by-Block Softmax" (Paper Notes), in base 2.
//  * At the end the states of the workgroup's lane groups meet in LDS and are
//    merged by the same rule into one (O, LSE) per query row for the
//    workgroup's chunk of keys.
// Workgroup x takes key chunk x % nsplit of head x / nsplit; with more than
// one chunk each writes its normalised fp32 output and LSE to the split-K/V
// partials, which fwd_combine merges.  Causal masking is bottom-right (query
// i sees key j when j <= i + nk - nq); with one query row it masks nothing.
#include "attn_device.h"
#include "attn_launch.h"

namespace attn {

namespace {

constexpr int kDecWaves = 4;  // waves per workgroup
constexpr int kDecLoads = 8;  // K (and V) load instructions per wave batch
constexpr int kDecMaxSplit = 64;  // chunks per head, at most (fwd_combine's limit)

// Sum of x over aligned groups of N lanes (N = 8 or 16), in every lane of
// the group: DPP quad swaps (lane ^ 1, lane ^ 2), then the half-row mirror
// (lane i <-> 7 - i within 8 lanes) and, for 16, the row mirror (i <-> 15 - i).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  x += __builtin_amdgcn_update_dpp(0.f, x, 0xB1, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0.f, x, 0x4E, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0.f, x, 0x141, 0xF, 0xF, false);
  if constexpr (N == 16) x += __builtin_amdgcn_update_dpp(0.f, x, 0x140, 0xF, 0xF, false);
  return x;
}

// q . k over the lane's 8 features, one v_dot2 per bf16 pair.  The pairs are
// taken from the bf16x8 view with shufflevector: a bit_cast of a u32 element
// to bf16x2 was compiled to the same register for all four pairs.
__device__ __forceinline__ float dot8(const u32x4& a, const u32x4& b, float acc) {
  const bf16x8 x = __builtin_bit_cast(bf16x8, a), y = __builtin_bit_cast(bf16x8, b);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 0, 1), __builtin_shufflevector(y, y, 0, 1), acc,
                                        false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 2, 3), __builtin_shufflevector(y, y, 2, 3), acc,
                                        false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 4, 5), __builtin_shufflevector(y, y, 4, 5), acc,
                                        false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, 6, 7), __builtin_shufflevector(y, y, 6, 7), acc,
                                        false);
  return acc;
}

// G: query rows per workgroup (nq <= G).  Q, O: [bh, nq, D]; K, V: [bh, nk, D];
// LSE: [bh, nq].  Chunk s covers keys [s * kchunk, min(nk, (s + 1) * kchunk)).
template <int D, int G, int NL = kDecLoads>
__global__ __launch_bounds__(kDecWaves * 64) void decode_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, float* __restrict__ opart, float* __restrict__ lpart,
    int nq, int nk, long long coff, int kchunk, int nsplit, float c) {
  constexpr int LPK = D / 8;                // lanes per key row
  constexpr int KPI = 64 / LPK;             // key rows per load instruction
  constexpr int KB = NL * KPI;              // keys per wave batch
  constexpr int NG = kDecWaves * KPI;       // lane groups per workgroup
  __shared__ float st_o[G][NG][D];
  __shared__ float st_m[G][NG], st_l[G][NG];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int g = lane / LPK, sub = lane % LPK;
  const int s = (int)(blockIdx.x % (unsigned)nsplit);
  const long long bh = blockIdx.x / (unsigned)nsplit;
  const int k0 = s * kchunk;
  const int k1 = min(nk, k0 + kchunk);
  const uint16_t* Kh = K + (size_t)bh * nk * D + 8 * sub;
  const uint16_t* Vh = V + (size_t)bh * nk * D + 8 * sub;

  u32x4 q[G];
  float m[G], l[G], acc[G][8];
  long long lim[G];  // last key row r sees
#pragma unroll
  for (int r = 0; r < G; ++r) {
    q[r] = r < nq ? *reinterpret_cast<const u32x4*>(Q + ((size_t)bh * nq + r) * D + 8 * sub) : u32x4{0, 0, 0, 0};
    m[r] = -INFINITY;
    l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.f;
    lim[r] = (long long)r + coff;
    if (lim[r] > k1 - 1) lim[r] = k1 - 1;
  }

  for (int kb = k0 + w * KB; kb < k1; kb += kDecWaves * KB) {
    u32x4 kr[NL], vr[NL];
#pragma unroll
    for (int t = 0; t < NL; ++t) {
      const int key = kb + t * KPI + g;
      kr[t] = key < k1 ? *reinterpret_cast<const u32x4*>(Kh + (size_t)key * D) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int t = 0; t < NL; ++t) {
      const int key = kb + t * KPI + g;
      vr[t] = key < k1 ? *reinterpret_cast<const u32x4*>(Vh + (size_t)key * D) : u32x4{0, 0, 0, 0};
    }
    float p[G][NL];
#pragma unroll
    for (int r = 0; r < G; ++r) {
      float mx = m[r];
#pragma unroll
      for (int t = 0; t < NL; ++t) {
        const int key = kb + t * KPI + g;
        const float sc = group_sum<LPK>(dot8(q[r], kr[t], 0.f)) * c;
        p[r][t] = key <= lim[r] ? sc : -INFINITY;
        mx = fmaxf(mx, p[r][t]);
      }
      // A row that has seen no key keeps m = -inf; its exponentials are then
      // taken against 0 and come out 0.
      const float ms = mx == -INFINITY ? 0.f : mx;
      const float corr = fast_exp2(m[r] - ms);
      float sum = 0.f;
#pragma unroll
      for (int t = 0; t < NL; ++t) {
        p[r][t] = fast_exp2(p[r][t] - ms);
        sum += p[r][t];
      }
      l[r] = l[r] * corr + sum;
      m[r] = mx;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[r][e] *= corr;
    }
#pragma unroll
    for (int t = 0; t < NL; ++t) {
      float vf[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vf[2 * i] = __uint_as_float(vr[t][i] << 16);
        vf[2 * i + 1] = __uint_as_float(vr[t][i] & 0xFFFF0000u);
      }
#pragma unroll
      for (int r = 0; r < G; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] += p[r][t] * vf[e];
    }
  }

  // Merge the lane groups' states: group gi = w * KPI + g.
  const int gi = w * KPI + g;
#pragma unroll
  for (int r = 0; r < G; ++r) {
#pragma unroll
    for (int e = 0; e < 8; ++e) st_o[r][gi][8 * sub + e] = acc[r][e];
    if (sub == 0) {
      st_m[r][gi] = m[r];
      st_l[r][gi] = l[r];
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += kDecWaves * 64) {
    const int r = idx / D, e = idx % D;
    if (r >= nq) break;
    float mx = -INFINITY;
#pragma unroll 8
    for (int i = 0; i < NG; ++i) mx = fmaxf(mx, st_m[r][i]);
    const float ms = mx == -INFINITY ? 0.f : mx;
    float lt = 0.f, ot = 0.f;
#pragma unroll 8
    for (int i = 0; i < NG; ++i) {
      const float wgt = fast_exp2(st_m[r][i] - ms);
      lt += wgt * st_l[r][i];
      ot += wgt * st_o[r][i][e];
    }
    // lt == 0: no key of the chunk is visible to row r (O = 0, LSE = -inf).
    const float out = lt > 0.f ? ot / lt : 0.f;
    const float lse = lt > 0.f ? (ms + fast_log2(lt)) * kLn2 : -INFINITY;
    const size_t row = (size_t)bh * nq + r;
    if (nsplit > 1) {
      const size_t prow = ((size_t)bh * nsplit + s) * nq + r;
      opart[prow * D + e] = out;
      if (e == 0) lpart[prow] = lse;
    } else {
      O[row * D + e] = (uint16_t)(pack_bf16x2(out, 0.f) & 0xFFFFu);
      if (e == 0) LSE[row] = lse;
    }
  }
}

template <int D, int G, int NL = kDecLoads>
static hipError_t launch_decode(const FwdArgs& a) {
  const int nsplit = a.nsplit;
  const int kchunk = nsplit > 1 ? a.kchunk : (int)a.nk;
  const long long coff = a.causal ? a.nk - a.n : (long long)a.nk;
  hipLaunchKernelGGL((decode_kernel<D, G, NL>), dim3((unsigned)(nsplit * a.bh)), dim3(kDecWaves * 64), 0,
                     a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (uint16_t*)a.o,
                     a.lse, a.opart, a.lpart, (int)a.n, (int)a.nk, coff, kchunk, nsplit, a.scale * kLog2e);
  return hipGetLastError();
}

template <int D>
static hipError_t decode_d(const FwdArgs& a) {
  if (a.n == 1) return launch_decode<D, 1>(a);
  if (a.n == 2) return launch_decode<D, 2>(a);
  // Four rows hold four output accumulators per lane: half as many loads per
  // batch keep the kernel at 126 VGPRs (four waves per SIMD instead of three;
  // 2-3% faster over 16384 keys, the same over 4096 and 65536).
  return launch_decode<D, 4, kDecLoads / 2>(a);
}

}  // namespace

int decode_max_rows() { return 4; }

int decode_wg_keys(int64_t d) { return kDecWaves * kDecLoads * (64 / (int)(d / 8)); }

hipError_t fwd_decode(const FwdArgs& a) {
  if (a.n < 1 || a.n > decode_max_rows() || a.nk < a.n) return hipErrorInvalidValue;
  if (a.nsplit < 1 || a.nsplit > kDecMaxSplit || (a.nsplit > 1 && (!a.opart || !a.lpart)))
    return hipErrorInvalidValue;
  return a.d == 64 ? decode_d<64>(a) : decode_d<128>(a);
}

}  // namespace attn
