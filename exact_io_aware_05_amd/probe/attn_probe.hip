// Diagnostic microbenchmarks for gfx950 behind design choices of the
// attention kernels.  Built into libattn_probe.so, separate from the
// attention library; run by `python bench.py --probes`.
//
//  * probe_atomic_dq: the fp32 atomic-add traffic a dQ accumulated with
//    atomics would need (one workgroup per head and 128-key block adding a
//    64 x d tile for each 64-row query tile it visits), against plain stores
//    of the same tiles.
//  * probe_issue_mix: cycles per iteration (s_memtime) of fixed instruction
//    mixes -- 16 v_mfma_f32_32x32x16_bf16 with vector instructions placed
//    between them or after them -- at one or two waves per SIMD.
//  * probe_mfma_rate: every SIMD of every CU runs independent MFMAs back to
//    back; the achieved bf16 rate and the shader clock under that load
//    (s_memtime cycles over event time).
//  * probe_read_bw: HBM read bandwidth of a plain streaming kernel -- each
//    workgroup reads a contiguous share of a buffer in 16-byte loads (1 KiB
//    per wave instruction, as the decode kernel's), a fixed number in flight
//    per thread -- for a given grid size.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <vector>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- atomics
template <int D, bool ATOMIC>
__global__ __launch_bounds__(256) void atomic_dq_kernel(float* acc, int heads, int n, int causal) {
  const int nblk = n / 128;
  const int pid = blockIdx.x;
  const int x = pid & 7, s = pid >> 3;  // XCD, then its workgroups: heads grouped per XCD
  const int hx = heads / 8;
  const int head = x * hx + s / nblk;
  const int blk = s % nblk;
  const int t0 = causal ? 2 * blk : 0;
  float* base = acc + (size_t)head * n * D;
  for (int t = t0; t < n / 64; ++t) {
    float* tile = base + (size_t)t * 64 * D;
#pragma unroll
    for (int j = 0; j < 64 * D / 256; ++j) {
      const int i = threadIdx.x + 256 * j;
      if constexpr (ATOMIC)
        __hip_atomic_fetch_add(tile + i, 1.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        tile[i] = 1.0f;
    }
  }
}

template <int D>
hipError_t run_atomic(int heads, int n, int causal, int atomic, int reps, float* ms, long long* bad) {
  const size_t elems = (size_t)heads * n * D;
  float* acc = nullptr;
  hipError_t e = hipMalloc(&acc, elems * sizeof(float));
  if (e != hipSuccess) return e;
  const int grid = heads * (n / 128);
  auto launch = [&]() {
    if (atomic)
      atomic_dq_kernel<D, true><<<grid, 256>>>(acc, heads, n, causal);
    else
      atomic_dq_kernel<D, false><<<grid, 256>>>(acc, heads, n, causal);
  };
  hipEvent_t a = nullptr, b = nullptr;
  std::vector<float> h;
  if ((e = hipMemset(acc, 0, elems * sizeof(float))) != hipSuccess) goto done;
  launch();  // warm-up
  if ((e = hipDeviceSynchronize()) != hipSuccess) goto done;
  if ((e = hipMemset(acc, 0, elems * sizeof(float))) != hipSuccess) goto done;
  if ((e = hipEventCreate(&a)) != hipSuccess || (e = hipEventCreate(&b)) != hipSuccess) goto done;
  if ((e = hipEventRecord(a)) != hipSuccess) goto done;
  for (int r = 0; r < reps; ++r) launch();
  if ((e = hipEventRecord(b)) != hipSuccess || (e = hipEventSynchronize(b)) != hipSuccess) goto done;
  if ((e = hipGetLastError()) != hipSuccess) goto done;
  if ((e = hipEventElapsedTime(ms, a, b)) != hipSuccess) goto done;
  *ms /= (float)reps;
  // Check: every element of row q was added once per key block that visits
  // its query tile, per repetition (plain stores leave 1).
  h.resize(elems);
  if ((e = hipMemcpy(h.data(), acc, elems * sizeof(float), hipMemcpyDeviceToHost)) != hipSuccess) goto done;
  *bad = 0;
  for (int hd = 0; hd < heads; ++hd)
    for (int q = 0; q < n; ++q) {
      const int t = q / 64;
      const int cnt = causal ? t / 2 + 1 : n / 128;
      const float want = atomic ? (float)(cnt * reps) : 1.0f;
      for (int d = 0; d < D; ++d) *bad += h[((size_t)hd * n + q) * D + d] != want;
    }
done:
  if (a) (void)hipEventDestroy(a);
  if (b) (void)hipEventDestroy(b);
  (void)hipFree(acc);
  return e;
}

// ---------------------------------------------------------------- issue mix
constexpr int kIters = 2000;
#define PF1(r) "v_fma_f32 %[x" #r "], %[x" #r "], %[y], %[z]\n\t"
#define PE1(r) "v_exp_f32 %[x" #r "], %[x" #r "]\n\t"
#define PMF(c) "v_mfma_f32_32x32x16_bf16 %[c" #c "], %[a], %[b], %[c" #c "]\n\t"
#define PG4 PF1(0) PF1(1) PF1(2) PF1(3)
#define PG6 PF1(0) PF1(1) PF1(2) PF1(3) PF1(4) PF1(5)
#define PG7 PF1(0) PF1(1) PF1(2) PF1(3) PF1(4) PF1(5) PF1(6)
#define PG8 PF1(0) PF1(1) PF1(2) PF1(3) PF1(4) PF1(5) PF1(6) PF1(7)
#define PGE PE1(0) PF1(1) PF1(2) PF1(3)
#define PGL "ds_read_b128 %[l], %[ad] offset:0\n\t" PF1(0) PF1(1) PF1(2) PF1(3) "s_waitcnt lgkmcnt(0)\n\t"
#define PX16(G) PMF(0) G PMF(1) G PMF(2) G PMF(3) G PMF(0) G PMF(1) G PMF(2) G PMF(3) G \
                PMF(0) G PMF(1) G PMF(2) G PMF(3) G PMF(0) G PMF(1) G PMF(2) G PMF(3) G
#define PM16 PMF(0) PMF(1) PMF(2) PMF(3) PMF(0) PMF(1) PMF(2) PMF(3) PMF(0) PMF(1) PMF(2) PMF(3) PMF(0) PMF(1) PMF(2) PMF(3)
#define PF16 PG4 PG4 PG4 PG4
#define PE16 PE1(0) PE1(1) PE1(2) PE1(3) PE1(0) PE1(1) PE1(2) PE1(3) PE1(0) PE1(1) PE1(2) PE1(3) PE1(0) PE1(1) PE1(2) PE1(3)
#define POUTS [c0] "+v"(c0), [c1] "+v"(c1), [c2] "+v"(c2), [c3] "+v"(c3), [x0] "+v"(x[0]), [x1] "+v"(x[1]), \
              [x2] "+v"(x[2]), [x3] "+v"(x[3]), [x4] "+v"(x[4]), [x5] "+v"(x[5]), [x6] "+v"(x[6]), \
              [x7] "+v"(x[7]), [l] "=&v"(l)
#define PINS [a] "v"(a), [b] "v"(b), [y] "v"(y), [z] "v"(z), [ad] "v"(ad)

// One workgroup per CU (the LDS pad keeps a second one off the CU), one or
// two waves per SIMD; each wave records its cycles for kIters iterations.
template <int MIX>
__global__ __launch_bounds__(512) void issue_mix_kernel(float* out, long long* cyc) {
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = threadIdx.x * 1e-3f + i;
  const float y = 0.999f, z = 1e-6f;
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  f32x4 l = {};
  const s16x8 a = {1, 2, 3, 4, 5, 6, 7, 8}, b = {1, 1, 1, 1, 1, 1, 1, 1};
  __shared__ float pad[23000];
  pad[threadIdx.x * 40] = x[0];  // threadIdx.x < 512: index < 20480
  __syncthreads();
  x[0] += pad[(threadIdx.x * 40 + 40) % 23000] * 0.f;
  const unsigned ad = (threadIdx.x & 63) * 16u;  // LDS bytes 0 .. 1023
  const long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < kIters; ++it) {
    if constexpr (MIX == 0) asm volatile(PM16 : POUTS : PINS);
    else if constexpr (MIX == 1) asm volatile(PX16(PG4) : POUTS : PINS);
    else if constexpr (MIX == 2) asm volatile(PX16(PG6) : POUTS : PINS);
    else if constexpr (MIX == 3) asm volatile(PX16(PG7) : POUTS : PINS);
    else if constexpr (MIX == 4) asm volatile(PX16(PG8) : POUTS : PINS);
    else if constexpr (MIX == 5) asm volatile(PX16(PGE) : POUTS : PINS);
    else if constexpr (MIX == 6) asm volatile(PM16 PF16 PF16 PF16 PF16 : POUTS : PINS);
    else if constexpr (MIX == 7) asm volatile(PF16 PF16 PF16 PF16 : POUTS : PINS);
    else if constexpr (MIX == 8) asm volatile(PE16 PE16 PE16 PE16 : POUTS : PINS);
    else if constexpr (MIX == 9) asm volatile(PX16(PGL) : POUTS : PINS);
    asm volatile("" : "+v"(l));
  }
  const long long t1 = __builtin_amdgcn_s_memtime();
  float sum = l[0] + l[1];
#pragma unroll
  for (int i = 0; i < 8; ++i) sum += x[i];
#pragma unroll
  for (int i = 0; i < 16; ++i) sum += c0[i] + c1[i] + c2[i] + c3[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = sum;
  if ((threadIdx.x & 63) == 0) cyc[blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64] = t1 - t0;
}

template <int MIX>
void launch_mix(int grid, int threads, float* out, long long* cyc) {
  issue_mix_kernel<MIX><<<grid, threads>>>(out, cyc);
}

// ---------------------------------------------------------------- MFMA rate
__global__ __launch_bounds__(256) void mfma_rate_kernel(float* out, long long* cyc, int iters) {
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  const s16x8 a = {1, 2, 3, 4, 5, 6, 7, 8}, b = {1, 1, 1, 1, 1, 1, 1, 1};
  const long long t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    asm volatile(PMF(0) PMF(1) PMF(2) PMF(3) : [c0] "+v"(c0), [c1] "+v"(c1), [c2] "+v"(c2), [c3] "+v"(c3)
                 : [a] "v"(a), [b] "v"(b));
  }
  const long long t1 = __builtin_amdgcn_s_memtime();
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) sum += c0[i] + c1[i] + c2[i] + c3[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = sum;
  if ((threadIdx.x & 63) == 0) cyc[blockIdx.x * 4 + threadIdx.x / 64] = t1 - t0;
}

// ---------------------------------------------------------------- HBM read
template <int U>
__global__ __launch_bounds__(256) void read_kernel(const uint4* __restrict__ p, long long n16, unsigned* out) {
  const long long per = (n16 + gridDim.x - 1) / gridDim.x;
  const long long c0 = (long long)blockIdx.x * per;
  const long long c1 = c0 + per < n16 ? c0 + per : n16;
  unsigned x = 0;
  for (long long i = c0 + threadIdx.x; i < c1; i += 256LL * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long long idx = i + 256LL * u;
      v[u] = idx < c1 ? p[idx] : uint4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = x;
}

}  // namespace

extern "C" {

// fp32 atomic adds of a dQ accumulated by key blocks: d (64 or 128), heads
// (a multiple of 8), n (a multiple of 128), causal (only query tiles at or
// after the block's first key), atomic (1: atomic adds; 0: plain stores of
// the same tiles), reps timed launches.  Writes the average ms per launch
// and the number of elements that end with the wrong count.  Returns a
// hipError_t (hipErrorInvalidValue for unsupported sizes).
int probe_atomic_dq(int d, int heads, int n, int causal, int atomic, int reps, float* ms, long long* mismatches) {
  if (!ms || !mismatches || heads <= 0 || heads % 8 || n <= 0 || n % 128 || reps <= 0) return hipErrorInvalidValue;
  if (d == 64) return run_atomic<64>(heads, n, causal, atomic, reps, ms, mismatches);
  if (d == 128) return run_atomic<128>(heads, n, causal, atomic, reps, ms, mismatches);
  return hipErrorInvalidValue;
}

// Cycles per iteration of instruction mix `mix` (0 .. 9) with one or two
// waves per SIMD on every CU: the mean over waves and the largest.
//   0: 16 MFMA                       5: 16 x (MFMA, exp, 3 FMA)
//   1: 16 x (MFMA, 4 FMA)            6: 16 MFMA, then 64 FMA
//   2: 16 x (MFMA, 6 FMA)            7: 64 FMA
//   3: 16 x (MFMA, 7 FMA)            8: 64 exp
//   4: 16 x (MFMA, 8 FMA)            9: 16 x (MFMA, LDS read, 4 FMA, wait for the read)
int probe_issue_mix(int mix, int waves_per_simd, int num_cus, double* mean_cycles, double* max_cycles) {
  if (!mean_cycles || !max_cycles || mix < 0 || mix > 9 || waves_per_simd < 1 || waves_per_simd > 2 || num_cus <= 0)
    return hipErrorInvalidValue;
  const int threads = 256 * waves_per_simd, grid = num_cus, nw = grid * threads / 64;
  float* out = nullptr;
  long long* cyc = nullptr;
  hipError_t e = hipMalloc(&out, (size_t)grid * threads * sizeof(float));
  if (e == hipSuccess) e = hipMalloc(&cyc, (size_t)nw * sizeof(long long));
  for (int rep = 0; rep < 2 && e == hipSuccess; ++rep) {  // the first launch warms up
    switch (mix) {
      case 0: launch_mix<0>(grid, threads, out, cyc); break;
      case 1: launch_mix<1>(grid, threads, out, cyc); break;
      case 2: launch_mix<2>(grid, threads, out, cyc); break;
      case 3: launch_mix<3>(grid, threads, out, cyc); break;
      case 4: launch_mix<4>(grid, threads, out, cyc); break;
      case 5: launch_mix<5>(grid, threads, out, cyc); break;
      case 6: launch_mix<6>(grid, threads, out, cyc); break;
      case 7: launch_mix<7>(grid, threads, out, cyc); break;
      case 8: launch_mix<8>(grid, threads, out, cyc); break;
      default: launch_mix<9>(grid, threads, out, cyc); break;
    }
    e = hipGetLastError();
    if (e == hipSuccess) e = hipDeviceSynchronize();
  }
  if (e == hipSuccess) {
    std::vector<long long> h(nw);
    e = hipMemcpy(h.data(), cyc, nw * sizeof(long long), hipMemcpyDeviceToHost);
    double s = 0.0, mx = 0.0;
    for (long long v : h) {
      s += (double)v;
      mx = (double)v > mx ? (double)v : mx;
    }
    *mean_cycles = s / nw / kIters;
    *max_cycles = mx / kIters;
  }
  (void)hipFree(out);
  (void)hipFree(cyc);
  return e;
}

// Back-to-back independent MFMAs on four waves (one per SIMD) of `num_cus`
// workgroups for `iters` iterations of 4 MFMAs: achieved bf16 TFLOP/s and
// the average shader clock in GHz (s_memtime cycles over event time).
int probe_mfma_rate(int num_cus, int iters, double* tflops, double* ghz) {
  if (!tflops || !ghz || num_cus <= 0 || iters <= 0) return hipErrorInvalidValue;
  const int grid = num_cus, nw = grid * 4;
  float* out = nullptr;
  long long* cyc = nullptr;
  hipEvent_t a = nullptr, b = nullptr;
  float ms = 0.f;
  hipError_t e = hipMalloc(&out, (size_t)grid * 256 * sizeof(float));
  if (e == hipSuccess) e = hipMalloc(&cyc, (size_t)nw * sizeof(long long));
  if (e == hipSuccess) e = hipEventCreate(&a);
  if (e == hipSuccess) e = hipEventCreate(&b);
  if (e == hipSuccess) {
    mfma_rate_kernel<<<grid, 256>>>(out, cyc, iters);  // warm-up
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipEventRecord(a);
  if (e == hipSuccess) {
    mfma_rate_kernel<<<grid, 256>>>(out, cyc, iters);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipEventRecord(b);
  if (e == hipSuccess) e = hipEventSynchronize(b);
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
  if (e == hipSuccess) {
    std::vector<long long> h(nw);
    e = hipMemcpy(h.data(), cyc, nw * sizeof(long long), hipMemcpyDeviceToHost);
    double s = 0.0;
    for (long long v : h) s += (double)v;
    const double flops = (double)nw * iters * 4 * (2.0 * 32 * 32 * 16);
    *tflops = flops / (ms * 1e-3) / 1e12;
    *ghz = s / nw / (ms * 1e-3) / 1e9;
  }
  if (a) (void)hipEventDestroy(a);
  if (b) (void)hipEventDestroy(b);
  (void)hipFree(out);
  (void)hipFree(cyc);
  return e;
}

// HBM read bandwidth: `bytes` (a multiple of 16) read by `grid` workgroups
// of 256 threads, `unroll` (4, 8 or 16) 16-byte loads in flight per thread;
// the average ms of `reps` launches after one warm-up launch.
int probe_read_bw(long long bytes, int grid, int unroll, int reps, float* ms) {
  if (!ms || bytes <= 0 || bytes % 16 || grid <= 0 || reps <= 0) return hipErrorInvalidValue;
  if (unroll != 4 && unroll != 8 && unroll != 16) return hipErrorInvalidValue;
  const long long n16 = bytes / 16;
  uint4* buf = nullptr;
  unsigned* out = nullptr;
  hipEvent_t a = nullptr, b = nullptr;
  hipError_t e = hipMalloc(&buf, (size_t)bytes);
  if (e == hipSuccess) e = hipMalloc(&out, (size_t)grid * 256 * sizeof(unsigned));
  if (e == hipSuccess) e = hipMemset(buf, 0x5A, (size_t)bytes);
  if (e == hipSuccess) e = hipEventCreate(&a);
  if (e == hipSuccess) e = hipEventCreate(&b);
  auto launch = [&]() {
    if (unroll == 4) read_kernel<4><<<grid, 256>>>(buf, n16, out);
    else if (unroll == 8) read_kernel<8><<<grid, 256>>>(buf, n16, out);
    else read_kernel<16><<<grid, 256>>>(buf, n16, out);
    return hipGetLastError();
  };
  if (e == hipSuccess) e = launch();
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipEventRecord(a);
  for (int r = 0; r < reps && e == hipSuccess; ++r) e = launch();
  if (e == hipSuccess) e = hipEventRecord(b);
  if (e == hipSuccess) e = hipEventSynchronize(b);
  if (e == hipSuccess) e = hipEventElapsedTime(ms, a, b);
  if (e == hipSuccess) *ms /= reps;
  if (a) (void)hipEventDestroy(a);
  if (b) (void)hipEventDestroy(b);
  (void)hipFree(buf);
  (void)hipFree(out);
  return e;
}

}  // extern "C"
