// Internal launch interface between the C ABI (attn_api.hip) and the kernels.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

// Dropout on the probabilities (bf16, square lengths, dense): the element
// (query i, key j) of head bh is kept when word j % 4 of
// Philox4x32-10(counter (j / 4, i, bh, offset), key (seed_lo, seed_hi)) is
// >= thr; kept probabilities are multiplied by keep_scale = 1 / (1 - p).
struct DropArgs {
  uint32_t thr = 0;
  float keep_scale = 1.f;
  uint32_t seed_lo = 0, seed_hi = 0;
  uint32_t offset = 0;
};

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t bh;  // batch * heads
  int64_t n;
  int64_t d;
  bool causal;
  float scale;
  hipStream_t stream;
  // Block-sparse variant (bf16 only): uint8 mask over 128 x 128 blocks of the
  // score matrix, [ceil(n / 128)]^2 per head, heads mask_stride bytes apart
  // (0: one mask for every head).  nullptr: dense.
  const uint8_t* bmask = nullptr;
  int64_t mask_stride = 0;
  // Unequal lengths (bf16 only): `n` is then the query length and nk the key
  // length (nk < 0: square); causal alignment is bottom-right.  With
  // nsplit > 1 the keys are cut into chunks of kchunk (a multiple of 64) and
  // each chunk's normalised output (fp32 [bh, nsplit, n, d]) and LSE
  // ([bh, nsplit, n]) go to opart / lpart, to be merged by fwd_combine.
  int64_t nk = -1;
  int nsplit = 1;
  int kchunk = 0;
  float* opart = nullptr;
  float* lpart = nullptr;
  bool dropout = false;  // with `drop`
  DropArgs drop;
  // Key padding (dense, square lengths): batch b = bh / heads attends only
  // its keys j < klen[b] (device int32 [bh / heads], clamped to [0, n] by the
  // kernels).  nullptr: every key.
  const int* klen = nullptr;
  int heads = 1;
  // Causal sliding window (dense, square lengths): query i sees keys
  // i - window + 1 .. i.  0: no window.
  int window = 0;
};

// Kernel-side view of the unequal-length arguments.
struct QkKernelArgs {
  int nk;      // key length
  int coff;    // causal offset nk - n: query i sees key j when j <= i + coff
  int kchunk;  // keys per split
  int nsplit;
  float* opart;
  float* lpart;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* dsum;  // workspace: D_i = sum_k dO_ik O_ik, float32 [bh, n]
  int64_t bh;
  int64_t n;
  int64_t d;
  bool causal;
  float scale;
  hipStream_t stream;
  const uint8_t* bmask = nullptr;  // as in FwdArgs
  int64_t mask_stride = 0;
  int64_t nk = -1;  // as in FwdArgs
  bool dropout = false;
  DropArgs drop;
  // Unequal lengths: the dQ pass split over nsplit chunks of kchunk keys
  // (whole 64-key tiles); chunk s writes its fp32 partial dQ (scale
  // applied) to dqpart[s][bh][n][d], and a second kernel sums the chunks in
  // order into dq.  nsplit = 1: no split, dqpart unused.
  int nsplit = 1;
  int kchunk = 0;
  float* dqpart = nullptr;
  // bf16 dQ launchers (no dQ split): form D from `o` and `dout` inside the
  // dQ kernel and write it to `dsum`, instead of reading it from there; the
  // dK/dV launch then follows the dQ launch.
  bool dq_forms_dsum = false;
  const int* klen = nullptr;  // as in FwdArgs
  int heads = 1;
  int window = 0;  // as in FwdArgs
};

// Compute units of the current device (cached after the first call).
inline int device_cu_count() {
  static int n = 0;
  if (n == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
  }
  return n;
}

// Start-up placement for heavy_first: pass = CUs per XCD, fill = pass times
// the workgroups of `kernel` that fit on one CU at once (0, 0 when only one
// does: nothing to balance at start).
template <typename K>
inline void start_fill(K kernel, int threads, int& pass, int& fill) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess) per_cu = 1;
  pass = device_cu_count() / 8;
  fill = per_cu > 1 ? pass * per_cu : 0;
  if (fill == 0) pass = 0;
}

// Key count of (batch, head) bh under key padding: klen[bh / heads] clamped
// to [0, n], or n without padding.
__device__ __forceinline__ int padded_keys(const int* klen, int heads, int bh, int n) {
  if (klen == nullptr) return n;
  const int v = klen[bh / heads];
  return v < 0 ? 0 : (v > n ? n : v);
}

// Block size of the block-sparse mask (query and key rows per block).
constexpr int kSparseBlock = 128;

hipError_t fwd_bf16(const FwdArgs& a);
// Merge of the split-K/V partial results into O (bf16) and LSE.
hipError_t fwd_combine(const FwdArgs& a);
// Forward for 1 <= n <= decode_max_rows() query rows over nk >= n keys
// (unequal lengths, no mask other than causal): vector-ALU kernel, split
// over keys as the matrix-core kernel (same partials, merged by fwd_combine).
hipError_t fwd_decode(const FwdArgs& a);
int decode_max_rows();
// Keys one decode workgroup covers in one pass of its waves (the smallest
// chunk that keeps every wave busy).
int decode_wg_keys(int64_t d);
hipError_t fwd_f32(const FwdArgs& a);
// Backward phases; `o` is read only by bwd_dsum, `dq` written only by the
// *_dq launchers, `dk`/`dv` only by the *_dkdv launchers.
hipError_t bwd_dsum(const BwdArgs& a, bool bf16);
hipError_t bwd_bf16_dkdv(const BwdArgs& a);
// dK, dV at d = 64 (dense, square lengths, no dropout): single-role waves.
hipError_t bwd_bf16_dkdv64(const BwdArgs& a);
hipError_t bwd_bf16_dq(const BwdArgs& a);
// Query rows per dQ workgroup of the bf16 kernels for head dimension d.
int bwd_dq_rows(int64_t d);
hipError_t bwd_f32_dkdv(const BwdArgs& a);
hipError_t bwd_f32_dq(const BwdArgs& a);

}  // namespace attn
