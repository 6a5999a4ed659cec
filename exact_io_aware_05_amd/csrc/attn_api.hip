// C ABI of the attention library: host-side validation and dispatch.
// Every check completes before the first HIP call, so an invalid argument
// returns a status without touching the device.
#include <math.h>

#include <mutex>

#include "attn.h"
#include "attn_launch.h"

// Scratch memory of attn_bwd_noalloc (D, float32 [B, H, N]): a fixed device
// array of ATTN_NOALLOC_SCRATCH_BYTES, one copy per GPU, held by the loaded
// code object until the process ends.  In host code `scratch` names a host
// stand-in, never the device memory: its device address is looked up per
// device (scratch_address below) and only that address is used.
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int64_t kMax31 = 2147483647LL;

int check_shape(int64_t B, int64_t H, int64_t N, int64_t d, int dtype) {
  if (dtype != ATTN_BF16 && dtype != ATTN_FP32) return ATTN_E_UNSUPPORTED;
  if (d != 64 && d != 128) return ATTN_E_UNSUPPORTED;
  if (B < 1 || H < 1 || N < 1) return ATTN_E_SHAPE;
  if (B > kMax31 || H > kMax31 || N > kMax31) return ATTN_E_SHAPE;
  if (B * H > kMax31 / N) return ATTN_E_SHAPE;  // B*H*N rows index in 31 bits
  if (N > (1LL << 30) / d) return ATTN_E_SHAPE;  // N*d <= 2^30: byte offsets in a head, plus a
                                                  // tile of padding rows, fit 32 bits
  return ATTN_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Alignment the kernels rely on: tensors are read and written with 16-byte
// vector and buffer->LDS accesses, the float32 row vectors (LSE, D) with
// 4-byte ones.  A contiguous view at an odd element offset is a valid
// pointer of its type and is still refused.
bool al16(const void* p) { return ((uintptr_t)p & 15) == 0; }
template <typename... P>
bool all16(P... p) {
  return (al16(p) && ...);
}
bool al4(const void* p) { return ((uintptr_t)p & 3) == 0; }

// Block-sparse mask arguments (shape already validated): a mask, bf16, and a
// head stride of 0 or at least nb * nb whose last head stays addressable.
int check_mask(const uint8_t* mask, int64_t stride, int64_t B, int64_t H, int64_t N, int dtype) {
  if (!mask) return ATTN_E_NULL;  // read byte by byte: any alignment
  if (dtype != ATTN_BF16) return ATTN_E_UNSUPPORTED;
  if (N > ATTN_SPARSE_MAX_N) return ATTN_E_SHAPE;  // the kernels list a row's tiles in LDS
  const int64_t nb = (N + ATTN_SPARSE_BLOCK - 1) / ATTN_SPARSE_BLOCK;
  if (stride < 0 || (stride != 0 && stride < nb * nb)) return ATTN_E_SHAPE;
  if (stride != 0 && B * H - 1 > (INT64_MAX - nb * nb) / stride) return ATTN_E_SHAPE;
  return ATTN_OK;
}

attn::BwdArgs make_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                       const float* lse, void* dq, void* dk, void* dv, float* dsum, int64_t B, int64_t H, int64_t N,
                       int64_t d, int causal, float scale, void* stream) {
  attn::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.dsum = dsum;
  a.bh = B * H;
  a.n = N;
  a.d = d;
  a.causal = causal != 0;
  a.scale = scale;
  a.stream = (hipStream_t)stream;
  return a;
}

// Split-K/V plan for attn_fwd_qk: number of chunks and keys per chunk.
struct SplitPlan {
  int nsplit;
  int kchunk;
};

// The forward of few query rows over at least as many keys runs the
// vector-ALU decode kernel.
bool use_decode(int64_t Nq, int64_t Nk) { return Nq <= attn::decode_max_rows() && Nq <= Nk; }

SplitPlan split_plan(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int num_splits) {
  const int64_t ktiles = (Nk + 63) / 64;
  int64_t want = num_splits;
  if (num_splits == 0) {
    if (use_decode(Nq, Nk)) {
      // Decode kernel: about four workgroups per CU (256 CUs), each chunk at
      // least one pass of the workgroup's waves.
      const int64_t wgs = B * H;
      const int64_t min_tiles = attn::decode_wg_keys(d) / 64;
      want = (1024 + wgs - 1) / wgs;
      want = want < ktiles / min_tiles ? want : ktiles / min_tiles;
    } else {
      // Matrix-core kernel: about 512 workgroups (two resident per CU over
      // 256 CUs, one round), each chunk at least 4 tiles.  Twice that many
      // was 10-27% slower on prefill shapes (B=1 H=16 1024 queries after
      // 7168 keys: 107 against 78 us): more chunks mostly add fp32
      // partials to write and merge.
      const int64_t wgs = B * H * ((Nq + 127) / 128);
      want = (512 + wgs - 1) / wgs;
      want = want < ktiles / 4 ? want : ktiles / 4;
    }
  }
  if (want > 64) want = 64;
  if (want > ktiles) want = ktiles;
  if (want < 2) return SplitPlan{1, (int)(ktiles * 64)};
  const int64_t tiles_per = (ktiles + want - 1) / want;
  const int64_t ns = (ktiles + tiles_per - 1) / tiles_per;
  if (ns < 2) return SplitPlan{1, (int)(ktiles * 64)};
  return SplitPlan{(int)ns, (int)(tiles_per * 64)};
}

// Split of the backward's dQ pass over keys (unequal lengths): with few
// (head, query block) workgroups, enough chunks for about 256 workgroups (one
// per CU), each chunk at least 4 tiles.  Targets of 512 and 1024 were 2-5%
// and 10-12% slower on prefill shapes (fp32 partials to write and merge),
// 128 was 10-20% slower.
SplitPlan dq_split_plan(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d) {
  const int64_t ktiles = (Nk + 63) / 64;
  const int64_t rows = attn::bwd_dq_rows(d);
  const int64_t wgs = B * H * ((Nq + rows - 1) / rows);
  int64_t want = (256 + wgs - 1) / wgs;
  want = want < ktiles / 4 ? want : ktiles / 4;
  if (want > 64) want = 64;
  if (want < 2) return SplitPlan{1, (int)(ktiles * 64)};
  const int64_t tiles_per = (ktiles + want - 1) / want;
  const int64_t ns = (ktiles + tiles_per - 1) / tiles_per;
  if (ns < 2) return SplitPlan{1, (int)(ktiles * 64)};
  return SplitPlan{(int)ns, (int)(tiles_per * 64)};
}

int check_qk(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int dtype) {
  int st = check_shape(B, H, Nq, d, dtype);
  if (st != ATTN_OK) return st;
  st = check_shape(B, H, Nk, d, dtype);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_BF16) return ATTN_E_UNSUPPORTED;
  return ATTN_OK;
}

// Device address of the current device's copy of `scratch`, looked up once
// per device (hipGetSymbolAddress with that device current) and kept.
constexpr int kMaxDevices = 256;
void* g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return ATTN_E_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

// The backward phases on one stream, D in a.dsum.  bf16: the dQ pass forms
// D (from O and dO) and writes it, then dK/dV reads it; fp32: D first, then
// dK/dV, then dQ.
int run_bwd(attn::BwdArgs a, bool bf16) {
  if (bf16) {
    a.dq_forms_dsum = true;
    if (attn::bwd_bf16_dq(a) != hipSuccess) return ATTN_E_HIP;
    if (attn::bwd_bf16_dkdv(a) != hipSuccess) return ATTN_E_HIP;
    return ATTN_OK;
  }
  if (attn::bwd_dsum(a, false) != hipSuccess) return ATTN_E_HIP;
  if (attn::bwd_f32_dkdv(a) != hipSuccess) return ATTN_E_HIP;
  if (attn::bwd_f32_dq(a) != hipSuccess) return ATTN_E_HIP;
  return ATTN_OK;
}

// Dropout arguments: p in [0, 1) (NaN fails the test); the keep threshold
// and the scale of kept probabilities.
int check_dropout(float p) { return (p >= 0.f && p < 1.f) ? ATTN_OK : ATTN_E_DROPOUT; }

attn::DropArgs make_drop(float p, uint64_t seed, uint64_t offset) {
  attn::DropArgs dr;
  const double t = floor((double)p * 4294967296.0);
  dr.thr = t >= 4294967295.0 ? 0xFFFFFFFFu : (uint32_t)t;
  dr.keep_scale = 1.0f / (1.0f - p);
  dr.seed_lo = (uint32_t)seed;
  dr.seed_hi = (uint32_t)(seed >> 32);
  dr.offset = (uint32_t)offset;
  return dr;
}

}  // namespace

extern "C" {

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_E_NULL: return "a required pointer is NULL";
    case ATTN_E_SHAPE:
      return "invalid shape (B, H, N must be >= 1 and within size limits), block-mask stride or window (>= 1)";
    case ATTN_E_UNSUPPORTED: return "unsupported head dimension (64 or 128) or dtype (bf16 or fp32; block-sparse: bf16)";
    case ATTN_E_SCALE: return "scale must be finite";
    case ATTN_E_WORKSPACE: return "workspace missing or too small";
    case ATTN_E_HIP: return "HIP kernel launch failed";
    case ATTN_E_DROPOUT: return "dropout probability must lie in [0, 1)";
    case ATTN_E_ALIGN: return "a tensor pointer is not 16-byte aligned (LSE and D: 4-byte)";
    case ATTN_E_SCRATCH: return "B * H * N float32 values exceed the fixed scratch of attn_bwd_noalloc";
    default: return "unknown status";
  }
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H, int64_t N,
             int64_t d, int dtype, int causal, float scale, void* stream) {
  if (!q || !k || !v || !o || !lse) return ATTN_E_NULL;
  if (!all16(q, k, v, o) || !al4(lse)) return ATTN_E_ALIGN;
  const int st = check_shape(B, H, N, d, dtype);
  if (st != ATTN_OK) return st;
  if (!isfinite(scale)) return ATTN_E_SCALE;
  attn::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.bh = B * H;
  a.n = N;
  a.d = d;
  a.causal = causal != 0;
  a.scale = scale;
  a.stream = (hipStream_t)stream;
  const hipError_t e = dtype == ATTN_BF16 ? attn::fwd_bf16(a) : attn::fwd_f32(a);
  return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

size_t attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int dtype) {
  if (check_shape(B, H, N, d, dtype) != ATTN_OK) return 0;
  return align256((size_t)(B * H * N) * sizeof(float));
}

int attn_bwd_dsum(const void* o, const void* dout, float* dsum, int64_t B, int64_t H, int64_t N, int64_t d,
                  int dtype, void* stream) {
  if (!o || !dout || !dsum) return ATTN_E_NULL;
  if (!all16(o, dout) || !al4(dsum)) return ATTN_E_ALIGN;
  const int st = check_shape(B, H, N, d, dtype);
  if (st != ATTN_OK) return st;
  attn::BwdArgs a = make_bwd(nullptr, nullptr, nullptr, o, dout, nullptr, nullptr, nullptr, nullptr, dsum, B, H,
                             N, d, 0, 1.0f, stream);
  return attn::bwd_dsum(a, dtype == ATTN_BF16) == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

int attn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, const float* lse, const float* dsum,
                  void* dk, void* dv, int64_t B, int64_t H, int64_t N, int64_t d, int dtype, int causal, float scale,
                  void* stream) {
  if (!q || !k || !v || !dout || !lse || !dsum || !dk || !dv) return ATTN_E_NULL;
  if (!all16(q, k, v, dout, dk, dv) || !al4(lse) || !al4(dsum)) return ATTN_E_ALIGN;
  const int st = check_shape(B, H, N, d, dtype);
  if (st != ATTN_OK) return st;
  if (!isfinite(scale)) return ATTN_E_SCALE;
  attn::BwdArgs a = make_bwd(q, k, v, nullptr, dout, lse, nullptr, dk, dv, (float*)dsum, B, H, N, d, causal,
                             scale, stream);
  const hipError_t e = dtype == ATTN_BF16 ? attn::bwd_bf16_dkdv(a) : attn::bwd_f32_dkdv(a);
  return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

int attn_bwd_dq(const void* q, const void* k, const void* v, const void* dout, const float* lse, const float* dsum,
                void* dq, int64_t B, int64_t H, int64_t N, int64_t d, int dtype, int causal, float scale,
                void* stream) {
  if (!q || !k || !v || !dout || !lse || !dsum || !dq) return ATTN_E_NULL;
  if (!all16(q, k, v, dout, dq) || !al4(lse) || !al4(dsum)) return ATTN_E_ALIGN;
  const int st = check_shape(B, H, N, d, dtype);
  if (st != ATTN_OK) return st;
  if (!isfinite(scale)) return ATTN_E_SCALE;
  attn::BwdArgs a = make_bwd(q, k, v, nullptr, dout, lse, dq, nullptr, nullptr, (float*)dsum, B, H, N, d, causal,
                             scale, stream);
  const hipError_t e = dtype == ATTN_BF16 ? attn::bwd_bf16_dq(a) : attn::bwd_f32_dq(a);
  return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

int attn_bwd_dq_dsum(const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, float* dsum, void* dq, int64_t B, int64_t H, int64_t N, int64_t d, int dtype,
                     int causal, float scale, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dsum || !dq) return ATTN_E_NULL;
  if (!all16(q, k, v, o, dout, dq) || !al4(lse) || !al4(dsum)) return ATTN_E_ALIGN;
  const int st = check_shape(B, H, N, d, dtype);
  if (st != ATTN_OK) return st;
  if (!isfinite(scale)) return ATTN_E_SCALE;
  attn::BwdArgs a = make_bwd(q, k, v, o, dout, lse, dq, nullptr, nullptr, dsum, B, H, N, d, causal, scale, stream);
  if (dtype == ATTN_BF16) {
    a.dq_forms_dsum = true;
    return attn::bwd_bf16_dq(a) == hipSuccess ? ATTN_OK : ATTN_E_HIP;
  }
  if (attn::bwd_dsum(a, false) != hipSuccess) return ATTN_E_HIP;
  return attn::bwd_f32_dq(a) == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
             void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N, int64_t d, int dtype, int causal,
             float scale, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return ATTN_E_NULL;
  if (!all16(q, k, v, o, dout, dq, dk, dv) || !al4(lse)) return ATTN_E_ALIGN;
  const int st = check_shape(B, H, N, d, dtype);
  if (st != ATTN_OK) return st;
  if (!isfinite(scale)) return ATTN_E_SCALE;
  if (!workspace || workspace_bytes < attn_bwd_workspace_bytes(B, H, N, d, dtype) ||
      ((uintptr_t)workspace & 255) != 0)
    return ATTN_E_WORKSPACE;
  attn::BwdArgs a =
      make_bwd(q, k, v, o, dout, lse, dq, dk, dv, (float*)workspace, B, H, N, d, causal, scale, stream);
  return run_bwd(a, dtype == ATTN_BF16);
}

int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N, int64_t d,
                     int dtype, int causal, float scale, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return ATTN_E_NULL;
  if (!all16(q, k, v, o, dout, dq, dk, dv) || !al4(lse)) return ATTN_E_ALIGN;
  const int st = check_shape(B, H, N, d, dtype);
  if (st != ATTN_OK) return st;
  if (!isfinite(scale)) return ATTN_E_SCALE;
  if ((size_t)(B * H * N) * sizeof(float) > (size_t)ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_E_SCRATCH;
  void* ws = nullptr;
  const int sst = scratch_address(&ws);
  if (sst != ATTN_OK) return sst;
  attn::BwdArgs a = make_bwd(q, k, v, o, dout, lse, dq, dk, dv, (float*)ws, B, H, N, d, causal, scale, stream);
  return run_bwd(a, dtype == ATTN_BF16);
}

int attn_fwd_kpad(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                  int64_t N, int64_t d, int dtype, int causal, float scale, const int32_t* key_len, void* stream) {
  if (!q || !k || !v || !o || !lse || !key_len) return ATTN_E_NULL;
  if (!all16(q, k, v, o) || !al4(lse) || !al4(key_len)) return ATTN_E_ALIGN;
  const int st = check_shape(B, H, N, d, dtype);
  if (st != ATTN_OK) return st;
  if (!isfinite(scale)) return ATTN_E_SCALE;
  attn::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.bh = B * H;
  a.n = N;
  a.d = d;
  a.causal = causal != 0;
  a.scale = scale;
  a.stream = (hipStream_t)stream;
  a.klen = key_len;
  a.heads = (int)H;
  const hipError_t e = dtype == ATTN_BF16 ? attn::fwd_bf16(a) : attn::fwd_f32(a);
  return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

int attn_bwd_kpad(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                  void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N, int64_t d, int dtype, int causal,
                  float scale, const int32_t* key_len, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !key_len) return ATTN_E_NULL;
  if (!all16(q, k, v, o, dout, dq, dk, dv) || !al4(lse) || !al4(key_len)) return ATTN_E_ALIGN;
  const int st = check_shape(B, H, N, d, dtype);
  if (st != ATTN_OK) return st;
  if (!isfinite(scale)) return ATTN_E_SCALE;
  if (!workspace || workspace_bytes < attn_bwd_workspace_bytes(B, H, N, d, dtype) ||
      ((uintptr_t)workspace & 255) != 0)
    return ATTN_E_WORKSPACE;
  attn::BwdArgs a =
      make_bwd(q, k, v, o, dout, lse, dq, dk, dv, (float*)workspace, B, H, N, d, causal, scale, stream);
  a.klen = key_len;
  a.heads = (int)H;
  return run_bwd(a, dtype == ATTN_BF16);
}

int attn_fwd_window(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                    int64_t N, int64_t d, int dtype, int64_t window, float scale, void* stream) {
  if (!q || !k || !v || !o || !lse) return ATTN_E_NULL;
  if (!all16(q, k, v, o) || !al4(lse)) return ATTN_E_ALIGN;
  const int st = check_shape(B, H, N, d, dtype);
  if (st != ATTN_OK) return st;
  if (window < 1) return ATTN_E_SHAPE;
  if (!isfinite(scale)) return ATTN_E_SCALE;
  attn::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.bh = B * H;
  a.n = N;
  a.d = d;
  a.causal = true;
  a.scale = scale;
  a.stream = (hipStream_t)stream;
  a.window = window < N ? (int)window : 0;  // a window of N keys or more is the causal mask
  const hipError_t e = dtype == ATTN_BF16 ? attn::fwd_bf16(a) : attn::fwd_f32(a);
  return e == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

int attn_bwd_window(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N, int64_t d,
                    int dtype, int64_t window, float scale, void* workspace, size_t workspace_bytes,
                    void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return ATTN_E_NULL;
  if (!all16(q, k, v, o, dout, dq, dk, dv) || !al4(lse)) return ATTN_E_ALIGN;
  const int st = check_shape(B, H, N, d, dtype);
  if (st != ATTN_OK) return st;
  if (window < 1) return ATTN_E_SHAPE;
  if (!isfinite(scale)) return ATTN_E_SCALE;
  if (!workspace || workspace_bytes < attn_bwd_workspace_bytes(B, H, N, d, dtype) ||
      ((uintptr_t)workspace & 255) != 0)
    return ATTN_E_WORKSPACE;
  attn::BwdArgs a =
      make_bwd(q, k, v, o, dout, lse, dq, dk, dv, (float*)workspace, B, H, N, d, 1, scale, stream);
  a.window = window < N ? (int)window : 0;
  return run_bwd(a, dtype == ATTN_BF16);
}

int attn_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                         int64_t N, int64_t d, int dtype, int causal, float scale, const uint8_t* block_mask,
                         int64_t mask_head_stride, void* stream) {
  if (!q || !k || !v || !o || !lse) return ATTN_E_NULL;
  if (!all16(q, k, v, o) || !al4(lse)) return ATTN_E_ALIGN;
  int st = check_shape(B, H, N, d, dtype);
  if (st != ATTN_OK) return st;
  st = check_mask(block_mask, mask_head_stride, B, H, N, dtype);
  if (st != ATTN_OK) return st;
  if (!isfinite(scale)) return ATTN_E_SCALE;
  attn::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.bh = B * H;
  a.n = N;
  a.d = d;
  a.causal = causal != 0;
  a.scale = scale;
  a.stream = (hipStream_t)stream;
  a.bmask = block_mask;
  a.mask_stride = mask_head_stride;
  return attn::fwd_bf16(a) == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

int attn_bwd_blocksparse(const void* q, const void* k, const void* v, const void* o, const void* dout,
                         const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N, int64_t d,
                         int dtype, int causal, float scale, const uint8_t* block_mask, int64_t mask_head_stride,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return ATTN_E_NULL;
  if (!all16(q, k, v, o, dout, dq, dk, dv) || !al4(lse)) return ATTN_E_ALIGN;
  int st = check_shape(B, H, N, d, dtype);
  if (st != ATTN_OK) return st;
  st = check_mask(block_mask, mask_head_stride, B, H, N, dtype);
  if (st != ATTN_OK) return st;
  if (!isfinite(scale)) return ATTN_E_SCALE;
  if (!workspace || workspace_bytes < attn_bwd_workspace_bytes(B, H, N, d, dtype) ||
      ((uintptr_t)workspace & 255) != 0)
    return ATTN_E_WORKSPACE;
  attn::BwdArgs a =
      make_bwd(q, k, v, o, dout, lse, dq, dk, dv, (float*)workspace, B, H, N, d, causal, scale, stream);
  a.bmask = block_mask;
  a.mask_stride = mask_head_stride;
  return run_bwd(a, true);
}

int attn_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H,
                     int64_t N, int64_t d, int dtype, int causal, float scale, float p_drop, uint64_t seed,
                     uint64_t offset, void* stream) {
  if (!q || !k || !v || !o || !lse) return ATTN_E_NULL;
  if (!all16(q, k, v, o) || !al4(lse)) return ATTN_E_ALIGN;
  int st = check_shape(B, H, N, d, dtype);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_BF16) return ATTN_E_UNSUPPORTED;
  if (!isfinite(scale)) return ATTN_E_SCALE;
  st = check_dropout(p_drop);
  if (st != ATTN_OK) return st;
  attn::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.bh = B * H;
  a.n = N;
  a.d = d;
  a.causal = causal != 0;
  a.scale = scale;
  a.stream = (hipStream_t)stream;
  a.dropout = true;
  a.drop = make_drop(p_drop, seed, offset);
  return attn::fwd_bf16(a) == hipSuccess ? ATTN_OK : ATTN_E_HIP;
}

int attn_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                     void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N, int64_t d, int dtype, int causal,
                     float scale, float p_drop, uint64_t seed, uint64_t offset, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return ATTN_E_NULL;
  if (!all16(q, k, v, o, dout, dq, dk, dv) || !al4(lse)) return ATTN_E_ALIGN;
  int st = check_shape(B, H, N, d, dtype);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_BF16) return ATTN_E_UNSUPPORTED;
  if (!isfinite(scale)) return ATTN_E_SCALE;
  st = check_dropout(p_drop);
  if (st != ATTN_OK) return st;
  if (!workspace || workspace_bytes < attn_bwd_workspace_bytes(B, H, N, d, dtype) ||
      ((uintptr_t)workspace & 255) != 0)
    return ATTN_E_WORKSPACE;
  attn::BwdArgs a =
      make_bwd(q, k, v, o, dout, lse, dq, dk, dv, (float*)workspace, B, H, N, d, causal, scale, stream);
  a.dropout = true;
  a.drop = make_drop(p_drop, seed, offset);
  return run_bwd(a, true);
}

size_t attn_fwd_qk_workspace_bytes(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int dtype,
                                   int num_splits) {
  if (check_qk(B, H, Nq, Nk, d, dtype) != ATTN_OK || num_splits < 0 || num_splits > 64) return 0;
  const SplitPlan sp = split_plan(B, H, Nq, Nk, d, num_splits);
  if (sp.nsplit < 2) return 0;
  const size_t rows = (size_t)(B * H * Nq) * (size_t)sp.nsplit;
  return align256(rows * (size_t)d * sizeof(float)) + align256(rows * sizeof(float));
}

int attn_fwd_qk(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t H, int64_t Nq,
                int64_t Nk, int64_t d, int dtype, int causal, float scale, int num_splits, void* workspace,
                size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !lse) return ATTN_E_NULL;
  if (!all16(q, k, v, o) || !al4(lse)) return ATTN_E_ALIGN;
  const int st = check_qk(B, H, Nq, Nk, d, dtype);
  if (st != ATTN_OK) return st;
  if (num_splits < 0 || num_splits > 64) return ATTN_E_SHAPE;
  if (!isfinite(scale)) return ATTN_E_SCALE;
  const SplitPlan sp = split_plan(B, H, Nq, Nk, d, num_splits);
  const size_t need = attn_fwd_qk_workspace_bytes(B, H, Nq, Nk, d, dtype, num_splits);
  if (need > 0 && (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255) != 0))
    return ATTN_E_WORKSPACE;
  attn::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.bh = B * H;
  a.n = Nq;
  a.d = d;
  a.causal = causal != 0;
  a.scale = scale;
  a.stream = (hipStream_t)stream;
  a.nk = Nk;
  a.nsplit = sp.nsplit;
  a.kchunk = sp.kchunk;
  if (sp.nsplit > 1) {
    const size_t rows = (size_t)(B * H * Nq) * (size_t)sp.nsplit;
    a.opart = (float*)workspace;
    a.lpart = (float*)((char*)workspace + align256(rows * (size_t)d * sizeof(float)));
  }
  if ((use_decode(Nq, Nk) ? attn::fwd_decode(a) : attn::fwd_bf16(a)) != hipSuccess) return ATTN_E_HIP;
  if (sp.nsplit > 1 && attn::fwd_combine(a) != hipSuccess) return ATTN_E_HIP;
  return ATTN_OK;
}

size_t attn_bwd_qk_workspace_bytes(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int dtype) {
  if (check_qk(B, H, Nq, Nk, d, dtype) != ATTN_OK) return 0;
  const size_t dbytes = align256((size_t)(B * H * Nq) * sizeof(float));
  const SplitPlan sp = dq_split_plan(B, H, Nq, Nk, d);
  if (sp.nsplit < 2) return dbytes;
  return dbytes + align256((size_t)sp.nsplit * (size_t)(B * H * Nq) * (size_t)d * sizeof(float));
}

int attn_bwd_qk(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int dtype,
                int causal, float scale, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return ATTN_E_NULL;
  if (!all16(q, k, v, o, dout, dq, dk, dv) || !al4(lse)) return ATTN_E_ALIGN;
  const int st = check_qk(B, H, Nq, Nk, d, dtype);
  if (st != ATTN_OK) return st;
  if (!isfinite(scale)) return ATTN_E_SCALE;
  if (!workspace || workspace_bytes < attn_bwd_qk_workspace_bytes(B, H, Nq, Nk, d, dtype) ||
      ((uintptr_t)workspace & 255) != 0)
    return ATTN_E_WORKSPACE;
  attn::BwdArgs a =
      make_bwd(q, k, v, o, dout, lse, dq, dk, dv, (float*)workspace, B, H, Nq, d, causal, scale, stream);
  a.nk = Nk;
  const SplitPlan sp = dq_split_plan(B, H, Nq, Nk, d);
  if (sp.nsplit > 1) {
    a.nsplit = sp.nsplit;
    a.kchunk = sp.kchunk;
    a.dqpart = (float*)((char*)workspace + align256((size_t)(B * H * Nq) * sizeof(float)));
  }
  // Without a dQ split the dQ pass forms D, as in attn_bwd; with one, each
  // chunk's workgroups would form it again, so D comes first.
  if (sp.nsplit <= 1) return run_bwd(a, true);
  if (attn::bwd_dsum(a, true) != hipSuccess) return ATTN_E_HIP;
  if (attn::bwd_bf16_dkdv(a) != hipSuccess) return ATTN_E_HIP;
  if (attn::bwd_bf16_dq(a) != hipSuccess) return ATTN_E_HIP;
  return ATTN_OK;
}

}  // extern "C"
