// C-ABI entry points: host-side validation, dispatch and error mapping.
// Every check runs before any HIP call, in the order the header states.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <mutex>

#include "../../include/fa.h"
#include "fa_launch.hpp"

namespace {

constexpr int kVersion = 100;  // 0.1.0
constexpr unsigned long long kSignKey = 0x5A17C0DEull;  // fixed rotation of FA_FP8_E4M3

bool log_enabled() {
  const char* e = std::getenv("FA_LOG");
  return e != nullptr && e[0] == '1';
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool bf16_dim_ok(int d) { return d == 64 || d == 96 || d == 128 || d == 256; }
bool bwd_dim_ok(int d) { return d == 64 || d == 96 || d == 128 || d == 256; }
bool split_dim_ok(int d) { return d == 64 || d == 96 || d == 128; }
bool fp8_dim_ok(int d) { return d == 64 || d == 128 || d == 256; }
bool pow2(int d) { return d > 0 && (d & (d - 1)) == 0; }

// A dispatch packet holds the grid size in work-items as a 32-bit number, so
// every launch (workgroups x threads) must stay at or below 2^32 - 1.
constexpr long long kMaxWorkItems = 0xFFFFFFFFLL;

// The forward, quantisation and backward kernels run one 256-thread
// workgroup per 128 rows of a head.
long long tile_grid_items(int B, int H, int N) {
  return (long long)((N + 127) / 128) * B * H * 256;
}

int sizes_check(int B, int H, int N, int d) {
  if ((long long)N * d > (1LL << 30)) return FA_ERR_TOO_LARGE;
  if ((long long)B * H >= (1LL << 31)) return FA_ERR_TOO_LARGE;
  if (tile_grid_items(B, H, N) > kMaxWorkItems) return FA_ERR_TOO_LARGE;
  return FA_OK;
}

// Stream-ordered scratch comes from one memory pool per device, created on
// first use and kept until the process ends. Its release threshold is
// unlimited, so memory freed at the end of one call is reused by the next
// call on the stream instead of being released (with the device's
// default pool each call paid for a fresh allocation, about 50 us).
constexpr int kMaxDevices = 64;

hipError_t scratch_pool(hipMemPool_t* out) {
  static std::mutex mu;
  static hipMemPool_t pools[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (pools[dev] == nullptr) {
    hipMemPoolProps props = {};
    props.allocType = hipMemAllocationTypePinned;
    props.handleTypes = hipMemHandleTypeNone;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t pool = nullptr;
    e = hipMemPoolCreate(&pool, &props);
    if (e != hipSuccess) return e;
    uint64_t keep = UINT64_MAX;
    e = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
    if (e != hipSuccess) {
      hipMemPoolDestroy(pool);
      return e;
    }
    pools[dev] = pool;
  }
  *out = pools[dev];
  return hipSuccess;
}

hipError_t scratch_alloc(void** p, size_t bytes, hipStream_t s) {
  hipMemPool_t pool = nullptr;
  hipError_t e = scratch_pool(&pool);
  if (e != hipSuccess) return e;
  return hipMallocFromPoolAsync(p, bytes, pool, s);
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return FA_OK;
  if (log_enabled()) std::fprintf(stderr, "[fa] %s: %s\n", what, hipGetErrorString(e));
  return FA_ERR_HIP;
}

int check_common(const void* q, const void* k, const void* v, void* o, int B, int H, int N) {
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return FA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

int run_fp8_path(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                 int H, int N, int d, int causal, float scale, hipStream_t stream) {
  // Stream-ordered scratch: e4m3 K and V, their block scales, the signs. Q
  // is quantised inside the forward kernel, block by block, with the same
  // arithmetic as the quantisation pass.
  const size_t elems = (size_t)B * H * N * d;
  const size_t nblk = (size_t)B * H * ((N + FA_FP8_BLOCK - 1) / FA_FP8_BLOCK);
  const size_t t_bytes = (elems + 255) & ~(size_t)255;
  const size_t s_bytes = (nblk * sizeof(float) + 255) & ~(size_t)255;
  const size_t total = 2 * t_bytes + 2 * s_bytes + 256 + d * sizeof(float);
  void* ws = nullptr;
  hipError_t e = scratch_alloc(&ws, total, stream);
  if (e != hipSuccess) return hip_status(e, "scratch allocation");
  char* base = static_cast<char*>(ws);
  void* k8 = base;
  void* v8 = base + t_bytes;
  float* sk = reinterpret_cast<float*>(base + 2 * t_bytes);
  float* sv = reinterpret_cast<float*>(base + 2 * t_bytes + s_bytes);
  float* signs = reinterpret_cast<float*>(base + 2 * t_bytes + 2 * s_bytes);
  e = fa::launch_quant_kv_fp8(k, v, k8, v8, sk, sv, signs, kSignKey, B, H, N, d, stream);
  if (e == hipSuccess)
    e = fa::launch_fwd_fp8_qbf16(q, signs, k8, v8, sk, sv, o, lse, B, H, N, d, causal != 0, scale,
                                 stream);
  hipError_t ef = hipFreeAsync(ws, stream);
  if (e != hipSuccess) return hip_status(e, "fp8 path launch");
  return hip_status(ef, "hipFreeAsync");
}

// The split-KV forward into stream-ordered scratch (the partial outputs and
// log-sum-exps of the splits); `splits` is already the normalised count.
int run_split_path(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                   int H, int Nq, int Nk, int d, int causal, float scale, int splits,
                   hipStream_t s) {
  void* ws = nullptr;
  hipError_t e = scratch_alloc(&ws, (size_t)splits * B * H * Nq * (d + 1) * sizeof(float), s);
  if (e != hipSuccess) return hip_status(e, "scratch allocation");
  e = fa::launch_fwd_split_bf16(q, k, v, o, lse, static_cast<float*>(ws), B, H, Nq, Nk, d,
                                causal != 0, splits, scale, s);
  hipError_t ef = hipFreeAsync(ws, s);
  if (e != hipSuccess) return hip_status(e, "fwd_split launch");
  return hip_status(ef, "hipFreeAsync");
}

// bf16 self-attention with few query-tile workgroups and at least 4096 keys
// leaves much of the GPU idle; the key axis then supplies the parallelism:
// such calls take the split-KV path (the forward kernel on key splits,
// partial results merged by LSE). Same-box timing against the one-pass
// kernel (TFLOP/s): non-causal at 128 query tiles, d = 128 (B=1 H=2 N=8192)
// 504 -> 854, d = 96 (B=1 H=4 N=4096) 518 -> 578, d = 64 (B=2 H=2 N=4096)
// 403 -> 435; causal at 128 tiles d = 96 (B=1 H=2 N=8192) 262 -> 540, at 192
// tiles (B=1 H=3 N=8192) 452 -> 623, at 224 (B=1 H=7 N=4096) 500 -> 566.
// Non-causal shapes above 128 tiles stay on the one-pass kernel (B=1 H=3
// N=8192: 925 against 911 with 2 splits), causal ones above 224 (B=1 H=15
// N=2048: 484 against 402), and so does d = 256 (no split instance).
// Returns the split count to use, or 0 for the one-pass kernel.
int fwd_splits_for(int B, int H, int N, int d, int causal) {
  if (!split_dim_ok(d) || N < 4096 || (long long)N * d > (1LL << 29)) return 0;
  if ((long long)B * H * ((N + 127) / 128) > (causal ? 224 : 128)) return 0;
  const int splits = fa::split_count(B, H, N, N, causal != 0, 0);
  if (splits < 2 || fa::split_work_items(B, H, N, d, splits) > kMaxWorkItems) return 0;
  return splits;
}

}  // namespace

namespace fa {
int debug_flags() {
  const char* e = std::getenv("FA_DEBUG");
  if (e == nullptr) return 0;
  return (int)(std::strtol(e, nullptr, 0) & 3);
}
}  // namespace fa

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
           int N, int d, int causal, float scale, int dtype, void* stream) {
  int st = check_common(q, k, v, o, B, H, N);
  if (st != FA_OK) return st;
  if (dtype == FA_BF16) {
    if (!bf16_dim_ok(d)) return FA_ERR_UNSUPPORTED;
  } else if (dtype == FA_FP8_E4M3) {
    if (!fp8_dim_ok(d) || !pow2(d)) return FA_ERR_UNSUPPORTED;
  } else {
    return FA_ERR_UNSUPPORTED;
  }
  if (!(scale > 0.f) || !std::isfinite(scale)) return FA_ERR_INVALID_ARG;
  st = sizes_check(B, H, N, d);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      (lse != nullptr && !aligned16(lse)))
    return FA_ERR_MISALIGNED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (log_enabled())
    std::fprintf(stderr, "[fa] fa_fwd dtype=%d B=%d H=%d N=%d d=%d causal=%d scale=%g\n", dtype,
                 B, H, N, d, causal, (double)scale);
  if (dtype == FA_BF16) {
    const int splits = fwd_splits_for(B, H, N, d, causal);
    if (splits > 0) return run_split_path(q, k, v, o, lse, B, H, N, N, d, causal, scale, splits, s);
    return hip_status(fa::launch_fwd_bf16(q, k, v, o, lse, B, H, N, d, causal != 0, scale, s),
                      "fwd_bf16 launch");
  }
  return run_fp8_path(q, k, v, o, lse, B, H, N, d, causal, scale, s);
}

int fa_quant_fp8(const void* x, void* x8, float* scales, int B, int H, int N, int d,
                 int per_tensor, const float* signs, void* stream) {
  if (x == nullptr || x8 == nullptr || scales == nullptr) return FA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1) return FA_ERR_INVALID_ARG;
  if (!bf16_dim_ok(d) || (signs != nullptr && !pow2(d))) return FA_ERR_UNSUPPORTED;
  int st = sizes_check(B, H, N, d);
  if (st != FA_OK) return st;
  if (!aligned16(x) || !aligned16(x8) || !aligned16(scales) ||
      (signs != nullptr && !aligned16(signs)))
    return FA_ERR_MISALIGNED;
  return hip_status(fa::launch_quant_fp8(x, x8, scales, B, H, N, d, per_tensor != 0, signs,
                                         static_cast<hipStream_t>(stream)),
                    "quant_fp8 launch");
}

int fa_fwd_fp8(const void* q8, const void* k8, const void* v8, const float* q_scale,
               const float* k_scale, const float* v_scale, void* o, float* lse, int B, int H,
               int N, int d, int causal, float scale, void* stream) {
  int st = check_common(q8, k8, v8, o, B, H, N);
  if (st != FA_OK) return st;
  if (q_scale == nullptr || k_scale == nullptr || v_scale == nullptr) return FA_ERR_INVALID_ARG;
  if (!fp8_dim_ok(d)) return FA_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || !std::isfinite(scale)) return FA_ERR_INVALID_ARG;
  st = sizes_check(B, H, N, d);
  if (st != FA_OK) return st;
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8) || !aligned16(o) ||
      !aligned16(q_scale) || !aligned16(k_scale) || !aligned16(v_scale) ||
      (lse != nullptr && !aligned16(lse)))
    return FA_ERR_MISALIGNED;
  return hip_status(fa::launch_fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, o, lse, B, H, N,
                                       d, causal != 0, scale, static_cast<hipStream_t>(stream)),
                    "fwd_fp8 launch");
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, int B, int H, int N, int d,
           int causal, float scale, void* stream) {
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr || lse == nullptr ||
      dout == nullptr || dq == nullptr || dk == nullptr || dv == nullptr)
    return FA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || N < 1) return FA_ERR_INVALID_ARG;
  if (!bwd_dim_ok(d)) return FA_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || !std::isfinite(scale)) return FA_ERR_INVALID_ARG;
  int st = sizes_check(B, H, N, d);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return FA_ERR_MISALIGNED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (log_enabled())
    std::fprintf(stderr, "[fa] fa_bwd B=%d H=%d N=%d d=%d causal=%d scale=%g\n", B, H, N, d,
                 causal, (double)scale);
  // Stream-ordered scratch: the per-row D and -LSE*log2(e) terms.
  void* ws = nullptr;
  hipError_t e = scratch_alloc(&ws, 2 * (size_t)B * H * N * sizeof(float), s);
  if (e != hipSuccess) return hip_status(e, "scratch allocation");
  e = fa::launch_bwd_bf16(q, k, v, o, lse, dout, dq, dk, dv, static_cast<float*>(ws), B, H, N,
                          d, causal != 0, scale, s);
  hipError_t ef = hipFreeAsync(ws, s);
  if (e != hipSuccess) return hip_status(e, "bwd_bf16 launch");
  return hip_status(ef, "hipFreeAsync");
}

}  // extern "C"

namespace {

// fa_fwd_splitkv's checks in the header's order up to the size limits;
// *splits receives the normalised split count.
int splitkv_check(const void* q, const void* k, const void* v, void* o, int B, int H, int Nq,
                  int Nk, int d, int causal, float scale, int num_splits, int* splits) {
  if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return FA_ERR_INVALID_ARG;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || num_splits < 0) return FA_ERR_INVALID_ARG;
  if (causal != 0 && Nq > Nk) return FA_ERR_INVALID_ARG;
  if (!split_dim_ok(d)) return FA_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || !std::isfinite(scale)) return FA_ERR_INVALID_ARG;
  if ((long long)Nk * d > (1LL << 30) || (long long)Nq * d > (1LL << 29) ||
      (long long)B * H >= (1LL << 31))
    return FA_ERR_TOO_LARGE;
  *splits = fa::split_count(B, H, Nq, Nk, causal != 0, num_splits);
  if (fa::split_work_items(B, H, Nq, d, *splits) > kMaxWorkItems) return FA_ERR_TOO_LARGE;
  return FA_OK;
}

bool splitkv_aligned(const void* q, const void* k, const void* v, void* o, float* lse) {
  return aligned16(q) && aligned16(k) && aligned16(v) && aligned16(o) &&
         (lse == nullptr || aligned16(lse));
}

}  // namespace

extern "C" {

int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                   int H, int Nq, int Nk, int d, int causal, float scale, int num_splits,
                   void* stream) {
  int splits = 0;
  const int st = splitkv_check(q, k, v, o, B, H, Nq, Nk, d, causal, scale, num_splits, &splits);
  if (st != FA_OK) return st;
  if (!splitkv_aligned(q, k, v, o, lse)) return FA_ERR_MISALIGNED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (log_enabled())
    std::fprintf(stderr, "[fa] fa_fwd_splitkv B=%d H=%d Nq=%d Nk=%d d=%d causal=%d splits=%d\n", B,
                 H, Nq, Nk, d, causal, splits);
  return run_split_path(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, splits, s);
}

int fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int Nq, int Nk, int d, int causal, float scale,
                           int num_splits, void* stream) {
  int splits = 0;
  const int st = splitkv_check(q, k, v, o, B, H, Nq, Nk, d, causal, scale, num_splits, &splits);
  if (st != FA_OK) return st;
  const unsigned long long need =
      (unsigned long long)splits * B * H * Nq * (d + 1) * sizeof(float);
  if (need > FA_NOALLOC_SCRATCH_BYTES) {
    if (log_enabled())
      std::fprintf(stderr, "[fa] fa_fwd_splitkv_noalloc needs %llu bytes of scratch, holds %u\n",
                   need, (unsigned)FA_NOALLOC_SCRATCH_BYTES);
    return FA_ERR_SCRATCH_LIMIT;
  }
  if (!splitkv_aligned(q, k, v, o, lse)) return FA_ERR_MISALIGNED;
  float* ws = nullptr;
  hipError_t e = fa::noalloc_scratch(&ws);
  if (e != hipSuccess) return hip_status(e, "scratch address");
  if (log_enabled())
    std::fprintf(stderr,
                 "[fa] fa_fwd_splitkv_noalloc B=%d H=%d Nq=%d Nk=%d d=%d causal=%d splits=%d\n",
                 B, H, Nq, Nk, d, causal, splits);
  return hip_status(fa::launch_fwd_split_bf16(q, k, v, o, lse, ws, B, H, Nq, Nk, d, causal != 0,
                                              splits, scale, static_cast<hipStream_t>(stream)),
                    "fwd_split launch");
}

int fa_splitkv_splits(int B, int H, int Nq, int Nk, int causal, int num_splits) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || num_splits < 0) return FA_ERR_INVALID_ARG;
  return fa::split_count(B, H, Nq, Nk, causal != 0, num_splits);
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported head dimension or dtype";
    case FA_ERR_MISALIGNED: return "tensor pointer not 16-byte aligned";
    case FA_ERR_HIP: return "HIP runtime error";
    case FA_ERR_TOO_LARGE: return "size beyond 32-bit index limits";
    case FA_ERR_SCRATCH_LIMIT:
      return "needs more scratch than the allocation-free entry point holds";
    default: return "unknown status";
  }
}

int fa_version(void) { return kVersion; }

}  // extern "C"
