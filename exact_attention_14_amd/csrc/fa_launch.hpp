// Host-side launchers of the attention kernels. Arguments are validated by the
// C-ABI layer (fa_api.cpp) before these are called.
#pragma once
#include <hip/hip_runtime.h>

namespace fa {

// Debug flags of the kernel launches (kDbgReverse | kDbgPoison of the device
// code), read from the environment variable FA_DEBUG at every call; 0 when
// it is unset. Forward and backward launchers pass them to their kernels in
// the top bits of the workgroup count.
int debug_flags();

// bf16 forward: d in {64, 96, 128, 256}.
hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o,
                           float* lse, int B, int H, int N, int d, bool causal,
                           float scale, hipStream_t stream);

// Block quantisation of one bf16 tensor to e4m3fn.
hipError_t launch_quant_fp8(const void* x, void* x8, float* scales, int B, int H,
                            int N, int d, bool per_tensor, const float* signs,
                            hipStream_t stream);

// FP8 forward: d in {64, 128, 256}.
hipError_t launch_fwd_fp8(const void* q8, const void* k8, const void* v8,
                          const float* sq, const float* sk, const float* sv,
                          void* o, float* lse, int B, int H, int N, int d,
                          bool causal, float scale, hipStream_t stream);

// bf16 backward: d in {64, 96, 128, 256}. ws: 2*B*H*N floats of scratch.
hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           float* ws, int B, int H, int N, int d, bool causal, float scale,
                           hipStream_t stream);

// Split-KV bf16 forward for Nq queries against Nk keys: d in {64, 96, 128}.
// ws: split_count(...) * B*H*Nq * (d + 1) floats of scratch.
hipError_t launch_fwd_split_bf16(const void* q, const void* k, const void* v, void* o,
                                 float* lse, float* ws, int B, int H, int Nq, int Nk, int d,
                                 bool causal, int splits, float scale, hipStream_t stream);

// The bf16 forward kernel on key splits (Nq = Nk = N, d in {64, 96, 128}):
// float32 partial outputs `op` and log-sum-exps `lp` of `splits` splits of
// tps 64-key tiles each, in the layout of launch_fwd_split_bf16's scratch.
hipError_t launch_fwd_bf16_partials(const void* q, const void* k, const void* v, float* op,
                                    float* lp, int B, int H, int N, int d, bool causal,
                                    int splits, int tps, float scale, hipStream_t stream);

// Number of key splits the split-KV forward uses (requested <= 0: automatic).
int split_count(int B, int H, int Nq, int Nk, bool causal, int requested);

// Work-items (workgroups x threads) of the larger of the split-KV forward's
// two launches, for the grid-size check.
long long split_work_items(int B, int H, int Nq, int d, int splits);

// FP8 forward with Q in bf16: each workgroup rotates (signs) and quantises
// its own 128-row Q block exactly as launch_quant_fp8 would.
hipError_t launch_fwd_fp8_qbf16(const void* qbf, const float* signs, const void* k8,
                                const void* v8, const float* sk, const float* sv, void* o,
                                float* lse, int B, int H, int N, int d, bool causal, float scale,
                                hipStream_t stream);

// The end-to-end FP8 path's K and V passes in one launch: K rotated by the
// signs of `key` (also written to `signs`, d floats), V not rotated; codes and
// scales as two launch_quant_fp8 calls would give.
hipError_t launch_quant_kv_fp8(const void* k, const void* v, void* k8, void* v8, float* sk,
                               float* sv, float* signs, unsigned long long key, int B, int H,
                               int N, int d, hipStream_t stream);

// The device address of this device's copy of the allocation-free entry
// point's scratch (FA_NOALLOC_SCRATCH_BYTES bytes); looked up once per
// device, with that device current, then reused. Allocates nothing.
hipError_t noalloc_scratch(float** ws);

}  // namespace fa
