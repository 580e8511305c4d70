// FP8 (OCP e4m3fn) attention path for gfx950: random signs, block
// quantisation with optional Hadamard rotation, and the e4m3 forward kernel.
//
// Method (QbitAI FlashAttention-3 article, FP8 section; FlashAttention-3 (HE),
// "3. FP8 with reduced quantisation error"; dibro.site FlashAttention-3 post,
// "Arquitectura y metodo"): Q, K, V are quantised block by block, each block
// with its own scale, instead of one scale per tensor; before quantising, Q
// and K are multiplied by a random orthogonal (Hadamard) matrix, which leaves
// Q K^T unchanged and spreads outliers over all coordinates; both matrix
// products run in FP8 with FP32 accumulation, the softmax stays in FP32
// (vikram-blog FlashAttention-3 post, "Production Gotchas"), and the V tile
// is presented transposed to the second product because the FP8 matrix
// instruction wants the reduction dimension contiguous (QbitAI article, FP8
// section).
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kBlock = 128;      // rows per quantisation block
constexpr float kE4m3Max = 448.f;
constexpr float kPScale = 256.f; // P is rounded to e4m3 as P * 2^8

// ----------------------------------------------------------------- signs ----

// SplitMix64 output function (Steele, Lea, Flood 2014) on counter i.
__device__ __forceinline__ unsigned long long splitmix64(unsigned long long x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

__global__ void fill_signs_kernel(float* signs, int d, unsigned long long key) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < d) signs[i] = (splitmix64(key + (unsigned long long)i) >> 63) ? -1.f : 1.f;
}

// ----------------------------------------------------------- quantiser ------

enum QuantMode { kPerBlock = 0, kAmaxOnly = 1, kGivenAmax = 2 };

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}

// Packs e4m3(a), e4m3(b) into the low (HI=false) or high 16 bits of `old`,
// round to nearest even (values beyond +-448 are clamped by the callers).
template <bool HI>
__device__ __forceinline__ int cvt_pk_fp8(float a, float b, int old) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

// One workgroup (256 threads) per 128-row block of one (batch, head). Each
// thread holds 8-element chunks; with rotation the CPR chunks of a row sit in
// CPR consecutive lanes, so the Walsh-Hadamard butterflies run in registers
// (strides 1, 2, 4) and across lanes (strides >= 8).
template <int D, bool ROTATE, int MODE>
__global__ __launch_bounds__(256) void quant_fp8_kernel(const u16* __restrict__ X,
                                                        uint8_t* __restrict__ X8,
                                                        float* __restrict__ scales,
                                                        const float* __restrict__ signs, int N,
                                                        int nblk, float rsqrt_d) {
  constexpr int CPR = D / 8;
  constexpr int NC = kBlock * CPR / 256;  // chunks per thread
  static_assert(!ROTATE || (64 % CPR == 0), "rotation needs a row inside one wave");
  const int tid = threadIdx.x;
  const int blk = blockIdx.x % nblk;
  const size_t bh = blockIdx.x / nblk;
  const int row0 = blk * kBlock;
  const size_t base = (bh * (size_t)N + row0) * D;
  const int nrows = min(kBlock, N - row0);

  float x[NC][8];
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int cid = k * 256 + tid;
    const int row = cid / CPR, ch = cid % CPR;
    uint4 w = {0u, 0u, 0u, 0u};
    if (row < nrows) w = *(const uint4*)(X + base + (size_t)row * D + ch * 8);
    const u16* e = (const u16*)&w;
#pragma unroll
    for (int j = 0; j < 8; ++j) x[k][j] = __uint_as_float((unsigned)e[j] << 16);
    if constexpr (ROTATE) {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[k][j] *= signs[ch * 8 + j];
      // strides 1, 2, 4 inside the chunk
#pragma unroll
      for (int s = 1; s < 8; s <<= 1)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if ((j & s) == 0) {
            const float a = x[k][j], b = x[k][j + s];
            x[k][j] = a + b;
            x[k][j + s] = a - b;
          }
      // strides 8 .. D/2 across the lanes holding one row
#pragma unroll
      for (int m = 1; m < CPR; m <<= 1) {
        const bool upper = (tid & m) != 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float other = __shfl_xor(x[k][j], m);
          x[k][j] = upper ? other - x[k][j] : x[k][j] + other;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(x[k][j]));
  }

  __shared__ float red[4];
  amax = wave_max(amax);
  if ((tid & 63) == 0) red[tid >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const size_t sidx = bh * nblk + blk;
  if constexpr (MODE == kAmaxOnly) {
    if (tid == 0) scales[sidx] = amax;
    return;
  }
  if constexpr (MODE == kGivenAmax) amax = scales[sidx];
  const float s = amax > 0.f ? amax / kE4m3Max : 1.f;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int cid = k * 256 + tid;
    const int row = cid / CPR, ch = cid % CPR;
    float t[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) t[j] = fminf(fmaxf(x[k][j] / s, -kE4m3Max), kE4m3Max);
    int lo = cvt_pk_fp8<false>(t[0], t[1], 0);
    lo = cvt_pk_fp8<true>(t[2], t[3], lo);
    int hi = cvt_pk_fp8<false>(t[4], t[5], 0);
    hi = cvt_pk_fp8<true>(t[6], t[7], hi);
    if (row < nrows) *(uint2*)(X8 + base + (size_t)row * D + ch * 8) = make_uint2(lo, hi);
  }
  if constexpr (MODE == kGivenAmax) __syncthreads();  // every thread has read scales[sidx]
  if (tid == 0) scales[sidx] = ROTATE ? s * rsqrt_d : s;
}

// Maximum over all block maxima, written back to every entry.
__global__ __launch_bounds__(256) void amax_all_kernel(float* scales, int n) {
  float m = 0.f;
  for (int i = threadIdx.x; i < n; i += 256) m = fmaxf(m, scales[i]);
  __shared__ float red[4];
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  for (int i = threadIdx.x; i < n; i += 256) scales[i] = m;
}

template <int D, bool ROTATE>
hipError_t quant_launch(const void* x, void* x8, float* scales, int B, int H, int N,
                        bool per_tensor, const float* signs, hipStream_t stream) {
  const int nblk = (N + kBlock - 1) / kBlock;
  const long long ngrid = (long long)nblk * B * H;
  if (ngrid >= (1LL << 31)) return hipErrorInvalidValue;
  const float rsqrt_d = (float)(1.0 / sqrt((double)D));
  if (!per_tensor) {
    hipLaunchKernelGGL((quant_fp8_kernel<D, ROTATE, kPerBlock>), dim3((unsigned)ngrid), dim3(256),
                       0, stream, (const u16*)x, (uint8_t*)x8, scales, signs, N, nblk, rsqrt_d);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((quant_fp8_kernel<D, ROTATE, kAmaxOnly>), dim3((unsigned)ngrid), dim3(256),
                     0, stream, (const u16*)x, (uint8_t*)x8, scales, signs, N, nblk, rsqrt_d);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(amax_all_kernel, dim3(1), dim3(256), 0, stream, scales, (int)ngrid);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((quant_fp8_kernel<D, ROTATE, kGivenAmax>), dim3((unsigned)ngrid), dim3(256),
                     0, stream, (const u16*)x, (uint8_t*)x8, scales, signs, N, nblk, rsqrt_d);
  return hipGetLastError();
}

// ------------------------------------------------------ e4m3 forward -------

constexpr int kBC = 64;  // keys per K/V tile

template <int D>
struct Geo8 {
  static constexpr int CPR = D / 16;       // 16-byte chunks per row (= slots)
  static constexpr int ROWB = D;           // bytes per LDS row
  static constexpr int TILEB = kBC * D;    // one K or V tile
  static constexpr int NKS = D / 64;       // k-steps of S^T = K Q^T (64 per step)
  static constexpr int NO = D / 32;        // 32-row blocks of O^T
};

// Chunk-slot XOR of LDS row `row` (bank model in the design notes).
template <int D>
__device__ __forceinline__ int swz8(int row) {
  const int r = row & 15;
  if constexpr (D == 64) {
    return (r >> 2) & 3;
  } else if constexpr (D == 128) {
    const int s = r >> 1;
    return ((s & 1) << 1) | ((s >> 2) << 2) | ((s >> 1) & 1);
  } else {
    return ((r & 3) << 2) | ((r >> 2) & 3);
  }
}

template <int D, int NW>
__device__ __forceinline__ void load_tile8(__amdgpu_buffer_rsrc_t rs, char* tile, int j0,
                                           int wave, int lane) {
  using G = Geo8<D>;
  constexpr int NCH = kBC * G::CPR;           // chunks per tile
  constexpr int NI = (NCH + 64 * NW - 1) / (64 * NW);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int w = i * NW + wave;              // 1 KiB wave copy index
    if (w * 64 < NCH) {
      const int slot = w * 64 + lane;
      const int row = slot / G::CPR;
      const int c = (slot % G::CPR) ^ swz8<D>(row);
      copy16_to_lds(rs, tile + w * 1024, (unsigned)(j0 + row) * D + c * 16);
    }
  }
}

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

__device__ __forceinline__ i32x2 tr8(const char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)p);
}

__device__ __forceinline__ f32x16 mfma8(i32x8 a, i32x8 b, f32x16 c) {
  // e4m3 x e4m3, unit block scales (exponent 127 = 2^0).
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

template <int D, bool CAUSAL, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(D == 256 ? 1 : 2, D == 256 ? 1 : 2)))
void fwd_fp8_kernel(const uint8_t* __restrict__ Q8, const uint8_t* __restrict__ K8,
                    const uint8_t* __restrict__ V8, const float* __restrict__ SQ,
                    const float* __restrict__ SK, const float* __restrict__ SV,
                    u16* __restrict__ O, float* __restrict__ LSE, int N, int ntq, int nwg,
                    int nblk, float scale) {
  using G = Geo8<D>;
  constexpr int BR = 32 * NW;
  __shared__ __attribute__((aligned(1024))) char ks0[G::TILEB];
  __shared__ __attribute__((aligned(1024))) char vs0[G::TILEB];
  __shared__ __attribute__((aligned(1024))) char ks1[G::TILEB];
  __shared__ __attribute__((aligned(1024))) char vs1[G::TILEB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  const int lid = xcd_grouped_id(blockIdx.x, nwg);
  const int qtr = lid % ntq;
  const int bh = lid / ntq;
  const int qt = CAUSAL ? (ntq - 1 - qtr) : qtr;
  const size_t head = (size_t)bh * (size_t)N;
  const unsigned head_bytes = (unsigned)N * D;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q8 + head * D, head_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(K8 + head * D, head_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(V8 + head * D, head_bytes);
  const float* sqh = SQ + (size_t)bh * nblk;
  const float* skh = SK + (size_t)bh * nblk;
  const float* svh = SV + (size_t)bh * nblk;

  const int q0w = qt * BR + wave * 32;
  const int qi = q0w + l32;
  const int q_last = min(N, qt * BR + BR) - 1;
  const int ntiles = CAUSAL ? (q_last / kBC + 1) : (N + kBC - 1) / kBC;

  load_tile8<D, NW>(rk, ks0, 0, wave, lane);
  load_tile8<D, NW>(rv, vs0, 0, wave, lane);

  i32x8 qreg[G::NKS];
#pragma unroll
  for (int ks = 0; ks < G::NKS; ++ks) {
    const unsigned off = (unsigned)qi * D + ks * 64 + half * 32;
    const i32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
    const i32x4 b = __builtin_amdgcn_raw_buffer_load_b128(rq, off + 16, 0, 0);
    qreg[ks] = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  const float sq = sqh[min(qi, N - 1) / kBlock];

  f32x16 oacc[G::NO];
#pragma unroll
  for (int i = 0; i < G::NO; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[i][v] = 0.f;
  // Softmax state in log2 units of the scaled score: z = scale * log2(e) * q.k.
  float m_ref = -INFINITY;
  float l_run = 0.f;
  float sv_cur = 1.f;  // V scale the accumulator is expressed in
  const float c = scale * kLog2e;

  const int krow = l32;
  const int g16 = lane >> 4, i16 = lane & 15;
  const int vq = i16 & 1, vt = i16 >> 1;  // tr8 source lane = 2 * vt + vq
  const int vrow = 8 * (vt >> 2) + 4 * half + (vt & 3);  // + 16 * r

  auto step = [&](const char* kt, const char* vt_, char* kn, char* vn, int t) {
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (t + 1 < ntiles) {
      load_tile8<D, NW>(rk, kn, (t + 1) * kBC, wave, lane);
      load_tile8<D, NW>(rv, vn, (t + 1) * kBC, wave, lane);
    }
    const int j0 = t * kBC;
    if (CAUSAL && j0 > q0w + 31) return;

    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 acc;
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[v] = 0.f;
      const int row = kb * 32 + krow;
      const int sw = swz8<D>(row);
#pragma unroll
      for (int ks = 0; ks < G::NKS; ++ks) {
        const int c0 = (ks * 4 + 2 * half) ^ sw;
        const int c1 = (ks * 4 + 2 * half + 1) ^ sw;
        const i32x4 lo = *(const i32x4*)(kt + row * G::ROWB + c0 * 16);
        const i32x4 hi = *(const i32x4*)(kt + row * G::ROWB + c1 * 16);
        acc = mfma8(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), qreg[ks], acc);
      }
      s[kb] = acc;
    }

    const bool need_mask = (j0 + kBC > N) || (CAUSAL && j0 + kBC - 1 > q0w);
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = j0 + kb * 32 + 8 * (v / 4) + 4 * half + (v % 4);
          if (key >= N || (CAUSAL && key > qi)) s[kb][v] = -INFINITY;
        }
    }

    const float cs = c * sq * skh[j0 / kBlock];  // raw MFMA result -> log2 units
    const float sv_t = svh[j0 / kBlock];
    float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = (kb == 0 ? 2 : 0); v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
    mx = fmaxf(mx, xor32(mx)) * cs;
    // Exact running maximum (P * 2^8 must stay within e4m3), and the
    // accumulator re-expressed in the V scale of this tile.
    if (__any(mx > m_ref) || sv_t != sv_cur) {
      const float m_new = fmaxf(m_ref, mx);
      const float alpha = (m_ref == -INFINITY) ? 0.f : fast_exp2(m_ref - m_new);
      const float f = alpha * (sv_cur / sv_t);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < G::NO; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[i][v] *= f;
      m_ref = m_new;
      sv_cur = sv_t;
    }
    const float mref = (m_ref == -INFINITY) ? 0.f : m_ref;
    float lsum = 0.f;
    int pw[8];  // P * 2^8 as e4m3, byte b = kb * 16 + v
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        float e[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          e[x] = fast_exp2(fmaf(s[kb][4 * v4 + x], cs, -mref));
          lsum += e[x];
        }
        const int w = cvt_pk_fp8<false>(e[0] * kPScale, e[1] * kPScale, 0);
        pw[kb * 4 + v4] = cvt_pk_fp8<true>(e[2] * kPScale, e[3] * kPScale, w);
      }
    l_run += lsum;
    const i32x8 pv = {pw[0], pw[1], pw[2], pw[3], pw[4], pw[5], pw[6], pw[7]};

#pragma unroll
    for (int i = 0; i < G::NO; ++i) {
      const int d = i * 32 + 16 * (g16 & 1) + 8 * vq;
      i32x2 part[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * r + vrow;
        const int ch = (d >> 4) ^ swz8<D>(row);
        part[r] = tr8(vt_ + row * G::ROWB + ch * 16 + (d & 15));
      }
      const i32x8 a = {part[0][0], part[0][1], part[1][0], part[1][1],
                       part[2][0], part[2][1], part[3][0], part[3][1]};
      oacc[i] = mfma8(a, pv, oacc[i]);
    }
  };
  for (int t = 0; t < ntiles; t += 2) {
    step(ks0, vs0, ks1, vs1, t);
    if (t + 1 < ntiles) step(ks1, vs1, ks0, vs0, t + 1);
  }

  const float l_tot = l_run + xor32(l_run);
  const float inv = sv_cur / (kPScale * l_tot);
  if (qi < N) {
    u16* orow = O + (head + qi) * D;
#pragma unroll
    for (int i = 0; i < G::NO; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 w;
#pragma unroll
        for (int x = 0; x < 4; ++x) w[x] = (__bf16)(oacc[i][4 * g + x] * inv);
        *(bf16x4*)(orow + i * 32 + 8 * g + 4 * half) = w;
      }
    if (LSE != nullptr && half == 0) LSE[head + qi] = (m_ref + __log2f(l_tot)) * kLn2;
  }
}

template <int D, bool CAUSAL>
hipError_t fwd_launch(const void* q8, const void* k8, const void* v8, const float* sq,
                      const float* sk, const float* sv, void* o, float* lse, int B, int H, int N,
                      float scale, hipStream_t stream) {
  constexpr int NW = 4;
  constexpr int BR = 32 * NW;
  const int ntq = (N + BR - 1) / BR;
  const long long nwg = (long long)ntq * B * H;
  if (nwg >= (1LL << 31)) return hipErrorInvalidValue;
  const int nblk = (N + kBlock - 1) / kBlock;
  hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL, NW>), dim3((unsigned)nwg), dim3(NW * 64), 0,
                     stream, (const uint8_t*)q8, (const uint8_t*)k8, (const uint8_t*)v8, sq, sk,
                     sv, (u16*)o, lse, N, ntq, (int)nwg, nblk, scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fill_signs(float* signs, int d, unsigned long long key, hipStream_t stream) {
  hipLaunchKernelGGL(fill_signs_kernel, dim3((d + 255) / 256), dim3(256), 0, stream, signs, d,
                     key);
  return hipGetLastError();
}

hipError_t launch_quant_fp8(const void* x, void* x8, float* scales, int B, int H, int N, int d,
                            bool per_tensor, const float* signs, hipStream_t stream) {
  const bool rot = signs != nullptr;
  switch (d) {
    case 64:
      return rot ? quant_launch<64, true>(x, x8, scales, B, H, N, per_tensor, signs, stream)
                 : quant_launch<64, false>(x, x8, scales, B, H, N, per_tensor, signs, stream);
    case 96:
      return rot ? hipErrorInvalidValue
                 : quant_launch<96, false>(x, x8, scales, B, H, N, per_tensor, signs, stream);
    case 128:
      return rot ? quant_launch<128, true>(x, x8, scales, B, H, N, per_tensor, signs, stream)
                 : quant_launch<128, false>(x, x8, scales, B, H, N, per_tensor, signs, stream);
    case 256:
      return rot ? quant_launch<256, true>(x, x8, scales, B, H, N, per_tensor, signs, stream)
                 : quant_launch<256, false>(x, x8, scales, B, H, N, per_tensor, signs, stream);
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_fwd_fp8(const void* q8, const void* k8, const void* v8, const float* sq,
                          const float* sk, const float* sv, void* o, float* lse, int B, int H,
                          int N, int d, bool causal, float scale, hipStream_t stream) {
#define FA_CASE(DD)                                                                       \
  case DD:                                                                                \
    return causal ? fwd_launch<DD, true>(q8, k8, v8, sq, sk, sv, o, lse, B, H, N, scale,  \
                                         stream)                                          \
                  : fwd_launch<DD, false>(q8, k8, v8, sq, sk, sv, o, lse, B, H, N, scale, \
                                          stream);
  switch (d) {
    FA_CASE(64)
    FA_CASE(128)
    FA_CASE(256)
    default:
      return hipErrorInvalidValue;
  }
#undef FA_CASE
}

}  // namespace fa
