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
#include <type_traits>

#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kBlock = 128;      // rows per quantisation block
constexpr float kE4m3Max = 448.f;

// ----------------------------------------------------------------- signs ----

// SplitMix64 output function (Steele, Lea, Flood 2014) on counter i.
__device__ __forceinline__ unsigned long long splitmix64(unsigned long long x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

// Sign i of the rotation with this key: -1 where the top bit of
// SplitMix64(key + i) is set, else +1.
__device__ __forceinline__ float sign_of(unsigned long long key, int i) {
  return (splitmix64(key + (unsigned long long)i) >> 63) ? -1.f : 1.f;
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
// Value of v in lane (lane ^ m). m = 1, 2, 8 through DPP lane permutes within
// 16-lane rows (quad permutes; row rotate by 8); m = 4 through one bit-mode
// ds_swizzle (two DPP moves before, a half-row mirror then a quad xor 3: the
// rotating quantisation pass ran 7-9% faster at d = 64 and 128 with the
// swizzle); m = 16 through the same swizzle (d = 256); wider strides through
// the LDS crossbar.
__device__ __forceinline__ float lane_xor(float v, int m) {
  const int b = __float_as_int(v);
  switch (m) {
    case 1: return __int_as_float(__builtin_amdgcn_mov_dpp(b, 0xB1, 0xF, 0xF, false));
    case 2: return __int_as_float(__builtin_amdgcn_mov_dpp(b, 0x4E, 0xF, 0xF, false));
    case 4:  // bit-mode swizzle within 32 lanes: and 0x1F, xor 4
      return __int_as_float(__builtin_amdgcn_ds_swizzle(b, (4 << 10) | 0x1F));
    case 8: return __int_as_float(__builtin_amdgcn_mov_dpp(b, 0x128, 0xF, 0xF, false));
    case 16:  // bit-mode swizzle within 32 lanes: and 0x1F, xor 16
      return __int_as_float(__builtin_amdgcn_ds_swizzle(b, (16 << 10) | 0x1F));
    default: return __shfl_xor(v, m);
  }
}

// The arithmetic of one 128-row block, shared by the quantisation pass and
// the e4m3 forward kernel's quantisation of its own Q block (both therefore
// give bit-identical codes and scales). 256 threads. With GR = 1 thread tid
// holds one 8-column chunk in each of NC rows (consecutive lanes, consecutive
// chunks: the loads of a wave cover whole rows). With rotation and GR = 4 it
// holds 4 consecutive chunks (32 columns) of each of NC/4 rows, so the
// Walsh-Hadamard butterflies of strides 1..16 run in registers and only
// strides >= 32 cross lanes (D/32 lanes per row): about 17% fewer VALU
// instructions, but each load instruction of a wave touches 4x as many cache
// lines. The quantisation passes are bound by memory access and keep GR = 1
// (GR = 4 measured 7-19% slower there); the forward kernel's quantisation of
// its own Q block is bound by instruction latency and uses GR = 4 (+1.5 to
// +2.5% end to end). Either way the butterflies are the same pairs in the
// same order (strides 1, 2, 4, ..., D/2), so the values do not depend on the
// layout.
template <int D, bool ROTATE, int GR = 1>
struct BlockQuant {
  static constexpr int CPR = D / 8;                // 8-column chunks per row
  static constexpr int NC = kBlock * CPR / 256;    // chunks per thread
  static constexpr int G = ROTATE ? GR : 1;        // consecutive chunks of a row per thread
  static constexpr int L = CPR / G;                // lanes per row
  static constexpr int RPT = NC / G;               // rows per thread
  static constexpr int RSTEP = 256 / L;            // rows between a thread's rows (G > 1)
  static_assert(NC % G == 0 && CPR % G == 0, "chunk groups tile the block");
  static_assert(!ROTATE || 64 % L == 0, "a row's lanes sit in one wave");
  float x[NC][8];

  // Row and chunk of the thread's chunk r * G + gi. One chunk per row: chunk
  // cid = r * 256 + tid of the block (consecutive lanes, consecutive chunks;
  // also when 256 is not a multiple of CPR, as for d = 96).
  __device__ __forceinline__ int row_of(int r, int tid) const {
    if constexpr (G == 1) return (r * 256 + tid) / CPR;
    else return r * RSTEP + tid / L;
  }
  __device__ __forceinline__ int chunk_of(int r, int gi, int tid) const {
    if constexpr (G == 1) return (r * 256 + tid) % CPR;
    else return (tid % L) * G + gi;
  }

  // Loads the rows from row0 on (zeros past the buffer's end), rotates them
  // if asked; returns this thread's largest magnitude.
  __device__ __forceinline__ float load(__amdgpu_buffer_rsrc_t rx, int row0,
                                        const float* __restrict__ signs, int tid) {
    float amax = 0.f;
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        const int row = row_of(r, tid), ch = chunk_of(r, gi, tid);
        const i32x4 w = __builtin_amdgcn_raw_buffer_load_b128(
            rx, (unsigned)((row0 + row) * D + ch * 8) * 2u, 0, 0);
        const u16* e = (const u16*)&w;
#pragma unroll
        for (int j = 0; j < 8; ++j) x[r * G + gi][j] = __uint_as_float((unsigned)e[j] << 16);
      }
      if constexpr (ROTATE) {
        float* y = &x[r * G][0];  // the thread's 8G consecutive columns of this row
        const int c0 = chunk_of(r, 0, tid) * 8;
        // stride 1 with the signs folded in: (s0 x0) +- (s1 x1), the
        // products exact, one rounding each, as sign-then-butterfly gives
#pragma unroll
        for (int j = 0; j < 8 * G; j += 2) {
          const float t = signs[c0 + j + 1] * y[j + 1];
          const float a = y[j];
          y[j] = fmaf(signs[c0 + j], a, t);
          y[j + 1] = fmaf(signs[c0 + j], a, -t);
        }
        // strides 2 .. 4G in registers
#pragma unroll
        for (int st = 2; st < 8 * G; st <<= 1)
#pragma unroll
          for (int j = 0; j < 8 * G; ++j)
            if ((j & st) == 0) {
              const float a = y[j], b = y[j + st];
              y[j] = a + b;
              y[j + st] = a - b;
            }
        // strides >= 8G across the lanes holding the row: the lane with the
        // bit m clear keeps x + other, the one with it set other - x.
#pragma unroll
        for (int m = 1; m < L; m <<= 1) {
          const float sgn = (tid & m) ? -1.f : 1.f;
#pragma unroll
          for (int j = 0; j < 8 * G; ++j) y[j] = fmaf(sgn, y[j], lane_xor(y[j], m));
        }
      }
#pragma unroll
      for (int gi = 0; gi < G; ++gi)
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(x[r * G + gi][j]));
    }
    return amax;
  }

  // e4m3 codes of the block, y * inv_s clamped to +-448 and rounded to
  // nearest even; sink(row, chunk, 8 packed bytes) stores them.
  template <class Sink>
  __device__ __forceinline__ void emit(float inv_s, int tid, Sink sink) const {
#pragma unroll
    for (int r = 0; r < RPT; ++r)
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        const float* xc = x[r * G + gi];
        float t[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) t[j] = fminf(fmaxf(xc[j] * inv_s, -kE4m3Max), kE4m3Max);
        int lo = cvt_pk_fp8<false>(t[0], t[1], 0);
        lo = cvt_pk_fp8<true>(t[2], t[3], lo);
        int hi = cvt_pk_fp8<false>(t[4], t[5], 0);
        hi = cvt_pk_fp8<true>(t[6], t[7], hi);
        const i32x2 packed = {lo, hi};
        sink(row_of(r, tid), chunk_of(r, gi, tid), packed);
      }
  }
};

// Largest of the 256 threads' values (red: 4 floats of LDS; contains a
// workgroup barrier).
__device__ __forceinline__ float block_max(float v, float* red, int tid) {
  v = wave_max(v);
  if ((tid & 63) == 0) red[tid >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// The block scale: amax / 448, or 1 for an all-zero block.
__device__ __forceinline__ float block_scale(float amax) {
  return amax > 0.f ? amax / kE4m3Max : 1.f;
}

template <int D, bool ROTATE, int MODE>
__global__ __launch_bounds__(256) void quant_fp8_kernel(const u16* __restrict__ X,
                                                        uint8_t* __restrict__ X8,
                                                        float* __restrict__ scales,
                                                        const float* __restrict__ signs, int N,
                                                        int nblk, float rsqrt_d) {
  const int tid = threadIdx.x;
  const int blk = blockIdx.x % nblk;
  const size_t bh = blockIdx.x / nblk;
  const int row0 = blk * kBlock;
  // Buffer resources over the head's rows: loads past row N return zeros and
  // stores there are dropped, so the ragged last block needs no branch.
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(X + bh * (size_t)N * D, (unsigned)N * D * 2u);
  const __amdgpu_buffer_rsrc_t rx8 = make_rsrc(X8 + bh * (size_t)N * D, (unsigned)N * D);

  BlockQuant<D, ROTATE> bq;
  __shared__ float red[4];
  float amax = block_max(bq.load(rx, row0, signs, tid), red, tid);
  const size_t sidx = bh * nblk + blk;
  if constexpr (MODE == kAmaxOnly) {
    if (tid == 0) scales[sidx] = amax;
    return;
  }
  if constexpr (MODE == kGivenAmax) amax = scales[sidx];
  const float s = block_scale(amax);
  const float inv_s = 1.f / s;  // the scale is applied through its float32 reciprocal
  bq.emit(inv_s, tid, [&](int row, int ch, i32x2 packed) {
    __builtin_amdgcn_raw_buffer_store_b64(packed, rx8, (unsigned)((row0 + row) * D + ch * 8), 0, 0);
  });
  if constexpr (MODE == kGivenAmax) __syncthreads();  // every thread has read scales[sidx]
  if (tid == 0) scales[sidx] = ROTATE ? s * rsqrt_d : s;
}

// The K and V passes of the end-to-end FP8 path in one launch: blockIdx.y = 0
// quantises K's blocks rotated by the signs of `key` (each workgroup makes
// them in LDS; workgroup (0, 0) also stores them for the forward kernel, which
// quantises Q with the same signs), blockIdx.y = 1 quantises V's blocks
// without rotation. Per block the arithmetic is quant_fp8_kernel's, so the
// codes and scales equal those of two quant_fp8_kernel launches bit for bit.
template <int D>
__global__ __launch_bounds__(256) void quant_kv_fp8_kernel(
    const u16* __restrict__ K, const u16* __restrict__ V, uint8_t* __restrict__ K8,
    uint8_t* __restrict__ V8, float* __restrict__ SK, float* __restrict__ SV,
    float* __restrict__ signs_out, unsigned long long key, int N, int nblk, float rsqrt_d) {
  const int tid = threadIdx.x;
  const int blk = blockIdx.x % nblk;
  const size_t bh = blockIdx.x / nblk;
  const int row0 = blk * kBlock;
  const size_t sidx = bh * nblk + blk;
  const unsigned nbytes = (unsigned)N * D * 2u;
  __shared__ float red[4];
  if (blockIdx.y == 0) {
    __shared__ float sgn[D];
    for (int i = tid; i < D; i += 256) {
      sgn[i] = sign_of(key, i);
      if (blockIdx.x == 0) signs_out[i] = sgn[i];
    }
    __syncthreads();
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(K + bh * (size_t)N * D, nbytes);
    const __amdgpu_buffer_rsrc_t rx8 = make_rsrc(K8 + bh * (size_t)N * D, (unsigned)N * D);
    BlockQuant<D, true> bq;
    const float s = block_scale(block_max(bq.load(rx, row0, sgn, tid), red, tid));
    bq.emit(1.f / s, tid, [&](int row, int ch, i32x2 packed) {
      __builtin_amdgcn_raw_buffer_store_b64(packed, rx8, (unsigned)((row0 + row) * D + ch * 8), 0,
                                            0);
    });
    if (tid == 0) SK[sidx] = s * rsqrt_d;
  } else {
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(V + bh * (size_t)N * D, nbytes);
    const __amdgpu_buffer_rsrc_t rx8 = make_rsrc(V8 + bh * (size_t)N * D, (unsigned)N * D);
    BlockQuant<D, false> bq;
    const float s = block_scale(block_max(bq.load(rx, row0, nullptr, tid), red, tid));
    bq.emit(1.f / s, tid, [&](int row, int ch, i32x2 packed) {
      __builtin_amdgcn_raw_buffer_store_b64(packed, rx8, (unsigned)((row0 + row) * D + ch * 8), 0,
                                            0);
    });
    if (tid == 0) SV[sidx] = s;
  }
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

typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

__device__ __forceinline__ i32x2 tr8(const char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)p);
}

__device__ __forceinline__ f32x16 mfma8(i32x8 a, i32x8 b, f32x16 c) {
  // e4m3 x e4m3, unit block scales (exponent 127 = 2^0).
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Per-lane byte offsets (tile row 0) of this wave's share of an e4m3 tile copy.
template <int D, int NW>
struct TileCopy8 {
  using G = Geo8<D>;
  static constexpr int NCH = kBC * G::CPR;                 // 16-byte chunks per tile
  static constexpr int NI = (NCH + 64 * NW - 1) / (64 * NW);
  unsigned off[NI];
  __device__ __forceinline__ TileCopy8(int wave, int lane) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int slot = (i * NW + wave) * 64 + lane;
      const int row = slot / G::CPR;
      const int c = (slot % G::CPR) ^ swz8<D>(row);
      off[i] = slot < NCH ? (unsigned)(row * D + c * 16) : kOutOfRange;
    }
  }
  static_assert(NCH % (64 * NW) == 0, "every wave issues the same number of copies");
  __device__ __forceinline__ void issue(i32x4 rs, char* tile, int j0, int wave, bool valid) const {
    const unsigned base = valid ? (unsigned)j0 * D : kOutOfRange;
#pragma unroll
    for (int i = 0; i < NI; ++i)
      copy16_to_lds_asm(rs, tile + (i * NW + wave) * 1024, off[i] + base);
  }
};


// Same software pipeline as the bf16 kernel: while the VALU runs the
// softmax of tile t, the matrix cores form the scores of tile t+1; the P V
// products of tile t then overlap the row maxima of tile t+1.
//   * P * 2^6 comes straight out of exp2 (6 is added to the exponent).
//   * V's block scales are folded into P instead of the accumulator: with
//     sv_ref a reference V scale of the wave, tile t's P is quantised as
//     P * 2^6 * r_t, r_t = sv_t / sv_ref (one more term in the exp2
//     argument), so the accumulator holds sum P V / sv_ref. sv_ref starts
//     at the head's largest V block scale and moves to sv_t whenever r_t
//     leaves [2^-4, 1] (a block larger than the reference, or one so much
//     smaller that its P * 2^6 * r would sink into e4m3's subnormal range:
//     an all-zero block, whose scale is 1, or blocks of very different
//     magnitudes); the fp32 accumulator is then rescaled by the old over
//     the new reference, which costs no precision. So every tile's P keeps
//     at least 2^4 * P of headroom above e4m3's normal threshold.
//   * The row sum is taken by one more e4m3 product per tile,
//     ones(32 x 64) . P^T, whose every output row is sum_k P*2^6*r_t for the
//     lane's query; divided by r_t it is the sum of exactly the
//     probabilities the P V product used.
//   * The reference maximum moves only when a row maximum exceeds it by more
//     than 2.75 (log2 units), so P * 2^6 <= 2^8.75 = 430 stays within e4m3.
//     (Scaling P by 2^8 with a 0.75 window made the accumulator rescale fire
//     on most tiles: same-box A/B against it, 2^7 / 1.75 ran +1.3 to +3.7%
//     at d = 64 and 128, 2^6 / 2.75 +1.9 to +5.4%, 2^5 / 3.75 +2.1 to +6.0%;
//     +16 / +27 / +31% at d = 256. The cost is the subnormal threshold: P
//     below 2^-12 of the reference maximum (2^-14 with 2^8) loses relative
//     precision. An fp64 emulation on the FP8 workload gives relative RMSE
//     against exact attention 0.0459 / 0.0458 / 0.0459 / 0.0474 for 2^8 /
//     2^7 / 2^6 / 2^5: 2^6 is the last step that costs nothing measurable.)
//   * QIN: Q arrives in bf16 and the workgroup quantises its own 128-row Q
//     block (one quantisation block) in the prologue, with the pass's own
//     arithmetic (BlockQuant: rotation by the random signs, block amax,
//     e4m3 codes through LDS into the Q registers): the result is bit for
//     bit the pre-quantised path's, without Q's round trip through HBM.
template <int D, bool CAUSAL, int NW, bool QIN>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd<D>, kWavesPerSimd<D>)))
void fwd_fp8_kernel(const uint8_t* __restrict__ Q8, const uint8_t* __restrict__ K8,
                    const uint8_t* __restrict__ V8, const float* __restrict__ SQ,
                    const float* __restrict__ SK, const float* __restrict__ SV,
                    u16* __restrict__ O, float* __restrict__ LSE, int N, int ntq, int nwg,
                    int hpx, int nblk, float scale, const u16* __restrict__ Qbf,
                    const float* __restrict__ signs, float rsqrt_d) {
  using G = Geo8<D>;
  using CP = TileCopy8<D, NW>;
  constexpr int BR = 32 * NW;
  constexpr float kPExp = 6.f;    // P is scaled by 2^kPExp before the e4m3 cast
  constexpr float kLazy = 2.75f;  // rescale window: P * 2^kPExp <= 2^8.75 = 430
  // The V fold ratio r stays in [2^-4, 1]: its reciprocal within
  // [kVLow, kVHigh] (kVLow allows sv_ref * (1/sv_t) to round below 1 when
  // the two scales are equal; P * 2^6 * r <= 430 * 1.0001 < 448).
  constexpr float kVLow = 0.9999f;
  constexpr float kVHigh = 16.f;
  constexpr int kDsFirst = 4;  // K fragment reads issued before stage A's first product
  __shared__ __attribute__((aligned(1024))) char ks0[G::TILEB];
  __shared__ __attribute__((aligned(1024))) char vs0[G::TILEB];
  __shared__ __attribute__((aligned(1024))) char ks1[G::TILEB];
  __shared__ __attribute__((aligned(1024))) char vs1[G::TILEB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;

  int bh, qtr;
  tile_of_workgroup(blockIdx.x, nwg, ntq, CAUSAL ? hpx : 0, bh, qtr);
  const int qt = CAUSAL ? (ntq - 1 - qtr) : qtr;
  const size_t head = (size_t)bh * (size_t)N;
  const unsigned head_bytes = (unsigned)N * D;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q8 + head * D, head_bytes);
  const i32x4 rk = make_rsrc_words(K8 + head * D, head_bytes);
  const i32x4 rv = make_rsrc_words(V8 + head * D, head_bytes);
  const float* sqh = SQ + (size_t)bh * nblk;
  const float* skh = SK + (size_t)bh * nblk;
  const float* svh = SV + (size_t)bh * nblk;

  const int q0w = qt * BR + wave * 32;
  const int qi = q0w + l32;
  const int q_last = min(N, qt * BR + BR) - 1;
  const int T = CAUSAL ? (q_last / kBC + 1) : (N + kBC - 1) / kBC;

  if (dbg_flags(nwg) & kDbgPoison) {
    poison_lds(ks0, G::TILEB, tid, NW * 64);
    poison_lds(vs0, G::TILEB, tid, NW * 64);
    poison_lds(ks1, G::TILEB, tid, NW * 64);
    poison_lds(vs1, G::TILEB, tid, NW * 64);
    __syncthreads();
  }

  // Prologue: copy K_0, load (or quantise) Q, copy V_0 and K_1.
  const CP cp(wave, lane);
  cp.issue(rk, ks0, 0, wave, true);
  i32x8 qreg[G::NKS];
  float sq;
  if constexpr (QIN) {
    static_assert(BR == kBlock, "a workgroup's queries are one quantisation block");
    __shared__ __attribute__((aligned(16))) char qcodes[kBlock * D];
    __shared__ float red[4];
    if (dbg_flags(nwg) & kDbgPoison) {
      poison_lds(qcodes, kBlock * D, tid, NW * 64);
      __syncthreads();
    }
    BlockQuant<D, true, 4> bq;
    const __amdgpu_buffer_rsrc_t rqb = make_rsrc(Qbf + head * D, (unsigned)N * D * 2u);
    const float s = block_scale(block_max(bq.load(rqb, qt * kBlock, signs, tid), red, tid));
    bq.emit(1.f / s, tid, [&](int row, int ch, i32x2 packed) {
      *(i32x2*)(qcodes + row * D + ch * 8) = packed;
    });
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < G::NKS; ++ks) {
      const char* p = qcodes + (wave * 32 + l32) * D + ks * 64 + half * 32;
      qreg[ks] = __builtin_shufflevector(*(const i32x4*)p, *(const i32x4*)(p + 16), 0, 1, 2, 3,
                                         4, 5, 6, 7);
    }
    sq = s * rsqrt_d;
  } else {
#pragma unroll
    for (int ks = 0; ks < G::NKS; ++ks) {
      const unsigned off = (unsigned)qi * D + ks * 64 + half * 32;
      const i32x4 a = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
      const i32x4 b = __builtin_amdgcn_raw_buffer_load_b128(rq, off + 16, 0, 0);
      qreg[ks] = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    sq = sqh[min(qi, N - 1) / kBlock];
  }
  cp.issue(rv, vs0, 0, wave, true);
  cp.issue(rk, ks1, kBC, wave, T > 1);

  f32x16 oacc[G::NO];
#pragma unroll
  for (int i = 0; i < G::NO; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[i][v] = 0.f;
  f32x16 zero16;
#pragma unroll
  for (int v = 0; v < 16; ++v) zero16[v] = 0.f;
  float l_run = 0.f;        // sum of P * 2^6 over the tiles so far
  float m_ref = -INFINITY;  // reference maximum, log2 units of scale * q.k
  // Largest V block scale of the head: the first reference of the V fold
  // (scales are positive; a non-positive scale is read as this maximum, and
  // a non-positive maximum as 1: finite output without meaning).
  float sv_max = 0.f;
  for (int b = lane; b < nblk; b += 64) sv_max = fmaxf(sv_max, svh[b]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) sv_max = fmaxf(sv_max, __shfl_xor(sv_max, o));
  if (!(sv_max > 0.f)) sv_max = 1.f;
  float sv_ref = sv_max;  // the reference V scale of the fold (wave-uniform)
  const float c = scale * kLog2e;
  // Per-block factors of the key tiles, lane b holding block b0 + b: the
  // score factor c * s_Q * s_K (raw MFMA result -> log2 units), the block's
  // V scale and its reciprocal. A tile reads its block's factors with
  // readlane, so the key loop has no scalar loads (whose waits also drain
  // the LDS reads) and no divisions; the table is reloaded every 64 blocks.
  // s_Q is the same for all of the workgroup's queries (one quantisation
  // block). Measured +5-9% at d = 64 and 128; at d = 256 (one wave per SIMD,
  // 460 registers) the table cost 3-9%, so there each tile computes its
  // factors from the scales directly (the same values).
  constexpr bool kTable = D <= 128;
  float tab_cs = 0.f, tab_sv = 1.f, tab_isv = 1.f, tab_l2sv = 0.f;
  auto pos_sv = [&](float sv_b) { return sv_b > 0.f ? sv_b : sv_max; };
  auto load_tab = [&](int b0) {
    const int b = min(b0 + lane, nblk - 1);
    const float sk_b = skh[b];
    const float sv_b = pos_sv(svh[b]);
    tab_cs = c * sq * sk_b;
    tab_sv = sv_b;
    tab_isv = 1.f / sv_b;
    tab_l2sv = __log2f(sv_b);
  };
  if constexpr (kTable) load_tab(0);
  i32x8 ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838,
                0x38383838, 0x38383838, 0x38383838, 0x38383838};  // e4m3 1.0
  // Kept in registers at d = 128 (rebuilt before every row-sum product they
  // cost eight moves per tile; at d = 64, three waves per SIMD, the
  // registers spill instead, and d = 256 ran 1% slower).
  if constexpr (D == 128) asm volatile("" : "+v"(ones));
  float l2_ref = __log2f(sv_ref);  // log2 of the reference V scale

  // Loop-invariant per-lane LDS offsets (row swizzles depend on row & 15 only).
  int koff[G::NKS][2];
  {
    const int sw = swz8<D>(l32);
#pragma unroll
    for (int ks = 0; ks < G::NKS; ++ks)
#pragma unroll
      for (int u = 0; u < 2; ++u) koff[ks][u] = l32 * G::ROWB + (((ks * 4 + 2 * half + u) ^ sw) << 4);
  }
  int voff[G::NO];
  {
    const int g16 = lane >> 4, i16 = lane & 15;
    const int vq = i16 & 1, vt = i16 >> 1;  // tr8 source lane = 2 * vt + vq
    const int vrow = 8 * (vt >> 2) + 4 * half + (vt & 3);
    const int sw = swz8<D>(vrow);
#pragma unroll
    for (int i = 0; i < G::NO; ++i) {
      const int d = i * 32 + 16 * (g16 & 1) + 8 * vq;
      voff[i] = vrow * G::ROWB + (((d >> 4) ^ sw) << 4) + (d & 15);
    }
  }

  auto scores = [&](const char* kt, f32x16* s) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) s[kb][v] = 0.f;
#pragma unroll
    for (int ks = 0; ks < G::NKS; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const char* row = kt + kb * 32 * G::ROWB;
        const i32x4 lo = *(const i32x4*)(row + koff[ks][0]);
        const i32x4 hi = *(const i32x4*)(row + koff[ks][1]);
        s[kb] = mfma8(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), qreg[ks], s[kb]);
      }
  };
  auto mask = [&](f32x16* s, int j0) {
    if ((j0 + kBC > N) || (CAUSAL && j0 + kBC - 1 > q0w)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = j0 + kb * 32 + 8 * (v / 4) + 4 * half + (v % 4);
          if (key >= N || (CAUSAL && key > qi)) s[kb][v] = -INFINITY;
        }
    }
  };
  auto rowmax = [&](const f32x16* s) {
    float a = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = (kb == 0 ? 2 : 0); v < 16; ++v) a = fmaxf(a, s[kb][v]);
    return max_with_other_half(a);
  };

  f32x16 s_cur[2], s_nxt[2];
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * G::NKS + 2 * CP::NI));  // K_0 landed
  __syncthreads();
  scores(ks0, s_cur);
  mask(s_cur, 0);
  float mt = rowmax(s_cur);  // raw row max of the tile about to be processed

  // KIND: 0 = steady state (tile t+1 needs no mask), 1 = tile t+1 may need
  // masking, 2 = last tile (t = T-1): there is no tile t+1 to score or copy.
  // The per-block factors of the tile (one quantisation block spans two
  // tiles): read at the even tile of a block, reused at the odd one.
  float cs_blk = 0.f, sv_blk = 1.f, isv_blk = 1.f, l2_blk = 0.f;
  auto step = [&](auto kind_tag, auto odd_tag, const char* kr, const char* vr, char* kl,
                  char* vl, int t) {
    constexpr int KIND = decltype(kind_tag)::value;
    constexpr bool MASK = KIND == 1;
    constexpr bool LAST = KIND == 2;
    // ODD: tile t is the second tile of its block and the previous step
    // handled the first, with the same factors; the V reference then already
    // lies within its window (it either stayed or moved to this block's
    // scale), so the move check is skipped.
    constexpr bool ODD = decltype(odd_tag)::value;
    // Tile t lies in key block t / 2 (kBC = 64, kBlock = 128); a new table
    // is loaded before the wait below, which also covers these loads.
    static_assert(kBlock == 2 * kBC, "two key tiles per quantisation block");
    const int blk = t >> 1;
    if (kTable && (blk & 63) == 0 && blk > 0 && (t & 1) == 0) load_tab(blk);
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // K_{t+1} and V_t landed
    __syncthreads();
    if constexpr (!LAST) {
      cp.issue(rk, kl, (t + 2) * kBC, wave, t + 2 < T);
      cp.issue(rv, vl, (t + 1) * kBC, wave, t + 1 < T);
    }
    if constexpr (!ODD) {
      if constexpr (kTable) {
        cs_blk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tab_cs), blk & 63));
        sv_blk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tab_sv), blk & 63));
        isv_blk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tab_isv), blk & 63));
        l2_blk = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tab_l2sv), blk & 63));
      } else {
        cs_blk = c * sq * skh[blk];
        sv_blk = pos_sv(svh[blk]);
        isv_blk = 1.f / sv_blk;
        l2_blk = __log2f(sv_blk);
      }
    }
    const float cs = cs_blk, sv_t = sv_blk, isv_t = isv_blk, l2_t = l2_blk;
    // 1 / r_t = sv_ref / sv_t (IEEE products: the accumulator's scaling and
    // the row sum use these; the fold factor inside exp2 only needs to be
    // close, its error cancels between P V and the row sum). The reference
    // moves when r_t > 1 (beyond rounding) or r_t < 2^-4.
    float inv_r = sv_ref * isv_t;
    const bool vmove = !ODD && (inv_r < kVLow || inv_r > kVHigh);
    const float mx = mt * cs;
    if (__any(vmove || mx - m_ref > kLazy)) {
      // New reference maximum (per lane) and, if the V fold ratio left its
      // window, new reference V scale sv_t: O and l follow the maximum, O
      // also the V reference (l counts probabilities, not P * r).
      const float m_new = fmaxf(m_ref, mx);
      const float am = (m_ref == -INFINITY) ? 0.f : fast_exp2(m_ref - m_new);
      const float alpha = vmove ? am * inv_r : am;
      l_run *= am;
#pragma unroll
      for (int i = 0; i < G::NO; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[i][v] *= alpha;
      m_ref = m_new;
      if (vmove) {
        sv_ref = sv_t;
        l2_ref = l2_t;
        inv_r = 1.f;
      }
    }
    // log2 r_t, from the logs of the two scales: 0 when they are equal.
    const float log2_r = l2_t - l2_ref;
    // exponent offset: 2^6 headroom, the reference maximum and the V fold
    const float mb = kPExp - ((m_ref == -INFINITY) ? 0.f : m_ref) + log2_r;
    // Stage A: scores of tile t+1; softmax of tile t -> P * 2^6 as e4m3.
    __builtin_amdgcn_s_setprio(1);
    if constexpr (!LAST) scores(kr, s_nxt);
    i32x8 pv;  // byte b = kb * 16 + v
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        float e[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) e[x] = fast_exp2(fmaf(s_cur[kb][4 * v4 + x], cs, mb));
        // Both halves are written, so the first conversion may start from
        // any register: e[0]'s, which it reads anyway (no zeroing move).
        const int w = cvt_pk_fp8<false>(e[0], e[1], __float_as_int(e[0]));
        pv[kb * 4 + v4] = cvt_pk_fp8<true>(e[2], e[3], w);
      }
    // d <= 128: V_t's fragments for stage B are read during stage A, behind
    // the K reads, so that the P V products do not wait on the LDS (+1 to
    // +2%); at d = 256 (one wave per SIMD) they are read in stage B (-1%
    // otherwise).
    auto read_v = [&](i32x8* vf) {
#pragma unroll
      for (int i = 0; i < G::NO; ++i) {
        const char* base = vr + voff[i];
        const i32x2 p0 = tr8(base);
        const i32x2 p1 = tr8(base + 16 * G::ROWB);
        const i32x2 p2 = tr8(base + 32 * G::ROWB);
        const i32x2 p3 = tr8(base + 48 * G::ROWB);
        vf[i] = (i32x8){p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
      }
    };
    constexpr bool kVPre = D <= 128;
    i32x8 vf[G::NO];
    if constexpr (kVPre) read_v(vf);
    if constexpr (!LAST) {
      constexpr int NMF = 2 * G::NKS;             // products of stage A
      constexpr int DS_K = 2 * NMF, DS_V = kVPre ? 4 * G::NO : 0;
      constexpr int DS_FIRST = kDsFirst;
      constexpr int DS_PER = (DS_K + DS_V - DS_FIRST + NMF - 1) / NMF;
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, DS_FIRST, 0);
#pragma unroll
      for (int i = 0; i < NMF; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedValu, 10, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, DS_PER, 0);
      }
    }
    // Nothing moves across: the softmax and the reads stay in stage A.
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    // Stage B: P V of tile t and the row sums; then the next tile's row max.
    if constexpr (!kVPre) read_v(vf);
#pragma unroll
    for (int i = 0; i < G::NO; ++i) oacc[i] = mfma8(vf[i], pv, oacc[i]);
    const f32x16 lt = mfma8(ones, pv, zero16);
    l_run = fmaf(lt[0], inv_r, l_run);
    if constexpr (!LAST) {
      if constexpr (MASK) mask(s_nxt, (t + 1) * kBC);
      mt = rowmax(s_nxt);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s_cur[kb] = s_nxt[kb];
    }
  };
  // Tiles j < J need no mask for any wave: every key of them precedes the
  // workgroup's first query (causal) and lies inside the sequence.
  const int J = CAUSAL ? min(N / kBC, (qt * BR + 1) / kBC) : N / kBC;
  using Steady = std::integral_constant<int, 0>;
  using Masked = std::integral_constant<int, 1>;
  using Last = std::integral_constant<int, 2>;
  using Even = std::false_type;
  using Odd = std::true_type;
  int t = 0;
  for (; t + 2 < J; t += 2) {  // steps whose next tile (t+1, t+2) is unmasked
    step(Steady{}, Even{}, ks1, vs0, ks0, vs1, t);
    step(Steady{}, Odd{}, ks0, vs1, ks1, vs0, t + 1);
  }
  for (; t + 2 < T; t += 2) {  // t is even here: stage parity stays static
    step(Masked{}, Even{}, ks1, vs0, ks0, vs1, t);
    step(Masked{}, Odd{}, ks0, vs1, ks1, vs0, t + 1);
  }
  if (t + 1 < T) {  // two tiles left
    step(Masked{}, Even{}, ks1, vs0, ks0, vs1, t);
    ++t;
  }
  // The last step only finishes tile t (reads V_t); one call site with the
  // stage chosen at run time.
  step(Last{}, Even{}, ks0, (t & 1) ? vs1 : vs0, ks1, (t & 1) ? vs0 : vs1, t);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // no copy lands after the exit

  // Stage the output rows through LDS (whole-row stores): once every wave
  // has finished the last step no stage is read and no copy is in flight,
  // and wave w uses stage w (an e4m3 tile of 64 x d bytes holds a wave's 32
  // rows of d bf16).
  static_assert(NW == 4 && 32 * 2 * D <= G::TILEB, "staging slots fit the stages");
  __syncthreads();
  char* const slot = wave == 0 ? ks0 : wave == 1 ? ks1 : wave == 2 ? vs0 : vs1;
  const float l_tot = l_run;  // sum of P * 2^6
  store_o_lse_staged<D>(O, LSE, head, N, q0w, lane, oacc, sv_ref / l_tot,
                        (m_ref + __log2f(l_tot) - kPExp) * kLn2, slot);
}

// q8 == nullptr: Q is qbf (bf16), quantised inside the kernel with `signs`.
template <int D, bool CAUSAL>
hipError_t fwd_launch(const void* q8, const void* k8, const void* v8, const float* sq,
                      const float* sk, const float* sv, void* o, float* lse, int B, int H, int N,
                      float scale, hipStream_t stream, const void* qbf = nullptr,
                      const float* signs = nullptr) {
  constexpr int NW = 4;
  constexpr int BR = 32 * NW;
  const int ntq = (N + BR - 1) / BR;
  const long long nwg = (long long)ntq * B * H;
  if (nwg >= (1LL << 31)) return hipErrorInvalidValue;
  const int nblk = (N + kBlock - 1) / kBlock;
  const int dbg = debug_flags();
  // Causal: whole heads per XCD, longest tiles first, when the heads split
  // evenly (not under the reversed debug order).
  const int hpx = ((long long)B * H) % 8 == 0 && !(dbg & 1) ? (int)(((long long)B * H) / 8) : 0;
  const int nwg_arg = (int)nwg | (dbg << kDbgShift);
  if (q8 == nullptr) {
    const float rsqrt_d = (float)(1.0 / sqrt((double)D));  // as the quantisation pass
    hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL, NW, true>), dim3((unsigned)nwg), dim3(NW * 64),
                       0, stream, nullptr, (const uint8_t*)k8, (const uint8_t*)v8, nullptr, sk,
                       sv, (u16*)o, lse, N, ntq, nwg_arg, hpx, nblk, scale, (const u16*)qbf,
                       signs, rsqrt_d);
  } else {
    hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL, NW, false>), dim3((unsigned)nwg), dim3(NW * 64),
                       0, stream, (const uint8_t*)q8, (const uint8_t*)k8, (const uint8_t*)v8, sq,
                       sk, sv, (u16*)o, lse, N, ntq, nwg_arg, hpx, nblk, scale, nullptr, nullptr,
                       0.f);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_kv_fp8(const void* k, const void* v, void* k8, void* v8, float* sk,
                               float* sv, float* signs, unsigned long long key, int B, int H,
                               int N, int d, hipStream_t stream) {
  const int nblk = (N + kBlock - 1) / kBlock;
  const long long ngrid = (long long)nblk * B * H;
  if (ngrid >= (1LL << 31)) return hipErrorInvalidValue;
  const float rsqrt_d = (float)(1.0 / sqrt((double)d));
#define FA_CASE(DD)                                                                         \
  case DD:                                                                                  \
    hipLaunchKernelGGL((quant_kv_fp8_kernel<DD>), dim3((unsigned)ngrid, 2), dim3(256), 0,   \
                       stream, (const u16*)k, (const u16*)v, (uint8_t*)k8, (uint8_t*)v8, sk, \
                       sv, signs, key, N, nblk, rsqrt_d);                                   \
    return hipGetLastError();
  switch (d) {
    FA_CASE(64)
    FA_CASE(128)
    FA_CASE(256)
    default:
      return hipErrorInvalidValue;
  }
#undef FA_CASE
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

hipError_t launch_fwd_fp8_qbf16(const void* qbf, const float* signs, const void* k8,
                                const void* v8, const float* sk, const float* sv, void* o,
                                float* lse, int B, int H, int N, int d, bool causal, float scale,
                                hipStream_t stream) {
#define FA_CASE(DD)                                                                           \
  case DD:                                                                                    \
    return causal ? fwd_launch<DD, true>(nullptr, k8, v8, nullptr, sk, sv, o, lse, B, H, N,   \
                                         scale, stream, qbf, signs)                           \
                  : fwd_launch<DD, false>(nullptr, k8, v8, nullptr, sk, sv, o, lse, B, H, N,  \
                                          scale, stream, qbf, signs);
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
