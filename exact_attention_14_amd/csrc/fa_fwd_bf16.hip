// FlashAttention forward, bf16 inputs, fp32 accumulation, gfx950 matrix cores.
//
// Method (droidorbit FlashAttention-3 explainer, "Mathematical Formulation:
// The Online Softmax Rescaling Trick"; dibro.site FlashAttention-3 post,
// "Arquitectura y metodo"): Q is split into tiles of Br rows and K, V into
// tiles of Bc rows; for each K/V tile the scores of a Q tile are formed on
// chip, the running row maximum m and row sum l are updated, the output
// accumulator is rescaled by exp(m_prev - m_new), and P V is accumulated.
// The normalisation by l happens once at the end. Causal query tiles stop at
// the last key tile that holds a key at or before their last query (dibro.site
// post, "Contribuciones clave").
//
// gfx950 mapping
//   * A workgroup owns Br = 128 queries of one (batch, head) as 4 waves of 32.
//   * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//     each lane then owns ONE query (lane % 32) and 16 of the 32 keys of a
//     32-key block, so the row maximum and row sum are in-lane reductions
//     plus one exchange with the other half of the wave.
//   * The output is accumulated transposed too, O^T += V^T P^T, so the
//     rescale by exp(m_prev - m_new) is a per-lane scalar.
//   * P^T is fed to the second product straight from the registers that hold
//     S^T. The reduction order over keys is free, so V is stored transposed in
//     LDS with its key columns permuted (bits 2 and 3 of the key index swapped)
//     to match the order in which P's registers hold the keys; each operand of
//     the second product is then one 16-byte LDS read.
//   * exp is evaluated as exp2 with scale*log2(e) folded into one FMA.
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kBR = 128;       // queries per workgroup
constexpr int kBC = 64;        // keys per K/V tile
constexpr int kThreads = 256;  // 4 waves
constexpr int kPad = 8;        // 16 bytes of padding per LDS row

// Column of key `key` (0..63 within a tile) in the transposed V tile.
__device__ __forceinline__ int vt_col(int key) {
  return (key & ~0xC) | ((key & 4) << 1) | ((key & 8) >> 1);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fwd_bf16_kernel(
    const u16* __restrict__ Q, const u16* __restrict__ K,
    const u16* __restrict__ V, u16* __restrict__ O, float* __restrict__ LSE,
    int H, int N, int ntq, float scale) {
  constexpr int KS = D + kPad;    // K tile row stride (elements)
  constexpr int VS = kBC + kPad;  // transposed V tile row stride (elements)
  constexpr int NK = D / 16;      // reduction steps of S^T = K Q^T
  constexpr int NO = D / 32;      // 32-row blocks of O^T
  __shared__ __attribute__((aligned(16))) u16 Ks[kBC * KS];
  __shared__ __attribute__((aligned(16))) u16 Vt[D * VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  // Workgroup -> (batch, head, query tile); causal tiles longest first.
  const int bid = blockIdx.x;
  const int qtr = bid % ntq;
  const int bh = bid / ntq;
  const int qt = CAUSAL ? (ntq - 1 - qtr) : qtr;
  const size_t head = (size_t)bh * (size_t)N;
  const u16* Qh = Q + head * D;
  const u16* Kh = K + head * D;
  const u16* Vh = V + head * D;

  const int q0w = qt * kBR + wave * 32;  // first query of this wave
  const int qi = q0w + l32;              // this lane's query
  const bool qvalid = qi < N;

  bf16x8 qreg[NK];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    uint4 w = {0u, 0u, 0u, 0u};
    if (qvalid) w = *(const uint4*)(Qh + (size_t)qi * D + kk * 16 + half * 8);
    qreg[kk] = __builtin_bit_cast(bf16x8, w);
  }

  f32x16 oacc[NO];
#pragma unroll
  for (int i = 0; i < NO; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[i][v] = 0.f;
  float m_run = -INFINITY;  // running max of the raw scores q.k
  float l_run = 0.f;        // this lane's half of the running row sum
  const float c = scale * kLog2e;

  const int q_last = min(N, qt * kBR + kBR) - 1;
  const int ntiles = CAUSAL ? (q_last / kBC + 1) : (N + kBC - 1) / kBC;

  for (int t = 0; t < ntiles; ++t) {
    const int j0 = t * kBC;
    __syncthreads();  // previous tile fully consumed
#pragma unroll
    for (int it = 0; it < D / 32; ++it) {
      const int id = it * kThreads + tid;
      const int row = id / (D / 8), ch = id % (D / 8);
      uint4 w = {0u, 0u, 0u, 0u};
      if (j0 + row < N) w = *(const uint4*)(Kh + (size_t)(j0 + row) * D + ch * 8);
      *(uint4*)(Ks + row * KS + ch * 8) = w;
    }
#pragma unroll
    for (int it = 0; it < D / 32; ++it) {
      const int id = it * kThreads + tid;
      const int key = id % kBC, ch = id / kBC;
      uint4 w = {0u, 0u, 0u, 0u};
      if (j0 + key < N) w = *(const uint4*)(Vh + (size_t)(j0 + key) * D + ch * 8);
      const u16* e = (const u16*)&w;
      const int col = vt_col(key);
#pragma unroll
      for (int x = 0; x < 8; ++x) Vt[(ch * 8 + x) * VS + col] = e[x];
    }
    __syncthreads();

    if (CAUSAL && j0 > q0w + 31) continue;  // every key after every query of this wave

    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 acc;
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const bf16x8 a = *(const bf16x8*)(Ks + (kb * 32 + l32) * KS + kk * 16 + half * 8);
        acc = mfma32(a, qreg[kk], acc);
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

    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;  // no (-inf) - (-inf)
    const float alpha = fast_exp2((m_run - m_use) * c);
    const float mc = m_use * c;
    float lsum = 0.f;
    bf16x8 p[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float e = fast_exp2(fmaf(s[kb][v], c, -mc));
        lsum += e;
        p[kb][v / 8][v % 8] = (__bf16)e;
      }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < NO; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) oacc[i][v] *= alpha;

#pragma unroll
    for (int i = 0; i < NO; ++i)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const bf16x8 vv =
              *(const bf16x8*)(Vt + (i * 32 + l32) * VS + kb * 32 + a * 16 + half * 8);
          oacc[i] = mfma32(vv, p[kb][a], oacc[i]);
        }
  }

  const float l_tot = l_run + xor32(l_run);
  const float inv = 1.f / l_tot;
  if (qvalid) {
    u16* orow = O + (head + qi) * D;
#pragma unroll
    for (int i = 0; i < NO; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 w;
#pragma unroll
        for (int x = 0; x < 4; ++x) w[x] = (__bf16)(oacc[i][4 * g + x] * inv);
        *(bf16x4*)(orow + i * 32 + 8 * g + 4 * half) = w;
      }
    if (LSE != nullptr && half == 0) LSE[head + qi] = m_run * scale + __logf(l_tot);
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int N, float scale, hipStream_t stream) {
  const int ntq = (N + kBR - 1) / kBR;
  const long long nwg = (long long)ntq * B * H;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3((unsigned)nwg), dim3(kThreads), 0,
                     stream, (const u16*)q, (const u16*)k, (const u16*)v, (u16*)o, lse, H, N,
                     ntq, scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           int B, int H, int N, int d, bool causal, float scale,
                           hipStream_t stream) {
#define FA_CASE(DD)                                                               \
  case DD:                                                                        \
    return causal ? launch<DD, true>(q, k, v, o, lse, B, H, N, scale, stream)     \
                  : launch<DD, false>(q, k, v, o, lse, B, H, N, scale, stream);
  switch (d) {
    FA_CASE(64)
    FA_CASE(96)
    FA_CASE(128)
    FA_CASE(256)
    default:
      return hipErrorInvalidValue;
  }
#undef FA_CASE
}

}  // namespace fa
