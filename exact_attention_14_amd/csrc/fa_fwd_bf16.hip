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
// post, "Contribuciones clave"). While one K/V tile is used the next one is
// already being copied into the other half of a double buffer (dibro.site
// post, "Arquitectura y metodo": two on-chip buffers in alternation; vikram-blog
// post, "System Topology & Data Flow").
//
// gfx950 mapping
//   * A workgroup owns Br = 32*NW queries of one (batch, head): NW waves of 32.
//   * K/V tiles of Bc = 64 keys move HBM -> LDS with buffer_load_dwordx4 ... lds
//     (direct to LDS, no registers, zero-filled past the sequence end by the
//     buffer's range check) into a two-stage LDS ring. Rows are 16-byte-chunk
//     XOR-swizzled so that both read patterns below are free of bank conflicts.
//   * Scores are formed transposed, S^T = K Q^T, on v_mfma_f32_32x32x16_bf16:
//     each lane owns ONE query (lane % 32) and 16 of the 32 keys of a 32-key
//     block, so the row max and row sum are in-lane reductions plus one
//     exchange with the other half of the wave. Q stays in registers.
//   * The output is accumulated transposed too, O^T += V^T P^T, so the
//     rescale is a per-lane scalar, and P^T is fed from the very registers that
//     held S^T. V stays row-major in LDS and is read transposed with
//     ds_read_b64_tr_b16, whose lane order matches P's register order.
//   * exp is evaluated as exp2 with scale*log2(e) folded into one FMA. The
//     accumulator is rescaled only when some row maximum of the wave grew by
//     more than 2^8 since the reference used so far; O and l always share the
//     same reference, so the result is unchanged (exp values stay <= 2^8).
//   * Workgroups are renumbered so that the query tiles of one (batch, head)
//     run on one XCD (workgroups are dealt to the 8 XCDs round-robin), which
//     keeps that head's K/V in one L2. Causal query tiles run longest first.
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {
namespace {

constexpr int kBC = 64;          // keys per K/V tile
constexpr float kLazyLog2 = 8.f; // rescale threshold, log2 units

template <int D>
struct Geo {
  static constexpr int CPR = D / 8;                                  // 16-B chunks of data per row
  static constexpr int CPRP = D == 64 ? 8 : (D == 256 ? 32 : 16);    // chunk slots per LDS row
  static constexpr int ROWB = CPRP * 16;                             // bytes per LDS row
  static constexpr int TILEB = kBC * ROWB;                           // one K or V tile
  static constexpr int STAGEB = 2 * TILEB;                           // K + V
  static constexpr int NK = D / 16;                                  // k-steps of S^T = K Q^T
  static constexpr int NO = D / 32;                                  // 32-row blocks of O^T
};

// Chunk-slot XOR for LDS row `row`; see the design notes for the bank model.
template <int CPRP>
__device__ __forceinline__ int swz(int row) {
  if constexpr (CPRP == 8) {
    const int s = row >> 1;
    return ((s & 1) << 2) | ((s >> 1) & 3);
  } else {
    return ((row & 3) << 2) | ((row >> 2) & 3);
  }
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ bf16x8 tr_pair(const char* lo, const char* hi) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)lo);
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)hi);
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

// Issue this wave's share of the direct-to-LDS copies of one K or V tile.
template <int D, int NW>
__device__ __forceinline__ void load_tile(__amdgpu_buffer_rsrc_t rs, char* tile, int j0,
                                          int wave, int lane) {
  using G = Geo<D>;
  constexpr int NI = G::CPRP / NW;  // 1 KiB wave copies per tile per wave
  static_assert(NI >= 1 && G::CPRP % NW == 0, "tile split");
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int slot = (i * NW + wave) * 64 + lane;  // chunk slot in the tile
    const int row = slot / G::CPRP;
    const int c = (slot % G::CPRP) ^ swz<G::CPRP>(row);
    const unsigned off = c < G::CPR ? ((unsigned)(j0 + row) * D + c * 8) * 2u : 0x80000000u;
    copy16_to_lds(rs, tile + (i * NW + wave) * 1024, off);
  }
}

template <int D, bool CAUSAL, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(D == 256 ? 1 : 2, D == 256 ? 1 : 2))) void fwd_bf16_kernel(
    const u16* __restrict__ Q, const u16* __restrict__ K, const u16* __restrict__ V,
    u16* __restrict__ O, float* __restrict__ LSE, int N, int ntq, int nwg, float scale) {
  using G = Geo<D>;
  constexpr int BR = 32 * NW;
  // One LDS object per (stage, tensor): with the loop unrolled by two every
  // read and every in-flight copy names a distinct object, so the compiler
  // need not wait for the next tile's copies before reading the current one.
  __shared__ __attribute__((aligned(1024))) char ks0[G::TILEB];
  __shared__ __attribute__((aligned(1024))) char vs0[G::TILEB];
  __shared__ __attribute__((aligned(1024))) char ks1[G::TILEB];
  __shared__ __attribute__((aligned(1024))) char vs1[G::TILEB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;

  // Workgroup id -> logical id with the tiles of one head on one XCD.
  const int lid = xcd_grouped_id(blockIdx.x, nwg);
  const int qtr = lid % ntq;
  const int bh = lid / ntq;
  const int qt = CAUSAL ? (ntq - 1 - qtr) : qtr;
  const size_t head = (size_t)bh * (size_t)N;
  const unsigned head_bytes = (unsigned)N * D * 2u;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + head * D, head_bytes);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(K + head * D, head_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(V + head * D, head_bytes);

  const int q0w = qt * BR + wave * 32;  // first query of this wave
  const int qi = q0w + l32;             // this lane's query
  const int q_last = min(N, qt * BR + BR) - 1;
  const int ntiles = CAUSAL ? (q_last / kBC + 1) : (N + kBC - 1) / kBC;

  load_tile<D, NW>(rk, ks0, 0, wave, lane);
  load_tile<D, NW>(rv, vs0, 0, wave, lane);

  bf16x8 qreg[G::NK];
#pragma unroll
  for (int kk = 0; kk < G::NK; ++kk) {
    const i32x4 w = __builtin_amdgcn_raw_buffer_load_b128(
        rq, (unsigned)(qi * D + kk * 16 + half * 8) * 2u, 0, 0);
    qreg[kk] = __builtin_bit_cast(bf16x8, w);
  }

  f32x16 oacc[G::NO];
#pragma unroll
  for (int i = 0; i < G::NO; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[i][v] = 0.f;
  float m_ref = -INFINITY;  // reference maximum (raw scores q.k) of O and l
  float l_run = 0.f;        // this lane's half of the row sum
  const float c = scale * kLog2e;

  // Per-lane LDS byte offsets inside a tile.
  const int krow = l32;                                   // + kb*32
  const int kswz = swz<G::CPRP>(krow);
  const int g16 = lane >> 4, i16 = lane & 15;             // tr16 lane group
  const int vrow = 4 * half + (i16 >> 2);                 // + kb*32 + a*16 + r*8
  const int vcol = (g16 & 1) * 2 + ((i16 & 3) >> 1);      // + blk*4 (chunk)
  const int vbyte = (i16 & 1) * 8;

  // One K/V tile: kt/vt hold tile t, kn/vn receive tile t+1.
  auto step = [&](const char* kt, const char* vt, char* kn, char* vn, int t) {
    // This wave's copies of tile t have landed (vmcnt counts LDS-DMA copies);
    // after the barrier every wave's have, and the other stage is free.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (t + 1 < ntiles) {
      load_tile<D, NW>(rk, kn, (t + 1) * kBC, wave, lane);
      load_tile<D, NW>(rv, vn, (t + 1) * kBC, wave, lane);
    }
    const int j0 = t * kBC;
    if (CAUSAL && j0 > q0w + 31) return;  // every key after every query of this wave

    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 acc;
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[v] = 0.f;
#pragma unroll
      for (int kk = 0; kk < G::NK; ++kk) {
        const int chunk = (2 * kk + half) ^ kswz;
        const bf16x8 a =
            *(const bf16x8*)(kt + (kb * 32 + krow) * G::ROWB + chunk * 16);
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

    float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = (kb == 0 ? 2 : 0); v < 16; ++v) mx = fmaxf(mx, s[kb][v]);
    mx = fmaxf(mx, xor32(mx));
    // Move the reference when a row maximum exceeds it by more than 2^8 (or
    // on the first keys a row sees); all lanes of the wave move together.
    if (__any((mx - m_ref) * c > kLazyLog2)) {
      const float m_new = fmaxf(m_ref, mx);
      const float alpha = (m_ref == -INFINITY) ? 0.f : fast_exp2((m_ref - m_new) * c);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < G::NO; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[i][v] *= alpha;
      m_ref = m_new;
    }
    const float mc = (m_ref == -INFINITY) ? 0.f : m_ref * c;
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
    l_run += lsum;

#pragma unroll
    for (int i = 0; i < G::NO; ++i)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const int row0 = kb * 32 + a * 16 + vrow;           // read r = 0
          const int row1 = row0 + 8;                          // read r = 1
          const int ch = i * 4 + vcol;
          const char* lo = vt + row0 * G::ROWB + ((ch ^ swz<G::CPRP>(row0)) * 16) + vbyte;
          const char* hi = vt + row1 * G::ROWB + ((ch ^ swz<G::CPRP>(row1)) * 16) + vbyte;
          oacc[i] = mfma32(tr_pair(lo, hi), p[kb][a], oacc[i]);
        }
    };
  for (int t = 0; t < ntiles; t += 2) {
    step(ks0, vs0, ks1, vs1, t);
    if (t + 1 < ntiles) step(ks1, vs1, ks0, vs0, t + 1);
  }

  const float l_tot = l_run + xor32(l_run);
  const float inv = 1.f / l_tot;
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
    if (LSE != nullptr && half == 0) LSE[head + qi] = m_ref * scale + __logf(l_tot);
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                  int H, int N, float scale, hipStream_t stream) {
  constexpr int NW = 4;
  constexpr int BR = 32 * NW;
  const int ntq = (N + BR - 1) / BR;
  const long long nwg = (long long)ntq * B * H;
  if (nwg >= (1LL << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, NW>), dim3((unsigned)nwg), dim3(NW * 64), 0,
                     stream, (const u16*)q, (const u16*)k, (const u16*)v, (u16*)o, lse, N, ntq,
                     (int)nwg, scale);
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
