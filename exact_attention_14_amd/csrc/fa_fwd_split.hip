// Split-KV attention forward (bf16, gfx950): Nq queries of each (batch, head)
// against Nk keys and values, the key range cut into `splits` parts that
// run as separate workgroups, their partial results merged by log-sum-exp.
//
// This is the FlashDecoding idea (droidorbit FlashAttention-3 explainer, FAQ
// on FlashDecoding: parallelise over the key/value length, for decode) on
// the forward's building blocks: when B*H*ceil(Nq/Br) workgroups cannot fill
// 256 compute units (decode: Nq = 1; or few heads), the key axis supplies the
// parallelism. With the causal mask the queries are the last Nq positions:
// query i attends keys j <= i + Nk - Nq.
//
// Each workgroup (NW waves, 32 queries per wave, one lane per query as in the
// forward kernel) runs the online softmax over its split's key tiles and
// writes, in float32, its partial output normalised by its own row sum and
// its partial log-sum-exp (-inf when the split holds no key the query
// attends). A second kernel merges the splits of each row:
//   LSE = log sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) O_s.
#include <algorithm>
#include <math.h>
#include <mutex>

#include <type_traits>

#include "../../include/fa.h"
#include "fa_common.hpp"
#include "fa_launch.hpp"
#include "fa_tiles_bf16.hpp"

namespace fa {
namespace {

// KT keys per tile, S stages in the LDS ring (tiles t+1 .. t+S-2 stay in
// flight while tile t is used). Decode runs NW = 1, KT = 32, S = 2: 32 KiB of
// LDS per workgroup (d = 128) lets five workgroups share a compute unit,
// which streams K and V faster than deeper rings with fewer workgroups
// (measured: 64 KiB rings of 64-key or 4 x 32-key tiles, two workgroups per
// unit, reached 10% less; K loaded straight into registers two tiles ahead,
// eight workgroups per unit, 2% less). Longer queries run NW = 4, KT = 64,
// S = 2.
template <int D, bool CAUSAL, int NW, int KT, int S>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2))) void fwd_split_kernel(
    const u16* __restrict__ Q, const u16* __restrict__ K, const u16* __restrict__ V,
    float* __restrict__ Op, float* __restrict__ Lp, int Nq, int Nk, int nqt, int splits, int tps,
    int nwg, float scale, int dbg) {
  using G = Geo<D>;
  using CP = TileCopy<D, NW, KT>;
  static_assert(KT == 32 || KT == 64, "32- or 64-key tiles");
  static_assert(S >= 2 && (S - 2) * 2 * CP::NI <= 63, "copies in flight fit the wait counter");
  constexpr int BR = 32 * NW;   // queries per workgroup
  constexpr int NB = KT / 32;   // 32-key blocks per tile
  constexpr int TB = KT * G::ROWB;  // bytes of one K or V tile
  __shared__ __attribute__((aligned(1024))) char ring[S * 2 * TB];  // stage st: K, then V

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = NW == 1 ? 0 : __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;

  // Non-causal (and decode): the (query tile, split) items of one head run
  // on one accelerator die (consecutive logical ids), query tiles fastest:
  // they share the split's key/value tiles in that die's L2. Causal with
  // several query tiles: items differ in length (a split past a query tile's
  // diagonal is empty), so they start longest first: the heads interleaved
  // (workgroup id modulo B*H, which also keeps each die on the same heads
  // when B*H divides 8 or 8 divides B*H), then query tiles from the last,
  // their splits consecutive. Grouping a head's items on one die would give
  // the die of its last query tiles most of the work.
  // dbg (kDbgReverse, kDbgPoison): the debug order and LDS poison of the
  // forward kernels, passed apart from nwg: one-wave workgroups make this
  // grid reach 2^26, past the bits the other kernels leave for the flags.
  const unsigned bid = (dbg & kDbgReverse) ? (unsigned)nwg - 1u - blockIdx.x : blockIdx.x;
  int bh, sp, qt;
  if constexpr (CAUSAL && NW > 1) {
    const int bht = nwg / (nqt * splits);
    bh = (int)(bid % (unsigned)bht);
    const int rank = (int)(bid / (unsigned)bht);
    qt = nqt - 1 - rank / splits;
    sp = rank % splits;
  } else {
    int rank;
    tile_of_id((int)bid, nwg, nqt * splits, 0, bh, rank);
    sp = rank / nqt;
    qt = rank % nqt;
  }
  const int q0w = qt * BR + wave * 32;
  const int qi = q0w + l32;
  const int delta = Nk - Nq;  // causal: query i attends keys <= i + delta

  // tps counts 64-key tiles; this kernel's tiles hold KT keys
  const int t_all = (Nk + KT - 1) / KT;
  const int t_begin = sp * tps * (kBC / KT);
  int t_end = min(t_all, t_begin + tps * (kBC / KT));
  if (CAUSAL) t_end = min(t_end, (min(Nq, qt * BR + BR) - 1 + delta) / KT + 1);
  if (t_begin >= t_end) {
    // None of the workgroup's queries attends a key of this split: only the
    // -inf log-sum-exps are written; the merge skips such a split without
    // reading its partial output.
    const size_t slab = ((size_t)bh * splits + sp) * (size_t)Nq;
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(Lp + slab, (unsigned)Nq * 4u);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(-INFINITY), rl,
                                          half == 0 ? (unsigned)qi * 4u : kOutOfRange, 0, 0);
    return;
  }

  const size_t qhead = (size_t)bh * (size_t)Nq;
  const size_t khead = (size_t)bh * (size_t)Nk;
  const unsigned kv_bytes = (unsigned)Nk * D * 2u;
  const i32x4 rk = make_rsrc_words(K + khead * D, kv_bytes);
  const i32x4 rv = make_rsrc_words(V + khead * D, kv_bytes);

  // Q rows of the lane's query (zeros past Nq) as B operands.
  bf16x8 qreg[G::NK];
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + qhead * D, (unsigned)Nq * D * 2u);
#pragma unroll
    for (int kk = 0; kk < G::NK; ++kk)
      qreg[kk] = __builtin_bit_cast(
          bf16x8, __builtin_amdgcn_raw_buffer_load_b128(
                      rq, (unsigned)(qi * D + kk * 16 + half * 8) * 2u, 0, 0));
  }
  // Let the Q loads land before any tile copy is issued: the compiler does
  // not see the copies, and a wait for Q placed inside the loop would also
  // wait for the copies issued ahead there.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  if (dbg & kDbgPoison) {
    poison_lds(ring, (int)sizeof(ring), tid, 64 * NW);
    __syncthreads();
  }
  const CP cp(wave, lane);
  auto issue = [&](int t) {
    char* const st = ring + ((t - t_begin) % S) * (2 * TB);
    cp.issue(rk, st, t * KT, wave, true);
    cp.issue(rv, st + TB, t * KT, wave, true);
  };
  for (int t = t_begin; t < min(t_end, t_begin + S - 1); ++t) issue(t);

  // Loop-invariant LDS offsets (the forward kernel's): K rows as A operands,
  // V read transposed as the A operand of O^T += V^T P^T.
  int koff[G::NK];
  {
    const int kswz = swz<G::CPRP>(l32);
#pragma unroll
    for (int kk = 0; kk < G::NK; ++kk) koff[kk] = l32 * G::ROWB + (((2 * kk + half) ^ kswz) << 4);
  }
  int voff[G::NO][2];
  {
    const int g16 = lane >> 4, i16 = lane & 15;
    const int vrow = 4 * half + (i16 >> 2);
    const int vcol = (g16 & 1) * 2 + ((i16 & 3) >> 1);
    const int vbyte = (i16 & 1) * 8;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int row = vrow + 8 * r;
      const int sw = swz<G::CPRP>(row);
#pragma unroll
      for (int i = 0; i < G::NO; ++i)
        voff[i][r] = row * G::ROWB + (((i * 4 + vcol) ^ sw) << 4) + vbyte;
    }
  }

  f32x16 oacc[G::NO];
#pragma unroll
  for (int i = 0; i < G::NO; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[i][v] = 0.f;
  float m_run = -INFINITY;  // running maximum of the raw scores
  float l_run = 0.f;        // this lane's share of the running row sum
  const float c = scale * kLog2e;

  for (int t = t_begin; t < t_end; ++t) {
    // Tile t has landed once at most the copies of tiles t+1 .. t+S-2 are
    // outstanding (fewer near the end of the split).
    const int ahead = min(S - 2, t_end - 1 - t);
    if (ahead <= 0) {
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    } else if (ahead == 1) {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * CP::NI));
    } else {
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * 2 * CP::NI));
    }
    __syncthreads();
    if (t + S - 1 < t_end) issue(t + S - 1);  // into the stage read in step t-1
    const char* const kc = ring + ((t - t_begin) % S) * (2 * TB);
    const char* const vc = kc + TB;
    const int j0 = t * KT;
    // Scores and softmax at raised issue priority, the P V products at the
    // normal one: two resident workgroups then interleave their phases on a
    // SIMD's matrix core (+4 to +7% on long-query shapes).
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    __builtin_amdgcn_sched_barrier(0);
    // S^T = K Q^T: lane = query, element v of block kb = key
    // j0 + kb*32 + 8*(v/4) + 4*half + v%4.
    f32x16 s[NB];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) s[kb][v] = 0.f;
#pragma unroll
      for (int kk = 0; kk < G::NK; ++kk) {
        const bf16x8 a = *(const bf16x8*)(kc + kb * 32 * G::ROWB + koff[kk]);
        s[kb] = mfma32(a, qreg[kk], s[kb]);
      }
    }
    // Keys past Nk (zero rows, score 0) and, causal, keys after the query
    // position are masked; a wave-uniform test keeps the mask to edge tiles.
    const bool edge = (j0 + KT > Nk) || (CAUSAL && j0 + KT - 1 > q0w + delta);
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = j0 + kb * 32 + 8 * (v / 4) + 4 * half + (v % 4);
        // a select, not a branch: with a lane-dependent branch here the
        // compiler may move matrix-core products under a partial exec mask
        const bool drop = edge & ((key >= Nk) | (CAUSAL & (key > qi + delta)));
        s[kb][v] = drop ? -INFINITY : s[kb][v];
        mt = fmaxf(mt, s[kb][v]);
      }
    const float m_new = fmaxf(m_run, max_with_other_half(mt));
    // alpha rescales the state to the new maximum; a row that has seen no
    // key yet keeps -inf and gets P = 0 (no NaN from -inf - -inf).
    const float alpha = m_new == m_run ? 1.f : fast_exp2((m_run - m_new) * c);
    const float mb = m_new == -INFINITY ? 0.f : m_new * c;
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < G::NO; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) oacc[i][v] *= alpha;
    bf16x8 p[NB][2];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float e = fast_exp2(fmaf(s[kb][v], c, -mb));
        l_run += e;
        p[kb][v / 8][v % 8] = (__bf16)e;
      }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    // O^T += V^T P^T
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int i = 0; i < G::NO; ++i) {
          const char* blk = vc + (kb * 32 + a * 16) * G::ROWB;
          oacc[i] = mfma32(tr_pair(blk + voff[i][0], blk + voff[i][1]), p[kb][a], oacc[i]);
        }
  }

  // Partial results, float32: O_s = O / l (0 where the split holds no key
  // the query attends) and LSE_s = scale*m + ln l (-inf there). Stores past
  // Nq fall outside the buffer range and are dropped; no branch.
  const float l_tot = l_run + xor32(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse = l_tot > 0.f ? m_run * scale + __logf(l_tot) : -INFINITY;
  const size_t slab = ((size_t)bh * splits + sp) * (size_t)Nq;
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(Op + slab * D, (unsigned)Nq * D * 4u);
#pragma unroll
  for (int i = 0; i < G::NO; ++i)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4 w;
#pragma unroll
      for (int x = 0; x < 4; ++x) w[x] = oacc[i][4 * g + x] * inv;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, w), ro,
                                             (unsigned)(qi * D + 32 * i + 8 * g + 4 * half) * 4u,
                                             0, 0);
    }
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(Lp + slab, (unsigned)Nq * 4u);
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(lse), rl,
                                        half == 0 ? (unsigned)qi * 4u : kOutOfRange, 0, 0);
}

// Merge of the splits: one thread per (row, 4 output columns), one pass
// over the splits with a running maximum (the loads of successive splits
// do not depend on each other, so several are in flight). A split whose
// log-sum-exp is -inf holds no key the row attends and is skipped: its
// partial output is zero or, for a wholly empty workgroup, never written.
template <int D>
__global__ __launch_bounds__(64) void split_combine_kernel(const float* __restrict__ Op,
                                                           const float* __restrict__ Lp,
                                                           u16* __restrict__ O,
                                                           float* __restrict__ LSE, long long rows,
                                                           int Nq, int splits) {
  constexpr int C = D / 4;
  const long long id = (long long)blockIdx.x * 64 + threadIdx.x;
  if (id >= rows * C) return;
  const long long r = id / C;
  const int cc = (int)(id % C);
  const long long bh = r / Nq;
  const int i = (int)(r % Nq);
  const size_t base = (size_t)bh * splits * Nq + i;  // split s at base + s*Nq
  float m = -INFINITY, l = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
  for (int s = 0; s < splits; ++s) {
    const float ls = Lp[base + (size_t)s * Nq];
    if (ls == -INFINITY) continue;  // no attended key in this split (partial output unwritten)
    const f32x4 o = *(const f32x4*)(Op + (base + (size_t)s * Nq) * D + cc * 4);
    const float m_new = fmaxf(m, ls);
    const float f = m == m_new ? 1.f : __expf(m - m_new);  // m = -inf: f = 0
    const float w = ls == -INFINITY ? 0.f : __expf(ls - m_new);
    acc = acc * f + w * o;
    l = l * f + w;
    m = m_new;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  bf16x4 out;
#pragma unroll
  for (int x = 0; x < 4; ++x) out[x] = (__bf16)(acc[x] * inv);
  *(bf16x4*)(O + r * D + cc * 4) = out;
  if (LSE != nullptr && cc == 0) LSE[r] = l > 0.f ? m + __logf(l) : -INFINITY;
}

// The merge for many splits: one workgroup per query row, kMergeGroups
// groups of d/4 threads; group g merges splits g, g + kMergeGroups, ... with
// a running maximum, then the groups' (max, sum, accumulator) are merged
// through LDS by group 0. With one thread per (row, 4 columns) looping over
// all splits, decode (few rows, 16-64 splits) left most of the GPU idle.
constexpr int kMergeGroups = 8;

template <int D>
__global__ __launch_bounds__(kMergeGroups * D / 4) void split_combine_rows_kernel(
    const float* __restrict__ Op, const float* __restrict__ Lp, u16* __restrict__ O,
    float* __restrict__ LSE, int Nq, int splits) {
  constexpr int C = D / 4;
  constexpr int G = kMergeGroups;
  __shared__ float sm[G][C], sl[G][C];
  __shared__ f32x4 sa[G][C];
  const long long r = blockIdx.x;
  const int g = threadIdx.x / C, cc = threadIdx.x % C;
  const long long bh = r / Nq;
  const int i = (int)(r % Nq);
  const size_t base = (size_t)bh * splits * Nq + i;  // split s at base + s*Nq
  float m = -INFINITY, l = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int s = g; s < splits; s += G) {
    const float ls = Lp[base + (size_t)s * Nq];
    if (ls == -INFINITY) continue;  // no attended key in this split (partial output unwritten)
    const f32x4 o = *(const f32x4*)(Op + (base + (size_t)s * Nq) * D + cc * 4);
    const float m_new = fmaxf(m, ls);
    const float f = m == m_new ? 1.f : __expf(m - m_new);  // m = -inf: f = 0
    const float w = ls == -INFINITY ? 0.f : __expf(ls - m_new);
    acc = acc * f + w * o;
    l = l * f + w;
    m = m_new;
  }
  sm[g][cc] = m;
  sl[g][cc] = l;
  sa[g][cc] = acc;
  __syncthreads();
  if (g != 0) return;
  float mm = sm[0][cc];
#pragma unroll
  for (int x = 1; x < G; ++x) mm = fmaxf(mm, sm[x][cc]);
  float ll = 0.f;
  f32x4 aa = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int x = 0; x < G; ++x) {
    const float w = sm[x][cc] == -INFINITY ? 0.f : __expf(sm[x][cc] - mm);
    ll += w * sl[x][cc];
    aa += w * sa[x][cc];
  }
  const float inv = ll > 0.f ? 1.f / ll : 0.f;
  bf16x4 out;
#pragma unroll
  for (int x = 0; x < 4; ++x) out[x] = (__bf16)(aa[x] * inv);
  *(bf16x4*)(O + r * D + cc * 4) = out;
  if (LSE != nullptr && cc == 0) LSE[r] = ll > 0.f ? mm + __logf(ll) : -INFINITY;
}

template <int D, bool CAUSAL, int NW, int KT, int S>
hipError_t split_launch(const void* q, const void* k, const void* v, void* o, float* lse,
                        float* ws, int B, int H, int Nq, int Nk, int splits, float scale,
                        hipStream_t stream) {
  constexpr int BR = 32 * NW;
  const int nqt = (Nq + BR - 1) / BR;
  const int t_all = (Nk + kBC - 1) / kBC;
  const int tps = (t_all + splits - 1) / splits;
  splits = (t_all + tps - 1) / tps;  // every split non-empty in key range
  const long long nwg = (long long)B * H * nqt * splits;
  if (nwg >= (1LL << 31)) return hipErrorInvalidValue;
  const long long rows = (long long)B * H * Nq;
  float* const op = ws;
  float* const lp = ws + rows * splits * D;
  if (NW > 1 && Nq == Nk) {
    // Self-attention shapes run the one-pass forward kernel on the key
    // splits (its software pipeline; same-box timing against this file's
    // split kernel: +17% at B=1 H=2 N=8192 non-causal, +23% at B=1 H=4
    // N=4096 causal, +13 to +27% at B=1 H=8 N=2048 causal); same partials,
    // same merge.
    const hipError_t e = launch_fwd_bf16_partials(q, k, v, op, lp, B, H, Nq, D, CAUSAL, splits,
                                                  tps, scale, stream);
    if (e != hipSuccess) return e;
  } else {
    hipLaunchKernelGGL((fwd_split_kernel<D, CAUSAL, NW, KT, S>), dim3((unsigned)nwg),
                       dim3(64 * NW), 0, stream, (const u16*)q, (const u16*)k, (const u16*)v, op,
                       lp, Nq, Nk, nqt, splits, tps, (int)nwg, scale, debug_flags());
  }
  if (splits >= kMergeGroups) {
    hipLaunchKernelGGL((split_combine_rows_kernel<D>), dim3((unsigned)rows),
                       dim3(kMergeGroups * D / 4), 0, stream, (const float*)op, (const float*)lp,
                       (u16*)o, lse, Nq, splits);
    return hipGetLastError();
  }
  const long long threads = rows * (D / 4);
  hipLaunchKernelGGL((split_combine_kernel<D>), dim3((unsigned)((threads + 63) / 64)),
                     dim3(64), 0, stream, (const float*)op, (const float*)lp, (u16*)o, lse, rows,
                     Nq, splits);
  return hipGetLastError();
}

template <int D>
hipError_t split_dispatch(const void* q, const void* k, const void* v, void* o, float* lse,
                          float* ws, int B, int H, int Nq, int Nk, bool causal, int splits,
                          float scale, hipStream_t stream) {
  // One wave per workgroup when the queries fit one wave (decode), else four.
  if (Nq <= 32)
    return causal ? split_launch<D, true, 1, 32, 2>(q, k, v, o, lse, ws, B, H, Nq, Nk, splits, scale,
                                                    stream)
                  : split_launch<D, false, 1, 32, 2>(q, k, v, o, lse, ws, B, H, Nq, Nk, splits,
                                                     scale, stream);
  return causal ? split_launch<D, true, 4, 64, 2>(q, k, v, o, lse, ws, B, H, Nq, Nk, splits, scale,
                                                  stream)
                : split_launch<D, false, 4, 64, 2>(q, k, v, o, lse, ws, B, H, Nq, Nk, splits, scale,
                                                   stream);
}

}  // namespace

int split_count(int B, int H, int Nq, int Nk, bool causal, int requested) {
  const int t_all = (Nk + kBC - 1) / kBC;
  long long s = requested;
  if (s <= 0) {
    const bool decode = Nq <= 32;  // one wave per workgroup
    const long long base = (long long)B * H * (decode ? 1 : (Nq + 127) / 128);
    if (decode) {
      // two rounds of workgroups (two per compute unit), >= 2 key tiles each
      s = std::min<long long>((1024 + base - 1) / base, std::max(1, t_all / 2));
    } else if (base >= 256) {
      s = 1;  // a round of workgroups already
    } else if (causal) {
      // causal items differ in length (the longest query tiles set the
      // makespan): about 768 items, at most 8 splits, >= 4 key tiles each
      // (measured at 128-224 query tiles: 6 splits at 128, 3-4 at 192-224)
      s = std::min<long long>(std::min<long long>(8, (768 + base / 2) / base),
                              std::max(1, t_all / 4));
    } else {
      // about 512 items (a round); >= 8 key tiles per split, since every
      // split adds a float32 partial output to write and merge
      s = std::min<long long>((512 + base - 1) / base, std::max(1, t_all / 8));
    }
  }
  s = std::max<long long>(1, std::min<long long>(s, t_all));
  const int tps = (int)((t_all + s - 1) / s);
  return (t_all + tps - 1) / tps;
}

long long split_work_items(int B, int H, int Nq, int d, int splits) {
  // Split kernel: one wave per 32 queries (Nq <= 32) or four per 128; the
  // merge: d/4 threads per query row in 64-thread workgroups, or, with at
  // least kMergeGroups splits, kMergeGroups * d/4 threads per row.
  const int nw = Nq <= 32 ? 1 : 4;
  const long long split_items = (long long)B * H * ((Nq + 32 * nw - 1) / (32 * nw)) * splits * 64 * nw;
  const long long rows = (long long)B * H * Nq;
  const long long merge_items = splits >= kMergeGroups ? rows * kMergeGroups * (d / 4)
                                                       : (rows * (d / 4) + 63) / 64 * 64;
  return split_items > merge_items ? split_items : merge_items;
}

hipError_t launch_fwd_split_bf16(const void* q, const void* k, const void* v, void* o,
                                 float* lse, float* ws, int B, int H, int Nq, int Nk, int d,
                                 bool causal, int splits, float scale, hipStream_t stream) {
  switch (d) {
    case 64:
      return split_dispatch<64>(q, k, v, o, lse, ws, B, H, Nq, Nk, causal, splits, scale, stream);
    case 96:
      return split_dispatch<96>(q, k, v, o, lse, ws, B, H, Nq, Nk, causal, splits, scale, stream);
    case 128:
      return split_dispatch<128>(q, k, v, o, lse, ws, B, H, Nq, Nk, causal, splits, scale, stream);
    default:
      return hipErrorInvalidValue;
  }
}

// Scratch of the allocation-free split-KV entry point (the partial outputs
// and log-sum-exps of the splits), for callers that cannot allocate device
// memory. Each device the library runs on holds its own copy until the
// process ends. In host code `scratch` names a host-side stand-in, never the
// device memory: its device address comes from hipGetSymbolAddress.
static __device__ __align__(256) char scratch[FA_NOALLOC_SCRATCH_BYTES];

hipError_t noalloc_scratch(float** ws) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    // once per device, with that device current: the address of its copy
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptrs[dev] = p;
  }
  *ws = static_cast<float*>(ptrs[dev]);
  return hipSuccess;
}

}  // namespace fa
