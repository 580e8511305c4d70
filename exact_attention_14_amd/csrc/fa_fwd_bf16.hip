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
#include <type_traits>

#include "fa_common.hpp"
#include "fa_launch.hpp"
#include "fa_tiles_bf16.hpp"

namespace fa {
namespace {

constexpr float kLazyLog2 = 8.f; // rescale threshold, log2 units

// Software-pipelined kernel: while the softmax of tile t runs on the VALU,
// the scores of tile t+1 are already being formed on the matrix cores, and
// the P V products of tile t overlap the row maximum of tile t+1 (QbitAI
// article: two-stage GEMM-softmax pipelining, S_cur / S_next). K is copied
// one tile further ahead than V through two-stage LDS rings; the copies are
// issued as assembly so that only the kernel's own waits order them.
//
// SPLIT: the key range of each (batch, head, query tile) is cut into `splits`
// parts of tps 64-key tiles that run as separate workgroups (few heads: the
// key axis supplies the parallelism). Each writes, in float32, its partial
// output normalised by its own row sum to Op and its partial log-sum-exp
// (-inf where it holds no key the query attends) to Lp, slab
// (batch*H + head)*splits + split of N rows each; a merge by log-sum-exp
// follows. A workgroup whose split holds no key of its queries writes only
// the -inf log-sum-exps.
template <int D, bool CAUSAL, int NW, bool SPLIT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd<D>, kWavesPerSimd<D>))) void fwd_bf16_kernel(
    const u16* __restrict__ Q, const u16* __restrict__ K, const u16* __restrict__ V,
    u16* __restrict__ O, float* __restrict__ LSE, int N, int ntq, int nwg, int hpx, float scale,
    float* __restrict__ Op, float* __restrict__ Lp, int splits, int tps) {
  using G = Geo<D>;
  using CP = TileCopy<D, NW>;
  constexpr int BR = 32 * NW;
  // K_j lives in ks[j % 2], V_j in vs[j % 2]. The copies are issued as
  // assembly, so the compiler adds no waits of its own for them.
  __shared__ __attribute__((aligned(1024))) char ks0[G::TILEB];
  __shared__ __attribute__((aligned(1024))) char vs0[G::TILEB];
  __shared__ __attribute__((aligned(1024))) char ks1[G::TILEB];
  __shared__ __attribute__((aligned(1024))) char vs1[G::TILEB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;

  int bh, qt, sp = 0;
  if constexpr (SPLIT && CAUSAL) {
    // Items differ in length (a split past a query tile's diagonal is
    // empty): longest first, the heads interleaved (workgroup id modulo
    // B*H, which also keeps each XCD on the same heads when B*H divides 8 or
    // 8 divides B*H), then query tiles from the last, their splits
    // consecutive.
    const int n = nwg & ((1 << kDbgShift) - 1);
    const int bid = (dbg_flags(nwg) & kDbgReverse) ? n - 1 - (int)blockIdx.x : (int)blockIdx.x;
    const int bht = n / (ntq * splits);
    bh = bid % bht;
    const int rank = bid / bht;
    qt = ntq - 1 - rank / splits;
    sp = rank % splits;
  } else if constexpr (SPLIT) {
    int rank;  // a head's items on one XCD, query tiles fastest
    tile_of_workgroup(blockIdx.x, nwg, ntq * splits, 0, bh, rank);
    sp = rank / ntq;
    qt = rank % ntq;
  } else {
    int qtr;
    tile_of_workgroup(blockIdx.x, nwg, ntq, CAUSAL ? hpx : 0, bh, qtr);
    qt = CAUSAL ? (ntq - 1 - qtr) : qtr;
  }
  const size_t head = (size_t)bh * (size_t)N;
  const unsigned head_bytes = (unsigned)N * D * 2u;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(Q + head * D, head_bytes);
  const i32x4 rk = make_rsrc_words(K + head * D, head_bytes);
  const i32x4 rv = make_rsrc_words(V + head * D, head_bytes);

  const int q0w = qt * BR + wave * 32;
  const int qi = q0w + l32;
  const int q_last = min(N, qt * BR + BR) - 1;
  const int T_all = CAUSAL ? (q_last / kBC + 1) : (N + kBC - 1) / kBC;
  // Key tiles tb .. tb+T-1 (all of them without SPLIT); below, t counts the
  // workgroup's own tiles and tile t holds keys (tb + t) * 64 ...
  const int tb = SPLIT ? sp * tps : 0;
  const int T = SPLIT ? min(T_all, tb + tps) - tb : T_all;
  if constexpr (SPLIT) {
    if (T <= 0) {
      const size_t slab = ((size_t)bh * splits + sp) * (size_t)N;
      const __amdgpu_buffer_rsrc_t rl = make_rsrc(Lp + slab, (unsigned)N * 4u);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(-INFINITY), rl,
                                            half == 0 ? (unsigned)qi * 4u : kOutOfRange, 0, 0);
      return;
    }
  }

  if (dbg_flags(nwg) & kDbgPoison) {
    poison_lds(ks0, G::TILEB, tid, NW * 64);
    poison_lds(vs0, G::TILEB, tid, NW * 64);
    poison_lds(ks1, G::TILEB, tid, NW * 64);
    poison_lds(vs1, G::TILEB, tid, NW * 64);
    __syncthreads();
  }

  // Prologue, in this order: copy K_0, load Q, copy V_0 and K_1. (The
  // compiler's waits for Q then cover K_0 but not the later copies.)
  const CP cp(wave, lane);
  cp.issue(rk, ks0, tb * kBC, wave, true);
  bf16x8 qreg[G::NK];
#pragma unroll
  for (int kk = 0; kk < G::NK; ++kk) {
    const i32x4 w = __builtin_amdgcn_raw_buffer_load_b128(
        rq, (unsigned)(qi * D + kk * 16 + half * 8) * 2u, 0, 0);
    qreg[kk] = __builtin_bit_cast(bf16x8, w);
  }
  cp.issue(rv, vs0, tb * kBC, wave, true);
  cp.issue(rk, ks1, (tb + 1) * kBC, wave, T > 1);

  f32x16 oacc[G::NO];
#pragma unroll
  for (int i = 0; i < G::NO; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[i][v] = 0.f;
  float m_ref = -INFINITY;  // reference maximum (raw scores) of O and l
  float l_run = 0.f;
  const float c = scale * kLog2e;

  // Loop-invariant per-lane LDS byte offsets. The swizzle of a row depends
  // only on its low 4 bits, which the 32- and 16-row block offsets keep, so
  // those offsets (and the stage base) fold into instruction immediates.
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

  auto scores = [&](const char* kt, f32x16* s) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) s[kb][v] = 0.f;
#pragma unroll
    for (int kk = 0; kk < G::NK; ++kk)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 a = *(const bf16x8*)(kt + kb * 32 * G::ROWB + koff[kk]);
        s[kb] = mfma32(a, qreg[kk], s[kb]);
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
  // K_0 has landed once at most the Q loads and the two younger copies (all
  // issued after it) are still in flight.
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(G::NK + 2 * CP::NI));
  __syncthreads();
  scores(ks0, s_cur);
  mask(s_cur, tb * kBC);
  float mt = rowmax(s_cur);

  // Tile t: S_t is in s_cur with its row max in mt; K_{t+1} (kr) and V_t (vr)
  // are in LDS once every wave passed the barrier; K_{t+2} goes to kl, V_{t+1}
  // to vl. The last step (t = T-1) only finishes tile t.
  // MASK: whether the scores of tile t+1 may need masking (edge tiles only;
  // the steady-state loop runs without the branch).
  // Where the softmax of tile t runs: all of it beside the scores of tile t+1
  // (stage A), leaving stage B to the P V products and the row maximum of
  // tile t+1; or, for d = 256, whose stages hold twice the matrix-core work,
  // half in each stage with the row maximum after stage B.
  constexpr bool SOFT_A = D <= 128;
  // VALU instructions placed after each matrix-core instruction: about 100
  // softmax instructions per tile spread over stage A's 2*NK products.
  constexpr int VALU_A = SOFT_A ? (100 + 2 * G::NK - 1) / (2 * G::NK) : 4;
  constexpr int VALU_B = SOFT_A ? 2 : 4;
  // LDS fragment reads run ahead of their MFMAs: at d <= 128 K fragments two
  // MFMAs ahead and V fragments (two transposed reads each) three ahead (two
  // ahead measured 1-3% slower); d = 256, one wave per SIMD with no other
  // wave to fill the gaps, reads both four MFMAs ahead (+2 to +7%).
  constexpr int RA_K = D == 256 ? 4 : 2;
  constexpr int RA_V = D == 256 ? 8 : 6;
  // Where the copies of V_{t+1} are issued: beside those of K_{t+2} in
  // stage A (d <= 128), so that they have a whole stage B more to land
  // before the next step's wait (same-box A/B against spreading them over
  // stage B: +0.1 to +2.6% at d <= 128, -1.8% at d = 256, which keeps them
  // in stage B). The stage of V_{t+1} (that of V_{t-1}) is free once every
  // wave has passed this step's barrier.
  constexpr bool V_IN_A = D <= 128;
  // KIND: 0 = steady state (tile t+1 needs no mask), 1 = tile t+1 may need
  // masking, 2 = last tile (t = T-1): there is no tile t+1 to score or copy.
  auto step = [&](auto kind_tag, const char* kr, const char* vr, char* kl, char* vl, int t) {
    constexpr int KIND = decltype(kind_tag)::value;
    constexpr bool MASK = KIND == 1;
    constexpr bool LAST = KIND == 2;
    // This wave's copies of K_{t+1} and V_t have landed; after the barrier
    // every wave's have, and the stages of K_t and V_{t-1} are free.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (__any((mt - m_ref) * c > kLazyLog2)) {
      const float m_new = fmaxf(m_ref, mt);
      const float alpha = (m_ref == -INFINITY) ? 0.f : fast_exp2((m_ref - m_new) * c);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < G::NO; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[i][v] *= alpha;
      m_ref = m_new;
    }
    const float mc = (m_ref == -INFINITY) ? 0.f : m_ref * c;
    bf16x8 p[2][2];
    float lsum = 0.f;
    auto softmax_half = [&](int kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float e = fast_exp2(fmaf(s_cur[kb][v], c, -mc));
        lsum += e;
        p[kb][v / 8][v % 8] = (__bf16)e;
      }
    };
    // Stage A: scores of tile t+1 on the matrix cores, softmax of tile t on
    // the VALU. A wave in this stage takes issue priority over the other
    // workgroup's wave on its SIMD, which then fills the matrix-core gaps
    // with its own stage (the pages' ping-pong of two warp groups, here
    // between the two resident workgroups). The NI copies of K_{t+2} are
    // spread over the stage: issued back to back, the copies of all waves of
    // a CU fill the texture unit's queues and stall the issuing waves.
    // (d <= 128 issues the copies of V_{t+1} here too, see V_IN_A.)
    __builtin_amdgcn_s_setprio(1);
    if constexpr (!LAST) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) s_nxt[kb][v] = 0.f;
#pragma unroll
      for (int kk = 0; kk < G::NK; ++kk) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 a = *(const bf16x8*)(kr + kb * 32 * G::ROWB + koff[kk]);
          s_nxt[kb] = mfma32(a, qreg[kk], s_nxt[kb]);
        }
#pragma unroll
        for (int ci = kk * CP::NI / G::NK; ci < (kk + 1) * CP::NI / G::NK; ++ci) {
          cp.issue_one(ci, rk, kl, (tb + t + 2) * kBC, wave, t + 2 < T);
          if constexpr (V_IN_A) cp.issue_one(ci, rv, vl, (tb + t + 1) * kBC, wave, t + 1 < T);
        }
      }
    }
    softmax_half(0);
    if constexpr (SOFT_A) softmax_half(1);
    // Issue order: K fragment reads run two MFMAs ahead; each MFMA is
    // followed by VALU_A VALU/transcendental instructions of the softmax.
    if constexpr (!LAST) {
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, RA_K, 0);
#pragma unroll
      for (int i = 0; i < 2 * G::NK; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedValu, VALU_A, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      }
    }
    // Nothing moves across: keeps stage B's V fragments out of stage A.
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    // Stage B: P V of tile t (d = 256: with the copies of V_{t+1} spread over it).
    float mt_next = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int i = 0; i < G::NO; ++i) {
          const char* blk = vr + (kb * 32 + a * 16) * G::ROWB;
          oacc[i] = mfma32(tr_pair(blk + voff[i][0], blk + voff[i][1]), p[kb][a], oacc[i]);
          const int slot = (kb * 2 + a) * G::NO + i;
          if constexpr (!LAST && !V_IN_A) {
#pragma unroll
            for (int ci = slot * CP::NI / (4 * G::NO); ci < (slot + 1) * CP::NI / (4 * G::NO); ++ci)
              cp.issue_one(ci, rv, vl, (tb + t + 1) * kBC, wave, t + 1 < T);
          }
        }
      if (kb == 0) {
        if constexpr (LAST) {
          if constexpr (!SOFT_A) softmax_half(1);
        } else if constexpr (SOFT_A) {
          // Tile t+1's scores are complete: mask them and take their row
          // maximum while the matrix cores work on P V.
          if constexpr (MASK) mask(s_nxt, (tb + t + 1) * kBC);
          mt_next = rowmax(s_nxt);
        } else {
          softmax_half(1);
        }
      }
    }
    l_run += lsum;
    // Issue order: V fragment reads run RA_V / 2 MFMAs ahead.
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, RA_V, 0);
#pragma unroll
    for (int i = 0; i < 4 * G::NO; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedValu, VALU_B, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!SOFT_A && !LAST) {
      if constexpr (MASK) mask(s_nxt, (tb + t + 1) * kBC);
      mt_next = rowmax(s_nxt);
    }
    if constexpr (!LAST) {
      mt = mt_next;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) s_cur[kb] = s_nxt[kb];
    }
  };

  // Tiles t < J need no mask for any wave: every key of them precedes the
  // workgroup's first query (causal) and lies inside the sequence (and the
  // count stops at the workgroup's own tiles).
  const int Jg = CAUSAL ? min(N / kBC, (qt * BR + 1) / kBC) : N / kBC;
  const int J = SPLIT ? min(Jg - tb, T) : Jg;
  using Steady = std::integral_constant<int, 0>;
  using Masked = std::integral_constant<int, 1>;
  using Last = std::integral_constant<int, 2>;
  int t = 0;
  for (; t + 2 < J; t += 2) {  // steps whose next tile (t+1, t+2) is unmasked
    step(Steady{}, ks1, vs0, ks0, vs1, t);
    step(Steady{}, ks0, vs1, ks1, vs0, t + 1);
  }
  for (; t + 2 < T; t += 2) {  // t is even here: stage parity stays static
    step(Masked{}, ks1, vs0, ks0, vs1, t);
    step(Masked{}, ks0, vs1, ks1, vs0, t + 1);
  }
  if (t + 1 < T) {  // two tiles left
    step(Masked{}, ks1, vs0, ks0, vs1, t);
    ++t;
  }
  // The last step reads only V_t; one call site with the stage chosen at run
  // time (two static-parity copies of the step raise register pressure into
  // spills).
  step(Last{}, ks0, (t & 1) ? vs1 : vs0, ks1, vs0, t);
  // No copy may land in LDS after the workgroup exits.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  // The last step read no K stage and no copy is in flight: each wave stages
  // its output rows in its own quarter of the two K stages.
  static_assert(NW == 4 && 2 * 32 * 2 * D <= G::TILEB, "staging slots fit the K stages");
  const float l_tot = l_run + xor32(l_run);
  if constexpr (SPLIT) {
    // Partial results, float32: O_s = O / l (0 where the split holds no key
    // the query attends) and LSE_s = scale*m + ln l (-inf there). Stores
    // past N fall outside the buffer range and are dropped.
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float lse = l_tot > 0.f ? m_ref * scale + __logf(l_tot) : -INFINITY;
    const size_t slab = ((size_t)bh * splits + sp) * (size_t)N;
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(Op + slab * D, (unsigned)N * D * 4u);
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
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(Lp + slab, (unsigned)N * 4u);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(lse), rl,
                                          half == 0 ? (unsigned)qi * 4u : kOutOfRange, 0, 0);
  } else {
    store_o_lse_staged<D>(O, LSE, head, N, q0w, lane, oacc, 1.f / l_tot,
                          m_ref * scale + __logf(l_tot),
                          (wave < 2 ? ks0 : ks1) + (wave & 1) * (32 * 2 * D));
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                  int H, int N, float scale, hipStream_t stream) {
  constexpr int NW = 4;
  const int ntq = (N + 32 * NW - 1) / (32 * NW);
  const long long nwg = (long long)ntq * B * H;
  if (nwg >= (1LL << 31)) return hipErrorInvalidValue;
  const int dbg = debug_flags();
  // Causal: whole heads per XCD, longest tiles first, when the heads split
  // evenly (not under the reversed debug order).
  const int hpx = ((long long)B * H) % 8 == 0 && !(dbg & 1) ? (int)(((long long)B * H) / 8) : 0;
  const int nwg_arg = (int)nwg | (dbg << kDbgShift);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, NW, false>), dim3((unsigned)nwg), dim3(NW * 64), 0,
                     stream, (const u16*)q, (const u16*)k, (const u16*)v, (u16*)o, lse, N, ntq,
                     nwg_arg, hpx, scale, nullptr, nullptr, 1, 0);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_partials(const void* q, const void* k, const void* v, float* op, float* lp,
                           int B, int H, int N, int splits, int tps, float scale,
                           hipStream_t stream) {
  constexpr int NW = 4;
  const int ntq = (N + 32 * NW - 1) / (32 * NW);
  const long long nwg = (long long)ntq * B * H * splits;
  if (nwg >= (1LL << 31)) return hipErrorInvalidValue;
  const int nwg_arg = (int)nwg | (debug_flags() << kDbgShift);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, NW, true>), dim3((unsigned)nwg), dim3(NW * 64), 0,
                     stream, (const u16*)q, (const u16*)k, (const u16*)v, nullptr, nullptr, N, ntq,
                     nwg_arg, 0, scale, op, lp, splits, tps);
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

hipError_t launch_fwd_bf16_partials(const void* q, const void* k, const void* v, float* op,
                                    float* lp, int B, int H, int N, int d, bool causal,
                                    int splits, int tps, float scale, hipStream_t stream) {
#define FA_CASE(DD)                                                                              \
  case DD:                                                                                       \
    return causal ? launch_partials<DD, true>(q, k, v, op, lp, B, H, N, splits, tps, scale, stream) \
                  : launch_partials<DD, false>(q, k, v, op, lp, B, H, N, splits, tps, scale, stream);
  switch (d) {
    FA_CASE(64)
    FA_CASE(96)
    FA_CASE(128)
    default:
      return hipErrorInvalidValue;
  }
#undef FA_CASE
}

}  // namespace fa
