// FlashAttention backward pass, bf16 inputs, fp32 accumulation, gfx950.
//
// What is computed (the gradients of sum(dO * O) for the forward pass of
// fa_fwd_bf16.hip; the QbitAI FlashAttention-3 article times this backward
// pass beside the forward): with P = softmax(scale * Q K^T) recomputed tile by
// tile from the forward's per-row log-sum-exp (no running maximum is needed
// on the way back),
//   D_i  = sum_c dO_ic O_ic                (= sum_j P_ij dP_ij)
//   dV   = P^T dO,  dP = dO V^T,  dS = P * (dP - D),
//   dQ   = scale * dS K,  dK = scale * dS^T Q.
// The N x N matrices never leave the chip. Two kernels share the work without
// atomics (results are deterministic): one owns a tile of queries and sweeps
// the key tiles for dQ, the other owns a tile of keys and sweeps the query
// tiles for dK and dV; both recompute S and dP. The dQ kernel runs first and
// also forms each of its rows' D and -LSE log2(e), which the dK/dV kernel
// then streams (a separate pass over O and dO for them cost a launch and
// about 11 us at B=4 H=16 N=2048 d=128).
//
// gfx950 mapping (same building blocks as the forward kernel)
//   * dK/dV: each lane owns one key. K and V stay in registers as the B
//     operands of S = Q K^T and dP = dO V^T (v_mfma_f32_32x32x16_bf16); the
//     outputs then hold, per lane, 16 queries of a 32-query block, which is
//     exactly the B-operand layout of dV^T += dO^T P and dK^T += Q^T dS, whose
//     A operands are the Q and dO tiles read transposed from LDS
//     (ds_read_b64_tr_b16). The per-query LSE and D are read per element.
//   * dQ: each lane owns one query (the forward's layout): S^T = K Q^T and
//     dP^T = V dO^T from the K and V tiles, then dQ^T += K^T dS^T with K read
//     transposed; LSE and D are per-lane scalars.
//   * Tiles of 64 rows move HBM -> LDS by direct-to-LDS copies into a
//     two-stage ring (one tile of prefetch), with the forward's swizzle.
//   * The gradients are stored with the forward's staged epilogue.
#include <type_traits>

#include "fa_common.hpp"
#include "fa_launch.hpp"
#include "fa_tiles_bf16.hpp"

namespace fa {
namespace {

// 4-byte HBM -> LDS copy per lane (lane l writes lds + 4 l), written as
// assembly for the same reason as the 16-byte tile copies: the kernel's own
// s_waitcnt decides when it is complete. `lds` must be wave-uniform.
__device__ __forceinline__ void copy4_to_lds_asm(i32x4 rsrc, const void* lds, unsigned byte_off) {
  const unsigned m0 = (unsigned)reinterpret_cast<unsigned long long>(
      (const __attribute__((address_space(3))) void*)lds);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(m0), "v"(byte_off), "s"(rsrc)
               : "memory", "m0");
}

// Offsets shared by both kernels: K-style row reads (lane = row l32 of a
// 32-row block, 16-byte chunk 2*kk + half) and V-style transposed reads (the
// forward's P V operand pattern), per lane, within a 64-row tile.
template <int D>
struct Offsets {
  using G = Geo<D>;
  // Chunk 2*kk + half of a row read sits at rb ^ (kk << 5), and the
  // transposed read of column block i, row group r at t[r] ^ (i << 6): the
  // swizzle is an XOR on the chunk index, whose bits above the lane's own
  // come from kk or i.
  int rb;
  int t[2];
  __device__ __forceinline__ Offsets(int lane) {
    const int half = lane >> 5, l32 = lane & 31;
    rb = l32 * G::ROWB + ((half ^ swz<G::CPRP>(l32)) << 4);
    const int g16 = lane >> 4, i16 = lane & 15;
    const int vrow = 4 * half + (i16 >> 2);
    const int vcol = (g16 & 1) * 2 + ((i16 & 3) >> 1);
    const int vbyte = (i16 & 1) * 8;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int rr = vrow + 8 * r;
      t[r] = rr * G::ROWB + ((vcol ^ swz<G::CPRP>(rr)) << 4) + vbyte;
    }
  }
};

// A copy of x that the compiler cannot see through: offsets derived from it
// are formed next to their use instead of being hoisted out of the loop and
// held in registers for the whole kernel.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// acc[i] += (rows rb*32 .. rb*32+31 of `tile`)^T . b, for the d blocks i:
// b[a] is the B operand of rows rb*32 + a*16 .. +15 in the permuted order of
// the transposed reads (the order in which a 32x32 product's result rows
// sit in a lane's registers).
template <int D>
__device__ __forceinline__ void block_t_times(const char* tile, int rb, const Offsets<D>& off,
                                              const bf16x8* b, f32x16* acc) {
  const int t0 = opaque(off.t[0]), t1 = opaque(off.t[1]);
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int i = 0; i < Geo<D>::NO; ++i) {
      const char* blk = tile + (rb * 32 + a * 16) * Geo<D>::ROWB;
      acc[i] = mfma32(tr_pair(blk + (t0 ^ (i << 6)), blk + (t1 ^ (i << 6))), b[a], acc[i]);
    }
}

// Two 32x32 products over d that share their A-row offsets:
// s = (rows rb*32.. of ta) . ra^T and t = (rows rb*32.. of tb) . rb_^T, with
// each LDS read issued next to the product that consumes it.
template <int D, bool SCHED = true>
__device__ __forceinline__ void two_rows_times_reg(const char* ta, const char* tb, int rb,
                                                   const Offsets<D>& off, const bf16x8* ra,
                                                   const bf16x8* rbreg, f32x16& s, f32x16& t) {
#pragma unroll
  for (int v = 0; v < 16; ++v) s[v] = t[v] = 0.f;
  const int r0 = opaque(off.rb);
#pragma unroll
  for (int kk = 0; kk < Geo<D>::NK; ++kk) {
    const bf16x8 a = *(const bf16x8*)(ta + rb * 32 * Geo<D>::ROWB + (r0 ^ (kk << 5)));
    s = mfma32(a, ra[kk], s);
  }
#pragma unroll
  for (int kk = 0; kk < Geo<D>::NK; ++kk) {
    const bf16x8 b = *(const bf16x8*)(tb + rb * 32 * Geo<D>::ROWB + (r0 ^ (kk << 5)));
    t = mfma32(b, rbreg[kk], t);
  }
  if constexpr (SCHED) {
#pragma unroll
    for (int kk = 0; kk < Geo<D>::NK; ++kk) {
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
    }
  }
}

// Row fragments of the lane's own row (row < N, else zeros) as B operands.
template <int D>
__device__ __forceinline__ void load_own_rows(__amdgpu_buffer_rsrc_t r, int row, int half,
                                              bf16x8* reg) {
#pragma unroll
  for (int kk = 0; kk < Geo<D>::NK; ++kk) {
    const i32x4 w = __builtin_amdgcn_raw_buffer_load_b128(
        r, (unsigned)(row * D + kk * 16 + half * 8) * 2u, 0, 0);
    reg[kk] = __builtin_bit_cast(bf16x8, w);
  }
}

// ------------------------------------------------------------------ dK, dV --

// Mask kinds of a step: the steady steps need none. Rows past N need no mask
// in the dK/dV kernel: their Q and dO rows are copied as zeros and their NL
// and D as zeros, so P = 1 and dS = 0 there and both products add nothing.
struct Plain {};
struct Diagonal {};

// Workgroup: 4 waves x 32 keys = one 128-key tile of one (batch, head); it
// sweeps the 64-query tiles that attend to it (causal: from its first key
// on, the first two tiles being the diagonal ones). Q, dO and the query
// tile's NL and D move HBM -> LDS one tile ahead. Grid: B*H*ceil(N/128);
// causal key tiles run lowest index (most query tiles) first. Two
// workgroups share a compute unit (256 registers per lane); at d = 256 the
// gradients alone take 256 registers and one workgroup runs per unit.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd<D>, kWavesPerSimd<D>))) void bwd_dkdv_kernel(
    const u16* __restrict__ Q, const u16* __restrict__ K, const u16* __restrict__ V,
    const u16* __restrict__ dO, const float* __restrict__ NL, const float* __restrict__ Dvec,
    u16* __restrict__ dK, u16* __restrict__ dV, int N, int nkt, int nwg, int hpx, float scale) {
  using G = Geo<D>;
  using CP = TileCopy<D, 4>;
  __shared__ __attribute__((aligned(1024))) char qs0[G::TILEB];
  __shared__ __attribute__((aligned(1024))) char gs0[G::TILEB];
  __shared__ __attribute__((aligned(1024))) char qs1[G::TILEB];
  __shared__ __attribute__((aligned(1024))) char gs1[G::TILEB];
  __shared__ __attribute__((aligned(16))) float rowt[2][2][kBC];  // [stage][NL, D][query]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5;
  const int l32 = lane & 31;

  int bh, kt;
  tile_of_workgroup(blockIdx.x, nwg, nkt, CAUSAL ? hpx : 0, bh, kt);
  const size_t head = (size_t)bh * (size_t)N;
  const unsigned head_bytes = (unsigned)N * D * 2u;
  const i32x4 rq = make_rsrc_words(Q + head * D, head_bytes);
  const i32x4 rg = make_rsrc_words(dO + head * D, head_bytes);
  // Waves 0 and 1 copy the NL and D rows of a query tile; queries past N
  // read as zeros.
  const i32x4 rr = make_rsrc_words((wave == 0 ? NL : Dvec) + head, (unsigned)N * 4u);

  const int k0w = kt * 128 + wave * 32;  // first key of the wave
  const int kj = k0w + l32;              // the lane's key
  const int u0 = CAUSAL ? (kt * 128) / kBC : 0;  // first query tile
  const int U = (N + kBC - 1) / kBC;
  const float c = scale * kLog2e;

  const CP cp(wave, lane);
  auto issue = [&](char* qn, char* gn, int st, int u) {
    cp.issue(rq, qn, u * kBC, wave, true);
    cp.issue(rg, gn, u * kBC, wave, true);
    if (wave < 2) copy4_to_lds_asm(rr, rowt[st][wave], (unsigned)(u * kBC + lane) * 4u);
  };
  issue(qs0, gs0, 0, u0);
  bf16x8 kreg[G::NK], vreg[G::NK];
  load_own_rows<D>(make_rsrc(K + head * D, head_bytes), kj, half, kreg);
  load_own_rows<D>(make_rsrc(V + head * D, head_bytes), kj, half, vreg);
  const Offsets<D> off(lane);

  f32x16 dk[G::NO], dv[G::NO];
#pragma unroll
  for (int i = 0; i < G::NO; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) dk[i][v] = dv[i][v] = 0.f;

  // Query tile u (in stage st): Q_u in qc, dO_u in gc; tile u+1 goes to the
  // other stage. One 32-query block at a time: S and dP, then P and dS, then
  // their products, so that only one block's scores are live.
  auto step = [&](auto kind, const char* qc, const char* gc, char* qn, char* gn, int st, int u) {
    constexpr bool DIAG = std::is_same_v<decltype(kind), Diagonal>;
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (u + 1 < U) issue(qn, gn, st ^ 1, u + 1);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qs = u * kBC + qb * 32;  // first query of the block
      // Diagonal tiles: a block whose queries all precede the wave's keys
      // adds nothing (a wave-uniform skip); the block with qs == k0w is
      // masked element by element (key <= query: l32 <= 8g + 4half + x).
      if (DIAG && k0w > qs) continue;
      f32x16 s, dp;
      // Scores and the P / dS arithmetic at raised issue priority: the other
      // wave on the SIMD is then usually in its products, and the matrix
      // core interleaves the two (1-5% measured).
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
      __builtin_amdgcn_sched_barrier(0);
      two_rows_times_reg<D, false>(qc, gc, qb, off, kreg, vreg, s, dp);  // S = Q K^T, dP = dO V^T
      bf16x8 pb[2], sb[2];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // NL and D of queries qs + 8g + 4half + x, x = 0..3
        const f32x4 nl4 = *(const f32x4*)&rowt[st][0][qb * 32 + 8 * g + 4 * half];
        const f32x4 d4 = *(const f32x4*)&rowt[st][1][qb * 32 + 8 * g + 4 * half];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int v = 4 * g + x;
          float p = fast_exp2(fmaf(s[v], c, nl4[x]));
          if (DIAG && k0w == qs && l32 > 8 * g + 4 * half + x) p = 0.f;
          pb[v / 8][v % 8] = (__bf16)p;
          sb[v / 8][v % 8] = (__bf16)(p * (dp[v] - d4[x]));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
      block_t_times<D>(gc, qb, off, pb, dv);  // dV^T += dO^T P
      block_t_times<D>(qc, qb, off, sb, dk);  // dK^T += Q^T dS
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  int u = u0;
  if constexpr (CAUSAL && D == 256) {
    // One step kind for the whole sweep: a second copy of the step for the
    // diagonal tiles pushed this kernel past its 512 registers. Off the
    // diagonal the kind's tests are wave-uniform and never taken.
    for (; u + 1 < U; u += 2) {
      step(Diagonal{}, qs0, gs0, qs1, gs1, 0, u);
      step(Diagonal{}, qs1, gs1, qs0, gs0, 1, u + 1);
    }
    if (u < U) step(Diagonal{}, qs0, gs0, qs1, gs1, 0, u);
  } else {
    if constexpr (CAUSAL) {
      step(Diagonal{}, qs0, gs0, qs1, gs1, 0, u);
      if (u + 1 < U) step(Diagonal{}, qs1, gs1, qs0, gs0, 1, u + 1);
      u += 2;
    }
    for (; u + 1 < U; u += 2) {
      step(Plain{}, qs0, gs0, qs1, gs1, 0, u);
      step(Plain{}, qs1, gs1, qs0, gs0, 1, u + 1);
    }
    if (u < U) step(Plain{}, qs0, gs0, qs1, gs1, 0, u);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();  // every wave is done with the tiles: they hold the staging slots
  static_assert(2 * 32 * 2 * D <= G::TILEB, "two staging slots per tile");
  char* const slot = (wave < 2 ? qs0 : qs1) + (wave & 1) * (32 * 2 * D);
  store_o_lse_staged<D>(dK, nullptr, head, N, k0w, lane, dk, scale, 0.f, slot);
  store_o_lse_staged<D>(dV, nullptr, head, N, k0w, lane, dv, 1.f, 0.f, slot);
}

// ---------------------------------------------------------------------- dQ --

// Workgroup: 4 waves x 32 queries = one 128-query tile of one (batch, head);
// it sweeps the 64-key tiles the queries attend to. Keys past N are copied
// as zero rows, but P there is exp(-LSE), not 0, so the tile holding them is
// masked; so are the two diagonal tiles of a causal sweep (the last two).
// Grid: B*H*ceil(N/128); causal query tiles run longest first. Two
// workgroups share a compute unit.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd<D>, kWavesPerSimd<D>))) void bwd_dq_kernel(
    const u16* __restrict__ Q, const u16* __restrict__ K, const u16* __restrict__ V,
    const u16* __restrict__ dO, const u16* __restrict__ O, const float* __restrict__ LSE,
    float* __restrict__ NL, float* __restrict__ Dvec, u16* __restrict__ dQ, int N, int ntq,
    int nwg, int hpx, float scale) {
  using G = Geo<D>;
  using CP = TileCopy<D, 4>;
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
  const unsigned head_bytes = (unsigned)N * D * 2u;
  const i32x4 rk = make_rsrc_words(K + head * D, head_bytes);
  const i32x4 rv = make_rsrc_words(V + head * D, head_bytes);

  const int q0w = qt * 128 + wave * 32;
  const int qi = q0w + l32;
  const int q_last = min(N, qt * 128 + 128) - 1;
  const int T = CAUSAL ? (q_last / kBC + 1) : (N + kBC - 1) / kBC;
  // tiles [0, T_plain) need no mask
  const int T_plain = CAUSAL ? 2 * qt : (N % kBC != 0 ? T - 1 : T);
  const float c = scale * kLog2e;

  const CP cp(wave, lane);
  cp.issue(rk, ks0, 0, wave, true);
  cp.issue(rv, vs0, 0, wave, true);
  bf16x8 qreg[G::NK], greg[G::NK];
  load_own_rows<D>(make_rsrc(Q + head * D, head_bytes), qi, half, qreg);
  load_own_rows<D>(make_rsrc(dO + head * D, head_bytes), qi, half, greg);
  // The row terms of the lane's query: D = sum_c dO O (this half-wave's
  // columns, then the other half's through lane ^ 32) and -LSE log2(e).
  // Queries past N read zeros (their rows are dropped at the store).
  float dd;
  {
    bf16x8 oreg[G::NK];
    load_own_rows<D>(make_rsrc(O + head * D, head_bytes), qi, half, oreg);
    float part = 0.f;
#pragma unroll
    for (int kk = 0; kk < G::NK; ++kk)
#pragma unroll
      for (int j = 0; j < 8; ++j) part = fmaf((float)greg[kk][j], (float)oreg[kk][j], part);
    dd = part + __shfl_xor(part, 32);
  }
  const float nl = -__uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                       make_rsrc(LSE + head, (unsigned)N * 4u), (unsigned)qi * 4u, 0, 0)) *
                   kLog2e;
  // Published for the dK/dV kernel, one lane per row (the second half-wave
  // and rows past N fall outside the buffer range and are dropped).
  {
    const unsigned so = half == 0 ? (unsigned)qi * 4u : kOutOfRange;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(nl),
                                          make_rsrc(NL + head, (unsigned)N * 4u), so, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(dd),
                                          make_rsrc(Dvec + head, (unsigned)N * 4u), so, 0, 0);
  }
  const Offsets<D> off(lane);

  f32x16 dq[G::NO];
#pragma unroll
  for (int i = 0; i < G::NO; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) dq[i][v] = 0.f;

  // Key tile t: K_t in kc, V_t in vc; K_{t+1}, V_{t+1} go to kn, vn.
  auto step = [&](auto kind, const char* kc, const char* vc, char* kn, char* vn, int t) {
    constexpr bool MASKED = std::is_same_v<decltype(kind), Diagonal>;
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (t + 1 < T) {
      cp.issue(rk, kn, (t + 1) * kBC, wave, true);
      cp.issue(rv, vn, (t + 1) * kBC, wave, true);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int ks = t * kBC + kb * 32;  // first key of the block
      // a block whose keys all follow the wave's queries adds nothing
      if (CAUSAL && MASKED && ks > q0w + 31) continue;
      f32x16 s, dp;
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);  // as in the dK/dV kernel
      __builtin_amdgcn_sched_barrier(0);
      two_rows_times_reg<D>(kc, vc, kb, off, qreg, greg, s, dp);  // S^T = K Q^T, dP^T = V dO^T
      bf16x8 sb[2];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = ks + 8 * (v / 4) + 4 * half + (v % 4);
        float p = fast_exp2(fmaf(s[v], c, nl));
        if (MASKED && (key >= N || (CAUSAL && key > qi))) p = 0.f;
        sb[v / 8][v % 8] = (__bf16)(p * (dp[v] - dd));
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
      block_t_times<D>(kc, kb, off, sb, dq);  // dQ^T += K^T dS^T
#pragma unroll
      for (int m = 0; m < 2 * G::NO; ++m) {
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  int t = 0;
  for (; t + 1 < T_plain; t += 2) {
    step(Plain{}, ks0, vs0, ks1, vs1, t);
    step(Plain{}, ks1, vs1, ks0, vs0, t + 1);
  }
  if (t < T_plain) {
    step(Plain{}, ks0, vs0, ks1, vs1, t);
    ++t;
  }
  // the masked tiles (at most two), stage chosen by parity at run time
  for (; t < T; ++t) {
    const bool odd = t & 1;
    step(Diagonal{}, odd ? ks1 : ks0, odd ? vs1 : vs0, odd ? ks0 : ks1, odd ? vs0 : vs1, t);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();  // every wave is done with the tiles: they hold the staging slots
  static_assert(2 * 32 * 2 * D <= G::TILEB, "two staging slots per tile");
  char* const slot = (wave < 2 ? ks0 : ks1) + (wave & 1) * (32 * 2 * D);
  store_o_lse_staged<D>(dQ, nullptr, head, N, q0w, lane, dq, scale, 0.f, slot);
}

template <int D, bool CAUSAL>
hipError_t bwd_launch(const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, void* dq, void* dk, void* dv,
                      float* ws, int B, int H, int N, float scale, hipStream_t stream) {
  const long long rows = (long long)B * H * N;
  float* const dvec = ws;
  float* const nl = ws + rows;
  const int nt = (N + 127) / 128;
  const long long nwg = (long long)nt * B * H;
  if (nwg >= (1LL << 31)) return hipErrorInvalidValue;
  const int dbg = debug_flags();
  // Causal: whole heads per XCD, longest tiles first, when the heads split
  // evenly (not under the reversed debug order).
  const int hpx = ((long long)B * H) % 8 == 0 && !(dbg & 1) ? (int)(((long long)B * H) / 8) : 0;
  const int nwg_arg = (int)nwg | (dbg << kDbgShift);
  // dQ first: it also writes the row terms D and -LSE log2(e) that the
  // dK/dV kernel reads (stream order makes them visible to it).
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)nwg), dim3(256), 0, stream,
                     (const u16*)q, (const u16*)k, (const u16*)v, (const u16*)dout, (const u16*)o,
                     lse, nl, dvec, (u16*)dq, N, nt, nwg_arg, hpx, scale);
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)nwg), dim3(256), 0, stream,
                     (const u16*)q, (const u16*)k, (const u16*)v, (const u16*)dout,
                     (const float*)nl, (const float*)dvec, (u16*)dk, (u16*)dv, N, nt, nwg_arg,
                     hpx, scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv,
                           float* ws, int B, int H, int N, int d, bool causal, float scale,
                           hipStream_t stream) {
#define FA_CASE(DD)                                                                          \
  case DD:                                                                                   \
    return causal ? bwd_launch<DD, true>(q, k, v, o, lse, dout, dq, dk, dv, ws, B, H, N,     \
                                         scale, stream)                                     \
                  : bwd_launch<DD, false>(q, k, v, o, lse, dout, dq, dk, dv, ws, B, H, N,    \
                                          scale, stream);
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
