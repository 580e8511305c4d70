// Device-side helpers shared by the attention kernels (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16;

// log2(e): the kernels evaluate exp(x) as exp2(x * log2 e).
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// One 32x32x16 bf16 matrix-core step, D = A B + C.
// A (32 x 16): lane l holds row l%32, reduction slots 8*(l/32) .. +7.
// B (16 x 32): lane l holds column l%32, reduction slots 8*(l/32) .. +7.
// C/D (32 x 32): lane l holds column l%32; element v is row
//   8*(v/4) + 4*(l/32) + v%4.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

// Maximum of x and the x of the lane 32 positions away (v_permlane32_swap).
__device__ __forceinline__ float max_with_other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Exchange with the lane 32 positions away (the other half of the wave).
__device__ __forceinline__ float xor32(float x) {
  return __shfl_xor(x, 32);
}

// s_waitcnt immediate: vmcnt = 0, expcnt and lgkmcnt left at their maxima.
constexpr int kWaitVmcnt0 = 0x0F70;

// s_waitcnt immediate for vmcnt = n (n < 64), expcnt and lgkmcnt at maxima.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }

// Buffer byte offset past any head buffer (head buffers are below 2 GiB):
// loads and copies there return zeros and stores are dropped, with no memory
// traffic.
constexpr unsigned kOutOfRange = 0x80000000u;

// Waves per SIMD the attention kernels are compiled for (their register
// budget: 512 / waves per lane). d = 256 needs the whole file for one wave;
// d = 64 fits three (<= 168 registers): measured on the forward +2% (bf16)
// and +5 to +9% (e4m3) at N = 8192, +5 to +13% (bf16) at N = 1024, -3% at
// N = 2048 non-causal (1024 workgroups: 1.33 rounds of three per compute
// unit instead of two rounds of two), and on the backward +2 to +5% at
// N = 8192; the rest run two.
template <int D>
constexpr int kWavesPerSimd = D == 256 ? 1 : (D == 64 ? 3 : 2);

// Instruction classes of __builtin_amdgcn_sched_group_barrier masks.
constexpr int kSchedValu = 0x002 | 0x400;  // VALU and transcendental
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// Raw buffer resource (gfx9 family dword 3: 32-bit data format). Loads at
// byte offsets >= `bytes` return zeros without touching memory.
constexpr int kBufferFlags = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                           kBufferFlags);
}


// Buffer resource as four dwords for inline assembly (base, stride 0,
// num_records = bytes, gfx9 dword 3).
__device__ __forceinline__ i32x4 make_rsrc_words(const void* p, unsigned bytes) {
  const unsigned long long a = reinterpret_cast<unsigned long long>(p);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(unsigned)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(unsigned)(a >> 32) & 0xFFFF);
  r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
  r[3] = kBufferFlags;
  return r;
}

// The same 16-byte HBM -> LDS copy, written as assembly so that the compiler
// does not treat it as an LDS store: it then inserts no conservative
// vmcnt(0) before unrelated LDS reads, and the kernel's own s_waitcnt
// vmcnt(n) decides when a copy is complete. `lds` must be wave-uniform. The
// instruction has no register results (the data goes to LDS).
__device__ __forceinline__ void copy16_to_lds_asm(i32x4 rsrc, const void* lds, unsigned byte_off) {
  const unsigned m0 = (unsigned)reinterpret_cast<unsigned long long>(
      (const __attribute__((address_space(3))) void*)lds);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m0), "v"(byte_off), "s"(rsrc)
               : "memory", "m0");
}

// Epilogue of one wave. O^T arrives as NO = D/32 blocks of 32 output columns
// x 32 queries (lane = query q0w + lane % 32, element v = column
// 8*(v/4) + 4*half + v%4 of its block); it is scaled by inv, rounded to bf16
// and staged through LDS: the wave writes its 32 rows x D bf16 into `slot`
// (32 * 2D bytes, 16-byte aligned, read by no other wave any more), 16-byte
// chunk c of row r at chunk (c + r) mod D/8 so that neither the 8-byte
// writes nor the 16-byte reads conflict; then each store instruction writes
// 1 KiB of whole rows (16 contiguous bytes per lane) instead of 8 bytes in
// each of 32 rows. There is no branch on the query bound: with a
// wave-divergent branch the compiler may move the last matrix-core products
// into it, where they would run under a partial exec mask. Rows past N fall
// outside the buffer range of the head's O rows and are dropped by the
// hardware range check, as is the LSE store of the second half-wave (and
// every LSE store when LSE is null).
template <int D>
__device__ __forceinline__ void store_o_lse_staged(u16* O, float* LSE, size_t head, int N,
                                                   int q0w, int lane, const f32x16* oacc,
                                                   float inv, float lse, char* slot) {
  constexpr int NO = D / 32;
  constexpr int CPR = D / 8;         // 16-byte chunks per row
  constexpr int ROWB = D * 2;        // bytes per row
  constexpr int NJ = 32 * ROWB / 1024;  // 1 KiB store instructions per wave
  const int half = lane >> 5, l32 = lane & 31;
#pragma unroll
  for (int i = 0; i < NO; ++i)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 w;
#pragma unroll
      for (int x = 0; x < 4; ++x) w[x] = (__bf16)(oacc[i][4 * g + x] * inv);
      const int chunk = (4 * i + g + l32) % CPR;
      *(bf16x4*)(slot + l32 * ROWB + chunk * 16 + 8 * half) = w;
    }
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(O + head * D, (unsigned)N * D * 2u);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int flat = j * 1024 + lane * 16;
    const int row = flat / ROWB, chunk = (flat % ROWB) / 16;
    const i32x4 v = *(const i32x4*)(slot + row * ROWB + ((chunk + row) % CPR) * 16);
    __builtin_amdgcn_raw_buffer_store_b128(v, ro, (unsigned)((q0w + row) * ROWB + chunk * 16), 0,
                                           0);
  }
  const __amdgpu_buffer_rsrc_t rl =
      make_rsrc(LSE != nullptr ? (const void*)(LSE + head) : nullptr,
                LSE != nullptr ? (unsigned)N * 4u : 0u);
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_int(lse), rl,
                                        half == 0 ? (unsigned)(q0w + l32) * 4u : kOutOfRange, 0, 0);
}

// Debug flags of a launch ride in the top bits of the workgroup-count
// argument (the forward and backward grids stay below 2^24 workgroups):
// kDbgReverse runs the workgroups in the reverse order and on other XCDs
// (the host also drops the per-XCD head grouping), kDbgPoison fills the
// kernel's LDS with 0xFF bytes (NaN in bf16, fp32 and e4m3) before any tile
// is copied in. Results must not change: each workgroup's output depends
// only on its own tile, and no tile may be read before its copy has landed.
constexpr int kDbgShift = 24;
constexpr int kDbgReverse = 1;
constexpr int kDbgPoison = 2;
__device__ __forceinline__ int dbg_flags(int nwg_arg) { return nwg_arg >> kDbgShift; }

// Fills `bytes` (a multiple of 16) of LDS from `p` with 0xFF, shared over
// `nthreads` threads; the caller waits for all of them (a barrier) before
// any copy into that memory is issued.
__device__ __forceinline__ void poison_lds(char* p, int bytes, int tid, int nthreads) {
  const i32x4 ff = {-1, -1, -1, -1};
  for (int o = tid * 16; o < bytes; o += nthreads * 16) *(i32x4*)(p + o) = ff;
}

// Workgroup id -> (head, query-tile rank). Workgroup ids are dealt to the 8
// XCDs round-robin. With hpx > 0 (B*H = 8*hpx heads) each XCD owns hpx whole
// heads and starts its workgroups in rank order across them (rank 0 = the
// longest causal tile first); otherwise consecutive logical ids, i.e. the
// tiles of one head, run on one XCD. `nwg` is the plain workgroup count.
__device__ __forceinline__ void tile_of_id(int bid, int nwg, int ntq, int hpx, int& bh,
                                           int& rank) {
  if (hpx > 0) {
    const int loc = bid >> 3;
    rank = loc / hpx;
    bh = (bid & 7) * hpx + loc % hpx;
    return;
  }
  const int q8 = nwg >> 3, r8 = nwg & 7;
  const int xcd = bid & 7, loc = bid >> 3;
  const int lid = xcd < r8 ? xcd * (q8 + 1) + loc : r8 * (q8 + 1) + (xcd - r8) * q8 + loc;
  rank = lid % ntq;
  bh = lid / ntq;
}

// The same for grids below 2^24 workgroups whose count argument carries the
// debug flags in its top bits (kDbgReverse: logical id nwg - 1 - bid).
__device__ __forceinline__ void tile_of_workgroup(int bid, int nwg, int ntq, int hpx, int& bh,
                                                  int& rank) {
  if (dbg_flags(nwg) & kDbgReverse) bid = (nwg & ((1 << kDbgShift) - 1)) - 1 - bid;
  tile_of_id(bid, nwg & ((1 << kDbgShift) - 1), ntq, hpx, bh, rank);
}


}  // namespace fa
