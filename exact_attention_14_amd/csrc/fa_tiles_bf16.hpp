// bf16 tiles in LDS shared by the attention kernels (gfx950 only): the
// geometry of a 64-row tile, its 16-byte-chunk swizzle, the direct-to-LDS
// copy of a tile spread over a workgroup's waves, and the transposed read of
// two 8-byte row fragments.
#pragma once
#include "fa_common.hpp"

namespace fa {

constexpr int kBC = 64;  // rows per tile (keys of a K/V tile, queries of a Q/dO tile)

template <int D>
struct Geo {
  static constexpr int CPR = D / 8;                                  // 16-B chunks of data per row
  static constexpr int CPRP = D == 64 ? 8 : (D == 256 ? 32 : 16);    // chunk slots per LDS row
  static constexpr int ROWB = CPRP * 16;                             // bytes per LDS row
  static constexpr int TILEB = kBC * ROWB;                           // one tile
  static constexpr int STAGEB = 2 * TILEB;                           // K + V
  static constexpr int NK = D / 16;                                  // 16-wide k-steps over d
  static constexpr int NO = D / 32;                                  // 32-row blocks of d
};

// Chunk-slot XOR for LDS row `row`: with it the 16-byte row reads (one per
// lane, 32 rows) and the transposed 8-byte reads are both free of bank
// conflicts.
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

// Byte offset for the chunk slots beyond the data width (d = 96). For heads
// below 1 GiB (N < 5592406 at d = 96) it lies past the head buffer, so those
// copies return zeros without memory traffic; for larger heads (up to the
// 2 GiB that N * d <= 2^30 allows) the pad slots receive real data from
// inside the head, which is harmless: no read of the kernels touches a pad
// slot. The offset stays at 1 GiB because it is added to the tile base,
// which is 2^31 for a tile past the sequence end: 2^31 + 2^30 still fits the
// 32-bit offset, a 2 GiB pad offset would wrap to the start of the buffer.
constexpr unsigned kPadOffset = 0x40000000u;

// Per-lane byte offsets (tile row 0) of this wave's share of a tile copy of
// ROWS rows; rows past the data width get an offset beyond any buffer (zero
// fill).
template <int D, int NW, int ROWS = kBC>
struct TileCopy {
  static constexpr int NI = Geo<D>::CPRP * ROWS / 64 / NW;
  static_assert(NI * NW * 64 == Geo<D>::CPRP * ROWS, "whole 1 KiB copies per wave");
  unsigned off[NI];
  __device__ __forceinline__ TileCopy(int wave, int lane) {
    using G = Geo<D>;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int slot = (i * NW + wave) * 64 + lane;
      const int row = slot / G::CPRP;
      const int c = (slot % G::CPRP) ^ swz<G::CPRP>(row);
      off[i] = c < G::CPR ? (unsigned)(row * D + c * 8) * 2u : kPadOffset;
    }
  }
  // Copy i (0 <= i < NI) of the tile starting at row j0 into `tile`
  // (zeros if !valid).
  __device__ __forceinline__ void issue_one(int i, i32x4 rs, char* tile, int j0, int wave,
                                            bool valid) const {
    const unsigned base = valid ? (unsigned)j0 * D * 2u : kOutOfRange;
    copy16_to_lds_asm(rs, tile + (i * NW + wave) * 1024, off[i] + base);
  }
  // All NI copies of the tile, back to back.
  __device__ __forceinline__ void issue(i32x4 rs, char* tile, int j0, int wave,
                                        bool valid = true) const {
#pragma unroll
    for (int i = 0; i < NI; ++i) issue_one(i, rs, tile, j0, wave, valid);
  }
};

}  // namespace fa
