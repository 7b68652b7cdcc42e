// attn_tile.h -- tile geometry, constants and lane-pair reductions shared by
// the gfx950 attention kernels (attn_fwd.hip, attn_wide.h).
#pragma once

#include "gfx950.h"

namespace libattn {

constexpr int BN = 64;           // keys per KV tile (the serial schedules also run 32 and 128)
constexpr float NEG_INF = -__builtin_inff();
constexpr float M_INIT = -1e30f; // finite start for the running max
constexpr float LN2 = 0.693147180559945309f;
// Sum-checked lazy rescaling: a tile's exponentials are first taken against
// the running max m (log2 units) as it stands.  If no row's sum over the tile
// exceeds RS_MAX, every P of the tile is at most RS_MAX (fp16 P and the fp32
// sums stay in range) and m stays; otherwise -- in practice only on a row's
// first tile -- m is raised to the tile max and the exponentials are redone.
// No tile max is needed in the common case, and the final O / l and
// LSE = m + log2(l) are exact for any m.
constexpr float RS_MAX = 256.0f;

// LDS layouts (bytes), per head dimension HD (64, 128 or 256) and keys per tile
// kBN.  A tile slot is a run of 1 KiB DMA instructions; where a K tile is not a
// whole number of them (kBN 32), its slot is rounded up and the last
// instruction's surplus lanes land past the tile.
//  K: kBN key rows of 2*HD + 16 B.  Consecutive keys fall 68 (HD 128), 36
//    (HD 64) or 132 (HD 256) banks apart, so the 16 keys of a ds_read_b128 pass at one
//    16-byte column cover all 64 banks once; every K fragment read is a
//    compile-time offset from one per-lane base.  One 16-byte lane slot per
//    row lands in the padding.
//  V: kBN key rows of 2*HD B whose 16-byte chunks are XOR-swizzled: by
//    4*(row & 3) for HD 128 and 256, by 4*((row >> 1) & 1) for HD 64.  A
//    ds_read_b64_tr_b16 group reads 4 consecutive rows x 32 B; with the
//    swizzle the 4 rows of the two groups of a half-wave (4 rows x 64 B) hit
//    all 64 banks once.  Across the 32-wide d blocks the per-lane address
//    changes by an XOR with 64*db.
template <int kHD, int kBN = BN>
struct Geo {
  static_assert(kHD == 64 || kHD == 128 || kHD == 256, "head dimension");
  static_assert(kBN == 32 || kBN == 64 || kBN == 128, "keys per tile");
  static constexpr int HD = kHD;
  static constexpr int KC = kHD / 8;                 // 16-byte chunks per K/V row
  static constexpr int K_ROWB = 2 * kHD + 16;
  static constexpr int K_TILEB = kBN * K_ROWB;       // kBN 64: 17408 | 9216 | 33792
  static constexpr int K_DMA = (K_TILEB + 1023) / 1024;  // kBN 64: 17 | 9 | 33
  static constexpr int K_SLOTB = 1024 * K_DMA;       // a K ring slot: the tile in whole instructions

  static constexpr int V_ROWB = 2 * kHD;
  static constexpr int V_TILEB = kBN * V_ROWB;       // kBN 64: 16384 | 8192 | 32768
  static constexpr int V_DMA = V_TILEB / 1024;       // kBN 64: 16 | 8 | 32

  static constexpr int V_ROWS_PER_DMA = 1024 / V_ROWB;
  static constexpr int NKK = kHD / 16;               // 16-wide d steps of QK^T
  static constexpr int NDB = kHD / 32;               // 32-wide d blocks of O^T
  static_assert(V_TILEB % 1024 == 0, "V tile slots are whole DMA instructions");
  static_assert(V_DMA % 8 == 0, "every wave of 4 or 8 issues the same number of V instructions");
  // physical 16-byte chunk of logical chunk c in V row r is c ^ vswz(r)
  __host__ __device__ static constexpr int vswz(int r) { return kHD == 64 ? 4 * ((r >> 1) & 1) : 4 * (r & 3); }
};
// acc += lo + hi of a packed fp16 pair, in fp32 (two v_fma_mix_f32, each
// adding one exactly widened half with one rounding).  The row sum of the
// softmax is taken this way from the fp16 P that the PV MFMAs consume.  Not
// v_dot2_f32_f16 against (1, 1): on gfx950 a dot2 does not issue beside a
// running MFMA and costs the matrix core about 18 cycles each, where a mix
// FMA costs it nothing (measured in a one-wave-per-SIMD probe).
__device__ __forceinline__ void add_pair_f16(float& acc, f16x2 pr) {
  asm("v_fma_mix_f32 %0, %1, 1.0, %0 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mix_f32 %0, %1, 1.0, %0 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
      : "+v"(acc)
      : "v"(pr));
}

__device__ __forceinline__ float pair_max(float x) {
  // lanes l and l^32 hold the same query: combine their partial results
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

}  // namespace libattn
