// variant.h -- the kernel variants libattn can launch and the choice among
// them per problem shape.  Host-only and free of HIP, so that the selection
// logic can be compiled and tested on its own.
//
// A variant is a point of the schedule space that the search in
// dnn_compiler_pipelining_amd/tune.py explores: the tile schedule, the depth
// of the fragment prefetch ring, where the softmax parts sit among the MFMAs
// (64-row and overlap schedules), the keys per K/V tile (serial schedules),
// the query rows per workgroup (64-row schedule) and two workgroup-order
// switches.  Variants with the same keys per tile compute
// bitwise identical results and differ only in speed; another tile size
// changes the rounding order of the online softmax.
// PipeThreader searches such a space of task orders with a validity check
// and profile feedback (page "PipeThreader: Software-Defined Pipelining ...
// (OSDI 2025)" summary, section "核心方法"); tuned_table.h is the outcome of
// that search for a set of measured shapes.
#pragma once

#include <cmath>

namespace libattn {

// Tile schedules (see attn_fwd.hip).  The first five compute bitwise identical
// results at 64-key tiles; SERIAL4_16 the same values up to rounding order.
//   SERIAL  : per tile, one wave runs QK^T, softmax and PV back to back; the
//             two waves that share a SIMD overlap each other's MFMA and VALU
//             work
//   OVERLAP : every wave overlaps, inside one instruction stream, the softmax
//             of tile j with the MFMAs of QK^T(j+1) and PV(j-1)
//   PINGPONG: two wave groups offset by half a tile alternate MFMA and softmax
//   SERIAL4 : the serial schedule in workgroups of four waves, one query head
//             each; two workgroups share a CU, so the two waves on a SIMD
//             come from independently synchronised workgroups and drift out
//             of phase (one's softmax beside the other's MFMAs)
//   WIDE    : 64 query rows per wave (attn_wide.h): one wave per SIMD, each
//             K/V fragment read from LDS feeds two MFMAs, the overlap
//             schedule inside each wave, K/V loaded two tiles ahead
//             (head dimension 128)
//   SERIAL4_16: SERIAL4 on 16 x 16 x 32 MFMAs (attn_s16.hip; head dimension
//             128, 64-key tiles); same values up to rounding order, not the
//             same bits
enum Schedule {
  SCHEDULE_SERIAL = 0,
  SCHEDULE_OVERLAP = 1,
  SCHEDULE_PINGPONG = 2,
  SCHEDULE_SERIAL4 = 3,
  SCHEDULE_WIDE = 4,
  SCHEDULE_SERIAL4_16 = 5
};

// Placements of the softmax parts among the MFMAs of the fused block of the
// 64-row schedule (WIDE) and of the overlap schedule (the other schedules
// have one placement, PLACE_EVEN):
//   PLACE_EVEN : the parts spread evenly over the block's steps
//   PLACE_FRONT: the first five parts (WIDE: of query half 0) before the
//                first MFMA, where the block waits for its first fragment,
//                the rest spread
//   PLACE_EARLY: the parts (WIDE: of half 1) end four steps before the
//                block, so that the sum check is settled when the block
//                ends; WIDE also holds each fp16 pack at its step (not sunk
//                to its first use)
enum Place { PLACE_EVEN = 0, PLACE_FRONT = 1, PLACE_EARLY = 2 };

// Keys per K/V tile of every schedule (BN in the kernels); SERIAL and SERIAL4
// at head dimension 128 also run 32 and 128.
constexpr int BN_STD = 64;

struct Variant {
  int schedule;  // Schedule
  int ring;      // fragment prefetch depth of the mma steps: 2 or 4
  int xcd;       // 1: each XCD gets whole (batch, kv head) groups
  int lpt;       // 1: longest causal query tiles of a group first
  int place;     // Place (SCHEDULE_WIDE and SCHEDULE_OVERLAP; PLACE_EVEN for the others)
  int bn;        // keys per K/V tile: 64; SERIAL and SERIAL4 also 32 and 128 (head dimension 128)
  int hpw;       // SCHEDULE_WIDE: query heads per workgroup, 4, 2 or 1 (64, 128 or 256 query rows of
                 // each), 0 for the largest of them that divides the GQA ratio; 0 for the others
};

// One measured shape and the fastest variant found for it.
struct TunedEntry {
  int B, Sq, Sk, Hq, Hkv;
  Variant v;
  double tflops;  // measured rate of that variant (documentation only)
};

#include "tuned_table.h"  // kTuned[], kTunedCount

inline bool variant_valid(const Variant& v) {
  return v.schedule >= SCHEDULE_SERIAL && v.schedule <= SCHEDULE_SERIAL4_16 && (v.ring == 2 || v.ring == 4) &&
         (v.xcd == 0 || v.xcd == 1) && (v.lpt == 0 || v.lpt == 1) && v.place >= PLACE_EVEN &&
         v.place <= PLACE_EARLY &&
         (v.schedule == SCHEDULE_WIDE || v.schedule == SCHEDULE_OVERLAP || v.place == PLACE_EVEN) &&
         (v.bn == BN_STD || ((v.bn == 32 || v.bn == 128) &&
                         (v.schedule == SCHEDULE_SERIAL || v.schedule == SCHEDULE_SERIAL4))) &&
         (v.hpw == 0 || ((v.hpw == 1 || v.hpw == 2 || v.hpw == 4) && v.schedule == SCHEDULE_WIDE));
}

// The variant tuned for the measured shape nearest to (B, Sq, Sk, Hq, Hkv):
// distance = sum of |log2| ratios of B, Sq, Sk and the GQA ratio Hq/Hkv, plus
// half that of Hkv.  The first entry wins ties.
inline Variant tuned_variant(int B, int Sq, int Sk, int Hq, int Hkv) {
  auto lr = [](double a, double b) { return std::fabs(std::log2(a / b)); };
  const double g = (double)Hq / Hkv;
  int best = 0;
  double best_d = 1e300;
  for (int i = 0; i < kTunedCount; ++i) {
    const TunedEntry& e = kTuned[i];
    const double d = lr(B, e.B) + lr(Sq, e.Sq) + lr(Sk, e.Sk) + lr(g, (double)e.Hq / e.Hkv) + 0.5 * lr(Hkv, e.Hkv);
    if (d < best_d) {
      best_d = d;
      best = i;
    }
  }
  return kTuned[best].v;
}

}  // namespace libattn
