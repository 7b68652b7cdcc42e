// attn_kernel.h -- internal interface between the C ABI (attn_api.cpp) and the
// gfx950 attention kernel (attn_fwd.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace libattn {

// Tile schedules of the kernel.  All compute bitwise identical results (each
// accumulator sees the same operations in the same order), so running one
// against another cross-checks them: an LDS race in any would show up.
//   SERIAL  : per tile, one wave runs QK^T, softmax and PV back to back; the
//             two waves that share a SIMD overlap each other's MFMA and VALU
//             work (the default: fastest measured, see below)
//   OVERLAP : every wave overlaps, inside one instruction stream, the softmax
//             of tile j with the MFMAs of QK^T(j+1) and PV(j-1)
//   PINGPONG: two wave groups offset by half a tile alternate MFMA and softmax
// Measured on MI355X all three land within a few percent of each other: the
// kernel runs at the chip's power limit, where the clock, not the issue
// order, sets the rate.
enum Schedule { SCHEDULE_SERIAL = 0, SCHEDULE_OVERLAP = 1, SCHEDULE_PINGPONG = 2 };

// Launch parameters.  Pointers are device pointers; strides are in elements.
struct Params {
  const _Float16* q;
  const _Float16* k;
  const _Float16* v;
  _Float16* o;
  float* lse;        // may be null
  int64_t q_bstride;  // Sq * Hq * D
  int64_t q_sstride;  // Hq * D
  int64_t kv_bstride; // Sk * Hkv * D
  int64_t kv_sstride; // Hkv * D
  int B, Sq, Sk, Hq, Hkv;
  int off;           // causal: Sk - Sq (query row i may attend keys j <= i + off); 0 otherwise
  int g;             // Hq / Hkv
  int pairs;         // ceil(g / 2): head pairs per KV head
  int n_qt;          // query tiles per head (over Sq)
  int causal;
  int neg;           // scale < 0: the kernel negates Q and uses |scale|
  float cs;          // |scale| * log2(e)
  int schedule;      // Schedule
};

// Grid size for p (number of workgroups), or -1 if it does not fit an int.
int64_t grid_blocks(const Params& p);

// Enqueue the forward kernel.  Returns the hipError_t of the launch.
hipError_t launch_attn_fwd(const Params& p, hipStream_t stream);

}  // namespace libattn
