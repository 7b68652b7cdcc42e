// attn_kernel.h -- internal interface between the C ABI (attn_api.cpp) and the
// gfx950 attention kernel (attn_fwd.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace libattn {

// Tile schedules of the kernel.  Both compute bitwise identical results; the
// serial one exists to cross-check the ping-pong one (an LDS race in either
// would make them differ).
enum Schedule { SCHEDULE_PINGPONG = 0, SCHEDULE_SERIAL = 1 };

// Launch parameters.  Pointers are device pointers; strides are in elements.
struct Params {
  const _Float16* q;
  const _Float16* k;
  const _Float16* v;
  _Float16* o;
  float* lse;        // may be null
  int64_t q_bstride;  // S * Hq * D
  int64_t q_sstride;  // Hq * D
  int64_t kv_bstride; // S * Hkv * D
  int64_t kv_sstride; // Hkv * D
  int B, S, Hq, Hkv;
  int g;             // Hq / Hkv
  int pairs;         // ceil(g / 2): head pairs per KV head
  int n_qt;          // query tiles per head
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
