// attn_kernel.h -- internal interface between the C ABI (attn_api.cpp) and the
// gfx950 attention kernel (attn_fwd.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "variant.h"

namespace libattn {

// Tile schedules and the variant choice: variant.h.  Measured on MI355X the
// serial, overlap and serial4 schedules land within a few percent of each
// other: the softmax's VALU instructions take issue from the MFMAs of every
// wave on a SIMD whatever the order, and the chip runs at its power limit.

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
  int pairs;         // workgroups per KV head and query tile: ceil(g / 2) head pairs, or g heads (SERIAL4)
  int n_qt;          // query tiles per head (over Sq)
  int causal;
  int neg;           // scale < 0: the kernel negates Q and uses |scale|
  float cs;          // |scale| * log2(e)
  int hd;            // head dimension: 64, 128 or 256
  int schedule;      // Schedule (HD 64: serial only)
  int ring;          // fragment prefetch depth of the mma steps: 2 or 4
  int xcd;           // 1: give each XCD whole (batch, kv head) groups
  int lpt;           // 1: longest causal query tiles of a group first
  int hpw;           // WIDE: query heads per workgroup (4, 2 or 1; 256 / hpw query rows each)
  int place;         // WIDE and OVERLAP: Place of the softmax parts (variant.h)
  int bn;            // keys per K/V tile: 64; SERIAL and SERIAL4 at HD 128 also 32 or 128
  // split-KV mode (attn_fwd_decode): n_qt counts 128-row tiles of the packed
  // (head, query row) rows of a KV group; the keys are cut into n_splits
  // splits of split_tiles 64-key tiles; partial results go to ws_o
  // [B][Hq][Sq][n_splits][D] and ws_lse [B][Hq][Sq][n_splits] (fp32)
  int n_splits;
  int split_tiles;
  float* ws_o;
  float* ws_lse;
};

// Grid size for p (number of workgroups), or -1 if it does not fit an int.
int64_t grid_blocks(const Params& p);

// Grid size of the split-KV kernel, or -1 if it does not fit an int.
int64_t grid_blocks_decode(const Params& p);

// Enqueue the split-KV kernel and the kernel that combines its splits into o
// and lse (SERIAL4 schedule, any ring).  Returns the hipError_t of the launches.
hipError_t launch_attn_decode(const Params& p, hipStream_t stream);

// Enqueue the forward kernel.  Returns the hipError_t of the launch.
hipError_t launch_attn_fwd(const Params& p, hipStream_t stream);

// Grid size and launch of the WIDE schedule's kernel (attn_wide.h; head
// dimension 128): p.pairs head groups of p.hpw heads per KV head, p.n_qt query
// tiles of 256 / p.hpw rows, placement p.place.
int64_t grid_blocks_wide(const Params& p);
hipError_t launch_attn_wide(const Params& p, hipStream_t stream);

// Grid size and launch of the SERIAL4_16 schedule's kernel (attn_s16.hip; head
// dimension 128, 64-key tiles): p.pairs = g one-head workgroups per KV head,
// p.n_qt query tiles of 128 rows, prefetch depth p.ring.
int64_t grid_blocks_s16(const Params& p);
hipError_t launch_attn_s16(const Params& p, hipStream_t stream);

}  // namespace libattn
