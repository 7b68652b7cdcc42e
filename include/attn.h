/*
 * attn.h -- C ABI of libattn: fused grouped-query softmax attention, forward
 * pass, for AMD Instinct MI355X (gfx950).
 *
 * The operation.  PipeThreader's FlashAttention workload (page "PipeThreader:
 * Software-Defined Pipelining for Efficient DNN Execution (OSDI 2025)"
 * summary, section "实验与结果", citing the paper's section 6.2 / Fig.12:
 * LLaMA3-8B/70B head shapes, sequence 512..8k, batch 1/64) is the attention
 * forward pass, which that page splits into load, mma and softmax sTasks
 * (section "核心方法").  For every batch entry b, query head h and query row i:
 *
 *   c = h / (Hq / Hkv)                         query head h reads KV head c
 *   allowed keys j: 0..i if causal, else 0..S-1
 *   s_j = scale * dot(q[b,i,h,:], k[b,j,c,:])
 *   o[b,i,h,:]  = sum_j softmax(s)_j * v[b,j,c,:]
 *   lse[b,h,i]  = log(sum_j exp(s_j))          natural log of the scaled scores
 *
 * Tensors (all device memory, owned and allocated by the caller, contiguous):
 *   q   fp16 [B][S][Hq][D]     k, v  fp16 [B][S][Hkv][D]
 *   o   fp16 [B][S][Hq][D]     (written; must not overlap q, k, v or lse)
 *   lse fp32 [B][Hq][S]        (written; must not overlap q, k, v or o; may be
 *                              NULL when not wanted)
 * Every pointer must be 16-byte aligned.  fp16 is IEEE binary16; o is rounded
 * to nearest even from fp32.  Internal offsets are 64-bit, so tensors larger
 * than 4 GiB are supported.
 *
 * Scalars: B, S, Hq, Hkv >= 1; S <= 2^30; Hq % Hkv == 0; D is 64, 128 or 256
 * (other head sizes return ATTN_ERR_UNSUPPORTED, and so does
 * Hkv * D * 2 * 64 >= 2^32, i.e. a 64-row K/V tile spanning 4 GiB or more);
 * causal is 0 or 1; scale is any finite float.
 *
 * attn_fwd_ex takes different query and key lengths (chunked prefill): q and
 * o are [B][Sq][Hq][D], k and v [B][Sk][Hkv][D], lse [B][Hq][Sq].  With
 * causal = 1 the mask is aligned at the bottom right: query row i sits at key
 * position i + Sk - Sq and attends keys 0..i + Sk - Sq, so the last query row
 * sees every key (Sq == Sk gives the square mask above); causal needs
 * Sq <= Sk, else ATTN_ERR_SHAPE.  Without causal any Sq, Sk >= 1 is allowed.
 *
 * Execution: the call validates its arguments, then enqueues one kernel on
 * the given HIP stream (attn_fwd uses the null stream) and returns without
 * waiting.  Faults during execution surface at the caller's next
 * synchronisation.  The library allocates no memory, keeps no state between
 * calls, is thread-safe, and gives bitwise identical results run to run.
 *
 * Kernel variants.  Every entry point runs the variant tuned for the nearest
 * measured shape (a table compiled into the library); attn_fwd_variant names
 * one explicitly.  Variants on the 32 x 32 x 16 MFMA with the same keys per
 * K/V tile give bitwise identical results, so each serves as a cross-check of
 * the others; a tile size other than 64 keys, or ATTN_SCHEDULE_SERIAL4_16 (the
 * 16 x 16 x 32 MFMA), changes only the rounding order.  The library reads no
 * environment.
 *
 * Errors: on invalid arguments nothing is launched and a nonzero ATTN_ERR_*
 * code is returned; a failed launch returns ATTN_ERR_HIP.  No exception
 * crosses the ABI and nothing is printed.  attn_status_string() names a code.
 */
#ifndef LIBATTN_ATTN_H
#define LIBATTN_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,        /* a required pointer is NULL */
  ATTN_ERR_SHAPE = 2,       /* a size < 1 or > 2^30, Hq % Hkv != 0, causal not 0/1, causal with Sq > Sk, scale not finite */
  ATTN_ERR_UNSUPPORTED = 3, /* D other than 64, 128 or 256, or Hkv * D * 2 * 64 >= 2^32; attn_fwd_variant: a
                               variant that does not exist or that the head dimension does not run */
  ATTN_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  ATTN_ERR_HIP = 5,         /* the HIP runtime reported an error at launch */
  ATTN_ERR_OVERLAP = 6,     /* o or lse overlaps another tensor; or the workspace overlaps any tensor */
  ATTN_ERR_WORKSPACE = 7,   /* attn_fwd_decode: workspace NULL, smaller than attn_decode_workspace_size(), or not
                               16-byte aligned */
  ATTN_ERR_TOO_LARGE = 8    /* attn_fwd_decode_static: the sizes need more workspace than
                               ATTN_STATIC_WORKSPACE_BYTES */
};

/* Forward pass on the null stream.  Returns ATTN_OK or an ATTN_ERR_* code. */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int S, int Hq, int Hkv, int D,
             int causal, float scale);

/* Same as attn_fwd, enqueued on `stream` (a hipStream_t; NULL means the null stream). */
int attn_fwd_stream(const void* q, const void* k, const void* v, void* o, float* lse, int B, int S, int Hq, int Hkv,
                    int D, int causal, float scale, void* stream);

/* Sq query rows against Sk keys (see above), enqueued on `stream`.  attn_fwd_stream(..., S, ...) is
 * attn_fwd_ex(..., S, S, ...). */
int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Sq, int Sk, int Hq,
                int Hkv, int D, int causal, float scale, void* stream);

/* Tile schedules of the forward kernel (attn_fwd_variant):
 *   SERIAL    8-wave workgroups, 32 query rows per wave; per tile QK^T, softmax, PV back to back
 *   OVERLAP   the same workgroups; each wave runs the softmax of tile j between the MFMAs of QK^T(j+1)
 *             and PV(j-1)
 *   PINGPONG  the same workgroups; two wave groups offset by half a tile alternate MFMA and softmax
 *   SERIAL4   the serial schedule in 4-wave, one-head workgroups, two per CU
 *   WIDE      4-wave workgroups, one wave per SIMD, 64 query rows per wave, the overlap schedule inside
 *             each wave, K/V loaded two tiles ahead (D = 128 only)
 *   SERIAL4_16  SERIAL4 on 16 x 16 x 32 MFMAs (D = 128, 64-key tiles); same values up to rounding order
 * D = 64 runs SERIAL and SERIAL4, D = 256 SERIAL4, D = 128 all six.  Every schedule stages K/V in tiles of
 * 64 keys; at D = 128 SERIAL and SERIAL4 also run tiles of 32 and 128 keys. */
enum {
  ATTN_SCHEDULE_SERIAL = 0,
  ATTN_SCHEDULE_OVERLAP = 1,
  ATTN_SCHEDULE_PINGPONG = 2,
  ATTN_SCHEDULE_SERIAL4 = 3,
  ATTN_SCHEDULE_WIDE = 4,
  ATTN_SCHEDULE_SERIAL4_16 = 5
};

/* Placement of the softmax work among the MFMAs of the main loop of ATTN_SCHEDULE_WIDE and
 * ATTN_SCHEDULE_OVERLAP: spread evenly, partly before the first MFMA (where the loop waits for its first
 * operands), or ending early (the sum check settled before the loop's next iteration).  The other
 * schedules have ATTN_PLACE_EVEN only. */
enum { ATTN_PLACE_EVEN = 0, ATTN_PLACE_FRONT = 1, ATTN_PLACE_EARLY = 2 };

/* attn_fwd_ex with an explicit kernel variant, for schedule search and cross-checks: `schedule` is an
 * ATTN_SCHEDULE_* value, `ring` the fragment prefetch depth (2 or 4), `xcd` 1 to give each XCD whole
 * (batch, KV head) groups, `lpt` 1 to run the longest causal query tiles first, `place` an ATTN_PLACE_*
 * value, `bn` the keys per K/V tile (64; 32 or 128 with SERIAL or SERIAL4 at D = 128), `hpw` the query
 * heads per workgroup of ATTN_SCHEDULE_WIDE (4, 2 or 1, i.e. 64, 128 or 256 query rows of each; 0 the
 * largest that divides Hq / Hkv); -1 in any of them takes the tuned value (place: ATTN_PLACE_EVEN for
 * schedules other than ATTN_SCHEDULE_WIDE and ATTN_SCHEDULE_OVERLAP; bn: 64 where the schedule or D has no
 * other; hpw: 0 for schedules other than ATTN_SCHEDULE_WIDE).  A value that does not exist, a
 * placement or tile size the schedule does not have, or a schedule the head dimension does not run,
 * returns ATTN_ERR_UNSUPPORTED and launches nothing.  Results are bitwise identical for every variant of one
 * tile size except ATTN_SCHEDULE_SERIAL4_16; another tile size, or that schedule, changes the rounding order. */
int attn_fwd_variant(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Sq, int Sk, int Hq,
                     int Hkv, int D, int causal, float scale, int schedule, int ring, int xcd, int lpt, int place,
                     int bn, int hpw, void* stream);

/* The variant attn_fwd_ex runs for these sizes (ATTN_SCHEDULE_* value, ring depth, xcd and lpt switches,
 * ATTN_PLACE_* value, keys per K/V tile, heads per workgroup as requested: 0 = the largest of 4, 2, 1
 * dividing Hq / Hkv), for reports and cross-checks.  Returns ATTN_OK, ATTN_ERR_NULL for a NULL output
 * pointer, ATTN_ERR_SHAPE for sizes attn_fwd_ex rejects, ATTN_ERR_UNSUPPORTED for a head dimension it does
 * not run.  No HIP call. */
int attn_tuned_variant(int B, int Sq, int Sk, int Hq, int Hkv, int D, int* schedule, int* ring, int* xcd, int* lpt,
                       int* place, int* bn, int* hpw);

/* Compute-unit count and peak shader clock (kHz) of HIP device `device`, as the runtime reports them: the
 * inputs of a peak-throughput figure (dense fp16 MFMA on gfx950: 4 SIMDs x 1024 FLOP per clock per compute
 * unit).  Returns ATTN_OK, ATTN_ERR_NULL or ATTN_ERR_HIP. */
int attn_device_clock(int device, int* compute_units, int* peak_clock_khz);

/* Split-KV path for few query rows against many keys (decode, short chunks): the same operation and
 * arguments as attn_fwd_ex, computed in two kernels.  The first packs the g = Hq / Hkv query heads of a KV
 * group with their Sq query rows into 128-row tiles, so each K/V tile is read once for all of them, and
 * cuts the keys into splits run by different workgroups, each writing its normalised partial O and LSE
 * (fp32) to `workspace`; the second merges the splits (O = sum_s exp(LSE_s - LSE) O_s, LSE = log sum_s
 * exp(LSE_s)) into o and lse.  Results match attn_fwd_ex within the attention tolerance, not bit for bit.
 * `workspace` is caller-owned device memory of at least attn_decode_workspace_size(...) bytes, 16-byte
 * aligned, not overlapping any tensor; its contents on entry do not matter and are overwritten.  Needs
 * (Hq / Hkv) * Sq <= 2^30.  Both kernels are enqueued on `stream`; the workspace must not be reused
 * before they complete.  The split length is chosen for about 512 workgroups. */
int attn_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Sq, int Sk, int Hq,
                    int Hkv, int D, int causal, float scale, void* workspace, size_t workspace_bytes, void* stream);
/* Workspace bytes attn_fwd_decode needs for these sizes (0 for sizes it rejects). */
size_t attn_decode_workspace_size(int B, int Sq, int Sk, int Hq, int Hkv, int D);

/* attn_fwd_decode with an explicit split length: `split_tiles` 64-key tiles per split (capped at the
 * number of key tiles; 0 or less takes the planned length).  The workspace must hold
 * attn_decode_workspace_size_split(..., split_tiles) bytes. */
int attn_fwd_decode_split(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Sq, int Sk,
                          int Hq, int Hkv, int D, int causal, float scale, int split_tiles, void* workspace,
                          size_t workspace_bytes, void* stream);
size_t attn_decode_workspace_size_split(int B, int Sq, int Sk, int Hq, int Hkv, int D, int split_tiles);

/* Size of the library's own split-KV workspace, per GPU (64 MiB). */
#define ATTN_STATIC_WORKSPACE_BYTES ((size_t)64 << 20)

/* attn_fwd_decode without a caller workspace, for callers that cannot allocate device memory: code under
 * HIP graph capture, serving loops and harnesses that forbid hipMalloc.  It calls no allocating routine;
 * the partial results go to a device array of ATTN_STATIC_WORKSPACE_BYTES that the library holds on every
 * GPU it runs on until the process ends (looked up on the first call on each device, which is the current
 * device: make it the one `stream` belongs to).  Same operation, arguments, split plan and results as
 * attn_fwd_decode (bit for bit).  Invalid arguments return attn_fwd_decode's codes (checked first); valid
 * sizes whose attn_decode_workspace_size() exceeds ATTN_STATIC_WORKSPACE_BYTES return ATTN_ERR_TOO_LARGE;
 * either way nothing is launched.  Every call on a GPU shares that GPU's array: calls on one stream are
 * ordered, but calls that overlap in time on one GPU (different streams, or threads without ordering)
 * race on it and give wrong results.  Nothing in the array has to start at zero. */
int attn_fwd_decode_static(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Sq, int Sk,
                           int Hq, int Hkv, int D, int causal, float scale, void* stream);

/* Measurement aid, not part of the attention path: the sustained dense fp16 MFMA rate of the current
 * device on random operands, in TFLOP/s, written to *tflops.  One workgroup of four waves per compute unit
 * (one wave per SIMD) issues `iters` x 16 back-to-back v_mfma_f32_32x32x16_f16 per wave on four independent
 * accumulators; one untimed launch, then one launch timed with HIP events on `stream` (NULL: the null
 * stream), whose completion the call waits for.  Under the chip's power limit this rate depends on the data
 * and on the box, and sits well below the published peak; kernel rates read against it say how much of the
 * box's matrix-core rate a kernel gets.  1 <= iters <= 10^7 (ATTN_ERR_SHAPE otherwise, nothing launched);
 * ATTN_ERR_NULL for a NULL tflops; ATTN_ERR_HIP if a HIP call fails.  Allocates no device memory (events
 * only); about 0.07 s per launch at iters = 200000 on MI355X. */
int attn_mfma_ceiling(int iters, void* stream, double* tflops);

/* attn_mfma_ceiling for a given instruction: `shape` 32 (v_mfma_f32_32x32x16_f16, what attn_mfma_ceiling
 * times) or 16 (v_mfma_f32_16x16x32_f16, 32 per iteration: the same FLOPs).  ATTN_ERR_UNSUPPORTED for
 * another shape, nothing launched; otherwise as attn_mfma_ceiling.  On random data the 16 x 16 x 32
 * instruction sustains the higher rate under the power limit. */
int attn_mfma_ceiling_shape(int shape, int iters, void* stream, double* tflops);

/* Static, NUL-terminated description of a status code ("unknown status" for others). */
const char* attn_status_string(int status);

/* Library version as major * 10000 + minor * 100 + patch. */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBATTN_ATTN_H */
