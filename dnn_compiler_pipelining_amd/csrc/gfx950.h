// gfx950.h -- device helpers shared by the attention and GEMM kernels.
//
// Layout facts these kernels rely on (checked on gfx950 with a lane probe):
//   mfma 32x32x16 f16, lane l, element i of the 8-half operands and r of the
//   16-float accumulator:  A[l%32][8*(l/32)+i],  B[8*(l/32)+i][l%32],
//   C[8*(r/4) + 4*(l/32) + r%4][l%32].
//   ds_read_b64_tr_b16: within each 16-lane group, result element j of lane i
//   is element i%4 of the 8 bytes addressed by lane 4*j + i/4 of the group.
//   global_load_lds_dwordx4: lane l writes its 16 bytes at LDS M0 + 16*l.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace libattn {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LDS __attribute__((address_space(3)))
// Lambdas of a kernel body are always inlined: an outlined lambda would pass
// its register arrays through scratch memory.
#define INL __attribute__((always_inline))

// Workgroup barrier that orders LDS accesses only: global loads issued before
// it stay in flight (a full __syncthreads would wait for them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One direct global -> LDS load of 16 B per lane: lane l writes LDS byte
// address lds_base + 16*l with the 16 bytes at base + off.  Issued as inline
// assembly so the compiler does not add conservative waits before unrelated
// LDS reads; the caller waits with dma_wait() before the barrier that
// publishes the tile.  M0 is restored afterwards.  An LDS DMA that reads M0
// needs one wait state after the scalar write of M0 (the compiler's hazard
// pass does not look inside inline assembly), hence the s_nop.
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(off), "s"(base), "s"(lds_base)
      : "memory");
}
// dma16 without saving M0: the assembly declares M0 clobbered, so the
// compiler keeps nothing of its own there across it.  Two instructions fewer
// per load, for kernels that issue loads back to back.
__device__ __forceinline__ void dma16_m0(const void* base, uint32_t off, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(off), "s"(base), "s"(lds_base)
      : "memory", "m0");
}
// dma16_m0 with the LDS address given as a wave-uniform base plus a
// compile-time byte offset, added straight into M0 (one scalar instruction
// per load instead of two).  The base is read from the first lane, so that
// it is a scalar operand even where the compiler cannot prove it uniform.
template <uint32_t kOff>
__device__ __forceinline__ void dma16_m0_plus(const void* base, uint32_t off, uint32_t lds_base) {
  asm volatile(
      "s_add_u32 m0, %2, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(off), "s"(base), "s"(__builtin_amdgcn_readfirstlane(lds_base)), "n"(kOff)
      : "memory", "m0", "scc");
}
// dma16_m0 for the lanes in `lanes` only (EXEC is set for the one load and
// restored): lane l of them still writes LDS byte lds_base + 16*l, so waves
// that pass disjoint lane sets with the same lds_base fill one 1 KiB run
// together, each with one instruction.
__device__ __forceinline__ void dma16_m0_lanes(const void* base, uint32_t off, uint32_t lds_base, uint64_t lanes) {
  uint64_t saved;
  asm volatile(
      "s_mov_b64 %0, exec\n\t"
      "s_mov_b64 exec, %4\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b64 exec, %0"
      : "=&s"(saved)
      : "v"(off), "s"(base), "s"(lds_base), "s"(lanes)
      : "memory", "m0");
}
__device__ __forceinline__ void dma_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0..N-1.
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

}  // namespace libattn
