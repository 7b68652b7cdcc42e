// mfma_ceiling.hip -- a measurement aid beside the attention path: the rate
// the dense fp16 matrix cores of the current device sustain on random
// operands (one workgroup of four waves per CU, one wave per SIMD, each wave
// issuing back-to-back v_mfma_f32_32x32x16_f16 on four independent
// accumulators, or v_mfma_f32_16x16x32_f16 on four, the same FLOPs per
// iteration).  Under the chip's power limit that rate depends on the
// operand data and differs from box to box; an attention or GEMM rate read
// against it says how much of what the box can deliver the kernel gets,
// where the published peak says how much of the data sheet.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "attn.h"
#include "gfx950.h"

namespace {

constexpr int kMaxBlocks = 1024;
constexpr int kMfmaPerIter = 16;
constexpr double kFlopPerMfma = 2.0 * 32 * 32 * 16;

__device__ float hash_unit(uint32_t x) {  // a value in [-0.5, 0.5) from a 32-bit integer hash
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return (float)(x & 0xffff) / 65536.0f - 0.5f;
}

template <int kShape>
__global__ __launch_bounds__(256, 1) void mfma_ceiling_kernel(int iters) {
  const uint32_t tid = blockIdx.x * 256u + threadIdx.x;
  libattn::f16x8 a[4], b[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[j][i] = (_Float16)hash_unit(tid * 64u + 8u * j + i);
      b[j][i] = (_Float16)hash_unit(tid * 64u + 32u + 8u * j + i);
    }
  using Acc = std::conditional_t<kShape == 32, libattn::f32x16, libattn::f32x4>;
  constexpr int kPerIter = kShape == 32 ? kMfmaPerIter : 2 * kMfmaPerIter;  // equal FLOPs per iteration
  Acc c[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < kPerIter; ++m) {
      if constexpr (kShape == 32)
        c[m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[m & 3], b[(m >> 2) & 3], c[m & 3], 0, 0, 0);
      else
        c[m & 3] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[m & 3], b[(m >> 2) & 3], c[m & 3], 0, 0, 0);
    }
  }
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < (kShape == 32 ? 16 : 4); ++e) r += c[i][e];
  // the sum is consumed by an (empty) assembly statement, so no MFMA can be
  // dropped as unused; nothing is written to memory
  asm volatile("" ::"v"(r));
}

}  // namespace

extern "C" int attn_mfma_ceiling_shape(int shape, int iters, void* stream, double* tflops) {
  if (!tflops) return ATTN_ERR_NULL;
  if (iters < 1 || iters > 10000000) return ATTN_ERR_SHAPE;
  if (shape != 32 && shape != 16) return ATTN_ERR_UNSUPPORTED;
  auto kernel = shape == 32 ? mfma_ceiling_kernel<32> : mfma_ceiling_kernel<16>;
  int dev = -1, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return ATTN_ERR_HIP;
  const int blocks = cus < kMaxBlocks ? cus : kMaxBlocks;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess) return ATTN_ERR_HIP;
  if (hipEventCreate(&e1) != hipSuccess) {
    (void)hipEventDestroy(e0);
    return ATTN_ERR_HIP;
  }
  int st = ATTN_OK;
  // one untimed launch brings the clock to the level the timed one runs at
  hipLaunchKernelGGL(kernel, dim3(blocks), dim3(256), 0, s, iters);
  float ms = 0.f;
  if (hipGetLastError() != hipSuccess || hipEventRecord(e0, s) != hipSuccess) {
    st = ATTN_ERR_HIP;
  } else {
    hipLaunchKernelGGL(kernel, dim3(blocks), dim3(256), 0, s, iters);
    if (hipGetLastError() != hipSuccess || hipEventRecord(e1, s) != hipSuccess ||
        hipEventSynchronize(e1) != hipSuccess || hipEventElapsedTime(&ms, e0, e1) != hipSuccess || ms <= 0.f)
      st = ATTN_ERR_HIP;
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (st != ATTN_OK) return st;
  *tflops = kFlopPerMfma * kMfmaPerIter * 4.0 * blocks * (double)iters / (ms * 1e-3) / 1e12;
  return ATTN_OK;
}

extern "C" int attn_mfma_ceiling(int iters, void* stream, double* tflops) {
  return attn_mfma_ceiling_shape(32, iters, stream, tflops);
}
