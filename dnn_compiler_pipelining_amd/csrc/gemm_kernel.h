// gemm_kernel.h -- host/device interface of the fp16 GEMM kernel (gemm_fwd.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace libattn {

struct GemmParams {
  const _Float16* a;  // [M][K]
  const _Float16* b;  // [K][N] (b_layout 0) or [N][K] (b_layout 1)
  _Float16* c;        // [M][N]
  int M, N, K;        // K >= 1, K % 8 == 0, N % 8 == 0
  int b_layout;
  int ntm, ntn;       // 256 x 256 output tiles along M and N
  int nkt;            // 64-deep K tiles
  int waves;          // waves per workgroup: 8 (two per SIMD) or 4 (one per SIMD)
};

// Enqueue C = A B (or A B^T) for K >= 1.  Returns the hipError_t of the launch.
hipError_t launch_gemm(const GemmParams& p, hipStream_t stream);
// Enqueue C = 0 for K == 0 (M * N fp16 elements, M * N a multiple of 8).
hipError_t launch_gemm_zero(_Float16* c, int64_t elems, hipStream_t stream);

}  // namespace libattn
