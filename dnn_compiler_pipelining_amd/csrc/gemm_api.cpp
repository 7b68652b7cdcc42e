// gemm_api.cpp -- the extern "C" fp16 GEMM entry point of libattn (declared in include/gemm.h).
//
// Validation runs before any HIP call, so every error path is reachable
// without a GPU.  Valid calls enqueue exactly one kernel and return.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "gemm.h"
#include "gemm_kernel.h"

namespace {

constexpr int kMaxMN = 1 << 24;  // M, N <= 2^24 and K <= 2^22 keep every
constexpr int kMaxK = 1 << 22;   // per-tile load offset below 2^32
constexpr int kDefaultWaves = 8;

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

bool overlaps(const void* a, uint64_t a_bytes, const void* b, uint64_t b_bytes) {
  if (!a || !b || a_bytes == 0 || b_bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + b_bytes && b0 < a0 + a_bytes;
}

int validate(const void* a, const void* b, const void* c, int M, int N, int K, int b_layout) {
  const bool empty = M == 0 || N == 0;
  if (!empty && (!a || !b || !c)) return ATTN_ERR_NULL;
  if (M < 0 || N < 0 || K < 0 || M > kMaxMN || N > kMaxMN || K > kMaxK) return ATTN_ERR_SHAPE;
  if (b_layout != GEMM_B_KN && b_layout != GEMM_B_NK) return ATTN_ERR_SHAPE;
  if (empty) return ATTN_OK;
  if ((K & 7) != 0 || (N & 7) != 0) return ATTN_ERR_UNSUPPORTED;
  if (!aligned16(a) || !aligned16(b) || !aligned16(c)) return ATTN_ERR_ALIGN;
  const uint64_t a_bytes = (uint64_t)M * K * 2, b_bytes = (uint64_t)K * N * 2, c_bytes = (uint64_t)M * N * 2;
  if (overlaps(c, c_bytes, a, a_bytes) || overlaps(c, c_bytes, b, b_bytes)) return ATTN_ERR_OVERLAP;
  return ATTN_OK;
}

}  // namespace

extern "C" {

int gemm_f16_waves(const void* a, const void* b, void* c, int M, int N, int K, int b_layout, int waves,
                   void* stream) {
  const int st = validate(a, b, c, M, N, K, b_layout);
  if (st != ATTN_OK) return st;
  if (waves != 0 && waves != 4 && waves != 8) return ATTN_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return ATTN_OK;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (K == 0) {  // the empty sum: C = 0
    const hipError_t e = libattn::launch_gemm_zero(static_cast<_Float16*>(c), (int64_t)M * N, s);
    return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
  }
  libattn::GemmParams p;
  p.a = static_cast<const _Float16*>(a);
  p.b = static_cast<const _Float16*>(b);
  p.c = static_cast<_Float16*>(c);
  p.M = M;
  p.N = N;
  p.K = K;
  p.b_layout = b_layout;
  p.ntm = (M + 255) / 256;
  p.ntn = (N + 255) / 256;
  p.nkt = (K + 63) / 64;
  p.waves = waves == 0 ? kDefaultWaves : waves;
  if ((int64_t)p.ntm * p.ntn > 0x7fffffff) return ATTN_ERR_SHAPE;
  const hipError_t e = libattn::launch_gemm(p, s);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int gemm_f16(const void* a, const void* b, void* c, int M, int N, int K, int b_layout, void* stream) {
  return gemm_f16_waves(a, b, c, M, N, K, b_layout, 0, stream);
}

}  // extern "C"
