// attn_static_ws.hip -- the split-KV attention path with a workspace the
// library owns, for callers that cannot allocate device memory (code under
// HIP graph capture, serving loops that must not call hipMalloc).
//
// The workspace is a file-scope device array: every GPU the library runs on
// gets its own copy when the code object is loaded there, and keeps it until
// the process ends.  Host code never passes the array's name to a kernel (on
// the host that name is only a stand-in for the symbol); it looks the
// device address up once per device with hipGetSymbolAddress and passes that.
#include <hip/hip_runtime.h>

#include <mutex>

#include "attn.h"

namespace {

constexpr size_t kStaticWsBytes = ATTN_STATIC_WORKSPACE_BYTES;
static_assert(kStaticWsBytes % 256 == 0, "the static workspace is a whole number of 256-byte blocks");

// Partial O and LSE of the split-KV kernels (fp32), as in attn_fwd_decode's
// caller-owned workspace.  Its contents on entry do not matter: the split
// kernel writes every element the combine kernel reads.
static __device__ __align__(256) float scratch[kStaticWsBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];  // device address of `scratch` per device, nullptr until looked up

// The device address of the current device's copy of `scratch`, looked up on
// the first call on that device.  Returns ATTN_OK or ATTN_ERR_HIP.
int device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return ATTN_ERR_HIP;
    g_ptr[dev] = ptr;
  }
  *out = g_ptr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" int attn_fwd_decode_static(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                                      int Sq, int Sk, int Hq, int Hkv, int D, int causal, float scale, void* stream) {
  // The split-KV path's own argument checks, without a workspace: any status
  // but ATTN_ERR_WORKSPACE is an invalid argument (nothing is launched).
  const int checked = attn_fwd_decode(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, D, causal, scale, nullptr, 0, stream);
  if (checked != ATTN_ERR_WORKSPACE) return checked;
  if (attn_decode_workspace_size(B, Sq, Sk, Hq, Hkv, D) > kStaticWsBytes) return ATTN_ERR_TOO_LARGE;
  void* ws = nullptr;
  const int st = device_scratch(&ws);
  if (st != ATTN_OK) return st;
  return attn_fwd_decode(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, D, causal, scale, ws, kStaticWsBytes, stream);
}
