// attn_api.cpp -- the extern "C" boundary of libattn (declared in include/attn.h).
//
// Validation runs before any HIP call, so every error path is reachable
// without a GPU.  Valid calls enqueue their kernels and return.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "attn.h"
#include "attn_kernel.h"

namespace {

constexpr int kVersion = 2 * 10000 + 0 * 100 + 0;
constexpr int kMaxSeq = 1 << 30;  // sequence lengths up to 2^30 keep all tile arithmetic in int

// Fields of a requested variant: -1 takes the tuned value (variant.h) for the
// nearest measured shape.  The library reads no environment and keeps no
// state: attn_fwd_variant passes a request explicitly (the schedule search
// and the tests use it), every other entry point asks for the tuned variant.
struct Request {
  int schedule, ring, xcd, lpt, place, bn, hpw;
};
constexpr Request kTunedRequest = {-1, -1, -1, -1, -1, -1, -1};

// The variant a call runs, or false if the request names a value that does
// not exist or a schedule the head dimension does not run.  D = 128 runs
// every schedule; D = 64 the serial ones (SERIAL4 unless SERIAL is asked for:
// its one-head workgroups, 142 VGPRs and 34 KiB of LDS, fit three to a CU,
// where SERIAL's eight-wave workgroups fit one; measured on MI355X at B=16
// S=8192 Hq=32 Hkv=8: 878 against 822 TFLOP/s); D = 256 SERIAL4 only.  Tiles
// of 32 or 128 keys: SERIAL and SERIAL4 at D = 128 (a tuned tile size other
// than 64 is dropped when the schedule or D does not have it).
bool choose_variant(const Request& r, int B, int Sq, int Sk, int Hq, int Hkv, int D, libattn::Variant& v) {
  v = libattn::tuned_variant(B, Sq, Sk, Hq, Hkv);
  if (D == 64) v.schedule = libattn::SCHEDULE_SERIAL4;
  if (D == 256) v.schedule = libattn::SCHEDULE_SERIAL4;
  if (r.schedule >= 0) v.schedule = r.schedule;
  if (r.ring >= 0) v.ring = r.ring;
  if (r.xcd >= 0) v.xcd = r.xcd;
  if (r.lpt >= 0) v.lpt = r.lpt;
  if (v.schedule != libattn::SCHEDULE_WIDE && v.schedule != libattn::SCHEDULE_OVERLAP)
    v.place = libattn::PLACE_EVEN;  // the only placement they have
  if (r.place >= 0) v.place = r.place;
  if (D != 128 || (v.schedule != libattn::SCHEDULE_SERIAL && v.schedule != libattn::SCHEDULE_SERIAL4))
    v.bn = libattn::BN_STD;
  if (r.bn >= 0) v.bn = r.bn;
  if (v.schedule != libattn::SCHEDULE_WIDE) v.hpw = 0;  // heads per workgroup: the 64-row schedule's
  if (r.hpw >= 0) v.hpw = r.hpw;
  if (!libattn::variant_valid(v)) return false;
  if (v.bn != libattn::BN_STD && D != 128) return false;
  if (D == 64) return v.schedule == libattn::SCHEDULE_SERIAL || v.schedule == libattn::SCHEDULE_SERIAL4;
  if (D == 256) return v.schedule == libattn::SCHEDULE_SERIAL4;
  return true;  // D = 128 runs every schedule
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

bool overlaps(const void* a, uint64_t a_bytes, const void* b, uint64_t b_bytes) {
  if (!a || !b || a_bytes == 0 || b_bytes == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + b_bytes && b0 < a0 + a_bytes;
}

int validate(const void* q, const void* k, const void* v, const void* o, const float* lse, int B, int Sq, int Sk,
             int Hq, int Hkv, int D, int causal, float scale) {
  if (!q || !k || !v || !o) return ATTN_ERR_NULL;
  if (B < 1 || Sq < 1 || Sk < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_ERR_SHAPE;
  if (Sq > kMaxSeq || Sk > kMaxSeq) return ATTN_ERR_SHAPE;
  if (causal != 0 && causal != 1) return ATTN_ERR_SHAPE;
  if (causal && Sq > Sk) return ATTN_ERR_SHAPE;
  if (!std::isfinite(scale)) return ATTN_ERR_SHAPE;
  if (D != 64 && D != 128 && D != 256) return ATTN_ERR_UNSUPPORTED;
  if ((int64_t)Hkv * D * 2 * 64 > 0xffffffffLL) return ATTN_ERR_UNSUPPORTED;  // 64 K/V rows must span < 4 GiB
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (lse && !aligned16(lse)))
    return ATTN_ERR_ALIGN;
  const uint64_t q_bytes = (uint64_t)B * Sq * Hq * D * 2;
  const uint64_t kv_bytes = (uint64_t)B * Sk * Hkv * D * 2;
  const uint64_t lse_bytes = (uint64_t)B * Hq * Sq * 4;
  if (overlaps(o, q_bytes, q, q_bytes) || overlaps(o, q_bytes, k, kv_bytes) || overlaps(o, q_bytes, v, kv_bytes) ||
      overlaps(o, q_bytes, lse, lse_bytes) || overlaps(lse, lse_bytes, q, q_bytes) ||
      overlaps(lse, lse_bytes, k, kv_bytes) || overlaps(lse, lse_bytes, v, kv_bytes))
    return ATTN_ERR_OVERLAP;
  return ATTN_OK;
}

libattn::Params base_params(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Sq, int Sk,
                            int Hq, int Hkv, int D, int causal, float scale) {
  libattn::Params p = {};
  p.q = static_cast<const _Float16*>(q);
  p.k = static_cast<const _Float16*>(k);
  p.v = static_cast<const _Float16*>(v);
  p.o = static_cast<_Float16*>(o);
  p.lse = lse;
  p.q_sstride = (int64_t)Hq * D;
  p.q_bstride = (int64_t)Sq * p.q_sstride;
  p.kv_sstride = (int64_t)Hkv * D;
  p.kv_bstride = (int64_t)Sk * p.kv_sstride;
  p.B = B;
  p.Sq = Sq;
  p.Sk = Sk;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.off = causal ? Sk - Sq : 0;
  p.g = Hq / Hkv;
  p.causal = causal;
  p.neg = scale < 0.f ? 1 : 0;
  p.cs = std::fabs(scale) * 1.44269504088896340736f;
  p.hd = D;
  p.bn = libattn::BN_STD;
  return p;
}

// Split-KV plan: the packed (head, query row) rows of a KV group in 128-row
// tiles, and the keys cut into splits of whole 64-key tiles so that the grid
// has about kDecodeTarget workgroups: one round of two per CU on 256 CUs.
// Measured on MI355X, fewer and longer splits stream K/V faster than more and
// shorter ones (each workgroup pays its Q load and first-tile latency once).
constexpr int64_t kDecodeTarget = 512;
struct DecodePlan {
  int n_pt, n_splits, split_tiles;
  int64_t ws_o_floats, ws_lse_floats;
};
DecodePlan decode_plan(int B, int Sq, int Sk, int Hq, int Hkv, int D, int split_tiles) {
  DecodePlan d;
  const int64_t g = Hq / Hkv;
  d.n_pt = (int)((g * Sq + 127) / 128);
  const int64_t tiles = ((int64_t)Sk + 63) / 64;
  const int64_t base = (int64_t)B * Hkv * d.n_pt;
  int64_t want = (kDecodeTarget + base - 1) / base;
  want = want < 1 ? 1 : (want > tiles ? tiles : want);
  d.split_tiles = (int)((tiles + want - 1) / want);
  // an explicit split length (attn_fwd_decode_split), for tuning and tests
  if (split_tiles > 0) d.split_tiles = (int)(split_tiles < tiles ? split_tiles : tiles);
  d.n_splits = (int)((tiles + d.split_tiles - 1) / d.split_tiles);
  const int64_t rows = (int64_t)B * Hq * Sq;
  d.ws_lse_floats = rows * d.n_splits;
  d.ws_o_floats = d.ws_lse_floats * D;
  return d;
}

// The forward pass with a variant request (attn_fwd_ex and attn_fwd_variant).
int forward(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Sq, int Sk, int Hq, int Hkv,
            int D, int causal, float scale, const Request& req, void* stream) {
  const int st = validate(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, D, causal, scale);
  if (st != ATTN_OK) return st;
  libattn::Variant var;
  if (!choose_variant(req, B, Sq, Sk, Hq, Hkv, D, var)) return ATTN_ERR_UNSUPPORTED;

  libattn::Params p = base_params(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, D, causal, scale);
  p.schedule = var.schedule;
  p.ring = var.ring;
  p.xcd = var.xcd;
  p.lpt = var.lpt;
  p.place = var.place;
  p.bn = var.bn;
  hipError_t e;
  if (p.schedule == libattn::SCHEDULE_WIDE) {
    // four heads of a KV group per workgroup at 64 query rows, or two at 128,
    // or one at 256: as the variant names it, else the largest that divides
    // the GQA ratio (with one that does not, the waves past the last head of
    // a KV group compute nothing that is stored)
    p.hpw = var.hpw ? var.hpw : p.g % 4 == 0 ? 4 : p.g % 2 == 0 ? 2 : 1;
    p.pairs = (p.g + p.hpw - 1) / p.hpw;
    const int rows = 256 / p.hpw;
    p.n_qt = (Sq + rows - 1) / rows;
    if (libattn::grid_blocks_wide(p) < 0) return ATTN_ERR_SHAPE;
    e = libattn::launch_attn_wide(p, static_cast<hipStream_t>(stream));
  } else if (p.schedule == libattn::SCHEDULE_SERIAL4_16) {
    p.n_qt = (Sq + 127) / 128;
    p.pairs = p.g;  // one query head per workgroup
    if (libattn::grid_blocks_s16(p) < 0) return ATTN_ERR_SHAPE;
    e = libattn::launch_attn_s16(p, static_cast<hipStream_t>(stream));
  } else {
    p.n_qt = (Sq + 127) / 128;
    // query heads per workgroup: a pair (two wave groups), or one for SERIAL4
    p.pairs = p.schedule == libattn::SCHEDULE_SERIAL4 ? p.g : (p.g + 1) / 2;
    if (libattn::grid_blocks(p) < 0) return ATTN_ERR_SHAPE;
    e = libattn::launch_attn_fwd(p, static_cast<hipStream_t>(stream));
  }
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // namespace

extern "C" {

int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Sq, int Sk, int Hq,
                int Hkv, int D, int causal, float scale, void* stream) {
  return forward(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, D, causal, scale, kTunedRequest, stream);
}

int attn_fwd_variant(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Sq, int Sk, int Hq,
                     int Hkv, int D, int causal, float scale, int schedule, int ring, int xcd, int lpt, int place,
                     int bn, int hpw, void* stream) {
  return forward(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, D, causal, scale,
                 Request{schedule, ring, xcd, lpt, place, bn, hpw}, stream);
}

int attn_fwd_stream(const void* q, const void* k, const void* v, void* o, float* lse, int B, int S, int Hq, int Hkv,
                    int D, int causal, float scale, void* stream) {
  return attn_fwd_ex(q, k, v, o, lse, B, S, S, Hq, Hkv, D, causal, scale, stream);
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int S, int Hq, int Hkv, int D,
             int causal, float scale) {
  return attn_fwd_stream(q, k, v, o, lse, B, S, Hq, Hkv, D, causal, scale, nullptr);
}

int attn_tuned_variant(int B, int Sq, int Sk, int Hq, int Hkv, int D, int* schedule, int* ring, int* xcd, int* lpt,
                       int* place, int* bn, int* hpw) {
  if (!schedule || !ring || !xcd || !lpt || !place || !bn || !hpw) return ATTN_ERR_NULL;
  if (B < 1 || Sq < 1 || Sk < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || Sq > kMaxSeq || Sk > kMaxSeq)
    return ATTN_ERR_SHAPE;
  if (D != 64 && D != 128 && D != 256) return ATTN_ERR_UNSUPPORTED;
  libattn::Variant var;
  if (!choose_variant(kTunedRequest, B, Sq, Sk, Hq, Hkv, D, var)) return ATTN_ERR_UNSUPPORTED;
  *schedule = var.schedule;
  *ring = var.ring;
  *xcd = var.xcd;
  *lpt = var.lpt;
  *place = var.place;
  *bn = var.bn;
  *hpw = var.hpw;
  return ATTN_OK;
}

int attn_device_clock(int device, int* compute_units, int* peak_clock_khz) {
  if (!compute_units || !peak_clock_khz) return ATTN_ERR_NULL;
  if (hipDeviceGetAttribute(compute_units, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
      hipDeviceGetAttribute(peak_clock_khz, hipDeviceAttributeClockRate, device) != hipSuccess)
    return ATTN_ERR_HIP;
  return ATTN_OK;
}

size_t attn_decode_workspace_size_split(int B, int Sq, int Sk, int Hq, int Hkv, int D, int split_tiles) {
  if (B < 1 || Sq < 1 || Sk < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || Sq > kMaxSeq || Sk > kMaxSeq) return 0;
  if (D != 64 && D != 128 && D != 256) return 0;
  if ((int64_t)(Hq / Hkv) * Sq > kMaxSeq) return 0;
  const DecodePlan d = decode_plan(B, Sq, Sk, Hq, Hkv, D, split_tiles);
  return (size_t)(d.ws_o_floats + d.ws_lse_floats) * sizeof(float);
}

size_t attn_decode_workspace_size(int B, int Sq, int Sk, int Hq, int Hkv, int D) {
  return attn_decode_workspace_size_split(B, Sq, Sk, Hq, Hkv, D, 0);
}

int attn_fwd_decode_split(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Sq, int Sk,
                          int Hq, int Hkv, int D, int causal, float scale, int split_tiles, void* workspace,
                          size_t workspace_bytes, void* stream) {
  const int st = validate(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, D, causal, scale);
  if (st != ATTN_OK) return st;
  if ((int64_t)(Hq / Hkv) * Sq > kMaxSeq) return ATTN_ERR_SHAPE;  // packed rows of a KV group stay below 2^30
  const DecodePlan d = decode_plan(B, Sq, Sk, Hq, Hkv, D, split_tiles);
  const size_t need = (size_t)(d.ws_o_floats + d.ws_lse_floats) * sizeof(float);
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return ATTN_ERR_WORKSPACE;
  const uint64_t q_bytes = (uint64_t)B * Sq * Hq * D * 2, kv_bytes = (uint64_t)B * Sk * Hkv * D * 2;
  const uint64_t lse_bytes = (uint64_t)B * Hq * Sq * 4;
  if (overlaps(workspace, need, q, q_bytes) || overlaps(workspace, need, k, kv_bytes) ||
      overlaps(workspace, need, v, kv_bytes) || overlaps(workspace, need, o, q_bytes) ||
      overlaps(workspace, need, lse, lse_bytes))
    return ATTN_ERR_OVERLAP;

  libattn::Params p = base_params(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, D, causal, scale);
  const libattn::Variant var = libattn::tuned_variant(B, Sq, Sk, Hq, Hkv);
  p.schedule = libattn::SCHEDULE_SERIAL4;
  p.ring = var.ring;
  p.xcd = var.xcd;
  p.lpt = 0;
  p.pairs = 1;
  p.n_qt = d.n_pt;
  p.n_splits = d.n_splits;
  p.split_tiles = d.split_tiles;
  p.ws_o = static_cast<float*>(workspace);
  p.ws_lse = p.ws_o + d.ws_o_floats;
  if (libattn::grid_blocks_decode(p) < 0) return ATTN_ERR_SHAPE;
  const hipError_t e = libattn::launch_attn_decode(p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Sq, int Sk, int Hq,
                    int Hkv, int D, int causal, float scale, void* workspace, size_t workspace_bytes, void* stream) {
  return attn_fwd_decode_split(q, k, v, o, lse, B, Sq, Sk, Hq, Hkv, D, causal, scale, 0, workspace, workspace_bytes,
                               stream);
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "invalid shape, layout, causal flag or scale";
    case ATTN_ERR_UNSUPPORTED:
      return "unsupported size: attention needs D of 64, 128 or 256 and K/V heads under 4 GiB per 64 rows, "
             "the GEMM K and N multiples of 8";
    case ATTN_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case ATTN_ERR_HIP: return "HIP launch error";
    case ATTN_ERR_OVERLAP: return "an output or the workspace overlaps an input or another output";
    case ATTN_ERR_WORKSPACE: return "workspace missing, too small or not 16-byte aligned";
    case ATTN_ERR_TOO_LARGE: return "the sizes need more workspace than the library's static array holds";
    default: return "unknown status";
  }
}

int attn_version(void) { return kVersion; }

}  // extern "C"
