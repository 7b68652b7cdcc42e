// attn_fwd.hip -- fused grouped-query softmax attention forward for gfx950 (CDNA4).
//
// One workgroup = 8 wavefronts = two wave groups of four.  Both groups work on
// the same 128 query positions of two query heads that share one KV head, so
// each K/V tile staged in LDS feeds 2 x 128 query rows (GQA sharing).  Wave w
// of a group owns 32 query rows.
//
// The tile loop follows the load / mma / softmax sTask split of PipeThreader
// (page "PipeThreader: Software-Defined Pipelining ... (OSDI 2025)" summary,
// section "核心方法"), mapped onto gfx950 units:
//   load    : K/V tiles of 64 keys, global -> registers -> swizzled LDS, one
//             tile ahead of the compute (double-buffered LDS ring; the
//             prologue / steady state / epilogue pattern of software
//             pipelining with ping-pong buffers, page "AI编译器融合技术 -- 5.
//             并行性与分布式融合", section 5.4.2)
//   mma     : S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_f16,
//             fp16 operands and fp32 accumulation (same page, section 5.2.2:
//             map the contraction onto the matrix instruction and conform the
//             register fragments to its layout)
//   softmax : online softmax in fp32 on the VALU; the per-query max and sum
//             need one cross-lane step (v_permlane32_swap) because the S^T
//             layout keeps each query in one lane pair (same page, section
//             5.2.1: subgroup reductions by lane exchange instead of LDS)
//
// Layout facts this file relies on (checked on gfx950 with a lane probe):
//   mfma 32x32x16 f16, lane l, element i of the 8-half operands and r of the
//   16-float accumulator:  A[l%32][8*(l/32)+i],  B[8*(l/32)+i][l%32],
//   C[8*(r/4) + 4*(l/32) + r%4][l%32].
//   ds_read_b64_tr_b16: within each 16-lane group, result element j of lane i
//   is element i%4 of the 8 bytes addressed by lane 4*j + i/4 of the group.
//   v_permlane32_swap(x, y): x's upper 32 lanes trade places with y's lower 32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_kernel.h"

namespace libattn {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LDS __attribute__((address_space(3)))

constexpr int HD = 128;                 // head dim
constexpr int BM = 128;                 // query rows per wave group
constexpr int BN = 64;                  // keys per KV tile
constexpr int NTHREADS = 512;           // 8 wavefronts
constexpr int TILE = BN * HD;           // halves per K or V tile (16 KiB)
constexpr float NEG_INF = -__builtin_inff();
constexpr float M_INIT = -1e30f;        // finite start for the running max
constexpr float LN2 = 0.693147180559945309f;

// 16-byte chunk swizzles (a row of a tile is 256 B = 16 chunks).
// K is read with ds_read_b128 by 32 consecutive rows per chunk column: XOR by
// row&7 spreads each 8-lane pass over 8 distinct 16-byte bank groups.
// V is read with ds_read_b64_tr_b16 in 4-row groups covering 4 chunks: XOR by
// 4*(row&3) keeps every 16- and 32-lane pass on distinct bank groups.
__device__ __forceinline__ int swz_k(int row) { return row & 7; }
__device__ __forceinline__ int swz_v(int row) { return (row & 3) << 2; }

__device__ __forceinline__ float wave_pair_max(float x) {
  // lanes l and l^32 hold the same query: combine their partial results
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float wave_pair_sum(float x) {
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Workgroup barrier that orders LDS accesses only: global loads issued before
// it stay in flight (a full __syncthreads would wait for them).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <bool kPingPong>
__global__ __launch_bounds__(NTHREADS, 1) void attn_fwd_kernel(Params p) {
  __shared__ __attribute__((aligned(16))) _Float16 k_smem[2 * TILE];
  __shared__ __attribute__((aligned(16))) _Float16 v_smem[2 * TILE];
  LDS _Float16* const k_lds = (LDS _Float16*)k_smem;
  LDS _Float16* const v_lds = (LDS _Float16*)v_smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = wave >> 2;  // wave group: which head of the pair
  const int wq = wave & 3;    // 32-row slice of the 128 query rows
  const int n = lane & 31;    // query column of this lane in S^T / O^T
  const int hh = lane >> 5;   // lane half

  // ---- workgroup -> (batch, kv head, head pair, query tile)
  // Workgroups are dealt round-robin to the 8 XCDs; give each XCD whole
  // (batch, kv head) groups so that co-resident workgroups share K/V in that
  // XCD's L2, and within a group run the longest causal tiles first.
  const int items = p.pairs * p.n_qt;  // workgroups per (b, c) group
  const int ngroups = p.B * p.Hkv;
  int group, item;
  {
    const int bid = blockIdx.x;
    if ((ngroups & 7) == 0) {
      const int x = bid & 7, y = bid >> 3;
      group = (y / items) * 8 + x;
      item = y % items;
    } else {
      group = bid / items;
      item = bid % items;
    }
  }
  const int b = group / p.Hkv;
  const int c = group % p.Hkv;
  const int t = p.n_qt - 1 - item / p.pairs;
  const int hl = 2 * (item % p.pairs) + grp;  // head index inside the KV group
  const bool active = hl < p.g;
  const int h = c * p.g + (active ? hl : 0);

  const int S = p.S;
  const int q0 = t * BM;
  const int qw = q0 + 32 * wq;  // first query row of this wave
  const int kv_tiles_all = (S + BN - 1) / BN;
  const int n_tiles = p.causal ? min(kv_tiles_all, (q0 + BM + BN - 1) / BN) : kv_tiles_all;

  const _Float16* qb = p.q + (int64_t)b * p.q_bstride + (int64_t)h * HD;
  const _Float16* kb_ = p.k + (int64_t)b * p.kv_bstride + (int64_t)c * HD;
  const _Float16* vb_ = p.v + (int64_t)b * p.kv_bstride + (int64_t)c * HD;

  // ---- Q^T fragments (B operand of S^T = K Q^T), resident for the whole loop
  f16x8 qf[8];
  {
    const int qrow = qw + n;
    const bool ok = active && qrow < S;
    const uint32_t flip = p.neg ? 0x80008000u : 0u;
    const _Float16* src = qb + (int64_t)qrow * p.q_sstride + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      u32x4 u = {0, 0, 0, 0};
      if (ok) u = *reinterpret_cast<const u32x4*>(src + 16 * kk);
      u ^= flip;
      qf[kk] = __builtin_bit_cast(f16x8, u);
    }
  }

  // ---- K/V staging: global -> registers -> swizzled LDS.  K and V each have
  // a two-slot ring (tile t lives in slot t & 1).  Every thread moves 2 K and
  // 2 V chunks of 16 B per staging step: of the whole tile in the serial
  // schedule, of its group's half of the tile in the ping-pong schedule.
  const int st_base = kPingPong ? grp * (TILE / 16) : 0;
  const int st_lt = kPingPong ? (tid & (NTHREADS / 2 - 1)) : tid;
  const int st_stride = kPingPong ? NTHREADS / 2 : NTHREADS;
  u32x4 kreg[2], vreg[2];
  auto fetch = [&](int tk, int tv) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int x = st_base + st_lt + st_stride * u;
      const int row = x >> 4, ch = x & 15;
      const int kkey = tk * BN + row, vkey = tv * BN + row;
      kreg[u] = u32x4{0, 0, 0, 0};
      vreg[u] = u32x4{0, 0, 0, 0};
      if (tk < n_tiles && kkey < S)
        kreg[u] = *reinterpret_cast<const u32x4*>(kb_ + (int64_t)kkey * p.kv_sstride + ch * 8);
      if (tv < n_tiles && vkey < S)
        vreg[u] = *reinterpret_cast<const u32x4*>(vb_ + (int64_t)vkey * p.kv_sstride + ch * 8);
    }
  };
  auto stash = [&](int tk, int tv) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int x = st_base + st_lt + st_stride * u;
      const int row = x >> 4, ch = x & 15;
      if (tk < n_tiles)
        *(LDS u32x4*)(&k_lds[(tk & 1) * TILE + row * HD + ((ch ^ swz_k(row)) << 3)]) = kreg[u];
      if (tv < n_tiles)
        *(LDS u32x4*)(&v_lds[(tv & 1) * TILE + row * HD + ((ch ^ swz_v(row)) << 3)]) = vreg[u];
    }
  };

  f32x16 o_acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o_acc[db] = f32x16{};
  float m_run = M_INIT;  // running max of the log2-scaled scores of query n
  float l_run = 0.f;     // running sum of exp2(score - m_run)
  const float cs = p.cs;
  f32x16 s[2];           // S^T of the current tile
  f16x8 pf[4];           // P^T of the current tile (PV operand)

  // a wave skips every tile that lies wholly above its causal diagonal
  auto skip = [&](int j) { return !active || (p.causal && j * BN > qw + 31); };

  // ---- mma sTask 1: S^T[key][query] for the 64 keys of tile j, two 32-key blocks
  auto mma_qk = [&](int j) {
    const LDS _Float16* ks = k_lds + (j & 1) * TILE;
    s[0] = f32x16{};
    s[1] = f32x16{};
    // the two 32-key blocks are independent accumulator chains: interleave them
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int ch = 2 * kk + hh;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        const int row = 32 * sb + n;
        const f16x8 kf = *(const LDS f16x8*)(&ks[row * HD + ((ch ^ swz_k(row)) << 3)]);
        s[sb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[kk], s[sb], 0, 0, 0);
      }
    }
  };

  // ---- softmax sTask: online softmax of tile j in the log2 domain
  auto softmax = [&](int j) {
    const int kj = j * BN;
    const bool need_mask = (p.causal && kj + BN - 1 > qw) || (kj + BN > S);
    const int query = qw + n;
    uint32_t keep = 0xffffffffu;  // bit (16*sb + r): key allowed
    if (need_mask) {
      keep = 0;
#pragma unroll
      for (int sb = 0; sb < 2; ++sb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kj + 32 * sb + 8 * (r >> 2) + 4 * hh + (r & 3);
          const bool ok = key < S && (!p.causal || key <= query);
          keep |= (ok ? 1u : 0u) << (16 * sb + r);
        }
    }
    float mt = NEG_INF;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float x = ((keep >> (16 * sb + r)) & 1u) ? s[sb][r] : NEG_INF;
        mt = fmaxf(mt, x);
      }
    mt = wave_pair_max(mt);
    const float mts = (mt == NEG_INF) ? NEG_INF : mt * cs;
    const float m_new = fmaxf(m_run, mts);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;

    float rs = 0.f;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][r], cs, -m_new));
        e = ((keep >> (16 * sb + r)) & 1u) ? e : 0.f;
        rs += e;
        pf[2 * sb + (r >> 3)][r & 7] = (_Float16)e;
      }
    rs = wave_pair_sum(rs);
    l_run = l_run * alpha + rs;
#pragma unroll
    for (int db = 0; db < 4; ++db) o_acc[db] *= alpha;
  };

  // ---- mma sTask 2: O^T[d][query] += V^T[d][key] P^T[key][query] for tile j
  auto mma_pv = [&](int j) {
    const LDS _Float16* vs = v_lds + (j & 1) * TILE;
    const int G = lane >> 4, sl = lane & 15;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int row1 = 16 * kk + 4 * (G >> 1) + (sl >> 2);
      const int row2 = row1 + 8;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int ch = 4 * db + 2 * (G & 1) + ((sl & 3) >> 1);
        const int within = (sl & 1) << 2;
        const i16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (LDS i16x4*)&vs[row1 * HD + ((ch ^ swz_v(row1)) << 3) + within]);
        const i16x4 a2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (LDS i16x4*)&vs[row2 * HD + ((ch ^ swz_v(row2)) << 3) + within]);
        const f16x4 h1 = __builtin_bit_cast(f16x4, a1);
        const f16x4 h2 = __builtin_bit_cast(f16x4, a2);
        const f16x8 vf = {h1[0], h1[1], h1[2], h1[3], h2[0], h2[1], h2[2], h2[3]};
        o_acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[kk], o_acc[db], 0, 0, 0);
      }
    }
  };

  if constexpr (!kPingPong) {
    // ---- serial schedule: every wave runs load-next / QK / softmax / PV per tile
    fetch(0, 0);
    stash(0, 0);
    lds_barrier();
    for (int j = 0; j < n_tiles; ++j) {
      fetch(j + 1, j + 1);
      if (!skip(j)) {
        mma_qk(j);
        softmax(j);
        mma_pv(j);
      }
      stash(j + 1, j + 1);
      lds_barrier();
    }
  } else {
    // ---- ping-pong schedule.  Time is cut into half-steps by workgroup
    // barriers.  Each wave alternates an mma block (PV of tile j-1, then QK
    // of tile j) and a softmax block (tile j); group 1 runs one half-step
    // behind group 0, so on every SIMD one wave keeps the matrix core busy
    // while the other runs softmax on the VALU.  Group 0 stages its half of
    // (K_{j+1}, V_j) during its softmax block j, group 1 its half of
    // (K_{j+2}, V_{j+1}) during its softmax block j; every slot is rewritten
    // only after both groups have read it.
    fetch(0, n_tiles);
    stash(0, n_tiles);
    if (grp == 1) fetch(1, 0);
    lds_barrier();
    for (int hs = 0; hs < 2 * n_tiles + 2; ++hs) {
      const int ph = hs - grp;
      if (ph == -1) {
        stash(1, 0);
      } else if (ph <= 2 * n_tiles) {
        const int j = ph >> 1;
        if ((ph & 1) == 0) {
          fetch(j + 1 + grp, j + grp);
          __builtin_amdgcn_s_setprio(1);
          if (j >= 1 && !skip(j - 1)) mma_pv(j - 1);
          if (j < n_tiles && !skip(j)) mma_qk(j);
          __builtin_amdgcn_s_setprio(0);
        } else {
          if (!skip(j)) softmax(j);
          stash(j + 1 + grp, j + grp);
        }
      }
      lds_barrier();
    }
  }

  // ---- epilogue: O = O^T / l (fp16, round to nearest even), LSE in natural log
  if (active) {
    const int qrow = qw + n;
    if (qrow < S) {
      const float inv = 1.0f / l_run;
      _Float16* dst = p.o + (int64_t)b * p.q_bstride + (int64_t)qrow * p.q_sstride + (int64_t)h * HD;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          f16x4 hv;
#pragma unroll
          for (int e = 0; e < 4; ++e) hv[e] = (_Float16)(o_acc[db][4 * r4 + e] * inv);
          *reinterpret_cast<f16x4*>(dst + 32 * db + 8 * r4 + 4 * hh) = hv;
        }
      if (p.lse && hh == 0)
        p.lse[((int64_t)b * p.Hq + h) * S + qrow] = (m_run + log2f(l_run)) * LN2;
    }
  }
}

int64_t grid_blocks(const Params& p) {
  const int64_t nb = (int64_t)p.B * p.Hkv * p.pairs * p.n_qt;
  return nb > 0x7fffffff ? -1 : nb;
}

hipError_t launch_attn_fwd(const Params& p, hipStream_t stream) {
  const int64_t nb = grid_blocks(p);
  if (nb <= 0) return hipErrorInvalidValue;
  if (p.schedule == SCHEDULE_SERIAL)
    hipLaunchKernelGGL(attn_fwd_kernel<false>, dim3((unsigned)nb), dim3(NTHREADS), 0, stream, p);
  else
    hipLaunchKernelGGL(attn_fwd_kernel<true>, dim3((unsigned)nb), dim3(NTHREADS), 0, stream, p);
  return hipGetLastError();
}

}  // namespace libattn
