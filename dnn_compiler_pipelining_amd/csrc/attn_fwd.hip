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
//   load    : K/V tiles of 64 keys, global -> registers -> padded LDS rows,
//             staged ahead of the compute in two-slot rings (the prologue /
//             steady state / epilogue pattern of software pipelining with
//             ping-pong buffers, page "AI编译器融合技术 -- 5. 并行性与分布式融合",
//             section 5.4.2)
//   mma     : S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_f16,
//             fp16 operands and fp32 accumulation (same page, section 5.2.2:
//             map the contraction onto the matrix instruction and conform the
//             register fragments to its layout)
//   softmax : online softmax in fp32 on the VALU; the per-query max and sum
//             need one cross-lane step (v_permlane32_swap) because the S^T
//             layout keeps each query in one lane pair (same page, section
//             5.2.1: subgroup reductions by lane exchange instead of LDS)
// and the two wave groups are offset by half a tile so that one group's
// softmax runs on the VALU while the other's MFMAs run on the matrix core.
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

#include <type_traits>

#include "attn_kernel.h"

namespace libattn {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LDS __attribute__((address_space(3)))

constexpr int HD = 128;          // head dim
constexpr int BM = 128;          // query rows per wave group
constexpr int BN = 64;           // keys per KV tile
constexpr int NTHREADS = 512;    // 8 wavefronts
constexpr float NEG_INF = -__builtin_inff();
constexpr float M_INIT = -1e30f; // finite start for the running max
constexpr float LN2 = 0.693147180559945309f;
// Lazy rescaling: the running max (log2 units) is only raised when a tile's
// max exceeds it by more than TAU, so P = 2^(s - m) stays below 2^TAU; the
// final O / l and LSE = m + log2(l) are exact for any m.
constexpr float TAU = 8.0f;

// LDS layouts (bytes).  Both tiles are staged through registers so that the
// global loads of a tile can stay in flight across a barrier.
//  K: 64 key rows of 256 + 16 B.  The 8 lanes of a ds_read_b128 pass (8
//    consecutive keys, same 16-byte column) fall 16 B apart in bank space and
//    a 16-lane pass covers all 64 banks once; every K fragment read is a
//    compile-time offset from one per-lane base.
//  V: stored transposed, V^T[d][key]: 128 d rows of 64 keys (128 B) + 16 B,
//    so a PV fragment (8 keys of one d) is one ds_read_b128 instead of two
//    transpose reads.  Inside each group of 16 keys the columns are ordered
//    0-3, 8-11, 4-7, 12-15: lane half h of the MFMA B operand P^T holds keys
//    {4h..4h+3, 8+4h..8+4h+3} of the group (the accumulator layout of S^T), and
//    reads exactly those 8 keys as 16 contiguous bytes.
constexpr int K_ROWB = 2 * HD + 16;     // 272
constexpr int K_TILEB = BN * K_ROWB;    // 17408
constexpr int VT_ROWB = 2 * BN + 16;    // 144
constexpr int VT_TILEB = HD * VT_ROWB;  // 18432
static_assert(2 * (K_TILEB + VT_TILEB) <= 160 * 1024, "two K and two V^T slots fit the 160 KiB LDS");
__host__ __device__ constexpr int vt_col(int key) {  // column of key (0..63) in a V^T row
  return (key & ~15) | (key & 3) | (((key >> 3) & 1) << 2) | (((key >> 2) & 1) << 3);
}
// Depth of the fragment prefetch ring of the mma block.
#ifndef ATTN_RING
#define ATTN_RING 4
#endif
constexpr int RING = ATTN_RING;

__device__ __forceinline__ float pair_max(float x) {
  // lanes l and l^32 hold the same query: combine their partial results
  auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
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

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0..N-1.
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Steps of an mma block.  A QK step (kk, x = sb) adds K[32sb.., 16kk..] x
// Q^T[16kk.., :] into S^T block sb; a PV step (kk, x = db) adds
// V^T[32db.., 16kk..] x P^T[16kk.., :] into O^T block db.  Mode 0 runs PV of
// tile j-1 and QK of tile j with the two kinds alternating, so consecutive
// MFMAs of one accumulator are >= 4 steps apart: per group g the order is
// PV(g,0) QK(2g,0) PV(g,1) QK(2g,1) PV(g,2) QK(2g+1,0) PV(g,3) QK(2g+1,1).
// Mode 1 is PV only, mode 2 QK only.
struct Step {
  bool pv;
  int kk, x;
};
__host__ __device__ constexpr Step step_of(int mode, int i) {
  return mode == 1   ? Step{true, i >> 2, i & 3}
         : mode == 2 ? Step{false, i >> 1, i & 1}
         : ((i & 7) & 1) == 0 ? Step{true, i >> 3, (i & 7) >> 1}
                              : Step{false, 2 * (i >> 3) + ((i & 7) >> 2), ((i & 7) >> 1) & 1};
}
constexpr int steps_of(int mode) { return mode == 0 ? 32 : 16; }
constexpr int reads_of(int, int) { return 1; }  // LDS reads per fragment

template <bool kPingPong>
__global__ __launch_bounds__(NTHREADS, 1) void attn_fwd_kernel(Params p) {
  __shared__ __attribute__((aligned(1024))) char k_smem[2 * K_TILEB];
  __shared__ __attribute__((aligned(1024))) char v_smem[2 * VT_TILEB];
  LDS char* const k_lds = (LDS char*)k_smem;
  LDS char* const v_lds = (LDS char*)v_smem;

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

  // ---- K/V staging through registers.  K_t and V_t live in slot t & 1 of
  // their rings.  Group 0 stages K tiles, group 1 V tiles; each of the 256
  // threads of a group moves 4 chunks of 16 B per tile.  Rows past the end of
  // the sequence are loaded from row S-1 (finite data whose scores and weights
  // are masked to zero).  Loads use a wave-uniform tile base plus a constant
  // per-thread 32-bit offset.
  const int gt = tid & (NTHREADS / 2 - 1);
  const uint32_t row_bytes = (uint32_t)p.kv_sstride * 2;
  // K: chunk x = gt + 256u -> key row x / 16, column chunk x % 16
  const int k_row0 = gt >> 4, k_ch = gt & 15;
  // V: key quad vq = gt % 16 (keys 4vq..4vq+3), d chunk vc = gt / 16 (d 8vc..8vc+7)
  const int vq = gt & 15, vc = gt >> 4;
  // row of chunk u = st_row0 + u * st_drow; byte offset = st_off0 + u * st_doff
  const int st_row0 = grp == 0 ? k_row0 : 4 * vq;
  const int st_drow = grp == 0 ? 16 : 1;
  const uint32_t st_col = (uint32_t)(grp == 0 ? k_ch : vc) * 16u;
  const uint32_t st_off0 = (uint32_t)st_row0 * row_bytes + st_col;
  const uint32_t st_doff = (uint32_t)st_drow * row_bytes;
  const char* st_src;
  {  // wave-uniform source pointer, so the tile base below lives in SGPRs
    const uintptr_t a = (uintptr_t)(grp == 0 ? (const char*)kb_ : (const char*)vb_);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    st_src = (const char*)(((uintptr_t)hi << 32) | lo);
  }
  u32x4 stg[4];
  auto stage_load = [&](int tile) {  // global -> registers (this group's tensor)
    tile = __builtin_amdgcn_readfirstlane(tile);
    if (tile >= n_tiles) return;
    if ((tile + 1) * BN <= S) {
      const char* base = st_src + (int64_t)tile * BN * row_bytes;
#pragma unroll
      for (int u = 0; u < 4; ++u) stg[u] = *reinterpret_cast<const u32x4*>(base + (st_off0 + u * st_doff));
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int key = min(tile * BN + st_row0 + u * st_drow, S - 1);
        stg[u] = *reinterpret_cast<const u32x4*>(st_src + (int64_t)key * row_bytes + st_col);
      }
    }
  };
  auto stage_store = [&](int tile) {  // registers -> LDS slot tile & 1
    if (tile >= n_tiles) return;
    if (grp == 0) {
      LDS char* dst = k_lds + (tile & 1) * K_TILEB + k_row0 * K_ROWB + k_ch * 16;
#pragma unroll
      for (int u = 0; u < 4; ++u) *(LDS u32x4*)(dst + 16 * u * K_ROWB) = stg[u];
    } else {
      // transpose: for each of the 8 d values of the chunk, the 4 keys of the
      // quad become one 8-byte word of V^T row d
      LDS char* dst = v_lds + (tile & 1) * VT_TILEB + vc * 8 * VT_ROWB + 2 * vt_col(4 * vq);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t lo0 = __builtin_amdgcn_perm(stg[1][m], stg[0][m], 0x05040100u);
        const uint32_t lo1 = __builtin_amdgcn_perm(stg[3][m], stg[2][m], 0x05040100u);
        const uint32_t hi0 = __builtin_amdgcn_perm(stg[1][m], stg[0][m], 0x07060302u);
        const uint32_t hi1 = __builtin_amdgcn_perm(stg[3][m], stg[2][m], 0x07060302u);
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        *(LDS u32x2*)(dst + (2 * m) * VT_ROWB) = u32x2{lo0, lo1};
        *(LDS u32x2*)(dst + (2 * m + 1) * VT_ROWB) = u32x2{hi0, hi1};
      }
    }
  };

  // per-lane fragment bases (bytes); everything else is a compile-time offset
  const int k_frag = n * K_ROWB + 16 * hh;    // A operand of QK^T: key row n, d column 8*hh
  const int v_frag = n * VT_ROWB + 16 * hh;   // A operand of PV: V^T row n, key columns of lane half hh

  f32x16 o_acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o_acc[db] = f32x16{};
  float m_run = M_INIT;  // running max (log2 units) of the scores of query n
  float l_run = 0.f;     // running sum of 2^(score - m_run), from the fp16 P
  const float cs = p.cs;
  f32x16 s[2];           // S^T of the current tile
  f16x8 pf[4];           // P^T of the current tile (PV operand)

  // a wave skips every tile that lies wholly above its causal diagonal
  auto skip = [&](int j) { return !active || (p.causal && j * BN > qw + 31); };

  // ---- mma sTasks
  auto frag_qk = [&](int j, int kk, int sb) -> f16x8 {
    return *(const LDS f16x8*)(k_lds + (j & 1) * K_TILEB + k_frag + 32 * sb * K_ROWB + 32 * kk);
  };
  auto frag_pv = [&](int j, int kk, int db) -> f16x8 {
    return *(const LDS f16x8*)(v_lds + (j & 1) * VT_TILEB + v_frag + 32 * db * VT_ROWB + 32 * kk);
  };
  // One mma block: the fragments of the next RING steps are always in
  // flight; the scheduler is pinned to "MFMA i, then the LDS reads of step
  // i + RING" so the matrix core never waits on a just-issued read.
  auto mma_block = [&](int j, auto mode_c) {
    constexpr int mode = decltype(mode_c)::value;  // 0: PV(j-1)+QK(j), 1: PV(j-1), 2: QK(j)
    constexpr int nsteps = steps_of(mode);
    auto load = [&](auto ic) -> f16x8 {
      constexpr Step st = step_of(mode, decltype(ic)::value);
      if constexpr (st.pv) return frag_pv(j - 1, st.kk, st.x);
      else return frag_qk(j, st.kk, st.x);
    };
    f16x8 fr[RING];
    static_for<RING>([&](auto ic) { fr[decltype(ic)::value] = load(ic); });
    static_for<nsteps>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      constexpr Step st = step_of(mode, i);
      const f16x8 a = fr[i % RING];
      if constexpr (i + RING < nsteps) fr[i % RING] = load(std::integral_constant<int, i + RING>{});
      if constexpr (st.pv)
        o_acc[st.x] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pf[st.kk], o_acc[st.x], 0, 0, 0);
      else if constexpr (st.kk == 0)
        s[st.x] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[0], f32x16{}, 0, 0, 0);
      else
        s[st.x] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[st.kk], s[st.x], 0, 0, 0);
    });
    static_for<RING>([&](auto ic) {
      __builtin_amdgcn_sched_group_barrier(0x100, reads_of(mode, decltype(ic)::value), 0);
    });
    static_for<nsteps>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if constexpr (i + RING < nsteps) __builtin_amdgcn_sched_group_barrier(0x100, reads_of(mode, i + RING), 0);
    });
  };
  auto mma = [&](int j) {  // PV of tile j-1 and QK of tile j, whichever this wave needs
    const bool do_pv = j >= 1 && !skip(j - 1);
    const bool do_qk = j < n_tiles && !skip(j);
    if (do_pv && do_qk) mma_block(j, std::integral_constant<int, 0>{});
    else if (do_pv) mma_block(j, std::integral_constant<int, 1>{});
    else if (do_qk) mma_block(j, std::integral_constant<int, 2>{});
  };

  // ---- softmax sTask: online softmax of tile j in the log2 domain
  auto softmax = [&](int j, auto masked) {
    constexpr bool kMasked = decltype(masked)::value;
    uint32_t keep = 0xffffffffu;  // bit (16*sb + r): key allowed
    if constexpr (kMasked) {
      const int kj = j * BN;
      const int query = qw + n;
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
    auto kept = [&](int sb, int r) { return !kMasked || ((keep >> (16 * sb + r)) & 1u); };

    float mt = NEG_INF;
#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, kept(sb, r) ? s[sb][r] : NEG_INF);
    mt = pair_max(mt);
    const float mts = (mt == NEG_INF) ? NEG_INF : mt * cs;
    if (__builtin_amdgcn_ballot_w64(mts > m_run + TAU)) {  // wave-uniform: rescale only when needed
      const float m_new = fmaxf(m_run, mts);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) o_acc[db] *= alpha;
    }

#pragma unroll
    for (int sb = 0; sb < 2; ++sb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[sb][r], cs, -m_run));
        if constexpr (kMasked) e = kept(sb, r) ? e : 0.f;
        pf[2 * sb + (r >> 3)][r & 7] = (_Float16)e;
      }
    // row sum of the fp16 P actually fed to PV: 16 dot2 products against (1, 1)
    float rs = 0.f;
    const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f16x2 pr = {pf[kk][2 * e], pf[kk][2 * e + 1]};
        rs = __builtin_amdgcn_fdot2(pr, ones, rs, false);
      }
    l_run += pair_sum(rs);
  };
  auto softmax_tile = [&](int j) {
    const int kj = j * BN;
    if ((p.causal && kj + BN - 1 > qw) || kj + BN > S)
      softmax(j, std::true_type{});
    else
      softmax(j, std::false_type{});
  };

  if constexpr (!kPingPong) {
    // ---- serial schedule: every wave runs load-next / QK / store-next /
    // softmax / PV per tile (group 0 moves K tiles, group 1 V tiles)
    stage_load(0);
    stage_store(0);
    lds_barrier();
    for (int j = 0; j < n_tiles; ++j) {
      stage_load(j + 1);  // slot (j+1) & 1 was last read in iteration j-1
      if (!skip(j)) mma_block(j, std::integral_constant<int, 2>{});
      stage_store(j + 1);
      if (!skip(j)) {
        softmax_tile(j);
        mma_block(j + 1, std::integral_constant<int, 1>{});
      }
      lds_barrier();
    }
  } else {
    // ---- ping-pong schedule.  Time is cut into half-steps by workgroup
    // barriers.  Each wave alternates an mma block (PV of tile j-1 and QK of
    // tile j) and a softmax block (tile j); group 1 runs one half-step behind
    // group 0, so on every SIMD one wave keeps the matrix core busy while the
    // other runs softmax on the VALU.  Staging: group 0 loads K_{j+1} during
    // its mma block j (half-step 2j) and stores it during its softmax block j
    // (2j+1); group 1 loads V_j during its mma block j-1 (2j-1) and stores it
    // during its softmax block j-1 (2j).  The slot a store overwrites was last
    // read in half-step 2j-1, and the tile is first read in half-step 2j+2.
    if (grp == 0) {
      stage_load(0);
      stage_store(0);
    } else {
      stage_load(0);
    }
    lds_barrier();
    for (int hs = 0; hs < 2 * n_tiles + 2; ++hs) {
      const int ph = hs - grp;
      if (ph == -1) {
        stage_store(0);  // group 1: V_0
      } else if (ph <= 2 * n_tiles) {
        const int j = ph >> 1;
        if ((ph & 1) == 0) {
          stage_load(j + 1);  // group 0: K_{j+1}; group 1: V_{j+1}
          __builtin_amdgcn_s_setprio(1);
          mma(j);
          __builtin_amdgcn_s_setprio(0);
        } else {
          stage_store(j + 1);
          if (!skip(j)) softmax_tile(j);
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
