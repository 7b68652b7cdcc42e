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
//   load    : K/V tiles of 64 keys, global -> LDS by direct loads
//             (global_load_lds_dwordx4), staged ahead of the compute in
//             two-slot rings (the prologue / steady state / epilogue pattern
//             of software pipelining with ping-pong buffers, page "AI编译器融合
//             技术 -- 5. 并行性与分布式融合", section 5.4.2)
//   mma     : S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16_f16,
//             fp16 operands and fp32 accumulation (same page, section 5.2.2:
//             map the contraction onto the matrix instruction and conform the
//             register fragments to its layout)
//   softmax : online softmax in fp32 on the VALU; the per-query max and sum
//             need one cross-lane step (v_permlane32_swap) because the S^T
//             layout keeps each query in one lane pair (same page, section
//             5.2.1: subgroup reductions by lane exchange instead of LDS)
// Four tile schedules (see Schedule in variant.h) order these tasks and give
// the same bits: serial, an overlap schedule that fuses the softmax of tile j
// with the MFMAs of QK^T(j+1) and PV(j-1) in every wave, a ping-pong schedule
// of two wave groups offset by half a tile, and serial4 (the serial schedule
// in four-wave, one-head workgroups).
//
// Besides the MFMA, transpose-read and direct-load layouts listed in gfx950.h,
// this file relies on v_permlane32_swap(x, y): x's upper 32 lanes trade places
// with y's lower 32 (checked on gfx950 with a lane probe).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "attn_kernel.h"
#include "attn_tile.h"
#include "gfx950.h"

namespace libattn {

constexpr int BM = 128;          // query rows per wave group
static_assert(BN == BN_STD, "the kernels' default tile is the variant table's");
// Waves per workgroup: 8 (two wave groups on two heads of a KV group), or 4
// (one head) for the SERIAL4 schedule.
__host__ __device__ constexpr int waves_of(int sched) { return sched == SCHEDULE_SERIAL4 ? 4 : 8; }
// K tiles rotate through three slots, V tiles through two: K_t stays in LDS
// for the whole iteration after its QK^T, so a softmax that has to be redone
// can recompute S^T from it.  The serial loop reads K_j while K_{j+1} arrives,
// so two K slots serve it: SERIAL4 keeps two so that two of its workgroups fit
// a CU, and so does SERIAL with 128-key tiles (three would take 166 KiB).
__host__ __device__ constexpr int k_slots_of(int sched, int bn = BN) {
  return sched == SCHEDULE_SERIAL4 || bn == 128 ? 2 : 3;
}
constexpr int V_SLOTS = 2;
// Workgroups per CU: SERIAL4 asks for two (one wave per SIMD each) while its
// rings fit half the LDS, i.e. for head dimensions up to 128 and tiles of up
// to 64 keys; every other instance for one.
__host__ __device__ constexpr int wgs_per_cu(int sched, int hd, int bn) {
  return sched == SCHEDULE_SERIAL4 && hd <= 128 && bn <= 64 ? 2 : 1;
}

// Steps of an mma block, for NKK = HD/16 k steps of QK^T, NDB = HD/32
// blocks of O^T and NSB = BN/32 blocks of S^T (32 keys each; P^T has 2 NSB
// 16-key steps).  A QK step (kk, x = sb) adds K[32sb.., 16kk..] x
// Q^T[16kk.., :] into S^T block sb; a PV step (kk, x = db) adds
// V^T[32db.., 16kk..] x P^T[16kk.., :] into O^T block db.
//   mode 0: PV and QK steps alternate, so consecutive MFMAs of one
//           accumulator are >= 4 steps apart: per group g the order is
//           PV(g,0) QK(2g,0) PV(g,1) QK(2g,1) PV(g,2) QK(2g+1,0) PV(g,3)
//           QK(2g+1,1)  (HD 128, NSB 2 only)
//   mode 1: PV only, k-major over the O^T blocks
//   mode 2: QK only, S^T block 0 first (so it is complete half-way)
//   mode 3: the QK steps of mode 2, then the PV steps of mode 1
// Each accumulator sees its k steps in increasing order in every mode, so all
// modes give the same bits.
struct Step {
  bool pv;
  int kk, x;
};
__host__ __device__ constexpr Step step_of(int mode, int i, int nkk, int ndb, int nsb = 2) {
  return mode == 1   ? Step{true, i / ndb, i % ndb}
         : mode == 2 ? Step{false, i % nkk, i / nkk}
         : mode == 3 ? (i < nsb * nkk ? Step{false, i % nkk, i / nkk}
                                      : Step{true, (i - nsb * nkk) / ndb, (i - nsb * nkk) % ndb})
         : ((i & 7) & 1) == 0 ? Step{true, i >> 3, (i & 7) >> 1}
                              : Step{false, 2 * (i >> 3) + ((i & 7) >> 2), ((i & 7) >> 1) & 1};
}
constexpr int steps_of(int mode, int nkk, int ndb, int nsb = 2) {
  return mode == 1 ? 2 * nsb * ndb : mode == 2 ? nsb * nkk : nsb * nkk + 2 * nsb * ndb;
}
constexpr int reads_of(int mode, int i, int nkk, int ndb, int nsb = 2) {
  return step_of(mode, i, nkk, ndb, nsb).pv ? 2 : 1;
}

// Placement of the ne exponential parts of the overlap schedule among the
// nsteps MFMAs of its block: the step before whose MFMA part e runs.
//   PLACE_EVEN : spread evenly over the block
//   PLACE_FRONT: parts 0..4 before the first MFMA, where the block waits for
//                its first fragments, the rest spread over steps 1..nsteps-1
//   PLACE_EARLY: spread over all but the last four steps, so that the sum
//                check that follows the block has its inputs in time
// The map is non-decreasing in e, so the parts keep their order.
constexpr int e_step(int place, int e, int nsteps, int ne) {
  return place == PLACE_FRONT   ? (e < 5 ? 0 : 1 + (e - 5) * (nsteps - 2) / (ne - 1 - 5))
         : place == PLACE_EARLY ? e * (nsteps - 5) / (ne - 1)
                                : e * (nsteps - 1) / (ne - 1);
}

// kSched: tile schedule; kRing: depth of the fragment prefetch ring of the mma
// steps (how many steps ahead the LDS reads run); kHD: head dimension.  The
// overlap and ping-pong schedules are written for HD 128.  A SERIAL4
// workgroup asks for two waves per SIMD (two workgroups per CU), except at
// HD 256: there one workgroup fills the LDS and each wave may use the whole
// register file of its SIMD (O^T alone is 128 registers).
//
// kSplit (SERIAL4 only): split-KV mode for few query rows against many keys
// (decode).  A workgroup takes one split of the keys (p.split_tiles tiles)
// and a 128-row tile of the KV group's packed query rows: packed row r is
// query head c*g + r / Sq, query row r % Sq, so the g heads that share K/V
// read each K/V tile once.  It writes the split's O (normalised, fp32) and
// LSE to the workspace; attn_combine_kernel merges the splits.
//
// kBN: keys per K/V tile.  64 for every schedule; the serial schedules at HD
// 128 also run 32 and 128 (a smaller or larger unit of the load / mma /
// softmax pipeline: with 128 the per-tile fixed costs -- wait, barrier, sum
// check -- are spread over twice the keys, with 32 the causal diagonal wastes
// less).  Per tile the softmax runs the same parts over more or fewer scores;
// a row's results differ from BN 64's only by rounding order.
//
// kPlace: placement of the softmax parts in the overlap schedule's block
// (e_step); the other schedules have PLACE_EVEN only.  Every placement runs
// the same parts in the same order, so the results are the same bits.
template <int kSched, int kRing, int kHD, bool kSplit = false, int kBN = BN, int kPlace = PLACE_EVEN>
__global__ __launch_bounds__(64 * waves_of(kSched), wgs_per_cu(kSched, kHD, kBN))
void attn_fwd_kernel(Params p) {
  using G = Geo<kHD, kBN>;
  static_assert(kHD == 128 || kSched == SCHEDULE_SERIAL || kSched == SCHEDULE_SERIAL4,
                "HD 64 runs the serial schedules");
  static_assert(kHD <= 128 || kSched == SCHEDULE_SERIAL4, "HD 256 runs the SERIAL4 schedule");
  static_assert(!kSplit || kSched == SCHEDULE_SERIAL4, "split-KV mode runs the SERIAL4 schedule");
  static_assert(kBN == BN || ((kSched == SCHEDULE_SERIAL || kSched == SCHEDULE_SERIAL4) && kHD == 128 && !kSplit),
                "32- and 128-key tiles: the serial schedules at HD 128");
  static_assert(kPlace == PLACE_EVEN || kSched == SCHEDULE_OVERLAP, "placements: the overlap schedule");
  constexpr int NW = waves_of(kSched);
  constexpr int K_SLOTS = k_slots_of(kSched, kBN);
  constexpr int HD = G::HD, NKK = G::NKK, NDB = G::NDB;
  constexpr int NSB = kBN / 32;  // 32-key blocks of S^T
  constexpr int NPK = kBN / 16;  // 16-key steps of P^T
  constexpr int K_ROWB = G::K_ROWB, K_SLOTB = G::K_SLOTB, K_DMA = G::K_DMA;
  constexpr int K_DMA_PER_WAVE = (K_DMA + NW - 1) / NW;  // wave w issues K instructions w, w+NW, ...
  constexpr int V_DMA_PER_WAVE = G::V_DMA / NW;          // wave w issues V instructions w, w+NW, ...
  constexpr int V_ROWB = G::V_ROWB, V_TILEB = G::V_TILEB;
  static_assert(wgs_per_cu(kSched, kHD, kBN) * (K_SLOTS * K_SLOTB + V_SLOTS * V_TILEB) <= 160 * 1024,
                "the rings of the workgroups on a CU fit its 160 KiB LDS");
  __shared__ __attribute__((aligned(1024))) char k_smem[K_SLOTS * K_SLOTB];
  __shared__ __attribute__((aligned(1024))) char v_smem[V_SLOTS * V_TILEB];
  LDS char* const k_lds = (LDS char*)k_smem;
  LDS char* const v_lds = (LDS char*)v_smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = NW == 8 ? wave >> 2 : 0;  // wave group: which head of the pair
  const int wq = wave & 3;    // 32-row slice of the 128 query rows
  const int n = lane & 31;    // query column of this lane in S^T / O^T
  const int hh = lane >> 5;   // lane half

  // ---- workgroup -> (batch, kv head, head pair, query tile)
  // Workgroups are dealt round-robin to the 8 XCDs.  With p.xcd, give each XCD
  // whole (batch, kv head) groups so that co-resident workgroups share K/V in
  // that XCD's L2; with p.lpt, run the longest causal tiles of a group first.
  const int items = (kSplit ? p.n_splits : p.pairs) * p.n_qt;  // workgroups per (b, c) group
  const int ngroups = p.B * p.Hkv;
  int group, item;
  {
    const int bid = blockIdx.x;
    if (p.xcd && (ngroups & 7) == 0) {
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
  const int t = kSplit ? item / p.n_splits : p.lpt ? p.n_qt - 1 - item / p.pairs : item / p.pairs;
  const int split = kSplit ? item % p.n_splits : 0;  // split-KV mode: which split of the keys
  const int hl = kSplit ? 0 : NW == 8 ? 2 * (item % p.pairs) + grp : item % p.pairs;  // head inside the KV group
  const bool active = hl < p.g;
  const int h = c * p.g + (active ? hl : 0);

  const int Sq = p.Sq, Sk = p.Sk;
  const int off = p.off;        // causal: query row i attends keys j <= i + off
  const int q0 = t * BM;
  const int qw = q0 + 32 * wq;  // first query row of this wave
  const int kv_tiles_all = (Sk + kBN - 1) / kBN;
  int n_tiles = p.causal ? min(kv_tiles_all, (q0 + off + BM + kBN - 1) / kBN) : kv_tiles_all;
  int j_lo = 0;  // first key tile

  // Split-KV mode: this lane's packed row, its query head and query row, and
  // wave-uniform bounds of the wave's query rows for the causal tests.
  int h_lane = h, qidx = qw + n, q_lo = qw, q_hi = qw + 31;
  bool lane_ok = active && qidx < Sq, wave_active = active;
  if constexpr (kSplit) {
    const int R = p.g * Sq;
    const int pr0 = q0 + 32 * wq, pr = pr0 + n;
    lane_ok = pr < R;
    const int prc = min(pr, R - 1);
    h_lane = c * p.g + prc / Sq;
    qidx = prc % Sq;
    wave_active = pr0 < R;
    const int pr_end = min(pr0 + 31, R - 1);
    q_lo = 0;
    q_hi = Sq - 1;
    if (pr_end - pr0 + 1 < Sq) {
      const int i0 = pr0 % Sq, i1 = pr_end % Sq;
      if (i1 >= i0) {
        q_lo = i0;
        q_hi = i1;
      }
    }
    j_lo = split * p.split_tiles;
    n_tiles = min(kv_tiles_all, j_lo + p.split_tiles);  // causal: row Sq-1 sees every key
  }

  const _Float16* qb = p.q + (int64_t)b * p.q_bstride + (int64_t)h * HD;
  const _Float16* kb_ = p.k + (int64_t)b * p.kv_bstride + (int64_t)c * HD;
  const _Float16* vb_ = p.v + (int64_t)b * p.kv_bstride + (int64_t)c * HD;

  // ---- Q^T fragments (B operand of S^T = K Q^T), resident for the whole loop
  f16x8 qf[NKK];
  {
    const int qrow = qw + n;
    const bool ok = kSplit ? lane_ok : active && qrow < Sq;
    const uint32_t flip = p.neg ? 0x80008000u : 0u;
    const _Float16* src = kSplit ? p.q + (int64_t)b * p.q_bstride + (int64_t)h_lane * HD +
                                       (int64_t)qidx * p.q_sstride + 8 * hh
                                 : qb + (int64_t)qrow * p.q_sstride + 8 * hh;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 u = {0, 0, 0, 0};
      if (ok) u = *reinterpret_cast<const u32x4*>(src + 16 * kk);
      u ^= flip;
      qf[kk] = __builtin_bit_cast(f16x8, u);
    }
  }

  // ---- K/V staging by direct global -> LDS loads.  K_t and V_t live in slots
  // t % K_SLOTS and t & 1 of their rings.  Wave w issues K instructions w,
  // w+NW, ... and V instructions w, w+NW, ... of a tile (HD 128, 64 keys: 33
  // per tile over 8 waves).  The lane offsets relative to a tile's first row
  // are fixed; rows past the end of the keys are loaded from row Sk-1 (finite
  // data whose scores and weights are masked to zero).
  const uint32_t row_bytes = (uint32_t)p.kv_sstride * 2;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t k_lds_base = (uint32_t)(uintptr_t)k_lds, v_lds_base = (uint32_t)(uintptr_t)v_lds;
  int k_row[K_DMA_PER_WAVE];
  uint32_t k_col[K_DMA_PER_WAVE];
#pragma unroll
  for (int u = 0; u < K_DMA_PER_WAVE; ++u) {
    const int o = 64 * (wave + NW * u) + lane;  // 16-byte lane slot inside the tile
    const int row = o / (K_ROWB / 16);
    const int cb = o - row * (K_ROWB / 16);
    k_col[u] = 16u * (uint32_t)(cb < G::KC ? cb : G::KC - 1);  // padding slot: any in-bounds chunk of the row
    // a partial last instruction (kBN 32): its surplus lanes land in the slot past the tile, read from any row
    if constexpr (G::K_SLOTB != G::K_TILEB) k_row[u] = min(row, kBN - 1);
    else k_row[u] = row;
  }
  const int v_rowl = lane / G::KC;  // row inside the instruction's rows (V_ROWS_PER_DMA * i + v_rowl)
  // chunk stored at slot lane % KC.  The swizzle reads row bits 0..1; the
  // rows of this wave's instructions i = wave + NW*u differ by multiples of
  // NW * V_ROWS_PER_DMA >= 8, so the column is the same for every u.
  static_assert(NW * G::V_ROWS_PER_DMA % 4 == 0, "one V column per lane");
  const uint32_t v_col = 16u * (uint32_t)((lane % G::KC) ^ G::vswz(G::V_ROWS_PER_DMA * wave + v_rowl));
  auto stage = [&](int tk, int tv) INL {  // issue this wave's DMA for K tile tk and V tile tv
    tk = __builtin_amdgcn_readfirstlane(tk);
    tv = __builtin_amdgcn_readfirstlane(tv);
    if (tk < n_tiles) {
      const char* base = (const char*)kb_ + (int64_t)tk * kBN * row_bytes;
      const bool full = (tk + 1) * kBN <= Sk;
#pragma unroll
      for (int u = 0; u < K_DMA_PER_WAVE; ++u) {
        const int i = wave_s + NW * u;
        if (i < K_DMA) {
          const int row = full ? k_row[u] : min(k_row[u], Sk - 1 - tk * kBN);
          dma16(base, (uint32_t)row * row_bytes + k_col[u], k_lds_base + (tk % K_SLOTS) * K_SLOTB + 1024 * i);
        }
      }
    }
    if (tv < n_tiles) {
      const char* base = (const char*)vb_ + (int64_t)tv * kBN * row_bytes;
      const bool full = (tv + 1) * kBN <= Sk;
#pragma unroll
      for (int u = 0; u < V_DMA_PER_WAVE; ++u) {
        const int i = wave_s + NW * u;
        const int row0 = G::V_ROWS_PER_DMA * i + v_rowl;
        const int row = full ? row0 : min(row0, Sk - 1 - tv * kBN);
        dma16(base, (uint32_t)row * row_bytes + v_col, v_lds_base + (tv & 1) * V_TILEB + 1024 * i);
      }
    }
  };

  // per-lane fragment bases (bytes); everything else is a compile-time offset
  const int k_frag = n * K_ROWB + 16 * hh;  // A operand of QK^T: key row n, d column 8*hh
  int v_frag[NDB];                          // transpose reads of V, one base per 32-wide d block
  {
    const int vg = lane >> 4, vsl = lane & 15;
    const int r0 = 4 * (vg >> 1) + (vsl >> 2);
    const int c0 = 2 * (vg & 1) + ((vsl & 3) >> 1);
    const int f0 = r0 * V_ROWB + ((c0 ^ G::vswz(r0)) << 4) + ((vsl & 1) << 3);
#pragma unroll
    for (int db = 0; db < NDB; ++db) v_frag[db] = f0 ^ (64 * db);
  }

  f32x16 o_acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o_acc[db] = f32x16{};
  float m_run = M_INIT;  // running max (log2 units) of the scores of query n
  float l_run = 0.f;     // running sum of 2^(score - m_run), from the fp16 P
  const float cs = p.cs;

  // A wave skips every tile that lies wholly above its causal diagonal.  The
  // tests take wave-uniform copies so that they compile to scalar branches.
  const int qw_u = __builtin_amdgcn_readfirstlane(qw);
  const bool active_u = __builtin_amdgcn_readfirstlane(active ? 1 : 0) != 0;
  const int qlo_u = __builtin_amdgcn_readfirstlane(q_lo), qhi_u = __builtin_amdgcn_readfirstlane(q_hi);
  const bool wact_u = __builtin_amdgcn_readfirstlane(wave_active ? 1 : 0) != 0;
  auto skip = [&](int j) INL {
    if constexpr (kSplit) return !wact_u || (p.causal && j * kBN > qhi_u + off);
    else return !active_u || (p.causal && j * kBN > qw_u + 31 + off);
  };
  auto is_masked = [&](int j) INL {
    if constexpr (kSplit) return (p.causal && j * kBN + kBN - 1 > qlo_u + off) || j * kBN + kBN > Sk;
    else return (p.causal && j * kBN + kBN - 1 > qw_u + off) || j * kBN + kBN > Sk;
  };

  // ---- fragments of the mma sTasks
  auto frag_qk = [&](int j, int kk, int sb) INL -> f16x8 {
    return *(const LDS f16x8*)(k_lds + (j % K_SLOTS) * K_SLOTB + k_frag + 32 * sb * K_ROWB + 32 * kk);
  };
  auto frag_pv = [&](int j, int kk, int db) INL -> f16x8 {
    const LDS char* a = v_lds + (j & 1) * V_TILEB + v_frag[db] + 16 * kk * V_ROWB;
    const f16x4 h1 = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)a));
    const f16x4 h2 = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)(a + 8 * V_ROWB)));
    return f16x8{h1[0], h1[1], h1[2], h1[3], h2[0], h2[1], h2[2], h2[3]};
  };

  // ---- softmax sTask: online softmax of tile j (scores sc) in the log2
  // domain, P^T into pd.  It yields the rescale factor alpha of O and whether
  // any lane needs it (wave-uniform); the caller applies O *= alpha once the
  // PV of the previous tile has been accumulated.
  //
  // The work is cut into parts with compile-time indices so that a fused mma
  // block can place each part between two MFMAs.  A lane holds NE = 16 NSB
  // scores of its query (NE = 32 for 64-key tiles):
  //   E0..E(NE-1)  P = 2^(s*cs - m) for score e; every second part also packs
  //           an earlier pair to fp16 and adds it to the row sum
  //           (add_pair_f16), one pair behind to hide the exponential's latency
  //   E(NE)   packs the last pair
  //   E(NE+1) row sum across the lane pair
  //   C       the check: does any row's tile sum exceed RS_MAX?  (ballot,
  //           wave-uniform)
  //   F       l = l * alpha + row sum (one fused multiply-add)
  // and, only on a wave's first tile or when C fires, before F:
  //   X0..X(2NC-1)  tile max: NC = 2 NSB chains of 8 scores, half a chain
  //           per part
  //   X(2NC), X(2NC+1)  lane-pair max, tile max in log2 units
  //   D       m = max(m, tile max), alpha = 2^(m_old - m), -m for the exponents
  //   E0..E33 again, with the new m
  // On the first tile this is the textbook online softmax step in order X,
  // D, E, F.  Every schedule runs the same parts on the same values in the
  // same order per tile, so they all produce the same bits.
  struct Rescale {
    bool any;
    float alpha;
  };
  constexpr int NC = 2 * NSB;    // max chains of 8 scores
  constexpr int NE = 16 * NSB;   // scores per lane and tile
  struct SmState {
    float mq[NC];    // chain maxima
    float sw[2];     // the lane pair's combined maxima after the swap
    float mts;       // tile max, log2 units
    float negm;      // -(running max) used by the exponentials
    float t[2][2];   // exponentials of the last two pairs
    float rq[2];     // row-sum partials
    float rs;        // row sum of the tile
    int lim;         // masked tiles: compile-time key offsets below lim are allowed
    Rescale rz;
  };
  // Key (sb, r) of this lane is j*kBN + 32sb + 8(r/4) + 4hh + r%4; it is
  // allowed iff it is below end = min(Sk, query + off + 1) (causal) or Sk, i.e. iff
  // the compile-time part 32sb + 8(r/4) + r%4 is below lim.
  auto sm_lim = [&](int j, auto masked, SmState& st) INL {
    if constexpr (decltype(masked)::value) {
      const int query = kSplit ? qidx : qw + n;
      const int end = p.causal ? min(Sk, query + off + 1) : Sk;
      st.lim = end - j * kBN - 4 * hh;
    }
  };
  auto sm_start = [&](SmState& st) INL {  // before the E parts
    st.negm = -m_run;
    st.rq[0] = 0.f;
    st.rq[1] = 0.f;
    st.rz.any = false;
    st.rz.alpha = 1.0f;
  };
  auto sm_x = [&](auto kc, f32x16 (&sc)[NSB], auto masked, SmState& st) INL {  // parts X0..X(2NC+1)
    constexpr int k = decltype(kc)::value;
    constexpr bool kMasked = decltype(masked)::value;
    auto kept = [&](int sb, int r) INL { return !kMasked || 32 * sb + 8 * (r >> 2) + (r & 3) < st.lim; };
    if constexpr (k < 2 * NC) {
      constexpr int q = k % NC, half = k / NC;
      if constexpr (half == 0) st.mq[q] = NEG_INF;
#pragma unroll
      for (int e = 4 * half; e < 4 * half + 4; ++e) {
        const int sb = q >> 1, r = 8 * (q & 1) + e;
        st.mq[q] = fmaxf(st.mq[q], kept(sb, r) ? sc[sb][r] : NEG_INF);
      }
    } else if constexpr (k == 2 * NC) {
      float m4;  // max of the chains, pairwise
      if constexpr (NC == 2) m4 = fmaxf(st.mq[0], st.mq[1]);
      else if constexpr (NC == 4) m4 = fmaxf(fmaxf(st.mq[0], st.mq[1]), fmaxf(st.mq[2], st.mq[3]));
      else
        m4 = fmaxf(fmaxf(fmaxf(st.mq[0], st.mq[1]), fmaxf(st.mq[2], st.mq[3])),
                   fmaxf(fmaxf(st.mq[4], st.mq[5]), fmaxf(st.mq[6], st.mq[7])));
      // lanes l and l^32 hold the same query: combine their partial maxima
      auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(m4), __float_as_uint(m4), false, false);
      st.sw[0] = __uint_as_float(x[0]);
      st.sw[1] = __uint_as_float(x[1]);
    } else {
      static_assert(k == 2 * NC + 1, "max part index");
      const float mt = fmaxf(st.sw[0], st.sw[1]);
      st.mts = (mt == NEG_INF) ? NEG_INF : mt * cs;
    }
  };
  auto sm_d = [&](SmState& st) INL {  // part D (rows without an allowed key keep m)
    const float m_new = fmaxf(m_run, st.mts);
    st.negm = -m_new;
    st.rq[0] = 0.f;
    st.rq[1] = 0.f;
    st.rz.any = true;
    st.rz.alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
  };
  auto sm_e = [&](auto kc, f32x16 (&sc)[NSB], f16x8 (&pd)[NPK], auto masked, SmState& st) INL {  // E0..E(NE+1)
    constexpr int e = decltype(kc)::value;
    constexpr bool kMasked = decltype(masked)::value;
    auto kept = [&](int sb, int r) INL { return !kMasked || 32 * sb + 8 * (r >> 2) + (r & 3) < st.lim; };
    auto pack = [&](auto pc) INL {  // pair pp to fp16 P^T and into the row sum
      constexpr int pp = decltype(pc)::value, kk = pp >> 2, c = 2 * (pp & 3);
      pd[kk][c] = (_Float16)st.t[pp & 1][0];
      pd[kk][c + 1] = (_Float16)st.t[pp & 1][1];
      add_pair_f16(st.rq[kk & 1], f16x2{pd[kk][c], pd[kk][c + 1]});
    };
    if constexpr (e < NE) {  // score e = pair e/2, element e%2: (sb, r)
      constexpr int pair = e >> 1, u = e & 1, sb = pair >> 3, r = 2 * (pair & 7) + u;
      float x = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[sb][r], cs, st.negm));
      if constexpr (kMasked) x = kept(sb, r) ? x : 0.f;
      st.t[pair & 1][u] = x;
      if constexpr (u == 1 && pair >= 1) pack(std::integral_constant<int, pair - 1>{});
    } else if constexpr (e == NE) {
      pack(std::integral_constant<int, NE / 2 - 1>{});
    } else {
      static_assert(e == NE + 1, "exp part index");
      st.rs = pair_sum(st.rq[0] + st.rq[1]);
    }
  };
  // part C; !(rs <= RS_MAX) also catches an infinite sum (m not yet set)
  auto sm_c = [&](SmState& st) INL { return __builtin_amdgcn_ballot_w64(!(st.rs <= RS_MAX)) != 0; };
  auto sm_f = [&](SmState& st) INL { l_run = __builtin_fmaf(l_run, st.rz.alpha, st.rs); };  // part F
  constexpr int SM_X = 2 * NC + 2, SM_E = NE + 2;
  // X, D, E: the tile with its max (first tile, or C fired)
  auto sm_full = [&](f32x16 (&sc)[NSB], f16x8 (&pd)[NPK], auto masked, SmState& st) INL {
    static_for<SM_X>([&](auto kc) INL { sm_x(kc, sc, masked, st); });
    sm_d(st);
    static_for<SM_E>([&](auto ec) INL { sm_e(ec, sc, pd, masked, st); });
  };
  auto softmax = [&](int j, f32x16 (&sc)[NSB], f16x8 (&pd)[NPK], auto masked, bool first) INL -> Rescale {
    SmState st;
    sm_lim(j, masked, st);
    sm_start(st);
    bool redo = first;
    if (!first) {
      static_for<SM_E>([&](auto ec) INL { sm_e(ec, sc, pd, masked, st); });
      redo = sm_c(st);
    }
    if (__builtin_expect(redo, 0)) sm_full(sc, pd, masked, st);
    sm_f(st);
    return st.rz;
  };
  auto rescale_o = [&](const Rescale& rz) INL {
    if (__builtin_expect(rz.any, 0)) {  // rare after a row's first tiles
#pragma unroll
      for (int db = 0; db < NDB; ++db) o_acc[db] *= rz.alpha;
    }
  };

  // ---- one block of mma steps, optionally fused with a softmax.  QK steps
  // read K tile jq into sd; PV steps read V tile jv with P^T from ps.  The
  // fragments of the next kRing steps are always in flight.  Without a
  // softmax the scheduler is pinned to "MFMA i, then the LDS reads of step
  // i + kRing".  With one, step i is fixed by
  // hand as "the softmax parts placed there (sm(i)), MFMA i, LDS reads of
  // step i + kRing" and nothing moves across steps, so each wave keeps the
  // matrix core, the LDS and the VALU busy together.
  struct NoSoftmax {};
  auto block = [&](auto mode_c, int jq, f32x16 (&sd)[NSB], int jv, f16x8 (&ps)[NPK], auto sm) INL {
    constexpr int mode = decltype(mode_c)::value;
    constexpr int nsteps = steps_of(mode, NKK, NDB, NSB);
    constexpr bool kSoftmax = !std::is_same_v<decltype(sm), NoSoftmax>;
    auto load = [&](auto ic) INL -> f16x8 {
      constexpr Step st = step_of(mode, decltype(ic)::value, NKK, NDB, NSB);
      if constexpr (st.pv) return frag_pv(jv, st.kk, st.x);
      else return frag_qk(jq, st.kk, st.x);
    };
    f16x8 fr[kRing];
    static_for<kRing>([&](auto ic) INL { fr[decltype(ic)::value] = load(ic); });
    auto step = [&](auto ic) INL {
      constexpr int i = decltype(ic)::value;
      constexpr Step st = step_of(mode, i, NKK, NDB, NSB);
      const f16x8 a = fr[i % kRing];
      if constexpr (i + kRing < nsteps) fr[i % kRing] = load(std::integral_constant<int, i + kRing>{});
      if constexpr (st.pv)
        o_acc[st.x] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, ps[st.kk], o_acc[st.x], 0, 0, 0);
      else if constexpr (st.kk == 0)
        sd[st.x] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[0], f32x16{}, 0, 0, 0);
      else
        sd[st.x] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, qf[st.kk], sd[st.x], 0, 0, 0);
    };
    if constexpr (!kSoftmax) {
      static_for<nsteps>(step);
      static_for<kRing>([&](auto ic) INL {
        __builtin_amdgcn_sched_group_barrier(0x100, reads_of(mode, decltype(ic)::value, NKK, NDB, NSB), 0);
      });
      static_for<nsteps>([&](auto ic) INL {
        constexpr int i = decltype(ic)::value;
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if constexpr (i + kRing < nsteps)
          __builtin_amdgcn_sched_group_barrier(0x100, reads_of(mode, i + kRing, NKK, NDB, NSB), 0);
      });
    } else {
      static_for<nsteps>([&](auto ic) INL {
        sm(ic);  // the softmax parts placed before MFMA i
        step(ic);
        __builtin_amdgcn_sched_barrier(0);
      });
    }
  };
  using M_BOTH = std::integral_constant<int, 0>;
  using M_PV = std::integral_constant<int, 1>;
  using M_QK = std::integral_constant<int, 2>;
  using M_FUSED = std::integral_constant<int, 3>;
  f16x8 pf[NPK];  // P^T of the tile whose softmax ran last
  f32x16 s[NSB];  // S^T of the tile whose QK^T ran last
  auto softmax_tile = [&](int j, bool first) INL {  // first: the wave's first tile
    const Rescale rz = is_masked(j) ? softmax(j, s, pf, std::true_type{}, first)
                                    : softmax(j, s, pf, std::false_type{}, first);
    rescale_o(rz);
  };

  if constexpr (kSched == SCHEDULE_SERIAL || kSched == SCHEDULE_SERIAL4) {
    // ---- serial schedule: every wave runs stage-next / QK / softmax / PV per
    // tile; K slot (j+1) % K_SLOTS and V slot (j+1) & 1 were last read in
    // iteration j-1 or earlier
    stage(j_lo, j_lo);
    dma_wait();
    lds_barrier();
    for (int j = j_lo; j < n_tiles; ++j) {
      stage(j + 1, j + 1);
      if (!skip(j)) {
        block(M_QK{}, j, s, 0, pf, NoSoftmax{});
        softmax_tile(j, j == j_lo);
        block(M_PV{}, 0, s, j, pf, NoSoftmax{});
      }
      dma_wait();
      lds_barrier();
    }
  } else if constexpr (kSched == SCHEDULE_PINGPONG) {
    // ---- ping-pong schedule.  Time is cut into half-steps by workgroup
    // barriers.  Each wave alternates an mma block (PV of tile j-1 and QK of
    // tile j) and a softmax block (tile j); group 1 runs one half-step behind
    // group 0, so on every SIMD one wave keeps the matrix core busy while the
    // other runs softmax on the VALU.  In half-step 2j all waves issue the
    // loads of K_{j+1} and V_j, whose slots were last read in half-step 2j-1,
    // and wait for them at the end of half-step 2j+1; the tiles are first read
    // in half-step 2j+2.
    stage(0, n_tiles);
    dma_wait();
    lds_barrier();
    for (int hs = 0; hs < 2 * n_tiles + 2; ++hs) {
      const int ph = hs - grp;
      if ((hs & 1) == 0) stage((hs >> 1) + 1, hs >> 1);
      if (ph >= 0 && ph <= 2 * n_tiles) {
        const int j = ph >> 1;
        if ((ph & 1) == 0) {
          const bool do_pv = j >= 1 && !skip(j - 1);
          const bool do_qk = j < n_tiles && !skip(j);
          __builtin_amdgcn_s_setprio(1);
          if (do_pv && do_qk) block(M_BOTH{}, j, s, j - 1, pf, NoSoftmax{});
          else if (do_pv) block(M_PV{}, j, s, j - 1, pf, NoSoftmax{});
          else if (do_qk) block(M_QK{}, j, s, j - 1, pf, NoSoftmax{});
          __builtin_amdgcn_s_setprio(0);
        } else if (!skip(j)) {
          softmax_tile(j, j == 0);
        }
      }
      if (hs & 1) dma_wait();
      lds_barrier();
    }
  } else {
    // ---- overlap schedule: all eight waves run the same phases, and the
    // overlap of MFMA and VALU work happens inside each wave.  The softmax is
    // pipelined across iterations.  Iteration j is one block of 32 MFMAs --
    // QK^T of tile j+1, then PV of tile j-1 -- with, between them, the
    // exponentials and row sum of tile j; then the sum check of tile j (and
    // in the rare case it fires, its max and the exponentials again),
    // O *= alpha_j and a barrier.
    // Iteration j reads K_{j+1} and V_{j-1} and loads K_{j+2} and V_j into
    // the slots that K_{j-1} and V_{j-2} left.  Per tile the softmax runs the
    // same parts in the same order as the serial schedule, and per
    // accumulator the MFMAs are the same, so the results are the same bits.
    //
    // No wave skips a tile here: the steady-state loop has one code path per
    // mask case, so O, S and P each keep a single set of registers.  A tile
    // wholly above a wave's diagonal (only ever the last one) is computed with
    // every key masked, which is an exact no-op: every P is 0, the sum check
    // passes so alpha = 1 and the running max stays, l gains 0 and PV adds
    // zeros.  Waves of a missing odd head (hl == g) compute head h of the pair
    // and store nothing.
    //
    // S^T and P^T alternate between two register sets (sa/sb, pa/pb) from
    // one iteration to the next, so the loops are unrolled twice.  On entry
    // to each loop S^T of the current tile is in sa and P^T of the previous
    // tile in pa; cur holds the softmax state of the current tile.
    f32x16 sa[NSB], sb[NSB];
    f16x8 pa[NPK], pb[NPK];
    SmState cur;
    // One iteration.  with_pv / with_qk: whether PV(j-1) / QK(j+1) exist;
    // mask_e / mask_x: whether tile j / tile j+1 need the key mask.
    auto iter = [&](int j, auto with_pv, auto with_qk, auto mask_e, auto mask_x, f32x16 (&sc)[NSB],
                    f32x16 (&sn)[NSB], f16x8 (&pp)[NPK], f16x8 (&pc)[NPK]) INL {
      constexpr bool kPV = decltype(with_pv)::value, kQK = decltype(with_qk)::value;
      stage(j + 2, j);
      SmState nx;  // tile j+1
      if constexpr (kQK) sm_lim(j + 1, mask_x, nx);
      sm_start(cur);
      // E part e runs before MFMA e_step(kPlace, e, nsteps, SM_E) of the
      // block; C, the rare X / D / E redo and F follow the block.
      constexpr int nsteps = kQK ? steps_of(kPV ? 3 : 2, NKK, NDB) : steps_of(1, NKK, NDB);
      auto sm = [&](auto ic) INL {
        constexpr int i = decltype(ic)::value;
        static_for<SM_E>([&](auto ec) INL {
          if constexpr (e_step(kPlace, decltype(ec)::value, nsteps, SM_E) == i) sm_e(ec, sc, pc, mask_e, cur);
        });
      };
      if constexpr (kPV && kQK) {
        block(M_FUSED{}, j + 1, sn, j - 1, pp, sm);
      } else if constexpr (kQK) {
        block(M_QK{}, j + 1, sn, j - 1, pp, sm);
      } else if constexpr (kPV) {
        block(M_PV{}, j + 1, sn, j - 1, pp, sm);
      } else {
        static_for<SM_E>([&](auto ec) INL { sm_e(ec, sc, pc, mask_e, cur); });
      }
      if (__builtin_expect(sm_c(cur), 0)) sm_full(sc, pc, mask_e, cur);
      sm_f(cur);
      rescale_o(cur.rz);
      if constexpr (kQK) cur = nx;
      dma_wait();
      lds_barrier();
    };
    auto to_a = [&]() INL {  // back to the loop-entry convention
#pragma unroll
      for (int i = 0; i < 2; ++i) sa[i] = sb[i];
#pragma unroll
      for (int i = 0; i < 4; ++i) pa[i] = pb[i];
    };
    // Tiles below j_ms need no mask for any wave of the workgroup; the
    // steady-state loop is split so that each loop has one code path.  The
    // first and the last iteration always take the masked path (with no key
    // masked it computes the same values).
    const int j_ms = min(n_tiles, p.causal ? min(q0 + off, Sk) / kBN : Sk / kBN);
    using T = std::true_type;
    using F = std::false_type;
    stage(0, n_tiles);
    stage(1, n_tiles);
    dma_wait();
    lds_barrier();
    // prologue: S^T of tile 0, its max and the first running max (K_0 keeps
    // its slot while iteration 0 loads K_2, so no barrier is needed here);
    // iteration 0 then runs the E parts of tile 0 against that max, as the
    // first tile of the serial schedule does
    block(M_QK{}, 0, sa, 0, pa, NoSoftmax{});
    sm_lim(0, T{}, cur);
    static_for<SM_X>([&](auto kc) INL { sm_x(kc, sa, T{}, cur); });
    sm_d(cur);
    int j = 0;
    if (n_tiles > 1) {
      iter(0, F{}, T{}, T{}, T{}, sa, sb, pa, pb);
      to_a();
      j = 1;
      // iterations with tiles j and j+1 both unmasked: [1, j_u)
      const int j_u = min(j_ms - 1, n_tiles - 1);
      for (; j + 1 < j_u; j += 2) {
        iter(j, T{}, T{}, F{}, F{}, sa, sb, pa, pb);
        iter(j + 1, T{}, T{}, F{}, F{}, sb, sa, pb, pa);
      }
      if (j < j_u) {
        iter(j, T{}, T{}, F{}, F{}, sa, sb, pa, pb);
        to_a();
        ++j;
      }
      for (; j + 1 < n_tiles - 1; j += 2) {
        iter(j, T{}, T{}, T{}, T{}, sa, sb, pa, pb);
        iter(j + 1, T{}, T{}, T{}, T{}, sb, sa, pb, pa);
      }
      if (j < n_tiles - 1) {
        iter(j, T{}, T{}, T{}, T{}, sa, sb, pa, pb);
        to_a();
        ++j;
      }
    }
    // the last tile (j = n_tiles - 1): with PV of the tile before if there is one
    if (j > 0) iter(j, T{}, F{}, T{}, T{}, sa, sb, pa, pb);
    else iter(j, F{}, F{}, T{}, T{}, sa, sb, pa, pb);
    // PV of the last tile, whose P^T the last iteration left in pb
    block(M_PV{}, 0, sa, n_tiles - 1, pb, NoSoftmax{});
  }

  // ---- split-KV epilogue: this split's O = O^T / l (fp32) and LSE (natural
  // log; -inf when the split holds no allowed key for the row) to the workspace
  if constexpr (kSplit) {
    if (lane_ok) {
      const int64_t row = ((int64_t)b * p.Hq + h_lane) * Sq + qidx;
      float* dst = p.ws_o + (row * p.n_splits + split) * HD;
      const bool any = l_run > 0.f;
      const float inv = any ? 1.0f / l_run : 0.f;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          f32x4 ov;
#pragma unroll
          for (int e = 0; e < 4; ++e) ov[e] = o_acc[db][4 * r4 + e] * inv;
          *reinterpret_cast<f32x4*>(dst + 32 * db + 8 * r4 + 4 * hh) = ov;
        }
      if (hh == 0) p.ws_lse[row * p.n_splits + split] = any ? (m_run + log2f(l_run)) * LN2 : NEG_INF;
    }
    return;
  }
  // ---- epilogue: O = O^T / l (fp16, round to nearest even), LSE in natural log
  if (active) {
    const int qrow = qw + n;
    if (qrow < Sq) {
      const float inv = 1.0f / l_run;
      _Float16* dst = p.o + (int64_t)b * p.q_bstride + (int64_t)qrow * p.q_sstride + (int64_t)h * HD;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          f16x4 hv;
#pragma unroll
          for (int e = 0; e < 4; ++e) hv[e] = (_Float16)(o_acc[db][4 * r4 + e] * inv);
          *reinterpret_cast<f16x4*>(dst + 32 * db + 8 * r4 + 4 * hh) = hv;
        }
      if (p.lse && hh == 0)
        p.lse[((int64_t)b * p.Hq + h) * Sq + qrow] = (m_run + log2f(l_run)) * LN2;
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
  const dim3 grid((unsigned)nb), block(64 * waves_of(p.schedule));
#define LIBATTN_LAUNCH(S, R, H) hipLaunchKernelGGL((attn_fwd_kernel<S, R, H>), grid, block, 0, stream, p)
#define LIBATTN_LAUNCH_BN(S, R, N) \
  hipLaunchKernelGGL((attn_fwd_kernel<S, R, 128, false, N>), grid, block, 0, stream, p)
  if (p.ring != 2 && p.ring != 4) return hipErrorInvalidValue;
  if (p.place != PLACE_EVEN && (p.schedule != SCHEDULE_OVERLAP || p.bn != BN || p.hd != 128))
    return hipErrorInvalidValue;
  const bool r2 = p.ring == 2;
  if (p.bn != BN) {  // 32- and 128-key tiles: the serial schedules at HD 128
    if (p.hd != 128 || (p.bn != 32 && p.bn != 128) ||
        (p.schedule != SCHEDULE_SERIAL && p.schedule != SCHEDULE_SERIAL4))
      return hipErrorInvalidValue;
    const bool s4 = p.schedule == SCHEDULE_SERIAL4;
    if (p.bn == 32) {
      if (s4) {
        if (r2) LIBATTN_LAUNCH_BN(SCHEDULE_SERIAL4, 2, 32);
        else LIBATTN_LAUNCH_BN(SCHEDULE_SERIAL4, 4, 32);
      } else {
        if (r2) LIBATTN_LAUNCH_BN(SCHEDULE_SERIAL, 2, 32);
        else LIBATTN_LAUNCH_BN(SCHEDULE_SERIAL, 4, 32);
      }
    } else {
      if (s4) {
        if (r2) LIBATTN_LAUNCH_BN(SCHEDULE_SERIAL4, 2, 128);
        else LIBATTN_LAUNCH_BN(SCHEDULE_SERIAL4, 4, 128);
      } else {
        if (r2) LIBATTN_LAUNCH_BN(SCHEDULE_SERIAL, 2, 128);
        else LIBATTN_LAUNCH_BN(SCHEDULE_SERIAL, 4, 128);
      }
    }
  } else if (p.schedule == SCHEDULE_SERIAL4) {
    if (p.hd == 64) {
      if (r2) LIBATTN_LAUNCH(SCHEDULE_SERIAL4, 2, 64);
      else LIBATTN_LAUNCH(SCHEDULE_SERIAL4, 4, 64);
    } else if (p.hd == 128) {
      if (r2) LIBATTN_LAUNCH(SCHEDULE_SERIAL4, 2, 128);
      else LIBATTN_LAUNCH(SCHEDULE_SERIAL4, 4, 128);
    } else if (p.hd == 256) {
      if (r2) LIBATTN_LAUNCH(SCHEDULE_SERIAL4, 2, 256);
      else LIBATTN_LAUNCH(SCHEDULE_SERIAL4, 4, 256);
    } else {
      return hipErrorInvalidValue;
    }
  } else if (p.hd == 64) {  // serial schedules only
    if (p.schedule != SCHEDULE_SERIAL) return hipErrorInvalidValue;
    if (r2) LIBATTN_LAUNCH(SCHEDULE_SERIAL, 2, 64);
    else LIBATTN_LAUNCH(SCHEDULE_SERIAL, 4, 64);
  } else if (p.hd != 128) {
    return hipErrorInvalidValue;
  } else if (p.schedule == SCHEDULE_OVERLAP) {
#define LIBATTN_LAUNCH_PL(R, P) \
  hipLaunchKernelGGL((attn_fwd_kernel<SCHEDULE_OVERLAP, R, 128, false, BN, P>), grid, block, 0, stream, p)
    if (p.place == PLACE_FRONT) {
      if (r2) LIBATTN_LAUNCH_PL(2, PLACE_FRONT);
      else LIBATTN_LAUNCH_PL(4, PLACE_FRONT);
    } else if (p.place == PLACE_EARLY) {
      if (r2) LIBATTN_LAUNCH_PL(2, PLACE_EARLY);
      else LIBATTN_LAUNCH_PL(4, PLACE_EARLY);
    } else {
      if (r2) LIBATTN_LAUNCH(SCHEDULE_OVERLAP, 2, 128);
      else LIBATTN_LAUNCH(SCHEDULE_OVERLAP, 4, 128);
    }
#undef LIBATTN_LAUNCH_PL
  } else if (p.schedule == SCHEDULE_PINGPONG) {
    if (r2) LIBATTN_LAUNCH(SCHEDULE_PINGPONG, 2, 128);
    else LIBATTN_LAUNCH(SCHEDULE_PINGPONG, 4, 128);
  } else {
    if (r2) LIBATTN_LAUNCH(SCHEDULE_SERIAL, 2, 128);
    else LIBATTN_LAUNCH(SCHEDULE_SERIAL, 4, 128);
  }
#undef LIBATTN_LAUNCH
#undef LIBATTN_LAUNCH_BN
  return hipGetLastError();
}

// ---- combine the splits of the split-KV kernel.  One wave per (b, h, row):
// LSE = log sum_s exp(LSE_s) and O = sum_s exp(LSE_s - LSE) O_s, the exact
// merge of softmax partials over disjoint key sets; O is rounded to fp16 (RNE).
template <int kHD>
__global__ __launch_bounds__(256) void attn_combine_kernel(Params p, int64_t rows) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  constexpr int PER = kHD / 64;  // head-dimension elements per lane
  const int ns = p.n_splits;
  const float* ls = p.ws_lse + row * ns;
  float mx = NEG_INF;
  for (int s = 0; s < ns; ++s) mx = fmaxf(mx, ls[s]);
  float sum = 0.f;
  for (int s = 0; s < ns; ++s) sum += (ls[s] == NEG_INF) ? 0.f : expf(ls[s] - mx);
  const float L = mx + logf(sum);
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  for (int s = 0; s < ns; ++s) {
    if (ls[s] == NEG_INF) continue;
    const float w = expf(ls[s] - L);
    const float* src = p.ws_o + (row * ns + s) * kHD + lane * PER;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = fmaf(w, src[e], acc[e]);
  }
  const int64_t hs = (int64_t)p.Hq * p.Sq;
  const int64_t b = row / hs, rem = row % hs;
  const int h = (int)(rem / p.Sq), i = (int)(rem % p.Sq);
  _Float16* dst = p.o + b * p.q_bstride + (int64_t)i * p.q_sstride + (int64_t)h * kHD + lane * PER;
#pragma unroll
  for (int e = 0; e < PER; ++e) dst[e] = (_Float16)acc[e];
  if (p.lse && lane == 0) p.lse[row] = L;
}

int64_t grid_blocks_decode(const Params& p) {
  const int64_t nb = (int64_t)p.B * p.Hkv * p.n_splits * p.n_qt;
  return nb > 0x7fffffff ? -1 : nb;
}

hipError_t launch_attn_decode(const Params& p, hipStream_t stream) {
  const int64_t nb = grid_blocks_decode(p);
  if (nb <= 0 || p.schedule != SCHEDULE_SERIAL4) return hipErrorInvalidValue;
  if (p.ring != 2 && p.ring != 4) return hipErrorInvalidValue;
  const dim3 grid((unsigned)nb), block(64 * waves_of(SCHEDULE_SERIAL4));
#define LIBATTN_SPLIT(R, H) hipLaunchKernelGGL((attn_fwd_kernel<SCHEDULE_SERIAL4, R, H, true>), grid, block, 0, stream, p)
  const bool r2 = p.ring == 2;
  if (p.hd == 64) {
    if (r2) LIBATTN_SPLIT(2, 64);
    else LIBATTN_SPLIT(4, 64);
  } else if (p.hd == 128) {
    if (r2) LIBATTN_SPLIT(2, 128);
    else LIBATTN_SPLIT(4, 128);
  } else if (p.hd == 256) {
    if (r2) LIBATTN_SPLIT(2, 256);
    else LIBATTN_SPLIT(4, 256);
  } else {
    return hipErrorInvalidValue;
  }
#undef LIBATTN_SPLIT
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)p.B * p.Hq * p.Sq;
  const int64_t cb = (rows + 3) / 4;
  if (cb > 0x7fffffff) return hipErrorInvalidValue;
  if (p.hd == 64)
    hipLaunchKernelGGL(attn_combine_kernel<64>, dim3((unsigned)cb), dim3(256), 0, stream, p, rows);
  else if (p.hd == 128)
    hipLaunchKernelGGL(attn_combine_kernel<128>, dim3((unsigned)cb), dim3(256), 0, stream, p, rows);
  else
    hipLaunchKernelGGL(attn_combine_kernel<256>, dim3((unsigned)cb), dim3(256), 0, stream, p, rows);
  return hipGetLastError();
}

}  // namespace libattn
