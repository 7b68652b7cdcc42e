// attn_wide.h -- the attention forward kernel with 64 query rows per wave
// (gfx950, CDNA4), as a template over the fragment prefetch depth and the
// placement of the softmax parts; attn_wide_even.hip, attn_wide_front.hip
// and attn_wide_early.hip compile one placement each (in parallel).
//
// One workgroup = 4 wavefronts, one per SIMD, one workgroup per CU.  A wave
// owns 64 query rows of one query head, as two 32-row halves (qb = 0, 1), so
// every K or V fragment read from LDS feeds two MFMAs (the 32-row kernel in
// attn_fwd.hip reads one fragment per MFMA): 0.75 LDS reads per MFMA instead
// of 1.5.  The four waves take four query heads of one KV head at the same 64
// query rows (hpw = 4 heads per workgroup; 2 heads x 128 rows or 1 head x 256
// rows when the GQA ratio is not a multiple of 4), so with hpw = 4 every wave
// has the same causal extent and no wave idles at a barrier.
//
// The tile loop is the overlap schedule of attn_fwd.hip re-cut for one wave
// per SIMD: iteration j runs the MFMAs of QK^T(j+1) and PV(j-1) with the
// softmax of tile j between them, in one instruction stream, so the matrix
// core, the VALU and the LDS work side by side inside each wave (the load /
// mma / softmax task split of page "PipeThreader: Software-Defined Pipelining
// ... (OSDI 2025)" summary, section "核心方法").  With no second wave on the
// SIMD to cover a wait, K/V tiles are loaded two iterations ahead into
// four-slot rings (the ping-pong buffers of page "AI编译器融合技术 -- 5.
// 并行性与分布式融合", section 5.4.2, two stages deeper): each wave waits only
// for the loads it issued in the previous iteration.
//
// Per query row the arithmetic is that of attn_fwd.hip -- the same MFMA k
// order, the same softmax parts in the same order, the sum check decided per
// 32-row half (one ballot per half, as one 32-row wave there decides) -- so
// the results are bitwise identical to its schedules.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "attn_kernel.h"
#include "attn_tile.h"
#include "gfx950.h"

namespace libattn {

namespace {

constexpr int W_NW = 4;      // waves per workgroup
constexpr int W_SLOTS = 4;   // slots of the K ring and of the V ring

// Steps of a wide mma block.  A QK step (kk, x = sb, qb) adds
// K[32sb.., 16kk..] x Q^T[16kk.., 32qb..] into S^T block (sb, qb); a PV step
// (kk, x = db, qb) adds V^T[32db.., 16kk..] x P^T[16kk.., 32qb..] into O^T
// block (db, qb).  Steps 2f and 2f+1 share fragment f (the two query halves).
//   mode 1 (32 steps): PV only, g = i/2: PV(g/4, g%4, i%2); the next MFMA on
//          the same O^T block is 8 steps later
//   mode 2 (32 steps): QK only, g = i/2: QK(g/2, g%2, i%2); the same S^T
//          block 4 steps later
//   mode 0 (64 steps): the PV steps of mode 1, then the QK steps of mode 2.
//          The next S^T is built only in the second half, while the first
//          half's softmax has already consumed half of the current S^T, so
//          the two S^T tiles are never both live in full.
// Every accumulator sees its k steps in increasing order.
struct WStep {
  bool pv;
  int kk, x, qb;
};
__host__ __device__ constexpr WStep wstep_of(int mode, int i) {
  return mode == 1 || mode == 3 ? WStep{true, (i >> 1) >> 2, (i >> 1) & 3, i & 1}
         : mode == 2 ? WStep{false, (i >> 1) >> 1, (i >> 1) & 1, i & 1}
         : i < 32    ? wstep_of(1, i)
                     : wstep_of(2, i - 32);
}
constexpr int wsteps_of(int mode) { return mode == 0 ? 64 : 32; }
// mode 3 is mode 1 for a last tile that is the causal diagonal at 64-row
// query blocks: P^T of query half 0 is zero for keys 32..63 of the tile, so
// those 8 PV steps issue no MFMA.
__host__ __device__ constexpr bool wstep_dropped(int mode, int i) {
  return mode == 3 && wstep_of(mode, i).kk >= 2 && wstep_of(mode, i).qb == 0;
}

}  // namespace

static_assert(W_SLOTS * (Geo<128>::K_TILEB + Geo<128>::V_TILEB) <= 160 * 1024, "the rings fit the 160 KiB LDS");

// The QK^T MFMAs are written as assembly so that their operands sit in the
// right register file: Q^T, only ever an MFMA operand, in AGPRs (an MFMA takes
// A and B from either file) and S^T, which the softmax reads, in VGPRs.  Left
// to itself the register allocator does the opposite at 64 query rows per
// wave and copies S^T out of AGPRs every tile.  The PV MFMAs stay builtins
// (their accumulator O^T lives in AGPRs either way).  The compiler's hazard
// pass does not see into assembly, so around the QK^T MFMAs the code keeps
// the dependency rules itself:
//  - a VALU access to an S^T written here comes 18 or more wait states
//    later: in the tile loop the softmax reads S^T an iteration after the
//    MFMAs wrote it; elsewhere s_drain() stands between, with S^T as an
//    operand so that no reader can be scheduled ahead of it;
//  - their operands are written by loads (K fragments from LDS, Q^T from
//    memory) or by the MFMA chain itself, not by the VALU just before;
//  - the accumulation chains reuse their destination as C exactly, which the
//    hardware orders by itself.
// tests/test_asm_hazards.py scans the compiled kernel for VALU accesses close
// to an MFMA result and for VALU writes just before an MFMA read.
__device__ __forceinline__ void qk_first(f32x16& d, const f16x8& a, const f16x8& q) {
  asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(q));
}
__device__ __forceinline__ void qk_next(f32x16& d, const f16x8& a, const f16x8& q) {
  asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(q));
}
// qk_first / qk_next with the dependency wait states inside the assembly:
// 5 before the MFMA (a VALU write of an operand just before it) and 19 after
// it (any access to the result), for code where the compiler may put copies
// of the operands or the result right next to the MFMA.
__device__ __forceinline__ void qk_first_guarded(f32x16& d, const f16x8& a, const f16x8& q) {
  asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, 0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 2"
               : "=&v"(d) : "v"(a), "a"(q));
}
__device__ __forceinline__ void qk_next_guarded(f32x16& d, const f16x8& a, const f16x8& q) {
  asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_f16 %0, %1, %2, %0\n\ts_nop 7\n\ts_nop 7\n\ts_nop 2"
               : "+v"(d) : "v"(a), "a"(q));
}
// 19 wait states after the MFMAs that wrote x and y, before any use of them
__device__ __forceinline__ void s_drain(f32x16& x, f32x16& y) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 2" : "+v"(x), "+v"(y));
}
// A Q^T fragment loaded straight into AGPRs (16 bytes per lane).  The caller
// makes sure the load has landed before an MFMA reads it.
__device__ __forceinline__ void load_agprs(f16x8& x, const void* src) {
  asm volatile("global_load_dwordx4 %0, %1, off" : "=a"(x) : "v"(src) : "memory");
}
// Zeroes an AGPR-resident fragment, one register at a time, inside assembly.
__device__ __forceinline__ void zero_agprs(f16x8& x) {
  u32x4 w = __builtin_bit_cast(u32x4, x);
  static_for<4>([&](auto ic) INL {
    uint32_t e = w[decltype(ic)::value];
    asm volatile("v_accvgpr_write_b32 %0, 0" : "=a"(e));
    w[decltype(ic)::value] = e;
  });
  x = __builtin_bit_cast(f16x8, w);
}
// o *= alpha on an AGPR-resident accumulator, one element at a time through a
// VGPR temporary, inside assembly.  Written as plain C++, the rare rescale of
// O^T (VALU work on the accumulator) leads the register allocator to stage
// all of O^T through VGPRs and spill at 64 query rows per wave; this way no
// VALU work on O^T is visible to it.  The hazard pass does not see the
// accumulator reads and writes inside: the caller puts the last MFMA that
// wrote o well before (a 16-MFMA recompute stands between), and the trailing
// s_nop keeps an MFMA that reads o right after at a distance.
__device__ __forceinline__ void scale_acc(f32x16& o, float alpha) {
  static_for<16>([&](auto ic) INL {
    constexpr int i = decltype(ic)::value;
    float e = o[i], tmp;
    asm volatile(
        "v_accvgpr_read_b32 %1, %0\n\t"
        "v_mul_f32 %1, %1, %2\n\t"
        "v_accvgpr_write_b32 %0, %1"
        : "+a"(e), "=&v"(tmp)
        : "v"(alpha));
    o[i] = e;
  });
  asm volatile("s_nop 4" ::: "memory");
}

// kRing: fragments (of two MFMAs each) read ahead of the MFMA that uses them.
// kPlace: where the softmax parts sit among the MFMAs of the fused block
// (Place in variant.h).
template <int kRing, int kPlace>
__global__ __launch_bounds__(64 * W_NW, 1) void attn_wide_kernel(Params p) {
  using G = Geo<128>;
  constexpr int NW = W_NW, NS = W_SLOTS;
  constexpr int K_ROWB = G::K_ROWB, K_TILEB = G::K_TILEB, K_DMA = G::K_DMA;
  constexpr int V_ROWB = G::V_ROWB, V_TILEB = G::V_TILEB;
  constexpr int K_DMA_PER_WAVE = (K_DMA + NW - 1) / NW;  // wave w issues K instructions w, w+4, ...
  constexpr int V_DMA_PER_WAVE = G::V_DMA / NW;          // and V instructions w, w+4, ...
  static_assert(G::V_DMA % NW == 0, "every wave issues the same number of V instructions");
  __shared__ __attribute__((aligned(1024))) char k_smem[NS * K_TILEB];
  __shared__ __attribute__((aligned(1024))) char v_smem[NS * V_TILEB];
  LDS char* const k_lds = (LDS char*)k_smem;
  LDS char* const v_lds = (LDS char*)v_smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;   // query column of this lane in a 32-row half of S^T / O^T
  const int hh = lane >> 5;  // lane half

  // ---- workgroup -> (batch, kv head, head group, query tile), as in
  // attn_fwd.hip: XCD-aware grouping and longest causal tiles first.
  const int hpw = p.hpw;           // heads per workgroup: 4, 2 or 1
  const int bmw = 64 * (NW / hpw); // query rows per workgroup and head
  const int items = p.pairs * p.n_qt;
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
  const int t = p.lpt ? p.n_qt - 1 - item / p.pairs : item / p.pairs;
  const int wh = wave % hpw, wr = wave / hpw;
  const int hl = hpw * (item % p.pairs) + wh;  // head inside the KV group
  const bool active = hl < p.g;
  const int h = c * p.g + (active ? hl : 0);

  const int Sq = p.Sq, Sk = p.Sk;
  const int off = p.off;          // causal: query row i attends keys j <= i + off
  const int q0 = t * bmw;
  const int qw = q0 + 64 * wr;    // first query row of this wave
  const int kv_tiles_all = (Sk + BN - 1) / BN;
  const int n_tiles = p.causal ? min(kv_tiles_all, (q0 + off + bmw + BN - 1) / BN) : kv_tiles_all;
  const int n_full = min(n_tiles, Sk / BN);  // tiles [0, n_full) exist and hold BN keys

  const _Float16* kb_ = p.k + (int64_t)b * p.kv_bstride + (int64_t)c * 128;
  const _Float16* vb_ = p.v + (int64_t)b * p.kv_bstride + (int64_t)c * 128;

  // ---- Q^T fragments of both halves (B operand of S^T = K Q^T), resident in
  // AGPRs for the whole loop, loaded straight into them; rows past Sq are
  // zero.  These loads precede every K/V load and loads complete in issue
  // order, so the prologue's wait for K_0 and K_1 also covers them.  A
  // negative scale is applied through the sign of the softmax's scale factor
  // rather than by negating Q, which leaves the same bits.
  f16x8 qf[2][8];
  {
    const _Float16* qb_ = p.q + (int64_t)b * p.q_bstride + (int64_t)h * 128;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qrow = qw + 32 * qb + n;
      const _Float16* src = qb_ + (int64_t)qrow * p.q_sstride + 8 * hh;
      if (active && qrow < Sq) {
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) load_agprs(qf[qb][kk], src + 16 * kk);
      } else {
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) zero_agprs(qf[qb][kk]);
      }
    }
  }

  // ---- K/V staging by direct global -> LDS loads: tile t goes to slot t % 4
  // of its ring.  Lane slots as in attn_fwd.hip; rows past the end of the
  // keys are loaded from row Sk-1 (finite data whose weights are masked).
  const uint32_t row_bytes = (uint32_t)p.kv_sstride * 2;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const uint32_t k_lds_base = (uint32_t)(uintptr_t)k_lds, v_lds_base = (uint32_t)(uintptr_t)v_lds;
  // K instruction u of this wave covers 16-byte lane slot 64*(wave + 4u) + lane
  // of the tile: key row o / 17, chunk o % 17 (the 17th, the padding slot,
  // loads the row's last chunk again)
  auto k_rowcol = [&](int u, int& row, uint32_t& col) INL {
    const int o = 64 * (wave + NW * u) + lane;
    row = o / (K_ROWB / 16);
    const int cb = o - row * (K_ROWB / 16);
    col = 16u * (uint32_t)(cb < G::KC ? cb : G::KC - 1);
  };
  // lane slot 1024 + lane of the tile (the 17th KiB), for every wave, and the
  // 16 lanes of it this wave loads in the steady state
  uint32_t k16_off;
  {
    const int o = 64 * 16 + lane, row = o / (K_ROWB / 16), cb = o - row * (K_ROWB / 16);
    k16_off = (uint32_t)row * (uint32_t)p.kv_sstride * 2 + 16u * (uint32_t)(cb < G::KC ? cb : G::KC - 1);
  }
  const uint64_t k16_lanes = 0xffffull << (16 * __builtin_amdgcn_readfirstlane(wave));
  uint32_t k_off[K_DMA_PER_WAVE];  // byte offsets inside a full tile
#pragma unroll
  for (int u = 0; u < K_DMA_PER_WAVE; ++u) {
    int row;
    uint32_t col;
    k_rowcol(u, row, col);
    k_off[u] = (uint32_t)row * row_bytes + col;
  }
  // V instruction u of this wave covers rows 4*(wave + 4u) .. +3, lane l the
  // 16 bytes of row l / 16 stored at swizzled chunk l % 16
  const int v_rowl = lane / G::KC;
  static_assert(NW * G::V_ROWS_PER_DMA % 4 == 0, "one V column per lane");
  const uint32_t v_col = 16u * (uint32_t)((lane % G::KC) ^ G::vswz(G::V_ROWS_PER_DMA * wave + v_rowl));
  const uint32_t v_off = (uint32_t)v_rowl * row_bytes + v_col;
  // Issues this wave's loads of K tile tk and V tile tv (tiles outside
  // [0, n_tiles): nothing) and returns how many load instructions it issued.
  auto stage = [&](int tk, int tv) INL -> int {
    tk = __builtin_amdgcn_readfirstlane(tk);
    tv = __builtin_amdgcn_readfirstlane(tv);
    int issued = 0;
    if (tk >= 0 && tk < n_tiles) {
      const char* base = (const char*)kb_ + (int64_t)tk * BN * row_bytes;
      const bool full = (tk + 1) * BN <= Sk;
      const uint32_t slot = k_lds_base + (uint32_t)(tk % NS) * K_TILEB;
#pragma unroll
      for (int u = 0; u < K_DMA_PER_WAVE; ++u) {
        const int i = wave_s + NW * u;
        if (i < K_DMA) {
          uint32_t o = k_off[u];
          if (!full) {
            int row;
            uint32_t col;
            k_rowcol(u, row, col);
            o = (uint32_t)min(row, Sk - 1 - tk * BN) * row_bytes + col;
          }
          dma16(base, o, slot + 1024 * i);
          ++issued;
        }
      }
    }
    if (tv >= 0 && tv < n_tiles) {
      const bool full = (tv + 1) * BN <= Sk;
      const uint32_t slot = v_lds_base + (uint32_t)(tv % NS) * V_TILEB;
#pragma unroll
      for (int u = 0; u < V_DMA_PER_WAVE; ++u) {
        const int i = wave_s + NW * u;
        const int row0 = G::V_ROWS_PER_DMA * i;  // first row of the instruction (wave-uniform)
        if (full) {
          const char* base = (const char*)vb_ + ((int64_t)tv * BN + row0) * row_bytes;
          dma16(base, v_off, slot + 1024 * i);
        } else {
          const char* base = (const char*)vb_ + (int64_t)tv * BN * row_bytes;
          const int row = min(row0 + v_rowl, Sk - 1 - tv * BN);
          dma16(base, (uint32_t)row * row_bytes + v_col, slot + 1024 * i);
        }
      }
      issued += V_DMA_PER_WAVE;
    }
    return issued;
  };
  // The steady-state case of stage(): both tiles exist and are full, so every
  // wave issues a fixed set of nine loads with no per-instruction tests (the
  // 17th K instruction is split over the four waves, 16 lanes each); returns
  // the count as stage() does.
  auto stage_full = [&](int tk, int tv) INL -> int {
    tk = __builtin_amdgcn_readfirstlane(tk);
    tv = __builtin_amdgcn_readfirstlane(tv);
    const char* kbase = (const char*)kb_ + (int64_t)tk * BN * row_bytes;
    const uint32_t kslot = k_lds_base + (uint32_t)(tk % NS) * K_TILEB + 1024u * (uint32_t)wave_s;
#pragma unroll
    for (int u = 0; u < 4; ++u) dma16_m0(kbase, k_off[u], kslot + 1024u * NW * u);
    const uint32_t vslot = v_lds_base + (uint32_t)(tv % NS) * V_TILEB + 1024u * (uint32_t)wave_s;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int row0 = G::V_ROWS_PER_DMA * (wave_s + NW * u);
      dma16_m0((const char*)vb_ + ((int64_t)tv * BN + row0) * row_bytes, v_off, vslot + 1024u * NW * u);
    }
    static_assert(K_DMA == 4 * NW + 1 && K_DMA_PER_WAVE == 5, "K tile: 16 instructions over the waves, one more");
    // the 17th KiB: every wave loads the 16 lane slots 16*wave .. 16*wave+15 of it
    dma16_m0_lanes(kbase, k16_off, kslot - 1024u * (uint32_t)wave_s + 1024u * 16, k16_lanes);
    return 9;
  };
  // Waits until at most `young` of this wave's loads are in flight.  Loads
  // complete in issue order, so with `young` no larger than the count issued
  // last, every older load has landed.
  auto wait_older = [&](int young) INL {
    if (young >= 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else if (young >= 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };

  // per-lane fragment bases (bytes), as in attn_fwd.hip
  const int k_frag = n * K_ROWB + 16 * hh;
  int v_frag[4];
  {
    const int vg = lane >> 4, vsl = lane & 15;
    const int r0 = 4 * (vg >> 1) + (vsl >> 2);
    const int c0 = 2 * (vg & 1) + ((vsl & 3) >> 1);
    const int f0 = r0 * V_ROWB + ((c0 ^ G::vswz(r0)) << 4) + ((vsl & 1) << 3);
#pragma unroll
    for (int db = 0; db < 4; ++db) v_frag[db] = f0 ^ (64 * db);
  }
  auto frag_qk = [&](uint32_t kslot, int kk, int sb) INL -> f16x8 {
    return *(const LDS f16x8*)(k_lds + kslot + k_frag + 32 * sb * K_ROWB + 32 * kk);
  };
  auto frag_pv = [&](uint32_t vslot, int kk, int db) INL -> f16x8 {
    const LDS char* a = v_lds + vslot + v_frag[db] + 16 * kk * V_ROWB;
    const f16x4 h1 = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)a));
    const f16x4 h2 = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)(a + 8 * V_ROWB)));
    return f16x8{h1[0], h1[1], h1[2], h1[3], h2[0], h2[1], h2[2], h2[3]};
  };
  auto kslot_of = [](int j) INL -> uint32_t { return (uint32_t)K_TILEB * (uint32_t)(j & (NS - 1)); };
  auto vslot_of = [](int j) INL -> uint32_t { return (uint32_t)V_TILEB * (uint32_t)(j & (NS - 1)); };

  f32x16 o_acc[4][2];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) o_acc[db][qb] = f32x16{};
  float m_run[2] = {M_INIT, M_INIT};  // running max (log2 units) per query half
  float l_run[2] = {0.f, 0.f};        // running sum of 2^(score - m_run), from the fp16 P
  const float cs = p.neg ? -p.cs : p.cs;  // scale * log2(e), with the sign of the scale

  // ---- softmax sTask of one tile, for both query halves.  The parts are
  // those of attn_fwd.hip, per half: E (exponential of one score; every
  // second part packs the previous pair to fp16 and adds it to the row sum),
  // the row sum across the lane pair, the sum check per half, and on its
  // failure (or the first tile) the tile max, the running-max update and the
  // exponentials again.
  //
  // Score k = 0..31 of a half (E order: pair k/2, element k%2, S^T block
  // sb = k/16, accumulator element r = 2((k/2) % 8) + k%2) is key
  // j*BN + 32sb + 8(r/4) + 4hh + r%4 of tile j.  Its offset 32sb + 8(r/4) +
  // r%4 grows with k, so the keys a mask keeps form a prefix in E order: a
  // masked tile carries one bit field per half, bit k set when score k is
  // kept, and a masked score costs a bit extract and an AND instead of a
  // compare (whose 64-bit lane-mask result would occupy scalar registers).
  struct WSm {
    uint32_t keep[2]; // masked tiles: bit k set when score k of the half is allowed
    float negm[2];    // -(running max) used by the exponentials
    float t[2][2][2]; // exponentials of the last two pairs, per half
    float rq[2][2];   // row-sum partials, per half
    float rs[2];      // row sums of the tile
    bool redo[2];     // the sum check failed for some row of the half
  };
  auto sm_keep = [&](int j, auto masked, WSm& st) INL {
    if constexpr (decltype(masked)::value) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int query = qw + 32 * qb + n;
        const int end = p.causal ? min(Sk, query + off + 1) : Sk;
        // kept offsets are those below lim; 4 of every 8 offsets belong to this lane
        const int lim = min(max(end - j * BN - 4 * hh, 0), 64);
        const int cnt = 4 * (lim >> 3) + min(lim & 7, 4);
        st.keep[qb] = cnt >= 32 ? 0xffffffffu : (1u << cnt) - 1u;
      }
    }
  };
  // all ones if score k is kept, else 0.  Written as assembly so that the
  // compiler cannot turn the one-bit extract back into a compare and select.
  auto keep_bits = [](uint32_t keep, auto kc) INL -> uint32_t {
    uint32_t m;
    asm("v_bfe_i32 %0, %1, %2, 1" : "=v"(m) : "v"(keep), "i"(decltype(kc)::value));
    return m;
  };
  // x where the mask is all ones, -inf where it is 0
  auto or_neg_inf = [](float x, uint32_t m) INL -> float {
    return __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, x) & m) | (0xff800000u & ~m));
  };
  auto sm_start = [&](WSm& st) INL {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      st.negm[qb] = -m_run[qb];
      st.rq[qb][0] = 0.f;
      st.rq[qb][1] = 0.f;
    }
  };
  // pack pair pp of half qb to fp16 P^T and into the row sum
  auto pack = [&](auto qbc, auto pc, f16x8 (&pd)[2][4], WSm& st) INL {
    constexpr int qb = decltype(qbc)::value, pp = decltype(pc)::value, kk = pp >> 2, c2 = 2 * (pp & 3);
    pd[qb][kk][c2] = (_Float16)st.t[qb][pp & 1][0];
    pd[qb][kk][c2 + 1] = (_Float16)st.t[qb][pp & 1][1];
    add_pair_f16(st.rq[qb][kk & 1], f16x2{pd[qb][kk][c2], pd[qb][kk][c2 + 1]});
    // PLACE_EARLY: the conversions stay at this step; otherwise the compiler
    // is free to sink them to the first use of the fragment
    if constexpr (kPlace == PLACE_EARLY) asm volatile("" : "+v"(pd[qb][kk]));
  };
  // E part e of half qb (e = 0..31: score e; 32: the last pack; 33: row sum)
  auto sm_eh = [&](auto qbc, auto ec, f32x16 (&sc)[2][2], f16x8 (&pd)[2][4], auto masked, WSm& st) INL {
    constexpr int qb = decltype(qbc)::value, e = decltype(ec)::value;
    if constexpr (e < 32) {
      constexpr int pair = e >> 1, u = e & 1, sb = pair >> 3, r = 2 * (pair & 7) + u;
      float arg = __builtin_fmaf(sc[sb][qb][r], cs, st.negm[qb]);
      // a masked score's exponent argument becomes -inf, whose exponential is exactly 0
      if constexpr (decltype(masked)::value) arg = or_neg_inf(arg, keep_bits(st.keep[qb], ec));
      st.t[qb][pair & 1][u] = __builtin_amdgcn_exp2f(arg);
      if constexpr (u == 1 && pair >= 1) pack(qbc, std::integral_constant<int, pair - 1>{}, pd, st);
    } else if constexpr (e == 32) {
      pack(qbc, std::integral_constant<int, 15>{}, pd, st);
    } else {
      static_assert(e == 33, "exp part index");
      st.rs[qb] = pair_sum(st.rq[qb][0] + st.rq[qb][1]);
      // the sum check (wave-uniform); !(rs <= RS_MAX) also catches an infinite sum
      st.redo[qb] = __builtin_amdgcn_ballot_w64(!(st.rs[qb] <= RS_MAX)) != 0;
    }
  };
  constexpr int SM_EH = 34;  // E parts of one half
  // tile max of half qb, running-max update; returns alpha = 2^(m_old - m_new)
  const bool neg = p.neg != 0;
  auto sm_max = [&](auto qbc, f32x16 (&sc)[2][2], auto masked, WSm& st) INL -> float {
    constexpr int qb = decltype(qbc)::value;
    float mq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) mq[q] = NEG_INF;
    static_for<32>([&](auto kc) INL {
      constexpr int k = decltype(kc)::value, pair = k >> 1, sb = pair >> 3, r = 2 * (pair & 7) + (k & 1);
      float s = neg ? -sc[sb][qb][r] : sc[sb][qb][r];  // scale * s = |scale| * (+-s)
      if constexpr (decltype(masked)::value) s = or_neg_inf(s, keep_bits(st.keep[qb], kc));
      mq[k >> 3] = fmaxf(mq[k >> 3], s);
    });
    const float mt = pair_max(fmaxf(fmaxf(mq[0], mq[1]), fmaxf(mq[2], mq[3])));
    const float mts = (mt == NEG_INF) ? NEG_INF : mt * p.cs;
    const float m_new = fmaxf(m_run[qb], mts);
    const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
    m_run[qb] = m_new;
    st.negm[qb] = -m_new;
    st.rq[qb][0] = 0.f;
    st.rq[qb][1] = 0.f;
    return alpha;
  };

  // ---- one block of mma steps with softmax parts placed before its MFMAs:
  // step i is "the parts placed there (sm(i)), MFMA i, then (after the second
  // MFMA of a fragment) the LDS reads of the fragment kRing ahead"; a
  // scheduling barrier keeps each step in place.
  auto block = [&](auto mode_c, uint32_t kslot, f32x16 (&sd)[2][2], uint32_t vslot, f16x8 (&ps)[2][4], auto sm) INL {
    constexpr int mode = decltype(mode_c)::value;
    constexpr int nsteps = wsteps_of(mode), nfr = nsteps / 2;
    auto load = [&](auto fc) INL -> f16x8 {
      constexpr WStep st = wstep_of(mode, 2 * decltype(fc)::value);
      if constexpr (st.pv) return frag_pv(vslot, st.kk, st.x);
      else return frag_qk(kslot, st.kk, st.x);
    };
    f16x8 fr[kRing];
    static_for<kRing>([&](auto fc) INL {
      if constexpr (decltype(fc)::value < nfr) fr[decltype(fc)::value] = load(fc);
    });
    static_for<nsteps>([&](auto ic) INL {
      constexpr int i = decltype(ic)::value, f = i >> 1;
      constexpr WStep st = wstep_of(mode, i);
      sm(ic);
      const f16x8 a = fr[f % kRing];
      if constexpr (st.pv) {
        if constexpr (!wstep_dropped(mode, i))
          o_acc[st.x][st.qb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, ps[st.qb][st.kk], o_acc[st.x][st.qb], 0, 0, 0);
      } else if constexpr (st.kk == 0) {
        qk_first(sd[st.x][st.qb], a, qf[st.qb][0]);
      } else {
        qk_next(sd[st.x][st.qb], a, qf[st.qb][st.kk]);
      }
      if constexpr ((i & 1) && f + kRing < nfr) fr[f % kRing] = load(std::integral_constant<int, f + kRing>{});
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  auto no_sm = [](auto) INL {};
  using M_FUSED = std::integral_constant<int, 0>;
  using M_PV = std::integral_constant<int, 1>;
  using M_QK = std::integral_constant<int, 2>;
  using T = std::true_type;
  using F = std::false_type;
  using Q0 = std::integral_constant<int, 0>;
  using Q1 = std::integral_constant<int, 1>;

  // S^T of one half of tile j again, from K_j (still in its slot): the QK
  // steps of that half in the order of mode 2
  auto recompute_half = [&](auto qbc, int j, f32x16 (&sc)[2][2]) INL {
    constexpr int qb = decltype(qbc)::value;
    const uint32_t kslot = kslot_of(j);
    static_for<16>([&](auto ic) INL {
      constexpr int i = decltype(ic)::value, kk = i >> 1, sb = i & 1;
      // The register allocator may move S^T between these MFMAs in this rare
      // path, so each one carries its own wait states on both sides.
      const f16x8 a = frag_qk(kslot, kk, sb);
      if constexpr (kk == 0) qk_first_guarded(sc[sb][qb], a, qf[qb][0]);
      else qk_next_guarded(sc[sb][qb], a, qf[qb][kk]);
      __builtin_amdgcn_sched_barrier(0);  // one fragment in flight: this path is rare
    });
  };
  // the sum check of half qb of tile j; on failure the tile max (S^T of the
  // half recomputed), the running-max update and the exponentials again, and
  // O^T of that half rescaled; then l.  In the last iteration (no QK^T, so no
  // second S^T set to make room for) S^T is kept instead of recomputed: Q^T
  // is then dead after the last QK^T block (kept alive for a recompute there,
  // it was spilled to scratch at every work item's end).  Same bits either
  // way: a recomputed S^T equals the first one.
  auto sm_finish = [&](auto qbc, int j, f32x16 (&sc)[2][2], f16x8 (&pd)[2][4], auto masked, WSm& st,
                       auto recompute) INL {
    constexpr int qb = decltype(qbc)::value;
    float alpha = 1.0f;
    if (__builtin_expect(st.redo[qb], 0)) {
      if constexpr (decltype(recompute)::value) {
        recompute_half(qbc, j, sc);  // 16 guarded MFMAs: O^T's last PV MFMA is far behind too
      } else {
        // O^T's last PV MFMA may be just before: keep the rescale below apart from it
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 2" ::: "memory");
      }
      alpha = sm_max(qbc, sc, masked, st);
      static_for<SM_EH>([&](auto ec) INL { sm_eh(qbc, ec, sc, pd, masked, st); });
      static_for<4>([&](auto dc) INL { scale_acc(o_acc[decltype(dc)::value][qb], alpha); });
    }
    l_run[qb] = __builtin_fmaf(l_run[qb], alpha, st.rs[qb]);
  };

  // ---- the tile loop.  Iteration j: PV of tile j-1 with the softmax of
  // half 0 of tile j between its MFMAs, then QK^T of tile j+1 with the
  // softmax of half 1; then the sum checks of tile j (O *= alpha_j after
  // PV(j-1)) and the loads: iteration j issues K_{j+3} and V_{j+1} into the
  // slots of K_{j-1} and V_{j-3} (last read in iteration j-1 and j-2), and at
  // its end waits for the loads it issued in iteration j-1 (K_{j+2}, V_j)
  // before the barrier.  K_j stays in its slot through iteration j, for a
  // redo.  S^T and P^T alternate between two register sets, so the loop is
  // unrolled twice; on entry to each loop S^T of tile j is in sa and P^T of
  // tile j-1 in pa.
  //
  // As in attn_fwd.hip's overlap schedule no wave skips a tile: a tile wholly
  // above a wave's diagonal (hpw < 4 only) is computed with every key masked,
  // an exact no-op.  Waves of a missing head (hl >= g) compute head c*g and
  // store nothing.
  f32x16 sa[2][2], sb[2][2];
  f16x8 pa[2][4], pb[2][4];
  const uint64_t tile_bytes = (uint64_t)BN * row_bytes;
  const uint64_t dv_wave = (uint64_t)(G::V_ROWS_PER_DMA * wave_s) * row_bytes;
  const char* dk_run = (const char*)kb_ + 4 * tile_bytes;
  const char* dv_run = (const char*)vb_ + 2 * tile_bytes + dv_wave;
  // dma_in: the loads of K_{j+3} and V_{j+1} are issued one by one between the
  // MFMAs of the fused block (steps 3, 10, ..., 59), both tiles full (j + 3 <
  // n_full); otherwise stage() issues them before the block
  auto iter = [&](int j, auto with_pv, auto with_qk, auto mask_e, auto dma_in, f32x16 (&sc)[2][2],
                  f32x16 (&sn)[2][2], f16x8 (&pp)[2][4], f16x8 (&pc)[2][4]) INL {
    constexpr bool kPV = decltype(with_pv)::value, kQK = decltype(with_qk)::value;
    constexpr bool kDmaIn = decltype(dma_in)::value;
    static_assert(!kDmaIn || (kPV && kQK), "loads inside the fused block only");
    int issued;
    if constexpr (kDmaIn) issued = 9;
    else issued = j + 3 < n_full ? stage_full(j + 3, j + 1) : stage(j + 3, j + 1);
    WSm st;
    sm_keep(j, mask_e, st);
    sm_start(st);
    const uint32_t kslot = kslot_of(j + 1), vslot = vslot_of(j + 3);  // K_{j+1}; V_{j-1} (slot (j-1) % 4)
    // the loads of the in-block case: d = 0..3 K instructions u = d, d = 4..7
    // V instructions u = d - 4, d = 8 this wave's quarter of the 17th K KiB
    const int tk = __builtin_amdgcn_readfirstlane(j + 3), tv = __builtin_amdgcn_readfirstlane(j + 1);
    const char* dk_base = dk_run;
    const uint32_t dk_slot = k_lds_base + ((uint32_t)tk & (NS - 1)) * K_TILEB + 1024u * (uint32_t)wave_s;
    const char* dv_base = dv_run;
    if constexpr (kDmaIn) {
      dk_run += tile_bytes;
      dv_run += tile_bytes;
    }
    const uint32_t dv_slot = v_lds_base + ((uint32_t)tv & (NS - 1)) * V_TILEB + 1024u * (uint32_t)wave_s;
    auto dma_at = [&](auto ic) INL {
      constexpr int i = decltype(ic)::value, d = (i - 3) / 7;
      if constexpr (kDmaIn && i >= 3 && (i - 3) % 7 == 0 && d < 9) {
        if constexpr (d < 4) {
          dma16_m0_plus<1024u * NW * d>(dk_base, k_off[d], dk_slot);
        } else if constexpr (d < 8) {
          constexpr int u = d - 4;
          dma16_m0_plus<1024u * NW * u>(dv_base + (int64_t)(G::V_ROWS_PER_DMA * NW * u) * row_bytes, v_off, dv_slot);
        } else {
          dma16_m0_lanes(dk_base, k16_off, dk_slot - 1024u * (uint32_t)wave_s + 1024u * 16, k16_lanes);
        }
      }
    };
    if constexpr (kPV && kQK) {
      // half 0's parts over the 32 PV steps, half 1's over the 32 QK steps:
      // part e of a half before step floor(e * 31 / 33) of its half
      // (PLACE_EVEN); PLACE_FRONT puts half 0's first five parts before the
      // first MFMA and spreads the rest over steps 1..31; PLACE_EARLY spreads
      // half 1's parts over its first 28 steps
      auto sm = [&](auto ic) INL {
        constexpr int i = decltype(ic)::value;
        dma_at(ic);
        static_for<SM_EH>([&](auto ec) INL {
          constexpr int e = decltype(ec)::value, at = e * 31 / (SM_EH - 1);
          constexpr int FR = 5;
          constexpr int at0 = kPlace == PLACE_FRONT ? (e < FR ? 0 : 1 + (e - FR) * 30 / (SM_EH - 1 - FR)) : at;
          constexpr int at1 = kPlace == PLACE_EARLY ? e * 27 / (SM_EH - 1) : at;
          if constexpr (i < 32 && at0 == i) sm_eh(Q0{}, ec, sc, pc, mask_e, st);
          if constexpr (i >= 32 && at1 == i - 32) sm_eh(Q1{}, ec, sc, pc, mask_e, st);
        });
      };
      block(M_FUSED{}, kslot, sn, vslot, pp, sm);
    } else if constexpr (kQK || kPV) {
      // both halves' parts over the 32 steps
      auto sm = [&](auto ic) INL {
        constexpr int i = decltype(ic)::value;
        static_for<2 * SM_EH>([&](auto ec) INL {
          constexpr int e = decltype(ec)::value;
          if constexpr (e * 31 / (2 * SM_EH - 1) == i) {
            if constexpr (e < SM_EH) sm_eh(Q0{}, ec, sc, pc, mask_e, st);
            else sm_eh(Q1{}, std::integral_constant<int, e - SM_EH>{}, sc, pc, mask_e, st);
          }
        });
      };
      if constexpr (kQK) block(M_QK{}, kslot, sn, vslot, pp, sm);
      else block(M_PV{}, kslot, sn, vslot, pp, sm);
    } else {
      static_for<SM_EH>([&](auto ec) INL { sm_eh(Q0{}, ec, sc, pc, mask_e, st); });
      static_for<SM_EH>([&](auto ec) INL { sm_eh(Q1{}, ec, sc, pc, mask_e, st); });
    }
    sm_finish(Q0{}, j, sc, pc, mask_e, st, with_qk);
    sm_finish(Q1{}, j, sc, pc, mask_e, st, with_qk);
    wait_older(issued);
    lds_barrier();
  };
  auto to_a = [&]() INL {
    s_drain(sb[0][0], sb[1][0]);
    s_drain(sb[0][1], sb[1][1]);
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 2; ++y) sa[x][y] = sb[x][y];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) pa[x][y] = pb[x][y];
  };
  // Tiles below j_ms need no mask for any wave of the workgroup.  The first
  // and the last iteration always take the masked path.
  const int j_ms = min(n_tiles, p.causal ? min(q0 + off, Sk) / BN : Sk / BN);
  // The last tile is the causal diagonal at 64-row query blocks when its
  // keys 32..63 all lie past the last key query half 0 of this wave may see:
  // the final PV block then drops those steps for that half (mode 3).
  const bool diag_tail = p.causal && (n_tiles - 1) * BN + 32 >= qw + 31 + off + 1;

  // prologue: K_0, V_0 and K_1 landed, K_2 in flight; S^T of tile 0 and its
  // max (the first tile of a row: the textbook online-softmax step, max
  // first).  Iteration 0 loads into fresh slots, so no barrier follows.
  stage(0, 0);
  stage(1, -1);
  const int issued2 = stage(2, -1);
  wait_older(issued2);
  lds_barrier();
  block(M_QK{}, kslot_of(0), sa, 0u, pa, no_sm);
  s_drain(sa[0][0], sa[1][0]);
  s_drain(sa[0][1], sa[1][1]);
  {
    WSm st;
    sm_keep(0, T{}, st);
    sm_max(Q0{}, sa, T{}, st);
    sm_max(Q1{}, sa, T{}, st);
  }
  // iterations [j, j_end) of the full mma block, in pairs that swap the
  // register sets; an odd one at the end hands its sets back
  auto run = [&](int& j, int j_end, auto mask_e, auto dma_in) INL {
    for (; j + 1 < j_end; j += 2) {
      iter(j, T{}, T{}, mask_e, dma_in, sa, sb, pa, pb);
      iter(j + 1, T{}, T{}, mask_e, dma_in, sb, sa, pb, pa);
    }
    if (j < j_end) {
      iter(j, T{}, T{}, mask_e, dma_in, sa, sb, pa, pb);
      to_a();
      ++j;
    }
  };
  int j = 0;
  if (n_tiles > 1) {
    iter(0, F{}, T{}, T{}, F{}, sa, sb, pa, pb);
    to_a();
    j = 1;
    // iterations whose tile j needs no mask: [1, j_u); the loads go inside the
    // block while both tiles they fetch are full
    const int j_u = min(j_ms, n_tiles - 1);
    run(j, min(j_u, n_full - 3), F{}, T{});
    run(j, j_u, F{}, F{});
    run(j, n_tiles - 1, T{}, F{});
  }
  // the last tile (j = n_tiles - 1): with PV of the tile before if there is one
  if (j > 0) iter(j, T{}, F{}, T{}, F{}, sa, sb, pa, pb);
  else iter(j, F{}, F{}, T{}, F{}, sa, sb, pa, pb);
  // PV of the last tile, whose P^T the last iteration left in pb
  if (diag_tail) block(std::integral_constant<int, 3>{}, 0u, sa, vslot_of(n_tiles - 1), pb, no_sm);
  else block(M_PV{}, 0u, sa, vslot_of(n_tiles - 1), pb, no_sm);

  // ---- epilogue: O = O^T / l (fp16, round to nearest even), LSE in natural
  // log.  O^T holds 4 consecutive columns of a row per lane and store, 32 rows
  // per instruction; it goes through LDS so that the stores write whole rows
  // instead (16 lanes per 256-byte row, 4 rows per instruction).  The K ring
  // is not read after the last iteration's barrier, and no load targets it
  // any more, so each wave takes one K slot: 64 rows at the padded K row
  // stride, which spreads the 32 rows a column write touches over the banks.
  // The reads are the wave's own writes, which LDS performs in order.
  if (active) {
    LDS char* const ob = k_lds + (uint32_t)K_TILEB * (uint32_t)wave;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float inv = 1.0f / l_run[qb];
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          f16x4 hv;
#pragma unroll
          for (int e = 0; e < 4; ++e) hv[e] = (_Float16)(o_acc[db][qb][4 * r4 + e] * inv);
          *(LDS f16x4*)(ob + (32 * qb + n) * K_ROWB + 2 * (32 * db + 8 * r4 + 4 * hh)) = hv;
        }
    }
    // O and LSE are written once and never read here again: non-temporal
    // stores keep them from displacing the K/V tiles that the other work
    // items of this KV group, running on the same XCD, still stream from L2.
    _Float16* const ob_g = p.o + (int64_t)b * p.q_bstride + (int64_t)h * 128 + 8 * (lane & 15);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      const int row = 4 * i + (lane >> 4);
      const f16x8 x = *(const LDS f16x8*)(ob + row * K_ROWB + 16 * (lane & 15));
      if (qw + row < Sq) __builtin_nontemporal_store(x, reinterpret_cast<f16x8*>(ob_g + (int64_t)(qw + row) * p.q_sstride));
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qrow = qw + 32 * qb + n;
      if (p.lse && hh == 0 && qrow < Sq)
        __builtin_nontemporal_store((m_run[qb] + log2f(l_run[qb])) * LN2, &p.lse[((int64_t)b * p.Hq + h) * Sq + qrow]);
    }
  }
}

// Launch of the kernel with placement kPlace, either prefetch depth
// (grid_blocks_wide() workgroups).
template <int kPlace>
hipError_t launch_attn_wide_placed(const Params& p, hipStream_t stream) {
  const int64_t nb = grid_blocks_wide(p);
  if (nb <= 0 || p.hd != 128 || (p.hpw != 1 && p.hpw != 2 && p.hpw != 4)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)nb), block(64 * W_NW);
  if (p.ring == 2) hipLaunchKernelGGL((attn_wide_kernel<2, kPlace>), grid, block, 0, stream, p);
  else if (p.ring == 4) hipLaunchKernelGGL((attn_wide_kernel<4, kPlace>), grid, block, 0, stream, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace libattn
