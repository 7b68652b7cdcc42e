// gemm_fwd.hip -- fp16 GEMM with fp32 accumulation for gfx950 (CDNA4):
// C[M][N] = A[M][K] B, B stored [K][N] (C = A B) or [N][K] (C = A B^T).
//
// This is the load / mma pipeline of the attention kernel without its softmax
// task: PipeThreader's MatMul workload (page "PipeThreader: Software-Defined
// Pipelining ... (OSDI 2025)" summary, sections "问题与动机" and "实验与结果")
// split into a load sTask (A and B tiles, global -> LDS by direct loads into a
// two-slot ring: prologue / steady state / epilogue, page "AI编译器融合技术 --
// 5. 并行性与分布式融合", section 5.4.2) and an mma sTask (v_mfma_f32_16x16x32_f16
// with 8 waves, v_mfma_f32_32x32x16_f16 with 4, fragments conformed to the
// instruction's layout, same page, section 5.2.2).  On random data under the
// chip's power limit the 16 x 16 x 32 instruction sustains a higher rate than
// the 32 x 32 x 16 one.
//
// One workgroup computes a 256 x 256 tile of C over 64-deep K tiles, with 8
// waves (two per SIMD) or 4 (one per SIMD, kNW = 4).  Wave (wm, wn) =
// (w % 2, w / 2) owns rows 128 wm .. +128 of the tile and columns
// 64 wn .. +64 (8 waves: 8 x 4 accumulators of 16 x 16) or 128 wn .. +128
// (4 waves: 4 x 4 accumulators of 32 x 32, 256 registers that live in AGPRs).
// The MFMA computes the transposed block, D[n][m] = sum_k B^T[n][k] A^T[k][m],
// so that each lane holds one row m of C and runs of 4 consecutive columns n:
// the epilogue writes 8-byte runs.
//
// LDS layouts (bytes; one slot of each ring is 32 KiB, both rings 128 KiB):
//   A tile and B tile stored [N][K]: 256 rows of 64 k = 128 B.  Its 16-byte
//     chunk c of row r sits at position c ^ ((r >> 1) & 7).  A fragment is
//     one ds_read_b128 per lane (16 x 32: row l % 16, chunk 4kk + l / 16;
//     32 x 16: row l % 32, chunk 2kk + l / 32); each 16-lane pass of it
//     touches rows r0..r0+15 at one chunk, which the swizzle spreads over
//     all 64 banks.
//   B tile stored [K][N]: 64 rows of 256 n = 512 B, chunk c of row r at
//     c ^ (4 * (r & 3)).  A B^T fragment (n rows, k columns) is two
//     ds_read_b64_tr_b16 of 4 k rows each; a half-wave of such a read covers
//     4 rows x 64 B, which the swizzle spreads over all 64 banks.
// The direct loads write 1 KiB per instruction in LDS order; each lane picks
// the global 16 bytes that belong at its LDS position.  Rows and columns past
// the end of A or B are loaded from the last valid ones (finite data that
// only reaches discarded outputs); K positions past the end are zeroed in LDS
// by the lane that loaded them, after its own load has landed.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "gemm_kernel.h"
#include "gfx950.h"

namespace libattn {

constexpr int GBM = 256, GBN = 256, GBK = 64;
constexpr int G_TILEB = 256 * GBK * 2;  // bytes of one A or B slot (32 KiB)
constexpr int G_BAND = 4;               // output tile rows per raster band (4 measured 0.5% ahead of 8, 16 5% behind)
static_assert(4 * G_TILEB <= 160 * 1024, "two slots of A and B fit the LDS");

// kBL 0: B stored [K][N]; 1: B stored [N][K].  kNW: waves per workgroup, 8 or 4.  kMI: the MFMA,
// 32 (v_mfma_f32_32x32x16_f16) or 16 (v_mfma_f32_16x16x32_f16).
template <int kBL, int kNW, int kMI = 32>
__global__ __launch_bounds__(64 * kNW, 1) void gemm_kernel(GemmParams p) {
  static_assert(kNW == 8 || kNW == 4, "8 or 4 waves");
  static_assert(kMI == 32 || kMI == 16, "32 x 32 x 16 or 16 x 16 x 32 MFMAs");
  constexpr int WNX = kNW == 8 ? 64 : 128;  // columns of C per wave
  constexpr int NFR = WNX / kMI;            // accumulator blocks per wave along n
  constexpr int MFB = 128 / kMI;            // accumulator blocks per wave along m (128 rows)
  constexpr int NSUB = 64 / (kMI == 32 ? 16 : 32);  // k substeps per 64-deep K tile
  constexpr int UPW = 32 / kNW;             // direct-load instructions per wave per tile, for A and for B
  __shared__ __attribute__((aligned(1024))) char a_smem[2 * G_TILEB];
  __shared__ __attribute__((aligned(1024))) char b_smem[2 * G_TILEB];
  LDS char* const a_lds = (LDS char*)a_smem;
  LDS char* const b_lds = (LDS char*)b_smem;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const int wm = wave_s & 1, wn = wave_s >> 1;

  // ---- workgroup -> output tile.  Workgroups are dealt round-robin to the 8
  // XCDs; when the tile count allows, XCD x takes the x-th eighth of the
  // raster, so the tiles that run together on one XCD are neighbours.  The
  // raster walks bands of G_BAND tile rows column by column, so concurrent
  // tiles share A row panels and B column panels in that XCD's L2.
  const int T = p.ntm * p.ntn;
  int t = blockIdx.x;
  if ((T & 7) == 0) t = (t & 7) * (T >> 3) + (t >> 3);
  const int band = t / (G_BAND * p.ntn);
  const int tm0 = band * G_BAND;
  const int gh = min(G_BAND, p.ntm - tm0);
  const int local = t - tm0 * p.ntn;
  const int tm = tm0 + local % gh, tn = local / gh;
  const int m0 = tm * GBM, n0 = tn * GBN;
  const int M = p.M, N = p.N, K = p.K;

  // ---- per-lane direct-load maps.  Wave w issues instructions w + kNW u
  // (u = 0..UPW-1) of each 32-instruction tile.
  //   [row][k] tiles (A, and B stored [N][K]): instruction i holds rows
  //     8i .. 8i+7; lane l has row 8i + l/8 and LDS chunk l % 8, i.e. logical
  //     chunk (l % 8) ^ ((row >> 1) & 7), the same for every u.
  //   [k][n] tile (B stored [K][N]): instruction i holds k rows 2i, 2i+1;
  //     lane l has k row 2i + l/32 and LDS chunk l % 32, i.e. logical chunk
  //     (l % 32) ^ (4 * (row & 3)), the same for every u.
  const uint32_t a_lds_base = (uint32_t)(uintptr_t)a_lds, b_lds_base = (uint32_t)(uintptr_t)b_lds;
  const int rk_row0 = 8 * wave + (lane >> 3);  // + 8 kNW u
  const int rk_chunk = (lane & 7) ^ ((4 * wave + (lane >> 4)) & 7);
  const int kn_row0 = 2 * wave + (lane >> 5);  // + 2 kNW u
  const int kn_chunk = (lane & 31) ^ (4 * ((2 * wave + (lane >> 5)) & 3));
  const int kchunks = K >> 3;  // 16-byte chunks per row of A (and of B stored [N][K])

  auto stage = [&](int kt) INL {  // this wave's loads of K tile kt into slot kt & 1
    const int k0 = kt * GBK;
    const uint32_t slot_off = (uint32_t)(kt & 1) * G_TILEB;
    // A: rows past M read row M-1, chunks past K read the last chunk (zeroed later)
    {
      const char* base = (const char*)(p.a + (int64_t)m0 * K + k0);
      const int c = min(rk_chunk, kchunks - 1 - (k0 >> 3));
#pragma unroll
      for (int u = 0; u < UPW; ++u) {
        const int row = min(rk_row0 + 8 * kNW * u, M - 1 - m0);
        dma16(base, (uint32_t)row * (uint32_t)(2 * K) + 16u * c,
              a_lds_base + slot_off + 1024u * (uint32_t)(wave_s + kNW * u));
      }
    }
    if constexpr (kBL == 1) {
      const char* base = (const char*)(p.b + (int64_t)n0 * K + k0);
      const int c = min(rk_chunk, kchunks - 1 - (k0 >> 3));
#pragma unroll
      for (int u = 0; u < UPW; ++u) {
        const int row = min(rk_row0 + 8 * kNW * u, N - 1 - n0);
        dma16(base, (uint32_t)row * (uint32_t)(2 * K) + 16u * c,
              b_lds_base + slot_off + 1024u * (uint32_t)(wave_s + kNW * u));
      }
    } else {
      const char* base = (const char*)(p.b + (int64_t)k0 * N + n0);
      const int c = min(kn_chunk, (N >> 3) - 1 - (n0 >> 3));
#pragma unroll
      for (int u = 0; u < UPW; ++u) {
        const int row = min(kn_row0 + 2 * kNW * u, K - 1 - k0);
        dma16(base, (uint32_t)row * (uint32_t)(2 * N) + 16u * c,
              b_lds_base + slot_off + 1024u * (uint32_t)(wave_s + kNW * u));
      }
    }
  };
  // After this wave's loads of the last K tile have landed: zero the LDS
  // positions it loaded that lie at k >= K.
  auto zero_tail = [&](int kt) INL {
    const int k0 = kt * GBK;
    const uint32_t slot_off = (uint32_t)(kt & 1) * G_TILEB;
    const u32x4 z = {0, 0, 0, 0};
    if (rk_chunk >= kchunks - (k0 >> 3)) {
#pragma unroll
      for (int u = 0; u < UPW; ++u) {
        *(LDS u32x4*)(a_lds + slot_off + 1024 * (wave_s + kNW * u) + 16 * lane) = z;
        if constexpr (kBL == 1) *(LDS u32x4*)(b_lds + slot_off + 1024 * (wave_s + kNW * u) + 16 * lane) = z;
      }
    }
    if constexpr (kBL == 0) {
#pragma unroll
      for (int u = 0; u < UPW; ++u)
        if (kn_row0 + 2 * kNW * u >= K - k0)
          *(LDS u32x4*)(b_lds + slot_off + 1024 * (wave_s + kNW * u) + 16 * lane) = z;
    }
  };

  // ---- per-lane fragment offsets (bytes) in a [row][k] tile.  kMI 32: row
  // l % 32 of a 32-row block and logical chunk 2kk + l/32, kk = 0..3 (the
  // 32 x 32 x 16 operand: row l % 32, k = 8 (l/32) .. +7).  kMI 16: row l % 16
  // of a 16-row block and logical chunk 4kk + l/16, kk = 0..1 (the 16 x 16 x 32
  // operand: row l % 16, k = 8 (l/16) .. +7).  Blocks start at multiples of 16
  // rows, so the swizzle of row r is that of r % 16.
  int rk_frag[NSUB];
#pragma unroll
  for (int kk = 0; kk < NSUB; ++kk)
    rk_frag[kk] = kMI == 32 ? (lane & 31) * 128 + 16 * ((2 * kk + (lane >> 5)) ^ ((lane >> 1) & 7))
                            : (lane & 15) * 128 + 16 * ((4 * kk + (lane >> 4)) ^ (((lane & 15) >> 1) & 7));
  // B stored [K][N]: lane (group g = l/16, s = l%16) of a transpose read
  // addresses 4 fp16 of one k row; the read hands lane s of each group the 4
  // k rows of the group's column s.  kMI 32: k row 8(g/2) + s/4 (+4 for the
  // second read, +16kk per step) and columns n = WNX wn + 32nf + 16(g%2) +
  // 4(s%4) .. +3.  kMI 16: k row 8g + s/4 (+4, +32kk) and columns
  // n = WNX wn + 16nf + 4(s%4) .. +3.
  int kn_frag[NFR];
  {
    const int g = lane >> 4, s = lane & 15;
    const int row = kMI == 32 ? 8 * (g >> 1) + (s >> 2) : 8 * g + (s >> 2);
    const int chunk = (WNX / 8) * wn + (kMI == 32 ? 2 * (g & 1) : 0) + ((s & 3) >> 1);  // 16-byte chunk, nf = 0
    const int f0 = row * 512 + ((chunk ^ (4 * (s >> 2))) << 4) + ((s & 1) << 3);
    // nf adds 4nf (kMI 32) or 2nf (kMI 16) to the chunk: bits that are zero in the nf = 0 chunk, so the
    // sum is an XOR, and XOR commutes with the swizzle
#pragma unroll
    for (int nf = 0; nf < NFR; ++nf) kn_frag[nf] = f0 ^ ((kMI == 32 ? 64 : 32) * nf);
  }

  auto frag_a = [&](int slot, int kk, int mf) INL -> f16x8 {  // B operand: A^T[k][m], m = 128wm + kMI mf + l%kMI
    return *(const LDS f16x8*)(a_lds + slot * G_TILEB + (128 * wm + kMI * mf) * 128 + rk_frag[kk]);
  };
  auto frag_b = [&](int slot, int kk, int nf) INL -> f16x8 {  // A operand: B^T[n][k], n = WNX wn + kMI nf + l%kMI
    if constexpr (kBL == 1) {
      return *(const LDS f16x8*)(b_lds + slot * G_TILEB + (WNX * wn + kMI * nf) * 128 + rk_frag[kk]);
    } else {
      const LDS char* a = b_lds + slot * G_TILEB + kn_frag[nf] + (64 / NSUB) * kk * 512;
      const f16x4 h1 = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)a));
      const f16x4 h2 = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)(a + 4 * 512)));
      return f16x8{h1[0], h1[1], h1[2], h1[3], h2[0], h2[1], h2[2], h2[3]};
    }
  };

  using Acc = std::conditional_t<kMI == 32, f32x16, f32x4>;
  Acc acc[MFB][NFR];
#pragma unroll
  for (int mf = 0; mf < MFB; ++mf)
#pragma unroll
    for (int nf = 0; nf < NFR; ++nf) acc[mf][nf] = Acc{};
  auto mma = [&](f16x8 bv, f16x8 av, Acc& c) INL {
    if constexpr (kMI == 32) c = __builtin_amdgcn_mfma_f32_32x32x16_f16(bv, av, c, 0, 0, 0);
    else c = __builtin_amdgcn_mfma_f32_16x16x32_f16(bv, av, c, 0, 0, 0);
  };

  // ---- mma task: a K tile is NSUB substeps (4 of 16 k, or 2 of 32 k), MFB
  // NFR MFMAs each (mf-major).  Fragments are double-buffered by substep; the
  // NFR + MFB (or 2 NFR + MFB, with transpose reads) fragment reads of the
  // next substep are issued one after each of the first MFMAs of the current
  // one (pinned below), so LDS latency hides behind the matrix core.
  constexpr int kSteps = MFB * NFR;
  constexpr int kReads = kBL == 1 ? NFR + MFB : 2 * NFR + MFB;
  static_assert(kReads <= kSteps, "one read after each MFMA at most");
  f16x8 bf[2][NFR], af[2][MFB];
  auto load_frags = [&](int slot, auto kc) INL {
    constexpr int kk = decltype(kc)::value;
#pragma unroll
    for (int nf = 0; nf < NFR; ++nf) bf[kk & 1][nf] = frag_b(slot, kk, nf);
#pragma unroll
    for (int mf = 0; mf < MFB; ++mf) af[kk & 1][mf] = frag_a(slot, kk, mf);
  };
  auto mfmas = [&](auto kc) INL {
    constexpr int kk = decltype(kc)::value;
#pragma unroll
    for (int j = 0; j < kSteps; ++j) {
      const int mf = j / NFR, nf = j % NFR;
      mma(bf[kk & 1][nf], af[kk & 1][mf], acc[mf][nf]);
    }
  };
  // Where the next substep's fragment reads sit among the MFMAs: with B stored [N][K] spread evenly over
  // the substep (measured 2% faster there), with B stored [K][N] one after each of the first MFMAs.
  auto pin_interleaved = [&]() INL {
    static_for<kSteps>([&](auto jc) INL {
      constexpr int j = decltype(jc)::value;
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if constexpr (kBL == 1) {
        constexpr int nr = (j + 1) * kReads / kSteps - j * kReads / kSteps;
        if constexpr (nr > 0) __builtin_amdgcn_sched_group_barrier(0x100, nr, 0);
      } else if constexpr (j < kReads) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    });
  };

  // ---- K loop, rotated by one substep across the barrier: iteration kt runs
  // substeps 0..NSUB-2 of tile kt, waits for tile kt+1's loads and the
  // barrier that publishes them, then runs the last substep of tile kt (its
  // fragments are already in registers) beside the substep-0 reads of tile
  // kt+1, and issues the loads of tile kt+2 into the slot tile kt has just
  // left.  The matrix
  // core stays busy while the waves meet at the barrier and while the first
  // reads of a tile are in flight.
  const int nkt = p.nkt;
  const bool tail = (K & (GBK - 1)) != 0;
  stage(0);
  dma_wait();
  if (tail && nkt == 1) zero_tail(0);
  lds_barrier();
  load_frags(0, std::integral_constant<int, 0>{});
  if (nkt > 1) stage(1);
  auto substeps_012 = [&](int slot) INL {  // substeps 0 .. NSUB-2
    static_for<NSUB - 1>([&](auto kc) INL {
      constexpr int kk = decltype(kc)::value;
      load_frags(slot, std::integral_constant<int, kk + 1>{});
      mfmas(kc);
      pin_interleaved();
    });
  };
  // Loads of a full K tile (every K position inside K): per-lane offsets
  // that do not change from tile to tile (rows past M or N already clamped),
  // running base addresses, and M0 = slot base + a compile-time offset.
  // Issued one beside each MFMA of substep 3 rather than as one block of
  // instructions, which would leave the matrix core without work while a
  // wave issues them (with one wave per SIMD nothing else fills the gap).
  uint32_t off_a[UPW], off_b[UPW];
#pragma unroll
  for (int u = 0; u < UPW; ++u) {
    off_a[u] = (uint32_t)min(rk_row0 + 8 * kNW * u, M - 1 - m0) * (uint32_t)(2 * K) + 16u * (uint32_t)rk_chunk;
    if constexpr (kBL == 1)
      off_b[u] = (uint32_t)min(rk_row0 + 8 * kNW * u, N - 1 - n0) * (uint32_t)(2 * K) + 16u * (uint32_t)rk_chunk;
    else
      off_b[u] = (uint32_t)(kn_row0 + 2 * kNW * u) * (uint32_t)(2 * N) +
                 16u * (uint32_t)min(kn_chunk, (N >> 3) - 1 - (n0 >> 3));
  }
  const int nfull = K / GBK;  // K tiles [0, nfull) lie wholly inside K
  const char* a_run = (const char*)(p.a + (int64_t)m0 * K) + 2 * 2 * GBK;  // tile 2
  const char* b_run = kBL == 1 ? (const char*)(p.b + (int64_t)n0 * K) + 2 * 2 * GBK
                               : (const char*)(p.b + (int64_t)2 * GBK * N + n0);
  const int64_t b_step = kBL == 1 ? 2 * GBK : (int64_t)2 * GBK * N;  // bytes from one K tile to the next
  // The last substep of tile kt beside the substep-0 reads of tile kt+1 (slot
  // slot ^ 1), with (kDmaIn) this wave's loads of tile kt+2 into `slot`.
  auto substep3 = [&](int slot, auto dma_in) INL {
    constexpr bool kDmaIn = decltype(dma_in)::value;
    const uint32_t a_m0 = a_lds_base + (uint32_t)slot * G_TILEB + 1024u * (uint32_t)wave_s;
    const uint32_t b_m0 = b_lds_base + (uint32_t)slot * G_TILEB + 1024u * (uint32_t)wave_s;
    static_for<kSteps>([&](auto jc) INL {
      constexpr int j = decltype(jc)::value, mf = j / NFR, nf = j % NFR;
      mma(bf[1][nf], af[1][mf], acc[mf][nf]);
      if constexpr (j < NFR) bf[0][j] = frag_b(slot ^ 1, 0, j);
      else if constexpr (j < NFR + MFB) af[0][j - NFR] = frag_a(slot ^ 1, 0, j - NFR);
      if constexpr (kDmaIn && j < UPW) dma16_m0_plus<1024u * kNW * j>(a_run, off_a[j], a_m0);
      if constexpr (kDmaIn && j >= UPW && j < 2 * UPW) dma16_m0_plus<1024u * kNW * (j - UPW)>(b_run, off_b[j - UPW], b_m0);
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (kDmaIn) {
      a_run += 2 * GBK;
      b_run += b_step;
    }
  };
  static_assert(2 * UPW <= kSteps && NFR + MFB <= kSteps, "one load and one fragment read beside each MFMA at most");
  static_assert((NSUB - 1) % 2 == 1, "the last substep's fragments are in buffer 1");
  // iteration kt: substeps 0..2, the barrier that publishes tile kt+1, substep 3
  auto iteration = [&](int kt, auto dma_in) INL {
    const int slot = kt & 1;
    substeps_012(slot);
    dma_wait();
    if (tail && kt + 2 == nkt) zero_tail(kt + 1);
    lds_barrier();
    substep3(slot, dma_in);
  };
  int kt = 0;
  // tile kt+2 full: its loads beside the MFMAs of substep 3
  for (; kt + 2 < nfull; ++kt) iteration(kt, std::true_type{});
  for (; kt + 1 < nkt; ++kt) {
    // the last iterations: tile kt+2 is the tail tile, or there is none
    iteration(kt, std::false_type{});
    if (kt + 2 < nkt) stage(kt + 2);
  }
  substeps_012(kt & 1);  // the last tile
  mfmas(std::integral_constant<int, NSUB - 1>{});

  if constexpr (kMI == 16) {
    // ---- epilogue: lane l holds C[m][n] for m = m0 + 128wm + 16mf + l%16 and
    // n = n0 + WNX wn + 16nf + 4(l/16) + r; fp16, round to nearest even
#pragma unroll
    for (int mf = 0; mf < MFB; ++mf) {
      const int m = m0 + 128 * wm + 16 * mf + (lane & 15);
      if (m >= M) continue;
      _Float16* crow = p.c + (int64_t)m * N;
#pragma unroll
      for (int nf = 0; nf < NFR; ++nf) {
        const int n = n0 + WNX * wn + 16 * nf + 4 * (lane >> 4);
        if (n < N) {  // N % 8 == 0 and n % 4 == 0: n .. n+3 lie inside N
          f16x4 hv;
#pragma unroll
          for (int e = 0; e < 4; ++e) hv[e] = (_Float16)acc[mf][nf][e];
          *reinterpret_cast<f16x4*>(crow + n) = hv;
        }
      }
    }
  } else {
    // ---- epilogue: lane l holds C[m][n] for m = m0 + 128wm + 32mf + l%32 and
    // n = n0 + WNX wn + 32nf + 8(r/4) + 4(l/32) + r%4; fp16, round to nearest even.
    const int h = lane >> 5;
#pragma unroll
    for (int mf = 0; mf < MFB; ++mf) {
      const int m = m0 + 128 * wm + 32 * mf + (lane & 31);
      if (m >= M) continue;
      _Float16* crow = p.c + (int64_t)m * N;
#pragma unroll
      for (int nf = 0; nf < NFR; ++nf)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int n = n0 + WNX * wn + 32 * nf + 8 * r4 + 4 * h;
          if (n < N) {
            f16x4 hv;
#pragma unroll
            for (int e = 0; e < 4; ++e) hv[e] = (_Float16)acc[mf][nf][4 * r4 + e];
            *reinterpret_cast<f16x4*>(crow + n) = hv;
          }
        }
    }
  }
}

__global__ void gemm_zero_kernel(u32x4* c, int64_t n16) {
  const u32x4 z = {0, 0, 0, 0};
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x)
    c[i] = z;
}

hipError_t launch_gemm(const GemmParams& p, hipStream_t stream) {
  const int64_t nb = (int64_t)p.ntm * p.ntn;
  if (nb <= 0 || nb > 0x7fffffff || p.nkt < 1) return hipErrorInvalidValue;
  if (p.waves != 4 && p.waves != 8) return hipErrorInvalidValue;
  const dim3 grid((unsigned)nb), block(64 * p.waves);
  // 8 waves run 16 x 16 x 32 MFMAs, 4 waves 32 x 32 x 16 (the faster shape of each, measured)
  if (p.b_layout == 0) {
    if (p.waves == 8) hipLaunchKernelGGL((gemm_kernel<0, 8, 16>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((gemm_kernel<0, 4, 32>), grid, block, 0, stream, p);
  } else if (p.b_layout == 1) {
    if (p.waves == 8) hipLaunchKernelGGL((gemm_kernel<1, 8, 16>), grid, block, 0, stream, p);
    else hipLaunchKernelGGL((gemm_kernel<1, 4, 32>), grid, block, 0, stream, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_zero(_Float16* c, int64_t elems, hipStream_t stream) {
  const int64_t n16 = elems / 8;  // 16-byte stores; elems is a multiple of 8
  if (n16 <= 0) return hipSuccess;
  const int64_t blocks = n16 / 256 + 1 < 4096 ? n16 / 256 + 1 : 4096;
  hipLaunchKernelGGL(gemm_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, reinterpret_cast<u32x4*>(c), n16);
  return hipGetLastError();
}

}  // namespace libattn
