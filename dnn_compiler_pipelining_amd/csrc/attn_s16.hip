// attn_s16.hip -- the serial4 schedule (four waves, one query head, 128 query
// rows per workgroup, 32 per wave, 64-key tiles, two-slot K and V rings) on
// v_mfma_f32_16x16x32_f16 instead of v_mfma_f32_32x32x16_f16 (head dimension
// 128).  On random data under the chip's power limit the 16 x 16 x 32
// instruction sustains a higher rate than the 32 x 32 x 16 one; this kernel
// measures what that is worth with the softmax beside the MFMAs.  The tile
// loop is the serial one of attn_fwd.hip (load / mma / softmax sTasks of page
// "PipeThreader: Software-Defined Pipelining ... (OSDI 2025)" summary, section
// "核心方法"), with the same sum-checked lazy rescale; its results differ from
// the 32-row schedules' only by rounding order (the row reductions run over
// four lane groups instead of two).
//
// Lane l: n = l % 16 (query within a 16-row block, or key / d row of an A
// operand), g = l / 16.
//   QK : S[kb][qb] (16 keys x 16 queries) += K[16kb + n][32kk + 8g ..] x
//        Q^T[32kk + 8g ..][16qb + n]; lane holds S for query 16qb + n, keys
//        16kb + 4g + r (r = 0..3)
//   PV : O[db][qb] (16 d x 16 queries) += V^T[16db + n][keys] x
//        P^T[keys][16qb + n], 32 keys per chunk c, k element e <-> key
//        32c + 4g + e (e < 4) or 32c + 16 + 4g + (e - 4) (e >= 4); lane holds
//        O for query 16qb + n, d = 16db + 4g + r
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_kernel.h"
#include "attn_tile.h"
#include "gfx950.h"

namespace libattn {

namespace s16 {
constexpr int NW = 4, BMW = 128, HD = 128;
constexpr int K_ROWB = 2 * HD + 16, K_TILEB = BN * K_ROWB, K_DMA = K_TILEB / 1024;  // 272, 17408, 17
constexpr int V_ROWB = 2 * HD, V_TILEB = BN * V_ROWB, V_DMA = V_TILEB / 1024;      // 256, 16384, 16
constexpr int KC = HD / 8;  // 16-byte chunks per row
// V chunk c of row r sits at c ^ vswz(r): row bits 0..1 select a 64-byte offset and row bit 2 a 32-byte
// one, so the two 16-lane groups of a half-wave transpose read (rows r0..r0+3 and r0+4..r0+7, 32 bytes
// each) hit all 64 banks once
__host__ __device__ constexpr int vswz(int r) { return 4 * (r & 3) + 2 * ((r >> 2) & 1); }
}  // namespace s16

// kRing: depth of the fragment prefetch ring of the two mma blocks (2 or 4)
template <int kRing>
__global__ __launch_bounds__(256, 2) void attn_s16_kernel(Params p) {
  using namespace s16;
  __shared__ __attribute__((aligned(1024))) char k_smem[2 * K_TILEB];
  __shared__ __attribute__((aligned(1024))) char v_smem[2 * V_TILEB];
  LDS char* const k_lds = (LDS char*)k_smem;
  LDS char* const v_lds = (LDS char*)v_smem;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);

  // ---- workgroup -> (batch, kv head, head, query tile), as the serial4 schedule
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
  const int b = group / p.Hkv, c = group % p.Hkv;
  const int t = p.lpt ? p.n_qt - 1 - item / p.pairs : item / p.pairs;
  const int hl = item % p.pairs;
  const int h = c * p.g + hl;
  const int Sq = p.Sq, Sk = p.Sk, off = p.off;
  const int q0 = t * BMW, qw = q0 + 32 * wave;
  const int kv_tiles_all = (Sk + BN - 1) / BN;
  const int n_tiles = p.causal ? min(kv_tiles_all, (q0 + off + BMW + BN - 1) / BN) : kv_tiles_all;

  const _Float16* qb_ = p.q + (int64_t)b * p.q_bstride + (int64_t)h * HD;
  const _Float16* kb_ = p.k + (int64_t)b * p.kv_bstride + (int64_t)c * HD;
  const _Float16* vb_ = p.v + (int64_t)b * p.kv_bstride + (int64_t)c * HD;

  // ---- Q^T fragments: qf[qb][kk] = Q[qw + 16qb + n][32kk + 8g .. +7]
  f16x8 qf[2][4];
  {
    const uint32_t flip = p.neg ? 0x80008000u : 0u;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int row = qw + 16 * qb + n;
      const _Float16* src = qb_ + (int64_t)row * p.q_sstride + 8 * g;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        u32x4 u = {0, 0, 0, 0};
        if (row < Sq) u = *reinterpret_cast<const u32x4*>(src + 32 * kk);
        u ^= flip;
        qf[qb][kk] = __builtin_bit_cast(f16x8, u);
      }
    }
  }

  // ---- K/V staging (direct loads; wave w issues K instructions w, w+4, ... and V instructions w, w+4, ...)
  const uint32_t row_bytes = (uint32_t)p.kv_sstride * 2;
  const uint32_t k_lds_base = (uint32_t)(uintptr_t)k_lds, v_lds_base = (uint32_t)(uintptr_t)v_lds;
  constexpr int K_PER_WAVE = (K_DMA + NW - 1) / NW, V_PER_WAVE = V_DMA / NW;
  int k_row[K_PER_WAVE];
  uint32_t k_col[K_PER_WAVE];
#pragma unroll
  for (int u = 0; u < K_PER_WAVE; ++u) {
    const int o = 64 * (wave + NW * u) + lane;
    k_row[u] = o / (K_ROWB / 16);
    const int cb = o - k_row[u] * (K_ROWB / 16);
    k_col[u] = 16u * (uint32_t)(cb < KC ? cb : KC - 1);
  }
  const int v_rowl = lane / KC;  // 4 rows per instruction; rows of instruction i: 4i .. 4i+3
  const uint32_t v_col = 16u * (uint32_t)((lane % KC) ^ vswz(4 * wave + v_rowl));  // same for every u (i & 1 = wave & 1)
  auto stage = [&](int tk) INL {
    tk = __builtin_amdgcn_readfirstlane(tk);
    if (tk >= n_tiles) return;
    const bool full = (tk + 1) * BN <= Sk;
    const char* kbase = (const char*)kb_ + (int64_t)tk * BN * row_bytes;
#pragma unroll
    for (int u = 0; u < K_PER_WAVE; ++u) {
      const int i = wave_s + NW * u;
      if (i < K_DMA) {
        const int row = full ? k_row[u] : min(k_row[u], Sk - 1 - tk * BN);
        dma16(kbase, (uint32_t)row * row_bytes + k_col[u], k_lds_base + (tk & 1) * K_TILEB + 1024 * i);
      }
    }
    const char* vbase = (const char*)vb_ + (int64_t)tk * BN * row_bytes;
#pragma unroll
    for (int u = 0; u < V_PER_WAVE; ++u) {
      const int i = wave_s + NW * u;
      const int row0 = 4 * i + v_rowl;
      const int row = full ? row0 : min(row0, Sk - 1 - tk * BN);
      dma16(vbase, (uint32_t)row * row_bytes + v_col, v_lds_base + (tk & 1) * V_TILEB + 1024 * i);
    }
  };

  // ---- fragment addresses
  const int k_frag = n * K_ROWB + 16 * g;  // + (16kb) K_ROWB + 64kk
  // V^T transpose reads: lane (g, n) addresses row 4g + n/4 (+16 for the second read, +32c), columns
  // 16db + 4(n%4) .. +3; it receives column 16db + n, rows 4g .. 4g+3 (and +16)
  const int v_row0 = 4 * g + (n >> 2);
  const int v_frag0 = v_row0 * V_ROWB + (((n & 3) >> 1) ^ vswz(v_row0)) * 16 + ((n & 1) << 3);  // db = 0, c = 0
  // db adds 2db to the logical chunk (bits 1..3, zero in the db = 0 chunk): an XOR, which commutes with the swizzle

  f32x4 o_acc[8][2];
#pragma unroll
  for (int db = 0; db < 8; ++db) o_acc[db][0] = o_acc[db][1] = f32x4{};
  float m_run[2] = {M_INIT, M_INIT}, l_run[2] = {0.f, 0.f};
  const float cs = p.cs;
  const int qw_u = __builtin_amdgcn_readfirstlane(qw);

  // reductions over the four lanes n, n+16, n+32, n+48 of a query: v_permlane32_swap pairs lanes l and
  // l^32, v_permlane16_swap lanes l and l^16 (rows of 16 lanes swapped in pairs)
  auto red_max = [&](float x) INL {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto c2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(c2[0]), __uint_as_float(c2[1]));
  };
  auto red_sum = [&](float x) INL {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto c2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(c2[0]) + __uint_as_float(c2[1]);
  };

  stage(0);
  dma_wait();
  lds_barrier();
  for (int j = 0; j < n_tiles; ++j) {
    stage(j + 1);
    const bool skip = p.causal && j * BN > qw_u + 31 + off;
    if (!skip) {
      const LDS char* ks = k_lds + (j & 1) * K_TILEB + k_frag;
      const LDS char* vs = v_lds + (j & 1) * V_TILEB;
      // QK^T: 16 K fragments (kb, kk), two MFMAs each; fragment f + R read after the MFMAs of f
      constexpr int R = kRing;
      f32x4 s[4][2];
      f16x8 kfr[R];
      auto kload = [&](int f) INL -> f16x8 { return *(const LDS f16x8*)(ks + 16 * (f >> 2) * K_ROWB + 64 * (f & 3)); };
      static_for<R>([&](auto ic) INL { kfr[decltype(ic)::value] = kload(decltype(ic)::value); });
      static_for<16>([&](auto fc) INL {
        constexpr int fi = decltype(fc)::value, kb = fi >> 2, kk = fi & 3;
        const f16x8 kf = kfr[fi % R];
        if constexpr (fi + R < 16) kfr[fi % R] = kload(fi + R);
        s[kb][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[0][kk], kk == 0 ? f32x4{} : s[kb][0], 0, 0, 0);
        s[kb][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf, qf[1][kk], kk == 0 ? f32x4{} : s[kb][1], 0, 0, 0);
      });
      static_for<R>([&](auto) INL { __builtin_amdgcn_sched_group_barrier(0x100, 1, 0); });
      static_for<16>([&](auto fc) INL {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        if constexpr (decltype(fc)::value + R < 16) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      });
      // softmax (sum-checked lazy rescale as the other kernels: exponentials against the running max;
      // the tile max only on the first tile or when a row's tile sum exceeds RS_MAX)
      const bool masked = (p.causal && j * BN + BN - 1 > qw_u + off) || j * BN + BN > Sk;
      int lim[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int query = qw + 16 * qb + n;
        const int end = p.causal ? min(Sk, query + off + 1) : Sk;
        lim[qb] = end - j * BN - 4 * g;  // key 16kb + 4g + r allowed iff 16kb + r < lim
      }
      f16x8 pf[2][2];
      float rs[2], alpha[2] = {1.f, 1.f};
      bool any_rescale = false;
      auto exps_t = [&](int qb, float negm, auto mk) INL {
        constexpr bool kMasked = decltype(mk)::value;
        float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const int kb = 2 * cc + (e >> 2), r = e & 3;
            float x0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][r], cs, negm));
            float x1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][r + 1], cs, negm));
            if constexpr (kMasked) {
              x0 = 16 * kb + r < lim[qb] ? x0 : 0.f;
              x1 = 16 * kb + r + 1 < lim[qb] ? x1 : 0.f;
            }
            pf[qb][cc][e] = (_Float16)x0;
            pf[qb][cc][e + 1] = (_Float16)x1;
            add_pair_f16((e & 2) ? acc1 : acc0, f16x2{pf[qb][cc][e], pf[qb][cc][e + 1]});
          }
        return red_sum(acc0 + acc1);
      };
      auto exps = [&](int qb, float negm) INL {
        return masked ? exps_t(qb, negm, std::true_type{}) : exps_t(qb, negm, std::false_type{});
      };
      auto full = [&](int qb) INL {  // tile max, new running max, exponentials again
        float mx = NEG_INF;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            mx = fmaxf(mx, (!masked || 16 * kb + r < lim[qb]) ? s[kb][qb][r] : NEG_INF);
        mx = red_max(mx);
        const float mts = mx == NEG_INF ? NEG_INF : mx * cs;
        const float m_new = fmaxf(m_run[qb], mts);
        alpha[qb] = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
        m_run[qb] = m_new;
        rs[qb] = exps(qb, -m_new);
      };
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        bool redo = j == 0;
        if (!redo) {
          rs[qb] = exps(qb, -m_run[qb]);
          redo = __builtin_amdgcn_ballot_w64(!(rs[qb] <= RS_MAX)) != 0;
        }
        if (__builtin_expect(redo, 0)) {
          full(qb);
          any_rescale = true;
        }
        l_run[qb] = __builtin_fmaf(l_run[qb], alpha[qb], rs[qb]);
      }
      if (__builtin_expect(any_rescale, 0)) {
#pragma unroll
        for (int db = 0; db < 8; ++db) {
          o_acc[db][0] *= alpha[0];
          o_acc[db][1] *= alpha[1];
        }
      }
      // PV: 16 V^T fragments (db, cc) of two transpose reads, two MFMAs each, ring as for QK
      f16x8 vfr[R];
      auto vload = [&](int f) INL -> f16x8 {
        const LDS char* base = vs + (v_frag0 ^ (32 * (f >> 1))) + 32 * (f & 1) * V_ROWB;
        const f16x4 h1 = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)base));
        const f16x4 h2 =
            __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS i16x4*)(base + 16 * V_ROWB)));
        return f16x8{h1[0], h1[1], h1[2], h1[3], h2[0], h2[1], h2[2], h2[3]};
      };
      static_for<R>([&](auto ic) INL { vfr[decltype(ic)::value] = vload(decltype(ic)::value); });
      static_for<16>([&](auto fc) INL {
        constexpr int fi = decltype(fc)::value, db = fi >> 1, cc = fi & 1;
        const f16x8 vf = vfr[fi % R];
        if constexpr (fi + R < 16) vfr[fi % R] = vload(fi + R);
        o_acc[db][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[0][cc], o_acc[db][0], 0, 0, 0);
        o_acc[db][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[1][cc], o_acc[db][1], 0, 0, 0);
      });
      static_for<R>([&](auto) INL { __builtin_amdgcn_sched_group_barrier(0x100, 2, 0); });
      static_for<16>([&](auto fc) INL {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        if constexpr (decltype(fc)::value + R < 16) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      });
    }
    dma_wait();
    lds_barrier();
  }

  // ---- epilogue: O = O^T / l (fp16, RNE), LSE
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qrow = qw + 16 * qb + n;
    if (qrow < Sq) {
      const float inv = 1.0f / l_run[qb];
      _Float16* dst = p.o + (int64_t)b * p.q_bstride + (int64_t)qrow * p.q_sstride + (int64_t)h * HD + 4 * g;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        f16x4 hv;
#pragma unroll
        for (int e = 0; e < 4; ++e) hv[e] = (_Float16)(o_acc[db][qb][e] * inv);
        *reinterpret_cast<f16x4*>(dst + 16 * db) = hv;
      }
      if (p.lse && g == 0) p.lse[((int64_t)b * p.Hq + h) * Sq + qrow] = (m_run[qb] + log2f(l_run[qb])) * LN2;
    }
  }
}

}  // namespace libattn

namespace libattn {

int64_t grid_blocks_s16(const Params& p) {
  const int64_t nb = (int64_t)p.B * p.Hkv * p.pairs * p.n_qt;
  return nb > 0x7fffffff ? -1 : nb;
}

hipError_t launch_attn_s16(const Params& p, hipStream_t stream) {
  const int64_t nb = grid_blocks_s16(p);
  if (nb <= 0 || p.hd != 128 || p.bn != BN || (p.ring != 2 && p.ring != 4)) return hipErrorInvalidValue;
  if (p.ring == 2) hipLaunchKernelGGL((attn_s16_kernel<2>), dim3((unsigned)nb), dim3(256), 0, stream, p);
  else hipLaunchKernelGGL((attn_s16_kernel<4>), dim3((unsigned)nb), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace libattn
