// bf16 MFMA split-KV latent decode for gfx950 (MI355X).
//
// What it computes ("Multi-Head Low-Rank Attention", 方法步骤详情 step 2 and
// 核心方法; "vllbc02MLA", 苏神思路): for one work item (a token range of one
// or more sequences, see PlanHeader) and a group of heads, the MQA-style
// attention of the absorbed query q_abs[h] = [q~ || rho] over the latent rows
// [c_t || k^R_t], one online softmax per branch j over the branch's latent
// slice plus the shared RoPE key, accumulating acc_j[h] = sum_t p_t c_t[S_j].
// It writes the unnormalised partial state (m, l, acc) that the combine merges.
//
// Mapping onto CDNA4:
//  * A workgroup owns one work item and 16*NW heads (16 per wave); when that
//    is less than all heads, the workgroups of one item's head groups are
//    placed on the same XCD back to back, reading each tile at about the same
//    time. The tiles use device-scope non-temporal loads even then: in paired
//    runs on one box plain loads were no faster for two workgroups per item
//    (MLA at 16 x 32K: 280.7 / 281.5 us against 275.4 / 279.6 us).
//  * KV tiles (32 tokens) stream HBM -> LDS with buffer_load_dwordx4 ... lds
//    (no VGPR staging) through an NS-stage ring shared by all waves; vmcnt
//    waits are placed by hand because the compiler does not order LDS-DMA
//    against ds_read.
//  * QK: S^T[t][h] = sum_d K[t][d] Q[h][d] on v_mfma_f32_16x16x32_bf16 with 16
//    tokens as M and the wave's 16 heads as N; Q^T stays in AGPRs for the
//    whole segment. The RoPE part is computed once per tile and shared by all
//    branches.
//  * The S^T accumulators (lane = head, 4 token rows per M block) are exactly
//    the B operand of PV, O^T[c][h] = sum_t V^T[c][t] P^T[t][h] with the 32
//    tile tokens as K, so P never moves between lanes. V^T is read from the
//    same row-major LDS tile with ds_read_b64_tr_b16. O^T keeps lane = head,
//    so a softmax rescale is one multiplier per lane.
//  * Lazy rescaling: the segment's first tile sets the reference max m; it only
//    moves (rescaling l and O in registers) when a tile's max exceeds it by
//    more than 16 in log2 units, so p <= 2^16, which fp32 and bf16 hold with
//    their usual relative precision. (m, l, acc) stay consistent.
//  * LDS rows are XOR-swizzled in 16-byte chunks so that the QK reads (16 rows
//    x 1 chunk per 16 lanes) and the transposed PV reads (4 rows x 2 chunks per
//    16 lanes) are free of bank conflicts.

#include <hip/hip_ext.h>

#include <type_traits>

#include "device_common.h"

namespace mlra {
namespace {

using namespace dev;

constexpr int kT = 32;   // tokens per tile
constexpr int kDR = 64;  // RoPE width
constexpr float kRescale = 16.f;  // log2 headroom before the running max moves

// Latent-row swizzle (16-byte chunk index XOR per row). Measured on gfx950
// (rocprofv3 SQ_LDS_BANK_CONFLICT on the two read patterns): for rows of
// >= 512 bytes, chunk ^ 2*(t & 15) makes both the QK reads (16 rows x one
// chunk per 16 lanes, ds_read_b128) and the transposed PV reads (4 rows x
// 32 bytes per 16 lanes, ds_read_b64_tr_b16) conflict-free. 256-byte rows
// (d_c = 128) keep a 4-bit swizzle.
template <int DC>
__device__ __forceinline__ int swz(int t) {
  if constexpr (DC >= 256) return 2 * (t & 15);
  else return ((t & 3) << 1) | ((t >> 2) & 1) | (((t >> 3) & 1) << 3);
}
// RoPE-row swizzle (128-byte rows): 16 rows of one chunk hit distinct banks.
__device__ __forceinline__ int swz_r(int t) { return (t >> 1) & 7; }

template <int DC, int NB, int NW>
struct Cfg {
  static constexpr int CPR = DC / 8;             // 16-byte chunks per latent row
  static constexpr int RPI = 64 / CPR;           // latent rows per 1 KB DMA instruction
  static constexpr int NL = kT / RPI;            // latent DMA instructions per tile
  static constexpr int NR = kT * kDR * 2 / 1024; // rope DMA instructions per tile
  static constexpr int NI = NL + NR;
  static constexpr int PER_HI = (NI + NW - 1) / NW;  // per wave (waves < NI % NW)
  static constexpr int PER_LO = NI / NW;             // per wave (the others)
  static constexpr int LAT_BYTES = kT * DC * 2;
  static constexpr int STAGE = LAT_BYTES + kT * kDR * 2;
  static constexpr int KS = DC / 32;             // latent k-steps (K = 32)
  static constexpr int KPB = KS / NB;            // latent k-steps per branch
  static constexpr int MB = DC / 16;             // PV output row blocks
  static constexpr int MPB = MB / NB;            // PV row blocks per branch
  static constexpr int HWG = 16 * NW;            // heads per workgroup
  static constexpr bool PRE_VOFF = PER_HI <= 9;  // DMA lane offsets held in VGPRs
  static_assert(CPR >= 16 && 64 % CPR == 0, "latent width must be 128, 256 or 512");
  static_assert(KPB >= 1 && MPB >= 1, "branch slice must be >= 32 columns");
};

// Row t and logical chunk of the u-th DMA instruction of this wave.
template <int DC, int NB, int NW>
__device__ __forceinline__ void dma_lane(int u, int wave, int lane, bool& rope, int& t, int& lc) {
  using C = Cfg<DC, NB, NW>;
  const int q = wave + NW * u;
  rope = q >= C::NL;
  if (!rope) {
    t = q * C::RPI + lane / C::CPR;
    lc = (lane % C::CPR) ^ swz<DC>(t);
  } else {
    t = (q - C::NL) * 8 + lane / 8;
    lc = (lane % 8) ^ swz_r(t);
  }
}

// DMA of one tile. Full tiles: per-lane offsets precomputed (voff), the tile
// offset in soffset. The tail tile clamps rows to the segment (tend - 1).
template <int DC, int NB, int NW, bool TAIL>
__device__ __forceinline__ void issue_tile(char LDS_AS* stage, i32x4 crs, i32x4 krs, int cts,
                                           int kts, int tstart, int tend, int wave, int lane,
                                           const uint32_t* voff) {
  using C = Cfg<DC, NB, NW>;
  const uint32_t sbase = (uint32_t)(uintptr_t)stage;
#pragma unroll
  for (int u = 0; u < C::PER_HI; ++u) {
    const int q = wave + NW * u;
    if (q >= C::NI) continue;
    const bool rope = q >= C::NL;
    const uint32_t ldsb = rope ? sbase + C::LAT_BYTES + (q - C::NL) * 1024 : sbase + q * 1024;
    const i32x4 rs = rope ? krs : crs;
    const int ts = rope ? kts : cts;
    if constexpr (!TAIL && C::PRE_VOFF) {
      dma16_stream(rs, ldsb, voff[u], (uint32_t)(tstart * ts * 2));
    } else if constexpr (!TAIL) {
      bool r_;
      int t, lc;
      dma_lane<DC, NB, NW>(u, wave, lane, r_, t, lc);
      dma16_stream(rs, ldsb, (uint32_t)(t * ts * 2 + lc * 16), (uint32_t)(tstart * ts * 2));
    } else {
      bool r_;
      int t, lc;
      dma_lane<DC, NB, NW>(u, wave, lane, r_, t, lc);
      const int row = min(tstart + t, tend - 1);
      dma16_stream(rs, ldsb, (uint32_t)(row * ts * 2 + lc * 16), 0u);
    }
  }
}

// Wait until at most `ahead` tiles of this wave's DMA are still in flight.
template <int PER, int NS>
__device__ __forceinline__ void wait_tiles_per(int ahead) {
  if constexpr (NS >= 4) {
    if (ahead >= 2) { wait_vm<2 * PER>(); return; }
  }
  if constexpr (NS >= 3) {
    if (ahead >= 1) { wait_vm<PER>(); return; }
  }
  wait_vm<0>();
}
template <int DC, int NB, int NW, int NS>
__device__ __forceinline__ void wait_tiles(int ahead, int wave) {
  using C = Cfg<DC, NB, NW>;
  if constexpr (C::PER_HI == C::PER_LO) {
    wait_tiles_per<C::PER_HI, NS>(ahead);
  } else {
    if (wave < C::NI % NW) wait_tiles_per<C::PER_HI, NS>(ahead);
    else wait_tiles_per<C::PER_LO, NS>(ahead);
  }
}

// Static schedule of one tile for one wave: group 0 is the RoPE part of the
// scores; then, per branch, QG groups of QK MFMAs (the last one followed by
// the branch softmax) and PG groups of PV MFMAs. Each group uses at most 8
// A-fragments read from LDS; the fragments of group g+1 are read while group
// g computes.
template <int DC, int NB, int GF = 8>
struct Sched {
  static constexpr int KS = DC / 32, KPB = KS / NB, MB = DC / 16, MPB = MB / NB;
  static constexpr int QG = (KPB + GF / 2 - 1) / (GF / 2);  // QK groups per branch
  static constexpr int QGK = KPB / QG;       // k-steps per QK group (2 M blocks each)
  static constexpr int PG = (MPB + GF - 1) / GF;  // PV groups per branch
  static constexpr int PGM = MPB / PG;       // output blocks per PV group
  static constexpr int GPB = QG + PG;
  static constexpr int NG = 1 + NB * GPB;
  static_assert(QG * QGK == KPB && PG * PGM == MPB && 2 * QGK <= GF && PGM <= GF, "schedule");
};

template <int DC, int NB, int NW, int NS, int HSPLIT, bool QLO>
__global__ __launch_bounds__(64 * NW, 1) void decode_mfma_kernel(DecodeParams p) {
  using C = Cfg<DC, NB, NW>;
  // groups of at most 4 fragments when the residue's registers are live at
  // the widest latent, else 8
  constexpr int GF = QLO && DC == 512 ? 4 : 8;
  using SC = Sched<DC, NB, GF>;
  constexpr int H = C::HWG * HSPLIT;
  __shared__ __attribute__((aligned(1024))) char smem_raw[NS * C::STAGE];
  char LDS_AS* smem = (char LDS_AS*)smem_raw;

  // workgroup -> (item, head group); the head groups of one item share an XCD
  int k, hg;
  if constexpr (HSPLIT == 1) {
    k = blockIdx.x;
    hg = 0;
  } else {
    const int i = blockIdx.x, x = i & 7, j = i >> 3;
    k = (j / HSPLIT) * 8 + x;
    hg = j % HSPLIT;
  }
  const PlanHeader hd = *p.hdr;
  if (k >= hd.n_items) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int l16 = lane & 15, kg = lane >> 4;
  const int head = hg * C::HWG + wave * 16 + l16;

  // per-lane DMA offsets of full tiles (fixed for the whole kernel; kept in
  // registers only when few)
  uint32_t voff[C::PRE_VOFF ? C::PER_HI : 1];
#pragma unroll
  for (int u = 0; u < (C::PRE_VOFF ? C::PER_HI : 0); ++u) {
    bool rope;
    int t, lc;
    dma_lane<DC, NB, NW>(u, wave, lane, rope, t, lc);
    voff[u] = (uint32_t)(t * (rope ? p.kr_ts : p.ckv_ts) * 2 + lc * 16);
  }
  // lane constants of the LDS reads (see the swizzle)
  const int qk_y = kg ^ swz<DC>(l16);
  const int rp_x = swz_r(l16);
  const int pv_r = l16 >> 2, pv_q = l16 & 3;
  const int pv_w = (pv_q >> 1) ^ swz<DC>(4 * kg + pv_r);
  const int pv_row_lo = (4 * kg + pv_r) * DC * 2 + 8 * (pv_q & 1);
  const int pv_row_hi = pv_row_lo + 16 * DC * 2;

  int start = k * hd.chunk;
  MLRA_DCHECK(p.hdr, start >= 0 && start < hd.total, 4);
  const int end = min(start + hd.chunk, hd.total);
  int b = find_seq(p.prefix, p.B, start);

  while (start < end) {
    while (p.prefix[b + 1] <= start) ++b;
    const int seg_end = min(end, p.prefix[b + 1]);
    const int t0 = start - p.prefix[b], t1 = seg_end - p.prefix[b];
    const int ntiles = (t1 - t0 + kT - 1) / kT;
    const i32x4 crs = seq_rsrc(p.ckv + (int64_t)b * p.ckv_bs, t1, p.ckv_ts);
    const i32x4 krs = seq_rsrc(p.krope + (int64_t)b * p.kr_bs, t1, p.kr_ts);
    const int slot = k + b;
    MLRA_DCHECK(p.hdr, b >= 0 && b < p.B, 1);
    MLRA_DCHECK(p.hdr, t0 >= 0 && t1 > t0 && t1 <= p.prefix[b + 1] - p.prefix[b], 2);
    MLRA_DCHECK(p.hdr, slot >= 0 && slot < hd.n_items + p.B, 3);
    _Float16* acc_row = reinterpret_cast<_Float16*>(p.acc) + ((int64_t)slot * H + head) * DC + 4 * kg;

    // earlier stores and loads of this wave done; all waves left the
    // previous segment's LDS tiles
    wait_vm<0>();
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();

    // Q^T as the B operand: lane (head, kg) holds q[head][32 ks + 8 kg .. +8];
    // with QLO also the bf16 residue of q~ (the latent k-steps), whose
    // products with the same K fragments go into the same score accumulators
    bf16x8 q[C::KS + 2];
    bf16x8 ql[QLO ? C::KS : 1];
    {
      const __bf16* qrow = p.q_abs + ((int64_t)b * H + head) * p.q_stride + 8 * kg;
#pragma unroll
      for (int ks = 0; ks < C::KS + 2; ++ks) q[ks] = *(const bf16x8*)(qrow + 32 * ks);
      if constexpr (QLO) {
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) ql[ks] = *(const bf16x8*)(qrow + p.q_lo + 32 * ks);
      }
    }
    // Q lives in AGPRs (MFMA reads its B operand from there), leaving the
    // VGPRs to the fragments and the softmax
#pragma unroll
    for (int ks = 0; ks < C::KS + 2; ++ks) asm volatile("" : "+a"(q[ks]));

    // Q complete before any DMA is in flight: the compiler then needs no vmcnt
    // wait for Q inside the tile loop (such a wait would also drain the DMA)
    wait_vm<0>();
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) {
      if (s < ntiles - 1)
        issue_tile<DC, NB, NW, false>(smem + s * C::STAGE, crs, krs, p.ckv_ts, p.kr_ts,
                                      t0 + s * kT, t1, wave, lane, voff);
      else if (s == ntiles - 1)
        issue_tile<DC, NB, NW, true>(smem + s * C::STAGE, crs, krs, p.ckv_ts, p.kr_ts,
                                     t0 + s * kT, t1, wave, lane, voff);
    }

    f32x4 o[C::MB];
#pragma unroll
    for (int i = 0; i < C::MB; ++i) o[i] = (f32x4){0.f, 0.f, 0.f, 0.f};
    float m_run[NB], l_run[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      m_run[j] = -INFINITY;
      l_run[j] = 0.f;
    }

    // one 32-token tile; valid < kT only for the segment's last tile
    auto tile = [&](const char LDS_AS* st, int valid, auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
      auto load = [&](int gid, bf16x8* F) {
        if (gid == 0) {
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
              F[2 * mb + ks] = *(const bf16x8 LDS_AS*)(st + C::LAT_BYTES +
                                                       (16 * mb + l16) * kDR * 2 +
                                                       16 * ((4 * ks + kg) ^ rp_x));
          return;
        }
        const int g = gid - 1, j = g / SC::GPB, r = g % SC::GPB;
        if (r < SC::QG) {
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int kk = 0; kk < SC::QGK; ++kk) {
              const int ks = j * SC::KPB + r * SC::QGK + kk;
              F[mb * SC::QGK + kk] = *(const bf16x8 LDS_AS*)(st + (16 * mb + l16) * DC * 2 +
                                                            512 * (ks >> 3) +
                                                            16 * ((4 * (ks & 7)) ^ qk_y));
            }
        } else {
#pragma unroll
          for (int i = 0; i < SC::PGM; ++i) {
            const int mb = j * SC::MPB + (r - SC::QG) * SC::PGM + i;
            const int coff = 512 * (mb >> 4) + 16 * ((2 * (mb & 15)) ^ pv_w);
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (i16x4 LDS_AS*)(st + pv_row_lo + coff));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (i16x4 LDS_AS*)(st + pv_row_hi + coff));
            const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            F[i] = __builtin_bit_cast(bf16x8, v);
          }
        }
      };

      f32x4 R[2], S[2];
      bf16x8 P;
      auto compute = [&](int gid, const bf16x8* F) {
        if (gid == 0) {
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) {
            R[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(F[2 * mb], q[C::KS],
                                                            (f32x4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            R[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(F[2 * mb + 1], q[C::KS + 1], R[mb],
                                                            0, 0, 0);
          }
          return;
        }
        const int g = gid - 1, j = g / SC::GPB, r = g % SC::GPB;
        if (r < SC::QG) {
#pragma unroll
          for (int mb = 0; mb < 2; ++mb) {
            if (r == 0) S[mb] = R[mb];
#pragma unroll
            for (int kk = 0; kk < SC::QGK; ++kk) {
              const int ks = j * SC::KPB + r * SC::QGK + kk;
              S[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(F[mb * SC::QGK + kk], q[ks], S[mb],
                                                              0, 0, 0);
              if constexpr (QLO)
                S[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(F[mb * SC::QGK + kk], ql[ks],
                                                                S[mb], 0, 0, 0);
            }
          }
          if (r == SC::QG - 1) {
            // softmax of branch j over this tile's 32 tokens; tokens past the
            // segment end (last tile only) get score -inf
            if constexpr (MASK) {
#pragma unroll
              for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  if (16 * mb + 4 * kg + e >= valid) S[mb][e] = -INFINITY;
            }
            float mx = fmaxf(fmaxf(fmaxf(S[0][0], S[0][1]), fmaxf(S[0][2], S[0][3])),
                             fmaxf(fmaxf(S[1][0], S[1][1]), fmaxf(S[1][2], S[1][3])));
            const float mt = max4(mx) * kLog2e;
            // the segment's first tile sets the reference; afterwards it only
            // moves when a tile max exceeds it by more than kRescale (rare)
            m_run[j] = m_run[j] == -INFINITY ? mt : m_run[j];
            const bool need = mt > m_run[j] + kRescale;
            if (__builtin_expect(__any(need), 0)) {
              const float mn = need ? mt : m_run[j];
              const float f = __builtin_amdgcn_exp2f(m_run[j] - mn);
              l_run[j] *= f;
#pragma unroll
              for (int mb = j * C::MPB; mb < (j + 1) * C::MPB; ++mb) o[mb] *= f;
              m_run[j] = mn;
            }
            float ps = 0.f;
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float pe =
                    __builtin_amdgcn_exp2f(__builtin_fmaf(S[mb][e], kLog2e, -m_run[j]));
                ps += pe;
                P[4 * mb + e] = (__bf16)pe;
              }
            l_run[j] += ps;
          }
        } else {
#pragma unroll
          for (int i = 0; i < SC::PGM; ++i) {
            const int mb = j * SC::MPB + (r - SC::QG) * SC::PGM + i;
            o[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(F[i], P, o[mb], 0, 0, 0);
          }
        }
      };

      bf16x8 F[2][GF];
      load(0, F[0]);
#pragma unroll
      for (int gid = 0; gid < SC::NG; ++gid) {
        if (gid + 1 < SC::NG) load(gid + 1, F[(gid + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
        compute(gid, F[gid & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    using MaskOn = std::integral_constant<bool, true>;
    using MaskOff = std::integral_constant<bool, false>;
    // steady tiles (it < ntiles - NS): NS - 2 tiles stay in flight, the tile
    // loaded is full and not the last, and no row is masked; the general body
    // handles the tail. Only for one branch: with two or four, the second
    // copy of the tile body makes the compiler spill.
    int it = 0;
    for (; NB == 1 && it < ntiles - NS; ++it) {
      wait_tiles<DC, NB, NW, NS>(NS - 2, wave);
      __builtin_amdgcn_s_barrier();
      const int nt = it + NS - 1;  // tile whose DMA goes out now
      issue_tile<DC, NB, NW, false>(smem + (nt % NS) * C::STAGE, crs, krs, p.ckv_ts, p.kr_ts,
                                    t0 + nt * kT, t1, wave, lane, voff);
      tile(smem + (it % NS) * C::STAGE, kT, MaskOff{});
    }
    for (; it < ntiles; ++it) {
      const int ahead = min(NS - 2, ntiles - 1 - it);
      wait_tiles<DC, NB, NW, NS>(ahead, wave);
      __builtin_amdgcn_s_barrier();
      const int nt = it + NS - 1;  // tile whose DMA goes out now
      if (nt < ntiles - 1)
        issue_tile<DC, NB, NW, false>(smem + (nt % NS) * C::STAGE, crs, krs, p.ckv_ts, p.kr_ts,
                                      t0 + nt * kT, t1, wave, lane, voff);
      else if (nt == ntiles - 1)
        issue_tile<DC, NB, NW, true>(smem + (nt % NS) * C::STAGE, crs, krs, p.ckv_ts, p.kr_ts,
                                     t0 + nt * kT, t1, wave, lane, voff);
      tile(smem + (it % NS) * C::STAGE, min(kT, t1 - (t0 + it * kT)), MaskOn{});
    }

    // partial state of this segment: m, l as [slot][n][H]; the accumulator
    // normalised by its branch's l (a weighted mean of cache rows) as fp16
    // [slot][H][d_c], 8-byte stores of 4 consecutive latent columns
    float inv[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const float lt = sum4(l_run[j]);
      if (kg == 0) {
        p.m[((int64_t)slot * NB + j) * H + head] = m_run[j];
        p.l[((int64_t)slot * NB + j) * H + head] = lt;
      }
      inv[j] = lt > 0.f ? 1.f / lt : 0.f;
    }
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
      store_f16x4_sat(acc_row + 16 * mb, o[mb] * inv[(16 * mb) / (DC / NB)]);
    start = seg_end;
    ++b;
  }
}

// Workgroups resident per CU: enough waves for all four SIMDs. At d_c = 128 a
// wave needs <= 256 registers, so two fit per SIMD; wider latents need up to
// 512 (Q and O of 16 heads), one per SIMD. The tile ring takes that share of
// the 160 KB of LDS.
constexpr int wgs_per_cu(int dc, int nw) { return (dc == 128 ? 8 : 4) / nw; }

template <int DC, int NB, int NW, int HSPLIT, bool QLO>
hipError_t launch_t(const Geom& g, const QView& q, const void* ckv, const void* krope,
                    const Workspace& ws, int items, hipStream_t s,
                    const KernelTiming& t) {
  using C = Cfg<DC, NB, NW>;
  // as many stages as this workgroup's share of LDS holds (<= 4) and the
  // 6-bit vmcnt can track
  constexpr int NS_LDS = (160 * 1024) / wgs_per_cu(DC, NW) / C::STAGE;
  constexpr int NS_VM = 2 * C::PER_HI < 64 ? 4 : 3;
  constexpr int NS = NS_LDS < NS_VM ? NS_LDS : NS_VM;
  static_assert(NS >= 2, "tile does not fit LDS");
  DecodeParams p;
  p.q_abs = (const __bf16*)q.q;
  p.q_stride = q.stride;
  p.q_lo = q.lo;
  p.ckv = (const __bf16*)ckv;
  p.krope = (const __bf16*)krope;
  p.ckv_bs = g.ckv_bs;
  p.ckv_ts = (int)g.ckv_ts;
  p.kr_bs = g.kr_bs;
  p.kr_ts = (int)g.kr_ts;
  p.hdr = ws.hdr;
  p.prefix = ws.prefix;
  p.m = ws.m;
  p.l = ws.l;
  p.acc = ws.acc;
  p.B = g.B;
  int grid = items;
  if (HSPLIT > 1) grid = ((items + 7) / 8) * 8 * HSPLIT;  // whole XCD rounds
  hipExtLaunchKernelGGL((decode_mfma_kernel<DC, NB, NW, NS, HSPLIT, QLO>), dim3(grid),
                        dim3(64 * NW), 0, s, t.start, t.stop, 0, p);
  return hipGetLastError();
}

// heads -> (waves per workgroup, head groups per item)
template <int DC, int NB, bool QLO>
hipError_t launch_hq(const Geom& g, const QView& q, const void* c, const void* k,
                     const Workspace& ws, int items, hipStream_t s,
                     const KernelTiming& t) {
  switch (g.H) {
    case 32: return launch_t<DC, NB, 2, 1, QLO>(g, q, c, k, ws, items, s, t);
    case 64: return launch_t<DC, NB, 4, 1, QLO>(g, q, c, k, ws, items, s, t);
    case 128: return launch_t<DC, NB, 4, 2, QLO>(g, q, c, k, ws, items, s, t);
  }
  return hipErrorNotSupported;
}

// With or without q~'s residue (mlra_decode gives it; a caller's q_abs in
// mla_decode_attn has it only with q_residue). A query rounded to one bf16
// moves every score by about 2^-9 of its spread; with one softmax over the
// whole latent (MLA at the pages' scales) that alone moves output rows by up
// to ~1.3e-2, and narrower latents at the pages' alpha spread their scores
// wider still.
template <int DC, int NB>
hipError_t launch_h(const Geom& g, const QView& q, const void* c, const void* k,
                    const Workspace& ws, int items, hipStream_t s,
                    const KernelTiming& t) {
  if (q.lo > 0) return launch_hq<DC, NB, true>(g, q, c, k, ws, items, s, t);
  return launch_hq<DC, NB, false>(g, q, c, k, ws, items, s, t);
}

template <int DC>
hipError_t launch_nb(const Geom& g, const QView& q, const void* c, const void* k,
                     const Workspace& ws, int items, hipStream_t s,
                     const KernelTiming& t) {
  switch (g.n) {
    case 1: return launch_h<DC, 1>(g, q, c, k, ws, items, s, t);
    case 2: return launch_h<DC, 2>(g, q, c, k, ws, items, s, t);
    case 4: return launch_h<DC, 4>(g, q, c, k, ws, items, s, t);
  }
  return hipErrorNotSupported;
}

}  // namespace

// q~'s residue for one or two branches: a softmax over one or two branch
// slices on a bf16 query alone moves output rows by up to ~1.1e-2 at the
// pages' scales; four branches average their errors (<= 8.6e-3 measured), as
// in the branch kernel, and the residue would double the latent k-steps.
bool decode_mfma_reads_residue(const Geom& g) { return g.n < 4; }

bool decode_mfma_supported(const Geom& g) {
  if (g.dr != kDR) return false;
  if (g.H != 32 && g.H != 64 && g.H != 128) return false;
  if (g.dc != 128 && g.dc != 256 && g.dc != 512) return false;
  if (g.n != 1 && g.n != 2 && g.n != 4) return false;
  if (g.dc / g.n < 32) return false;
  return true;
}

// Work items that keep every CU busy: workgroups resident per CU over the
// workgroups (head groups) of one item.
int decode_mfma_target_items(const Geom& g, int cus) {
  const int nw = g.H == 32 ? 2 : 4, hsplit = g.H == 128 ? 2 : 1;
  return cus * wgs_per_cu(g.dc, nw) / hsplit;
}

hipError_t launch_decode_mfma(const Geom& g, const QView& q, const void* ckv,
                              const void* krope, const Workspace& ws, int items,
                              hipStream_t s, const KernelTiming& t) {
  switch (g.dc) {
    case 128: return launch_nb<128>(g, q, ckv, krope, ws, items, s, t);
    case 256: return launch_nb<256>(g, q, ckv, krope, ws, items, s, t);
    case 512: return launch_nb<512>(g, q, ckv, krope, ws, items, s, t);
  }
  return hipErrorNotSupported;
}

}  // namespace mlra
