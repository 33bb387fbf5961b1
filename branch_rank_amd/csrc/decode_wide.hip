// Wide MFMA split-KV decode for a 512-wide latent at 128 heads, gfx950
// (MI355X): MLA (one branch over the whole latent).
//
// What it computes ("Multi-Head Low-Rank Attention", 核心方法 and 方法步骤详情
// step 2; "vllbc02MLA", 苏神思路: the decode works like MQA over the latent):
// for one work item (a token range of one or more sequences, see PlanHeader),
// each branch j's online softmax over the scores q~_j[h]·c_t[S_j] + rho[h]·k^R_t
// and its accumulator acc_j[h] = sum_t p_t c_t[S_j], written as the same
// partial state (m, l, acc) as the other MFMA decodes, so the same merge
// follows.
//
// Mapping onto CDNA4:
//  * One workgroup of NW waves per work item holds all 128 heads, so every
//    byte of a tile is streamed into LDS once per CU. The work of a tile is
//    split two ways:
//      - scores and softmax by heads: wave w owns heads [HPW w, HPW w + HPW)
//        across the whole 576-wide row (Q^T stays in its registers);
//      - P V by columns: wave w owns latent columns [CPW w, CPW w + CPW) for
//        all 128 heads (its O^T stays in its registers), reading every head's
//        P^T from LDS, where each wave leaves its own after the softmax.
//    So each transposed V^T read from LDS (the slow LDS read on this chip)
//    feeds eight MFMAs, one per 16-head block, and a wave's registers hold
//    Q of HPW heads plus O of CPW columns: 72 + 128 with eight waves, which
//    leaves room for a second wave on every SIMD to hide LDS latency.
//  * The RoPE score is computed once per head and tile and shared by every
//    branch (the method's flop count).
//  * 32-token tiles stream HBM -> LDS by LDS-DMA (device-scope, non-temporal)
//    into a ring of NS stages of 36 KB; the waves share a tile's 36 1 KB
//    instructions. Two workgroup barriers per tile: one before the scores
//    (the tile is in LDS and converted, the previous tile's P V is done, so
//    its stage takes the DMA NS - 1 tiles ahead and its P^T can be
//    overwritten) and one before P V (every head's P^T is in LDS).
//  * F16: the MFMAs run in fp16. After its own DMA of the next tile lands,
//    each lane converts the 16 bytes it loaded from bf16 to fp16 in place
//    (exact for |x| in [2^-14, 65504]: bf16's 8 significant bits fit fp16's
//    11; round toward zero saturates beyond, flushes the negligible tail
//    below). q~ (its bf16 parts summed in fp32) and P are rounded to fp16,
//    2^-11 relative, where a bf16 query's 2^-8 alone moves one softmax's
//    output rows by up to ~1.3e-2 at MLA's scales on the pages. P is kept
//    <= 2^15 (the reference moves when a tile's max passes it by 15 in log2
//    units), within fp16's range; the factor that rescales a head's
//    accumulators then goes to LDS beside its P^T for the column owners.
//  * QK: S^T[t][h] on v_mfma_f32_16x16x32_{f16,bf16}, 16 tokens as M and 16
//    heads as N, from a per-row bias (0, or -inf past the segment's end), in
//    two accumulator sets (even and odd k-steps) so that more MFMAs are
//    independent. The S^T accumulators (lane = head) are P^T, the B operand
//    of O^T[c][h] += V^T[c][t] P^T[t][h], with V^T read by ds_read_b64_tr_b16
//    from the same LDS tile. The LDS rows are XOR-swizzled in 16-byte chunks
//    (chunk ^ 2 (t & 15) for latent rows, ^ ((t >> 1) & 7) for RoPE rows), as
//    in the head-group kernel, so both read patterns are free of bank
//    conflicts.

#include <hip/hip_ext.h>

#include <type_traits>

#include "device_common.h"

#ifndef MLRA_WIDE_WAVES
#define MLRA_WIDE_WAVES 8
#endif

namespace mlra {
namespace {

using namespace dev;

constexpr int kT = 32;                   // tokens per tile
constexpr int kDC = 512;                 // latent width
constexpr int kDR = 64;                  // RoPE width
constexpr int kLat = kT * kDC * 2;       // latent bytes of a stage
constexpr int kStage = kLat + kT * kDR * 2;  // 36 KB
constexpr int kHMax = 128;               // most heads
constexpr int kNI = kT + 4;              // DMA instructions per tile (32 latent rows + 4 RoPE)
constexpr int kKS = kDC / 32;            // latent k-steps
constexpr int kNS = 4;                   // tile stages (144 KB of LDS)
// fp8 codes: 18 KB per stage, 16 latent DMA instructions (two rows each) and
// two RoPE instructions (16 rows each) per tile
constexpr int kLat8 = kT * kDC;
constexpr int kStage8 = kLat8 + kT * kDR;
constexpr int kLR8 = kT / 2;

typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;

// MFMA operand type: fp16 (cache converted in LDS) or bf16 (as stored).
template <bool F16>
struct Op;
template <>
struct Op<true> {
  using V = f16x8;
  using E = _Float16;
  static __device__ __forceinline__ f32x4 mfma(V a, V b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Op<false> {
  using V = bf16x8;
  using E = __bf16;
  static __device__ __forceinline__ f32x4 mfma(V a, V b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

__device__ __forceinline__ int swz(int t) { return 2 * (t & 15); }
__device__ __forceinline__ int swz_r(int t) { return (t >> 1) & 7; }


// Wave shape for H heads: the score waves (the first QW; with fewer than 16
// heads per wave the others only load, convert and accumulate) own
// HPW = 16 NBQ heads each; every wave accumulates CPW latent columns of all H
// heads.
template <int NW, int H>
struct WCfg {
  static constexpr int HB = H / 16;                  // 16-head blocks
  static constexpr int QW = HB < NW ? HB : NW;       // score waves
  static constexpr int HPW = H / QW;                 // heads per score wave
  static constexpr int NBQ = HPW / 16;               // 16-head blocks per score wave
  static constexpr int CPW = kDC / NW;               // latent columns per wave (P V)
  static constexpr int CBW = CPW / 16;               // PV column blocks per wave
  static constexpr int LR = kT / NW;                 // latent rows each wave loads per tile
  static constexpr int PB = HB < 4 ? HB : 4;         // P^T fragments read at a time
  static_assert(H % 16 == 0 && H <= kHMax && HPW % 16 == 0 && CPW % 16 == 0 && kT % NW == 0 &&
                    NW >= 4 && HB % PB == 0,
                "wave shape");
};

template <int NB, bool F16, int NW, bool FP8, int H>
__global__ __launch_bounds__(64 * NW, 1) void decode_wide_kernel(DecodeParams p) {
  using O_ = Op<F16>;
  using V = typename O_::V;
  using E = typename O_::E;
  using C = WCfg<NW, H>;
  constexpr int NBQ = C::NBQ, CBW = C::CBW, kHB = C::HB, QW = C::QW, PB = C::PB;
  constexpr int KPB = kKS / NB;  // latent k-steps per branch
  constexpr float kRescale = F16 ? 15.f : 16.f;
  static_assert(kKS % NB == 0, "branches");
  static_assert(!FP8 || F16, "fp8 codes are converted to fp16");

  // LDS: the tile ring (bf16: kNS stages of 36 KB, converted in place; fp8:
  // two 36 KB fp16 tiles, the one in use and the next, then kNS stages of
  // 18 KB of codes), then the P exchange (P^T fragments of NB branches x
  // H / 16 16-head blocks, 1 KB each: lane l's 16 bytes at 16 l, the B-operand
  // layout), the rescale factors per (branch, head) and one flag per (score
  // wave, branch) that says whether any of its heads' references moved
  constexpr int kPBytes = NB * kHB * 1024;
  constexpr int kRing = FP8 ? 2 * kStage + kNS * kStage8 : kNS * kStage;
  __shared__ __attribute__((aligned(1024))) char smem_raw[kRing + kPBytes];
  __shared__ float fl_raw[NB * H];
  __shared__ int flags_raw[NW * NB];
  char LDS_AS* smem = (char LDS_AS*)smem_raw;
  char LDS_AS* pl = smem + kRing;
  float LDS_AS* fl = (float LDS_AS*)fl_raw;
  int LDS_AS* flags = (int LDS_AS*)flags_raw;
  const uint32_t sbase = (uint32_t)(uintptr_t)smem;

  const int k = blockIdx.x;
  const PlanHeader hd = *p.hdr;
  if (k >= hd.n_items) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int l16 = lane & 15, kg = lane >> 4;
  __builtin_assume(wave >= 0 && wave < NW);
  const int jq = wave * NB / NW;  // branch of this wave's columns

  // DMA of a tile: wave w loads latent rows w + NW u (u < LR; lane l: LDS
  // chunk l, global chunk l ^ swz(row), the row's offset in the scalar
  // offset) and, for w < 4, RoPE rows 8 w .. 8 w + 7 (lane l: row 8 w + l / 8,
  // LDS chunk l % 8, global chunk (l % 8) ^ swz_r(row)). The DMA writes lane
  // l's 16 bytes at a wave-uniform LDS offset + 16 l.
  //
  // fp8: a stage holds the codes row after row (latent rows of 512 bytes,
  // then RoPE rows of 64), unswizzled: wave w loads latent rows 2 q, 2 q + 1
  // for q = w + NW u (u < 16 / NW; lane l: row 2 q + l / 32, bytes
  // 16 (l % 32) of it) and, for w < 2, RoPE rows 16 w .. 16 w + 15 (lane l:
  // row 16 w + l / 4, bytes 16 (l % 4)); rows are clamped per lane. Each lane
  // later converts the 16 codes it loaded into the swizzled fp16 tile.
  const bool rope_wave = FP8 ? wave < 2 : wave < 4;
  auto lat_lds = [&](int u) { return (uint32_t)((wave + NW * u) * 1024); };
  const uint32_t rope_lds = (uint32_t)((FP8 ? kLat8 : kLat) + wave * 1024);
  const int rope_rt = FP8 ? 16 * wave + (lane >> 2) : 8 * wave + (lane >> 3);
  const uint32_t rope_c = FP8 ? (uint32_t)(16 * (lane & 3))
                              : (uint32_t)(16 * ((lane & 7) ^ swz_r(rope_rt)));
  // QK A fragments: row 16 mb + l16, logical chunk 4 ks + kg, physical chunk
  // (4 ks + kg) ^ 2 l16 = 4 ks ^ (kg ^ 2 l16); the XOR touches address bits
  // 6-9 only, which the lane base and every stage base leave zero.
  const int qk_base = l16 * 1024 + 16 * (kg ^ (2 * l16));
  const int rp_base = kLat + l16 * 128 + 16 * (kg ^ swz_r(l16));
  // PV transposed reads (as in the head-group kernel)
  const int pv_r = l16 >> 2, pv_q = l16 & 3;
  const int pv_w = (pv_q >> 1) ^ swz(4 * kg + pv_r);
  const int pv_lo = (4 * kg + pv_r) * 1024 + 8 * (pv_q & 1);

  int start = k * hd.chunk;
  MLRA_DCHECK(p.hdr, start >= 0 && start < hd.total, 4);
  const int end = min(start + hd.chunk, hd.total);
  int bseq = find_seq(p.prefix, p.B, start);

  while (start < end) {
    while (p.prefix[bseq + 1] <= start) ++bseq;
    const int seg_end = min(end, p.prefix[bseq + 1]);
    const int t0 = start - p.prefix[bseq], t1 = seg_end - p.prefix[bseq];
    const int ntiles = (t1 - t0 + kT - 1) / kT;
    // cache bytes per element: 2 (bf16) or 1 (fp8 codes)
    constexpr int EB = FP8 ? 1 : 2;
    const i32x4 crs = seq_rsrc_bytes((const char*)p.ckv + (int64_t)bseq * p.ckv_bs * EB, t1,
                                     p.ckv_ts * EB);
    const i32x4 krs = seq_rsrc_bytes((const char*)p.krope + (int64_t)bseq * p.kr_bs * EB, t1,
                                     p.kr_ts * EB);
    const int slot = k + bseq;
    MLRA_DCHECK(p.hdr, bseq >= 0 && bseq < p.B, 1);
    MLRA_DCHECK(p.hdr, t0 >= 0 && t1 > t0 && t1 <= p.prefix[bseq + 1] - p.prefix[bseq], 2);
    MLRA_DCHECK(p.hdr, slot >= 0 && slot < hd.n_items + p.B, 3);

    // earlier stores and loads of this wave done; all waves left the
    // previous segment's LDS tiles
    wait_vm<0>();
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();

    // Q^T as the B operand: lane (head, kg) holds 8 consecutive k of its
    // head; k-steps 0..15 latent, 16..17 RoPE. The fp16 query is q~'s bf16
    // parts summed in fp32, then rounded once (without a residue in the view
    // the residue loads re-read q~ and are weighted by 0).
    V q[kKS + 2][NBQ];
    const float wlo = p.q_lo > 0 ? 1.f : 0.f;
#pragma unroll
    for (int nb = 0; nb < NBQ; ++nb) {
      const __bf16* qrow =
          p.q_abs + ((int64_t)bseq * H + C::HPW * (wave < QW ? wave : 0) + 16 * nb + l16) *
                        p.q_stride +
          8 * kg;
      const __bf16* lrow = qrow + p.q_lo;
#pragma unroll
      for (int ks = 0; ks < kKS + 2; ++ks) {
        const int off = ks < kKS ? 32 * ks : kDC + 32 * (ks - kKS);
        const bf16x8 hi = *(const bf16x8*)(qrow + off);
        if constexpr (F16) {
          V v;
          if (ks < kKS) {
            const bf16x8 lo = *(const bf16x8*)(lrow + off);
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = (E)__builtin_fmaf(wlo, (float)lo[i], (float)hi[i]);
          } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = (E)(float)hi[i];
          }
          q[ks][nb] = v;
        } else {
          q[ks][nb] = hi;
        }
      }
    }
    // Q complete before any DMA is in flight: the loop's vmcnt waits then
    // count DMA only
    wait_vm<0>();

    // DMA instruction u of this wave for `tile`; the segment's last tile
    // clamps its rows to t1 - 1 (the segment's rows bound the buffer range)
    auto issue = [&](int tile) {
      const int ts0 = t0 + tile * kT;
      if constexpr (FP8) {
        const uint32_t sa = sbase + (uint32_t)(2 * kStage + (tile & (kNS - 1)) * kStage8);
#pragma unroll
        for (int u = 0; u < kLR8 / NW; ++u) {
          const int row = min(ts0 + 2 * (wave + NW * u) + (lane >> 5), t1 - 1);
          dma16_stream(crs, sa + lat_lds(u), (uint32_t)(row * p.ckv_ts + 16 * (lane & 31)), 0u);
        }
        if (rope_wave) {
          const int row = min(ts0 + rope_rt, t1 - 1);
          dma16_stream(krs, sa + rope_lds, (uint32_t)(row * p.kr_ts) + rope_c, 0u);
        }
        return;
      }
      const uint32_t sa = sbase + (uint32_t)((tile & (kNS - 1)) * kStage);
#pragma unroll
      for (int u = 0; u < C::LR; ++u) {
        const int qi = wave + NW * u;
        const int row = min(ts0 + qi, t1 - 1);
        dma16_stream(crs, sa + lat_lds(u), (uint32_t)(16 * (lane ^ swz(qi))),
                     (uint32_t)(row * p.ckv_ts * 2));
      }
      if (rope_wave) {
        const int row = min(ts0 + rope_rt, t1 - 1);
        dma16_stream(krs, sa + rope_lds, (uint32_t)(row * p.kr_ts * 2) + rope_c, 0u);
      }
    };
    // wait until this wave's DMA of `tile` has landed, given the tiles
    // issued after it that may stay in flight (at most kNS - 2)
    auto wait_own = [&](int tile) {
      constexpr int L = FP8 ? kLR8 / NW : C::LR, LH = L + 1;
      const int after = min(tile + kNS - 2, ntiles - 1) - tile;
      if (rope_wave) {
        if (after >= 2) wait_vm<2 * LH>();
        else if (after == 1) wait_vm<LH>();
        else wait_vm<0>();
      } else {
        if (after >= 2) wait_vm<2 * L>();
        else if (after == 1) wait_vm<L>();
        else wait_vm<0>();
      }
      asm volatile("" ::: "memory");
    };
    // this lane's 16-byte chunks of `tile` from bf16 to fp16, in place; fp8:
    // its 16 codes per instruction into the fp16 tile (tile & 1), swizzled
    // as the bf16 tiles: latent row t, codes 16 cc .. 16 cc + 15 are fp16
    // chunks 2 cc, 2 cc + 1, at chunks 2 (cc ^ (t & 15)) and the next (one
    // 32-byte store); RoPE row t's chunks 2 cc, 2 cc + 1 at (2 cc) ^ swz_r(t)
    // and (2 cc + 1) ^ swz_r(t)
    auto convert = [&](int tile) {
      if constexpr (FP8) {
        // the lane's offsets are recomputed here from an opaque copy of the
        // lane id: kept live across the loop they would be spilled, and a
        // reload waits for every load in flight, the DMA included
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const char LDS_AS* src = smem + 2 * kStage + (tile & (kNS - 1)) * kStage8 + 16 * ln;
        char LDS_AS* dst = smem + (tile & 1) * kStage;
        i32x4 x[kLR8 / NW], r;
#pragma unroll
        for (int u = 0; u < kLR8 / NW; ++u) x[u] = *(const i32x4 LDS_AS*)(src + lat_lds(u));
        if (rope_wave) r = *(const i32x4 LDS_AS*)(src + kLat8 + wave * 1024);
#pragma unroll
        for (int u = 0; u < kLR8 / NW; ++u) {
          const int tr = 2 * (wave + NW * u) + (ln >> 5), cc = ln & 31;
          i32x4 lo, hi;
          fp8x16_to_f16(x[u], lo, hi);
          char LDS_AS* d = dst + tr * 1024 + 32 * (cc ^ (tr & 15));
          *(i32x4 LDS_AS*)d = lo;
          *(i32x4 LDS_AS*)(d + 16) = hi;
        }
        if (rope_wave) {
          const int cc = ln & 3, rt = 16 * wave + (ln >> 2);
          i32x4 lo, hi;
          fp8x16_to_f16(r, lo, hi);
          char LDS_AS* d = dst + kLat + rt * 128;
          *(i32x4 LDS_AS*)(d + 16 * ((2 * cc) ^ swz_r(rt))) = lo;
          *(i32x4 LDS_AS*)(d + 16 * ((2 * cc + 1) ^ swz_r(rt))) = hi;
        }
        return;
      }
      char LDS_AS* st = smem + (tile & (kNS - 1)) * kStage + 16 * lane;
      i32x4 x[C::LR], r;
#pragma unroll
      for (int u = 0; u < C::LR; ++u) x[u] = *(const i32x4 LDS_AS*)(st + lat_lds(u));
      if (rope_wave) r = *(const i32x4 LDS_AS*)(st + rope_lds);
#pragma unroll
      for (int u = 0; u < C::LR; ++u) *(i32x4 LDS_AS*)(st + lat_lds(u)) = bf16_to_f16x8(x[u]);
      if (rope_wave) *(i32x4 LDS_AS*)(st + rope_lds) = bf16_to_f16x8(r);
    };

#pragma unroll
    for (int s = 0; s < kNS - 1; ++s)
      if (s < ntiles) issue(s);

    // O^T of this wave's columns (column blocks CBW wave + c) for every
    // 16-head block
    f32x4 o[CBW][kHB];
#pragma unroll
    for (int c = 0; c < CBW; ++c)
#pragma unroll
      for (int hb = 0; hb < kHB; ++hb) o[c][hb] = (f32x4){0.f, 0.f, 0.f, 0.f};
    float m_run[NB][NBQ], l_run[NB][NBQ];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int nb = 0; nb < NBQ; ++nb) {
        m_run[j][nb] = -INFINITY;
        l_run[j][nb] = 0.f;
      }
    if constexpr (F16) {
      wait_own(0);
      convert(0);
    }

    auto barrier = [&] {
      // this wave's LDS writes complete and its reads returned: s_barrier
      // waits for neither
      wait_lgkm0();
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    };

    for (int t = 0; t < ntiles; ++t) {
      if constexpr (!F16) wait_own(t);
      barrier();  // tile t in LDS (converted); P V of tile t - 1 done
      if (t + kNS - 1 < ntiles) issue(t + kNS - 1);
      const char LDS_AS* st = smem + (FP8 ? (t & 1) : (t & (kNS - 1))) * kStage;
      // V^T fragment of column block cb
      auto pv_frag = [&](int cb) -> V {
        const int coff = 512 * (cb >> 4) + 16 * ((2 * (cb & 15)) ^ pv_w);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)(st + pv_lo + coff));
        const i16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)(st + pv_lo + 16 * 1024 + coff));
        const i16x8 vv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(V, vv);
      };

      // scores and softmax (score waves); the others convert their share of
      // the next tile
      if (wave >= QW) {
        if constexpr (F16) {
          if (t + 1 < ntiles) {
            wait_own(t + 1);
            convert(t + 1);
          }
        }
      } else {
      // score bias per token row: 0, or -inf past the segment's end
      f32x4 bias[2];
      const int valid = t1 - (t0 + t * kT);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) bias[mb][e] = 16 * mb + 4 * kg + e < valid ? 0.f : -INFINITY;

      // RoPE score of this wave's heads, shared by the branches
      f32x4 R[2][NBQ];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const V a0 = *(const V LDS_AS*)(st + rp_base + mb * 2048);
        const V a1 =
            *(const V LDS_AS*)((const char LDS_AS*)(((uintptr_t)(st + rp_base + mb * 2048)) ^ 64));
#pragma unroll
        for (int nb = 0; nb < NBQ; ++nb) {
          R[mb][nb] = O_::mfma(a0, q[kKS][nb], bias[mb]);
          R[mb][nb] = O_::mfma(a1, q[kKS + 1][nb], R[mb][nb]);
        }
      }

      // A fragments of k-step ks (rows 0-15 and 16-31)
      auto qk_frag = [&](int ks, V* a) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          a[mb] = *(const V LDS_AS*)((const char LDS_AS*)(((uintptr_t)(st + qk_base +
                                                                       mb * 16 * 1024)) ^
                                                          (64 * ks)));
      };


#pragma unroll
      for (int j = 0; j < NB; ++j) {
        // two accumulator sets (even and odd k-steps): more independent MFMA
        // chains per wave
        // with one wave per SIMD, two accumulator sets (even and odd k-steps)
        // make more MFMA chains independent; with two, the other wave hides
        // the chain's latency and the registers are needed for Q and O
        constexpr bool kDual = NW < 8;
        constexpr int kPf = kDual ? 2 : 1;  // k-steps of fragments read ahead
        f32x4 S[2][NBQ], S2[2][NBQ];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < NBQ; ++nb) {
            S[mb][nb] = R[mb][nb];
            if constexpr (kDual) S2[mb][nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
          }
        // software pipeline: the fragments of k-step ks + kPf are read while
        // k-step ks computes; fences keep the compiler from hoisting every
        // read of the tile (their registers would not fit beside Q and O)
        V A[kPf + 1][2];
#pragma unroll
        for (int i = 0; i < kPf && i < KPB; ++i) qk_frag(j * KPB + i, A[i]);
#pragma unroll
        for (int kk = 0; kk < KPB; ++kk) {
          const int ks = j * KPB + kk;
          if (kk + kPf < KPB) qk_frag(ks + kPf, A[(kk + kPf) % (kPf + 1)]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < NBQ; ++nb) {
              const V& a = A[kk % (kPf + 1)][mb];
              if (kDual && (kk & 1)) S2[mb][nb] = O_::mfma(a, q[ks][nb], S2[mb][nb]);
              else S[mb][nb] = O_::mfma(a, q[ks][nb], S[mb][nb]);
            }
          __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (kDual) {
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < NBQ; ++nb) S[mb][nb] += S2[mb][nb];
        }
        // the next tile's conversion runs while these MFMAs drain
        if constexpr (F16) {
          if (j == 0 && t + 1 < ntiles) {
            wait_own(t + 1);
            convert(t + 1);
          }
        }
        // branch j's online softmax over the tile for this wave's heads; P^T
        // and the factor that rescales the heads' accumulators (1 unless the
        // reference moved) go to LDS for the waves that own the columns
        bool moved = false;
#pragma unroll
        for (int nb = 0; nb < NBQ; ++nb) {
          const float mx =
              fmaxf(fmaxf(fmaxf(S[0][nb][0], S[0][nb][1]), fmaxf(S[0][nb][2], S[0][nb][3])),
                    fmaxf(fmaxf(S[1][nb][0], S[1][nb][1]), fmaxf(S[1][nb][2], S[1][nb][3])));
          const float mt = max4(mx) * kLog2e;
          const bool need = mt > m_run[j][nb] + kRescale;
          float f = 1.f;
          if (__builtin_expect(__any(need), 0)) {
            const float mn = need ? mt : m_run[j][nb];
            f = __builtin_amdgcn_exp2f(m_run[j][nb] - mn);
            l_run[j][nb] *= f;
            m_run[j][nb] = mn;
            moved = true;
          }
          V P;
          float ps = 0.f;
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(S[mb][nb][e], kLog2e,
                                                                     -m_run[j][nb]));
              ps += pe;
              P[4 * mb + e] = (E)pe;
            }
          l_run[j][nb] += ps;
          const int hb = NBQ * wave + nb;
          *(V LDS_AS*)(pl + ((j * kHB + hb) * 64 + lane) * 16) = P;
          if (kg == 0) fl[j * H + 16 * hb + l16] = f;
        }
        if (lane == 0) flags[wave * NB + j] = moved ? 1 : 0;
      }
      }

      barrier();  // every head's P^T is in LDS

      // rescale this wave's accumulators of the heads whose reference moved
      {
        int any = 0;
#pragma unroll
        for (int w = 0; w < QW; ++w) any |= flags[w * NB + jq];
        if (__builtin_expect(any != 0, 0)) {
#pragma unroll
          for (int hb = 0; hb < kHB; ++hb) {
            const float f = fl[jq * H + 16 * hb + l16];
#pragma unroll
            for (int c = 0; c < CBW; ++c) o[c][hb] *= f;
          }
        }
      }
      // O^T += V^T P^T over this wave's columns for all heads: every V^T
      // fragment feeds one MFMA per 16-head block; P^T fragments PB at a time
#pragma unroll
      for (int h0 = 0; h0 < kHB; h0 += PB) {
        V Pf[PB];
#pragma unroll
        for (int i = 0; i < PB; ++i)
          Pf[i] = *(const V LDS_AS*)(pl + ((jq * kHB + h0 + i) * 64 + lane) * 16);
        V Vf[3];
#pragma unroll
        for (int c = 0; c < 2 && c < CBW; ++c) Vf[c] = pv_frag(CBW * wave + c);
#pragma unroll
        for (int c = 0; c < CBW; ++c) {
          if (c + 2 < CBW) Vf[(c + 2) % 3] = pv_frag(CBW * wave + c + 2);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = 0; i < PB; ++i) o[c][h0 + i] = O_::mfma(Vf[c % 3], Pf[i], o[c][h0 + i]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }

    // partial state of this segment: m, l as [slot][n][H] (a score wave's
    // heads); the accumulator normalised by l (a weighted mean of cache rows)
    // as fp16 [slot][H][d_c] (this wave's columns, all heads), 8-byte stores
    // of 4 consecutive latent columns. The score waves pass 1/l to the column
    // owners through the rescale table, once every wave has left the last
    // P V (which read it).
    barrier();
#pragma unroll
    for (int nb = 0; nb < NBQ; ++nb) {
      const int head = C::HPW * wave + 16 * nb + l16;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const float lt = sum4(l_run[j][nb]);
        if (kg == 0 && wave < QW) {
          p.m[((int64_t)slot * NB + j) * H + head] = m_run[j][nb];
          p.l[((int64_t)slot * NB + j) * H + head] = lt;
          fl[j * H + head] = lt > 0.f ? 1.f / lt : 0.f;
        }
      }
    }
    barrier();
#pragma unroll
    for (int hb = 0; hb < kHB; ++hb) {
      const float inv = fl[jq * H + 16 * hb + l16];
      _Float16* row = reinterpret_cast<_Float16*>(p.acc) + ((int64_t)slot * H + 16 * hb + l16) * kDC +
                      C::CPW * wave + 4 * kg;
#pragma unroll
      for (int c = 0; c < CBW; ++c) store_f16x4_sat(row + 16 * c, o[c][hb] * inv);
    }
    start = seg_end;
    ++bseq;
  }
}

template <int NB, bool F16, int NW, bool FP8, int H>
hipError_t launch_w(const Geom& g, const QView& q, const void* ckv, const void* krope,
                    const Workspace& ws, int items, hipStream_t s, const KernelTiming& t) {
  DecodeParams p;
  p.q_abs = (const __bf16*)q.q;
  p.q_stride = q.stride;
  p.q_lo = F16 ? q.lo : 0;
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
  hipExtLaunchKernelGGL((decode_wide_kernel<NB, F16, NW, FP8, H>), dim3(items), dim3(64 * NW), 0, s,
                        t.start, t.stop, 0, p);
  return hipGetLastError();
}

}  // namespace

// MLA: one branch over a 512-wide latent, 64-wide RoPE key, 32, 64 or 128
// heads (all of MLA's heads, or one device's share of them under 2- or 4-way
// tensor parallelism). (The kernel is written for n branches with a shared
// RoPE score; only n = 1 is built, with the MFMAs' results selected into
// VGPRs: this compiler's pass that moves them to AGPRs fails on a four-branch
// instantiation.)
bool decode_wide_supported(const Geom& g, bool) {
  return g.dc == kDC && g.dr == kDR && (g.H == 32 || g.H == 64 || g.H == 128) && g.n == 1;
}

// fp16 MFMAs on q~ with its residue
bool decode_wide_reads_residue(const Geom&) { return true; }

template <bool FP8>
hipError_t launch_wh(const Geom& g, const QView& q, const void* ckv, const void* krope,
                     const Workspace& ws, int items, hipStream_t s, const KernelTiming& t) {
  switch (g.H) {
    case 32: return launch_w<1, true, MLRA_WIDE_WAVES, FP8, 32>(g, q, ckv, krope, ws, items, s, t);
    case 64: return launch_w<1, true, MLRA_WIDE_WAVES, FP8, 64>(g, q, ckv, krope, ws, items, s, t);
    case 128: return launch_w<1, true, MLRA_WIDE_WAVES, FP8, 128>(g, q, ckv, krope, ws, items, s, t);
  }
  return hipErrorNotSupported;
}

hipError_t launch_decode_wide(const Geom& g, const QView& q, const void* ckv, const void* krope,
                              const Workspace& ws, int items, hipStream_t s,
                              const KernelTiming& t, bool fp8) {
  if (!decode_wide_supported(g, fp8)) return hipErrorNotSupported;
  return fp8 ? launch_wh<true>(g, q, ckv, krope, ws, items, s, t)
             : launch_wh<false>(g, q, ckv, krope, ws, items, s, t);
}

}  // namespace mlra
