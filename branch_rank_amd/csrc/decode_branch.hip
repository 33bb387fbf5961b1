// Branch-per-wave bf16 MFMA split-KV decode for MLRA-n with 128-wide branch
// slices, gfx950 (MI355X).
//
// What it computes ("Multi-Head Low-Rank Attention", 核心方法 and 方法步骤详情
// step 2; "vllbc02MLA", 苏神思路): for one work item (a token range of one or
// more sequences) and a set of branches, each branch j's own online softmax
// over the scores q~_j[h]·c_t[S_j] + rho[h]·k^R_t of every head and its
// accumulator acc_j[h] = sum_t p_t c_t[S_j]. Branch j only ever touches its
// latent slice S_j (128 columns) and the shared RoPE key, so branches can be
// split between workgroups and waves that never talk to each other.
//
// Mapping onto CDNA4 (the partial state it writes is the same as the
// head-group kernel's, so both feed the same merge):
//  * The NBR branches are split over NSPLIT workgroups per work item: the
//    workgroup for part hg owns branches [hg*NBW, (hg+1)*NBW) for all heads
//    and streams only those branches' latent columns plus the RoPE key
//    (640 of the 1152 bytes of a token row at MLRA-4), so the workgroups of an
//    item read disjoint data and every CU streams its own bytes from HBM.
//    The parts of one item are placed 8 apart in launch order (same XCD), so
//    the RoPE rows that both read come from that XCD's L2 the second time.
//  * A workgroup has NBW x NHG waves: wave (b, g) owns branch hg*NBW + b for
//    the HPW heads of head group g. Its registers hold Q for those heads over
//    the branch slice plus the RoPE part and O over the slice, small enough
//    for two waves per SIMD.
//  * Every tile runs in two phases between workgroup barriers: a matrix phase
//    (PV of the previous tile, QK of this one) and a vector phase (softmax,
//    V^T fragments into registers). Waves w and w + NW/2 share a SIMD and the
//    second group runs one phase behind the first, so on every SIMD one
//    wave's MFMAs run beside the other wave's softmax instead of both waves
//    doing the same kind of work at once.
//  * 32-token tiles stream HBM -> LDS with buffer_load_dwordx4 ... lds (no
//    VGPR staging): one instruction per two 512-byte latent half-rows and per
//    eight 128-byte RoPE rows, shared by all waves, through an NS-stage ring
//    (20 KB per stage, so several tiles are in flight per CU); a stage is
//    reloaded once the lagging group's vector phase has read it. All but a
//    segment's last few tiles run a branch-free steady body (fixed wait depth,
//    full tiles, no row mask); the general body handles the tail. LDS rows are
//    XOR-swizzled in 16-byte chunks (chunk ^ 2*(row & 15) for latent rows,
//    measured free of bank conflicts for both read patterns below).
//  * QK: S^T[t][h] on v_mfma_f32_16x16x32_bf16, 16 tokens as M, 16 heads as N;
//    the S^T accumulators (lane = head) are the B operand of PV,
//    O^T[c][h] = V^T[c][t] P^T[t][h] with V^T read by ds_read_b64_tr_b16, so P
//    never moves between lanes and a rescale is one multiplier per lane.
//  * Lazy rescaling without a per-tile max: P is computed against a running
//    reference; only when some p would pass 2^20 (seen from the per-lane sum
//    of P) does the exact tile max move the reference to 16 below it, with O
//    and l rescaled. fp32 and bf16 hold such p with their usual relative
//    precision.

#include <hip/hip_ext.h>

#include <type_traits>

#include "branch_tiles.h"

namespace mlra {
namespace {

using namespace dev;
using namespace bt;

typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;

// Operand type of the MFMAs: bf16 (the cache as stored), or fp16 (F16: each
// tile converted in LDS, q~ from its two bf16 parts, P in fp16, 2^-11 where
// bf16 gives 2^-9).
template <bool F16>
struct BOp {
  using V = bf16x8;
  using E = __bf16;
  static constexpr float kRes = kRescale, kSum = kSumLimit;
  static __device__ __forceinline__ f32x4 mfma(V a, V b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct BOp<true> {
  using V = f16x8;
  using E = _Float16;
  // P stays below fp16's 65504: a per-lane sum of 8 values above 2^15 moves
  // the reference, to 12 below the tile max (so 8 p <= 2^15 after a move)
  static constexpr float kRes = 12.f, kSum = 32768.f;
  static __device__ __forceinline__ f32x4 mfma(V a, V b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

template <int NBR, int NSPLIT, int HPW, int NHG, int NS, bool QLO, bool FP8, bool F16>
__global__ __launch_bounds__(64 * (NBR / NSPLIT) * NHG, 1) void decode_branch_kernel(DecodeParams p) {
  using C = BCfg<NBR, NSPLIT, HPW, NHG>;
  using O_ = BOp<F16>;
  using VT = typename O_::V;
  using ET = typename O_::E;
  static_assert(!(F16 && QLO), "fp16: q~'s two parts are summed, not multiplied apart");
  constexpr int H = C::H;
  constexpr int DC = C::DC;
  constexpr int D = NS - 1;  // tiles issued ahead of the one in use
  static_assert(D >= 2 && D <= 6, "tile ring");
  // fp8 codes: a stage holds the tile's codes row after row (the branch
  // pair's 256 latent codes per row, then the 64 RoPE codes), unswizzled,
  // 10 KB; each lane converts the 16 codes it loaded into one of two bf16
  // tiles (the one in use and the next) laid out as the bf16 stages.
  static_assert(!FP8 || (C::ROWB == 512 && C::NW == 8), "fp8: two branches per workgroup, 8 waves");
  constexpr int LAT8 = kT * C::ROWB / 2;
  constexpr int STAGE8 = LAT8 + kT * kDR;
  constexpr int RING = FP8 ? 2 * C::STAGE + NS * STAGE8 : NS * C::STAGE;
  __shared__ __attribute__((aligned(1024))) char smem_raw[RING];
  char LDS_AS* smem = (char LDS_AS*)smem_raw;
  const uint32_t sbase = (uint32_t)(uintptr_t)smem;

  // workgroup -> (item, branch part); the parts of one item share an XCD
  int k, hg;
  if constexpr (NSPLIT == 1) {
    k = blockIdx.x;
    hg = 0;
  } else {
    const int i = blockIdx.x, x = i & 7, jj = i >> 3;
    k = (jj / NSPLIT) * 8 + x;
    hg = jj % NSPLIT;
  }
  const PlanHeader hd = *p.hdr;
  if (k >= hd.n_items) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int b = wave % C::NBW;       // branch of this wave within the workgroup
  const int g = wave / C::NBW;       // head group of this wave
  const int j = hg * C::NBW + b;     // branch of this wave
  const int l16 = lane & 15, kg = lane >> 4;
  const int head0 = g * HPW;         // first head of this wave
  const bool lag = wave >= C::NW / 2;  // second group: one phase behind

  // Per-lane LDS byte offsets within a stage. QK A operand: token row
  // 16 mb + l16 (+ 16 rows for mb = 1), branch columns 32 ks + 8 kg .. +7.
  // RoPE: chunk 4 ks + kg of row 16 mb + l16. PV (transposed reads): token
  // rows 4 kg + (l16 >> 2) (+ 16), columns 16 cb + 4 (l16 & 3) .. +3.
  // The swizzle only flips address bits 6-7 (QK, per k-step ks) and 5-7 (PV,
  // per column block cb), which these lane offsets and every stage base (a
  // multiple of 20 KB from a 1 KB-aligned array) leave zero: the address of
  // k-step ks is (base + qk_lat) ^ (64 ks), of block cb (base + pv_lat) ^
  // (32 cb), and the second RoPE k-step is (base + qk_rp) ^ 64.
  static_assert(C::STAGE % 4096 == 0 && (C::ROWB == 512 || C::ROWB == 256), "XOR addressing");
  const int qk_lat = l16 * C::ROWB + 16 * ((16 * b + kg) ^ swz_l<C::ROWB>(l16));
  const int qk_rp = C::LAT + l16 * 128 + 16 * (kg ^ swz_r(l16));
  int pv_lat;
  {
    const int t = 4 * kg + (l16 >> 2), half = l16 & 3;
    pv_lat = t * C::ROWB + 16 * ((16 * b + (half >> 1)) ^ swz_l<C::ROWB>(t)) + 8 * (half & 1);
  }
  // DMA lane constants. Latent: lane -> row RPI*q + lat_row of the
  // instruction, LDS chunk lat_p, which holds logical chunk lat_p ^ swz_l<C::ROWB>(row);
  // the row's parity within 16 (2 q + lat_row with q = wave + NW u, NW even)
  // is the same for every instruction of the wave. RoPE: this lane's part of
  // the wave's instruction (waves < NR).
  static_assert((C::RPI * C::NW) % (C::ROWB / 32) == 0, "row parity per wave");
  const int lat_row = lane / (64 / C::RPI), lat_p = lane % (64 / C::RPI);
  const int lat_c = 16 * (lat_p ^ swz_l<C::ROWB>(C::RPI * wave + lat_row)) + hg * C::ROWB;
  const int rope_t = wave * 8 + (lane >> 3);
  const int rope_c = 16 * ((lane & 7) ^ swz_r(rope_t));

  int start = k * hd.chunk;
  MLRA_DCHECK(p.hdr, start >= 0 && start < hd.total, 4);
  const int end = min(start + hd.chunk, hd.total);
  int bseq = find_seq(p.prefix, p.B, start);

  while (start < end) {
    while (p.prefix[bseq + 1] <= start) ++bseq;
    const int seg_end = min(end, p.prefix[bseq + 1]);
    const int t0 = start - p.prefix[bseq], t1 = seg_end - p.prefix[bseq];
    const int ntiles = (t1 - t0 + kT - 1) / kT;
    constexpr int EB = FP8 ? 1 : 2;  // cache bytes per element
    const i32x4 crs = seq_rsrc_bytes((const char*)p.ckv + (int64_t)bseq * p.ckv_bs * EB, t1,
                                     p.ckv_ts * EB);
    const i32x4 krs = seq_rsrc_bytes((const char*)p.krope + (int64_t)bseq * p.kr_bs * EB, t1,
                                     p.kr_ts * EB);
    const int slot = k + bseq;
    MLRA_DCHECK(p.hdr, bseq >= 0 && bseq < p.B, 1);
    MLRA_DCHECK(p.hdr, t0 >= 0 && t1 > t0 && t1 <= p.prefix[bseq + 1] - p.prefix[bseq], 2);
    MLRA_DCHECK(p.hdr, slot >= 0 && slot < hd.n_items + p.B, 3);
    const uint32_t lat_voff = (uint32_t)(lat_row * p.ckv_ts * 2 + lat_c);
    // fp8 latent instruction `wave`: rows 4 wave .. + 3 of the tile, lane l
    // row 4 wave + l / 16, codes hg 256 + 16 (l % 16) .. of it
    const int lat8_c = hg * 256 + 16 * (lane & 15);
    const uint32_t lat8_voff = (uint32_t)((lane >> 4) * p.ckv_ts + lat8_c);

    // earlier stores and loads of this wave done; all waves left the
    // previous segment's LDS tiles
    wait_vm<0>();
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();

    // Q^T as the B operand: lane (head, kg) holds 8 consecutive k of its head;
    // with QLO also q~'s bf16 residue over the branch's latent k-steps, whose
    // products with the same K fragments go into the same scores
    VT q[C::KS][C::NBLK];
    bf16x8 ql[QLO ? C::KL : 1][C::NBLK];
    // fp16: q~ is its two bf16 parts summed in fp32, rounded once (a view
    // without the residue re-reads q~ and weights it by 0)
    auto to_q = [&](const __bf16* hi, const __bf16* lo, float wlo) -> VT {
      const bf16x8 h = *(const bf16x8*)hi;
      if constexpr (F16) {
        const bf16x8 l = *(const bf16x8*)lo;
        VT v;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (_Float16)__builtin_fmaf(wlo, (float)l[i], (float)h[i]);
        return v;
      } else {
        return h;
      }
    };
    const float wlo = p.q_lo > 0 ? 1.f : 0.f;
#pragma unroll
    for (int nb = 0; nb < C::NBLK; ++nb) {
      const __bf16* qrow = p.q_abs + ((int64_t)bseq * H + head0 + 16 * nb + l16) * p.q_stride;
#pragma unroll
      for (int ks = 0; ks < C::KL; ++ks)
        q[ks][nb] = to_q(qrow + kBW * j + 32 * ks + 8 * kg,
                         qrow + p.q_lo + kBW * j + 32 * ks + 8 * kg, wlo);
      if constexpr (QLO) {
#pragma unroll
        for (int ks = 0; ks < C::KL; ++ks)
          ql[ks][nb] = *(const bf16x8*)(qrow + p.q_lo + kBW * j + 32 * ks + 8 * kg);
      }
#pragma unroll
      for (int ks = C::KL; ks < C::KS; ++ks)
        q[ks][nb] = to_q(qrow + DC + 32 * (ks - C::KL) + 8 * kg,
                         qrow + DC + 32 * (ks - C::KL) + 8 * kg, 0.f);
    }
    // Q complete before any DMA is in flight: no vmcnt wait for Q is then
    // needed inside the tile loop (it would also drain the DMA)
    wait_vm<0>();
    // LDS byte offset of a tile's stage, advanced one tile at a time
    // (fp8: the tiles read by the phases alternate between the two bf16
    // tiles, the loads go round the ring of code stages after them)
    auto next_stage = [](int off) {
      if constexpr (FP8) return off ^ C::STAGE;
      return off + C::STAGE == NS * C::STAGE ? 0 : off + C::STAGE;
    };
    auto next_ring = [&](int off) {
      if constexpr (FP8) return off + STAGE8 == NS * STAGE8 ? 0 : off + STAGE8;
      return next_stage(off);
    };
    int dma_off = 0;  // stage of the next tile to load
    // fp8: DMA of a tile's codes; the latent rows of the segment's last tile
    // are clamped per lane
    auto issue8 = [&](int tile, bool tail) {
      const uint32_t sa = sbase + 2 * C::STAGE + dma_off;
      dma_off = next_ring(dma_off);
      const int ts0 = t0 + tile * kT;
      if (!tail) {
        dma16_stream(crs, sa + wave * 1024, lat8_voff, (uint32_t)((ts0 + 4 * wave) * p.ckv_ts));
      } else {
        const int row = min(ts0 + 4 * wave + (lane >> 4), t1 - 1);
        dma16_stream(crs, sa + wave * 1024, (uint32_t)(row * p.ckv_ts + lat8_c), 0u);
      }
      if (wave < 2) {
        const int row = min(ts0 + 16 * wave + (lane >> 2), t1 - 1);
        dma16_stream(krs, sa + LAT8 + wave * 1024, (uint32_t)(row * p.kr_ts + 16 * (lane & 3)),
                     0u);
      }
    };
    // fp8: this lane's codes of the next tile to convert, into its bf16 tile
    // (the swizzles of the bf16 stages: latent row t's codes 16 cc .. are
    // chunks 2 cc, 2 cc + 1, at 2 (cc ^ (t & 15)) and the next; RoPE row t's
    // chunk c at c ^ swz_r(t)). The offsets come from an opaque copy of the
    // lane id, so that they are recomputed instead of kept live (spilled).
    int cv_off = 0, cv_buf = 0;
    auto convert8 = [&]() {
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const char LDS_AS* src = smem + 2 * C::STAGE + cv_off + 16 * ln;
      char LDS_AS* dst = smem + cv_buf;
      cv_off = next_ring(cv_off);
      cv_buf ^= C::STAGE;
      const i32x4 x = *(const i32x4 LDS_AS*)(src + wave * 1024);
      i32x4 r;
      if (wave < 2) r = *(const i32x4 LDS_AS*)(src + LAT8 + wave * 1024);
      {
        const int t = 4 * wave + (ln >> 4), cc = ln & 15;
        i32x4 lo, hi;
        if constexpr (F16) fp8x16_to_f16(x, lo, hi);
        else fp8x16_to_bf16(x, lo, hi);
        char LDS_AS* d = dst + t * C::ROWB + 32 * (cc ^ (t & 15));
        *(i32x4 LDS_AS*)d = lo;
        *(i32x4 LDS_AS*)(d + 16) = hi;
      }
      if (wave < 2) {
        const int t = 16 * wave + (ln >> 2), cc = ln & 3;
        i32x4 lo, hi;
        if constexpr (F16) fp8x16_to_f16(r, lo, hi);
        else fp8x16_to_bf16(r, lo, hi);
        char LDS_AS* d = dst + C::LAT + t * 128;
        *(i32x4 LDS_AS*)(d + 16 * ((2 * cc) ^ swz_r(t))) = lo;
        *(i32x4 LDS_AS*)(d + 16 * ((2 * cc + 1) ^ swz_r(t))) = hi;
      }
    };
    auto issue = [&](int tile) {
      if constexpr (FP8) {
        issue8(tile, t0 + tile * kT + kT > t1);
        return;
      }
      const uint32_t sa = sbase + dma_off;
      dma_off = next_stage(dma_off);
      const int ts0 = t0 + tile * kT;
      if (ts0 + kT <= t1)
        issue_tile<C, false>(sa, crs, krs, p.ckv_ts, p.kr_ts, ts0, t1, wave, lane, lat_voff,
                             lat_c, rope_t, rope_c);
      else
        issue_tile<C, true>(sa, crs, krs, p.ckv_ts, p.kr_ts, ts0, t1, wave, lane, lat_voff, lat_c,
                            rope_t, rope_c);
    };
#pragma unroll
    for (int s = 0; s < D; ++s)
      if (s < ntiles) issue(s);

    f32x4 o[C::CB][C::NBLK];
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
      for (int nb = 0; nb < C::NBLK; ++nb) o[cb][nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
    float m_run[C::NBLK], l_run[C::NBLK];
#pragma unroll
    for (int nb = 0; nb < C::NBLK; ++nb) {
      m_run[nb] = kNoRef;
      l_run[nb] = 0.f;
    }
    // score bias per token row: 0, or -inf past the segment's end (its last
    // tile only); the QK accumulators start from it, so masking costs nothing
    // on full tiles
    f32x4 bias[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) bias[mb] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // Two phases per tile, each between two workgroup barriers: the matrix
    // phase M(t) (PV of tile t - 1, then QK of tile t) and the vector phase
    // V(t) (softmax of tile t, V^T fragments of tile t into registers). The
    // waves w and w + NW/2 share a SIMD; the second group runs one phase
    // behind the first, so on every SIMD one wave's MFMAs run beside the
    // other wave's softmax.
    f32x4 S[2][C::NBLK];   // scores of the tile between M(t) and V(t)
    VT P[C::NBLK];         // P^T of tile t, from V(t) to M(t + 1)
    VT V[C::CB];           // V^T of tile t, from V(t) to M(t + 1)
    int m_off = 0, v_off = 0;  // stages of the tiles the next M and V phases read

    // a phase boundary: no instruction is scheduled across it (the phases
    // exist to keep MFMA and VALU work apart), and no LDS access moves over it
    auto bar = [] {
      __builtin_amdgcn_sched_barrier(0);
      // fp8: this wave's converted tile written (s_barrier does not wait)
      if constexpr (FP8 || F16) wait_lgkm0();
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    };
    // wait for this wave's loads of tile t (fp8: two instructions per tile on
    // waves 0 and 1, one on the others), then (fp8) convert its codes
    // (fp8: nothing to wait for here; conv(u) below waits for tile u's codes
    // and converts them in the phase before the barrier that opens M(u))
    // fp16 from the bf16 cache: once this wave's loads of the tile at stage
    // `off` have landed, its lanes convert the 16 bytes each loaded, in
    // place (its latent instructions wave + NW u and, on waves < NR, its
    // RoPE one), before the barrier that opens the tile's first matrix
    // phase. The lane offsets come from an opaque copy of the lane id, so
    // that they are recomputed instead of kept live (spilled).
    auto convert16 = [&](int off) {
      if constexpr (F16 && !FP8) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        char LDS_AS* st = smem + off + 16 * ln;
        i32x4 x[C::NL / C::NW], r;
#pragma unroll
        for (int u = 0; u < C::NL / C::NW; ++u)
          x[u] = *(const i32x4 LDS_AS*)(st + (wave + C::NW * u) * 1024);
        if (wave < C::NR) r = *(const i32x4 LDS_AS*)(st + C::LAT + wave * 1024);
#pragma unroll
        for (int u = 0; u < C::NL / C::NW; ++u)
          *(i32x4 LDS_AS*)(st + (wave + C::NW * u) * 1024) = bf16_to_f16x8(x[u]);
        if (wave < C::NR) *(i32x4 LDS_AS*)(st + C::LAT + wave * 1024) = bf16_to_f16x8(r);
      }
    };
    auto wait_tile = [&](int t) {
      if constexpr (!FP8) wait_tiles<C, NS - 2>(min(NS - 2, ntiles - 1 - t), wave);
      convert16(m_off);  // fp16: the tile the next matrix phase reads
    };
    // fp8: this wave's codes of tile u have landed (the tiles issued after it,
    // up to u + D - 1, may be in flight), then its lanes convert them
    auto conv = [&](int u) {
      if constexpr (FP8) {
        if (wave < 2) wait_tiles_per<2, D - 1>(min(D - 1, ntiles - 1 - u));
        else wait_tiles_per<1, D - 1>(min(D - 1, ntiles - 1 - u));
        asm volatile("" ::: "memory");
        convert8();
      }
    };
    auto issue_if = [&](int t) {
      if (t < ntiles) issue(t);
    };
    // steady tiles (1 <= t < ntiles - D - 1): the wait keeps NS - 2 tiles in
    // flight, the tile loaded is full and not the last, and no row is masked
    auto wait_steady = [&] {
      if constexpr (FP8) return;
      if (wave < C::NR) wait_vm<(NS - 2) * (C::NL / C::NW + 1)>();
      else wait_vm<(NS - 2) * (C::NL / C::NW)>();
      convert16(m_off);
    };
    auto issue_full = [&](int tile) {
      if constexpr (FP8) {
        issue8(tile, false);
        return;
      }
      const uint32_t sa = sbase + dma_off;
      dma_off = next_stage(dma_off);
      issue_tile<C, false>(sa, crs, krs, p.ckv_ts, p.kr_ts, t0 + tile * kT, t1, wave, lane, lat_voff,
                           lat_c, rope_t, rope_c);
    };
    const int steady_end = ntiles - D - 1;

    auto mphase = [&](int t, auto pv_tag, auto qk_tag, auto steady_tag) {
      constexpr bool PV = decltype(pv_tag)::value, QK = decltype(qk_tag)::value;
      constexpr bool STEADY = decltype(steady_tag)::value;
      VT A[2][C::KS];
      if constexpr (QK) {
        const char LDS_AS* st = smem + __builtin_amdgcn_readfirstlane(m_off);
        m_off = next_stage(m_off);
        const int valid = t1 - (t0 + t * kT);
        if (!STEADY && valid < kT) {
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int e = 0; e < 4; ++e) bias[mb][e] = 16 * mb + 4 * kg + e < valid ? 0.f : -INFINITY;
        }
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
          for (int ks = 0; ks < C::KL; ++ks)
            A[mb][ks] = *(const VT LDS_AS*)((const char LDS_AS*)(((uintptr_t)(st + qk_lat)) ^ (64 * ks)) +
                                                mb * 16 * C::ROWB);
          A[mb][C::KL] = *(const VT LDS_AS*)(st + qk_rp + mb * 2048);
          A[mb][C::KL + 1] =
              *(const VT LDS_AS*)((const char LDS_AS*)(((uintptr_t)(st + qk_rp)) ^ 64) + mb * 2048);
        }
      }
      if constexpr (PV) {
#pragma unroll
        for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
          for (int nb = 0; nb < C::NBLK; ++nb)
            o[cb][nb] = O_::mfma(V[cb], P[nb], o[cb][nb]);
      }
      if constexpr (QK) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < C::NBLK; ++nb) {
            S[mb][nb] = O_::mfma(A[mb][0], q[0][nb], bias[mb]);
#pragma unroll
            for (int ks = 1; ks < C::KS; ++ks)
              S[mb][nb] = O_::mfma(A[mb][ks], q[ks][nb], S[mb][nb]);
            if constexpr (QLO) {
#pragma unroll
              for (int ks = 0; ks < C::KL; ++ks)
                S[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mb][ks], ql[ks][nb],
                                                                    S[mb][nb], 0, 0, 0);
            }
          }
      }
    };

    // V(t): this branch's online softmax of S, per 16-head block. P is taken
    // against the running reference m_run without a tile max: a per-lane sum
    // of P above kSumLimit (or inf: no reference yet, or an overflow) means
    // some score passed the reference by more than 2^16, and only then
    // (rare) the exact tile max moves the reference, O and l are rescaled and
    // P is recomputed. Otherwise every p stays below 2^20. O holds the tiles
    // before t here (PV of tile t - 1 ran in M(t)).
    auto vphase = [&]() {
      const char LDS_AS* st = smem + __builtin_amdgcn_readfirstlane(v_off);
      v_off = next_stage(v_off);
#pragma unroll
      for (int cb = 0; cb < C::CB; ++cb) {
        const char LDS_AS* a = (const char LDS_AS*)(((uintptr_t)(st + pv_lat)) ^ (32 * cb));
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)a);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)(a + 16 * C::ROWB));
        const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        V[cb] = __builtin_bit_cast(VT, v);
      }
      float ps[C::NBLK];
      bool need = false;
      auto probs = [&](int nb) {
        ps[nb] = 0.f;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(S[mb][nb][e], kLog2e, -m_run[nb]));
            ps[nb] += pe;
            P[nb][4 * mb + e] = (ET)pe;
          }
      };
#pragma unroll
      for (int nb = 0; nb < C::NBLK; ++nb) {
        probs(nb);
        need |= !(ps[nb] <= O_::kSum);
      }
      if (__builtin_expect(__any(need), 0)) {
#pragma unroll
        for (int nb = 0; nb < C::NBLK; ++nb) {
          const float mx = fmaxf(fmaxf(fmaxf(S[0][nb][0], S[0][nb][1]), fmaxf(S[0][nb][2], S[0][nb][3])),
                                 fmaxf(fmaxf(S[1][nb][0], S[1][nb][1]), fmaxf(S[1][nb][2], S[1][nb][3])));
          const float mt = max4(mx) * kLog2e;
          const float mr = m_run[nb] == kNoRef ? mt : m_run[nb];  // first tile sets it
          const float mn = fmaxf(mr, mt - O_::kRes);
          const float f = __builtin_amdgcn_exp2f(mr - mn);
          l_run[nb] *= f;
#pragma unroll
          for (int cb = 0; cb < C::CB; ++cb) o[cb][nb] *= f;
          m_run[nb] = mn;
          probs(nb);
        }
      }
#pragma unroll
      for (int nb = 0; nb < C::NBLK; ++nb) l_run[nb] += ps[nb];
    };

    using T_ = std::integral_constant<bool, true>;
    using F_ = std::integral_constant<bool, false>;
    // Barriers: b(2t + 1) opens M(t) of the first group, b(2t + 2) its V(t);
    // the second group's M(t) and V(t) start one barrier later. Tile t is in
    // LDS (every wave waited for its own loads) before b(2t + 1); its stage
    // is read for the last time in the second group's V(t), which ends at
    // b(2t + 4), after which tile t + NS (same stage) is loaded: tile
    // u + NS - 1 is issued right after b(2u + 2), at the start of V(u) in the
    // first group and of M(u) in the second. Both groups pass 2 ntiles + 2
    // barriers per segment.
    // fp8: tile u is converted in the phase before b(2u + 1): the first group
    // at the start of V(u - 1), the second at the start of M(u - 1); the bf16
    // tile it overwrites (u - 2) was last read in the second group's V(u - 2),
    // which ends at b(2u)
    if (!lag) {
      conv(0);
      wait_tile(0);
      bar();
      mphase(0, F_{}, T_{}, F_{});
      bar();
      issue_if(D);
      if (1 < ntiles) conv(1);
      vphase();
      int t = 1;
      for (; t < steady_end; ++t) {
        wait_steady();
        bar();
        mphase(t, T_{}, T_{}, T_{});
        bar();
        issue_full(t + D);
        conv(t + 1);
        vphase();
      }
      for (; t < ntiles; ++t) {
        wait_tile(t);
        bar();
        mphase(t, T_{}, T_{}, F_{});
        bar();
        issue_if(t + D);
        if (t + 1 < ntiles) conv(t + 1);
        vphase();
      }
      bar();
      mphase(ntiles, T_{}, F_{}, F_{});
      bar();
    } else {
      conv(0);
      wait_tile(0);
      bar();
      bar();
      issue_if(D);
      if (1 < ntiles) conv(1);
      mphase(0, F_{}, T_{}, F_{});
      if (1 < ntiles) wait_tile(1);
      bar();
      vphase();
      bar();
      int t = 1;
      for (; t < steady_end; ++t) {
        issue_full(t + D);
        conv(t + 1);
        mphase(t, T_{}, T_{}, T_{});
        wait_steady();
        bar();
        vphase();
        bar();
      }
      for (; t < ntiles; ++t) {
        issue_if(t + D);
        if (t + 1 < ntiles) conv(t + 1);
        mphase(t, T_{}, T_{}, F_{});
        if (t + 1 < ntiles) wait_tile(t + 1);
        bar();
        vphase();
        bar();
      }
      mphase(ntiles, T_{}, F_{}, F_{});
    }

    // partial state of this segment: m, l as [slot][n][H]; the accumulator
    // normalised by l (a weighted mean of cache rows) as fp16 [slot][H][d_c],
    // this branch's 128 columns, 8-byte stores
#pragma unroll
    for (int nb = 0; nb < C::NBLK; ++nb) {
      const int head = head0 + 16 * nb + l16;
      const float lt = sum4(l_run[nb]);
      if (kg == 0) {
        p.m[((int64_t)slot * NBR + j) * H + head] = m_run[nb];
        p.l[((int64_t)slot * NBR + j) * H + head] = lt;
      }
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      _Float16* row = reinterpret_cast<_Float16*>(p.acc) + ((int64_t)slot * H + head) * DC +
                      kBW * j + 4 * kg;
#pragma unroll
      for (int cb = 0; cb < C::CB; ++cb) store_f16x4_sat(row + 16 * cb, o[cb][nb] * inv);
    }
    start = seg_end;
    ++bseq;
  }
}

template <int NBR, int NSPLIT, int HPW, int NHG, bool QLO, bool FP8 = false, bool F16 = false>
hipError_t launch_b(const Geom& g, const QView& q, const void* ckv, const void* krope,
                    const Workspace& ws, int items, hipStream_t s, const KernelTiming& t) {
  using C = BCfg<NBR, NSPLIT, HPW, NHG>;
  // a deep ring: up to 7 stages of 20 KB keep up to 6 tiles in flight per CU
  constexpr int NS = (160 * 1024) / C::STAGE < 7 ? (160 * 1024) / C::STAGE : 7;
  static_assert(NS >= 3, "tile ring does not fit LDS");
  DecodeParams p;
  p.q_abs = (const __bf16*)q.q;
  p.q_stride = q.stride;
  p.q_lo = QLO || F16 ? q.lo : 0;
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
  if (NSPLIT > 1) grid = ((items + 7) / 8) * 8 * NSPLIT;  // whole XCD rounds
  hipExtLaunchKernelGGL((decode_branch_kernel<NBR, NSPLIT, HPW, NHG, NS, QLO, FP8, F16>), dim3(grid),
                        dim3(64 * C::NW), 0, s, t.start, t.stop, 0, p);
  return hipGetLastError();
}

}  // namespace

// MLRA-4 with 128-wide branches (two workgroups per item, one per branch
// pair) and one such branch alone, a tensor-parallel shard (one workgroup
// per item).
bool decode_branch_supported(const Geom& g, bool fp8) {
  if (g.dr != kDR) return false;
  if (fp8) return g.dc == 4 * kBW && g.n == 4 && g.H == 128;
  if (g.dc == 4 * kBW && g.n == 4) return g.H == 64 || g.H == 128;
  return g.dc == kBW && g.n == 1 && g.H == 128;
}

// Workgroups per work item; one workgroup per CU.
int decode_branch_wgs_per_item(const Geom& g) { return g.n == 1 ? 1 : 2; }

// The one-branch shard always adds q~'s residue to its bf16 scores. The
// four-branch kernel at 128 heads reads it, and then runs in fp16 (q~ from
// both parts, the tiles converted in LDS, P in fp16), with an fp8 cache (whose
// tiles are converted anyway, so the fp16 form costs about 3%) or when the
// caller asks for it (cfg->q_residue; about 19% more time on a bf16 cache).
bool decode_branch_reads_residue(const Geom& g, bool fp8, bool want) {
  return g.n == 1 || (g.n == 4 && g.H == 128 && (fp8 || want));
}

hipError_t launch_decode_branch(const Geom& g, const QView& q, const void* ckv,
                                const void* krope, const Workspace& ws, int items,
                                hipStream_t s, const KernelTiming& t, bool fp8) {
  if (!decode_branch_supported(g, fp8)) return hipErrorNotSupported;
  // one branch alone (a tensor-parallel shard) is one softmax over the
  // branch: a bf16 query alone moves its output rows by up to ~1.1e-2 at the
  // pages' scales, so the shard adds q~'s residue when the view has it. With
  // four branches the summed output averages the branches' errors (<= 9.8e-3
  // measured) and a residue in the scores would need registers that cost the
  // second wave per SIMD; with the residue in the view the kernel runs in
  // fp16 instead (<= 2.0e-3 measured).
  if (g.n == 1) {
    if (q.lo > 0) return launch_b<1, 1, 16, 8, true>(g, q, ckv, krope, ws, items, s, t);
    return launch_b<1, 1, 16, 8, false>(g, q, ckv, krope, ws, items, s, t);
  }
  if (fp8) return launch_b<4, 2, 32, 4, false, true, true>(g, q, ckv, krope, ws, items, s, t);
  if (g.H == 64) return launch_b<4, 2, 16, 4, false>(g, q, ckv, krope, ws, items, s, t);
  if (q.lo > 0) return launch_b<4, 2, 32, 4, false, false, true>(g, q, ckv, krope, ws, items, s, t);
  return launch_b<4, 2, 32, 4, false>(g, q, ckv, krope, ws, items, s, t);
}

}  // namespace mlra
