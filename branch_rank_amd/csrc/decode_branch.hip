// Branch-per-wave bf16 MFMA split-KV decode for MLRA-n with 128-wide branch
// slices, gfx950 (MI355X).
//
// What it computes ("Multi-Head Low-Rank Attention", 核心方法 and 方法步骤详情
// step 2; "vllbc02MLA", 苏神思路): for one work item (a token range of one or
// more sequences) and a group of heads, each branch j's own online softmax over
// the scores q~_j[h]·c_t[S_j] + rho[h]·k^R_t and its accumulator
// acc_j[h] = sum_t p_t c_t[S_j]. Branch j only ever touches its latent slice
// S_j (128 columns) and the shared RoPE key, so one wave can own one branch
// for all of its heads without talking to the other branches' waves.
//
// Mapping onto CDNA4 (the partial state it writes is the same as the
// head-group kernel's, so both feed the same merge):
//  * A workgroup has NBR x NHG waves: wave (j, g) owns branch j for the HPW
//    heads of head group g. Its registers hold Q for those heads over the
//    branch slice plus the RoPE part (48 VGPRs at HPW = 32) and O over the
//    slice (64 AGPRs), small enough for two waves per SIMD: while one wave runs
//    its softmax on the VALU, the other keeps the matrix core busy.
//  * Per tile, a wave reads only its branch's columns from LDS (32 tokens x
//    (128 + 64) for QK, 32 x 128 for PV), and each fragment feeds HPW / 16
//    MFMAs; this is 1.7x fewer LDS bytes per head than reading whole rows.
//  * 32-token tiles stream HBM -> LDS with buffer_load_dwordx4 ... lds: one
//    instruction per 1024-byte latent row, 8 RoPE rows per instruction,
//    shared by all waves, through an NS-stage ring. Latent rows sit at a
//    1056-byte stride (32-byte pad), which keeps both LDS read patterns free
//    of bank conflicts and every read address a constant offset from one
//    per-lane base. RoPE rows (128 bytes) are XOR-swizzled in 16-byte chunks.
//  * QK: S^T[t][h] on v_mfma_f32_16x16x32_bf16, 16 tokens as M, 16 heads as N;
//    the S^T accumulators (lane = head) are the B operand of PV,
//    O^T[c][h] = V^T[c][t] P^T[t][h] with V^T read by ds_read_b64_tr_b16, so P
//    never moves between lanes and a rescale is one multiplier per lane.
//  * Lazy rescaling as in the head-group kernel: the segment's first tile
//    sets the reference max; it moves only when exceeded by more than 2^16.

#include "device_common.h"

namespace mlra {
namespace {

using namespace dev;

constexpr int kT = 32;    // tokens per tile
constexpr int kDR = 64;   // RoPE width
constexpr int kBW = 128;  // latent width of one branch
constexpr float kRescale = 16.f;  // log2 headroom before the running max moves

template <int NBR, int HPW, int NHG>
struct BCfg {
  static constexpr int DC = NBR * kBW;            // total latent width
  static constexpr int NW = NBR * NHG;            // waves per workgroup
  static constexpr int HWG = HPW * NHG;           // heads per workgroup
  static constexpr int NBLK = HPW / 16;           // MFMA N blocks (16 heads) per wave
  static constexpr int RS = DC * 2 + 32;          // latent row stride in LDS (bytes)
  static constexpr int LAT = kT * RS;             // latent part of a stage
  static constexpr int STAGE = LAT + kT * kDR * 2;
  static constexpr int NL = kT;                   // latent DMA instructions per tile (1 row each)
  static constexpr int NR = kT * kDR * 2 / 1024;  // RoPE DMA instructions per tile (8 rows each)
  static constexpr int NI = NL + NR;
  static constexpr int PER_HI = (NI + NW - 1) / NW;  // per wave, waves < NI % NW
  static constexpr int PER_LO = NI / NW;             // per wave, the others
  static constexpr int KL = kBW / 32;             // latent k-steps of a branch score
  static constexpr int KS = KL + kDR / 32;        // plus the RoPE k-steps
  static constexpr int CB = kBW / 16;             // PV output row blocks of a branch
  static_assert(DC * 2 == 1024, "one latent row per DMA instruction (d_c = 512)");
  static_assert(HPW % 16 == 0 && NW <= 16, "wave shape");
};

// RoPE-row swizzle (128-byte rows): 16 rows of one chunk hit distinct banks.
__device__ __forceinline__ int swz_r(int t) { return (t >> 1) & 7; }

// DMA of one tile into the stage at LDS byte address `stage`. Latent rows:
// lane offset 16 * lane, the row in soffset (a wave-uniform value). RoPE
// rows: 8 per instruction, chunk-swizzled. The segment's last tile clamps
// rows to tend - 1 so that every load stays inside the sequence.
template <class C, bool TAIL>
__device__ __forceinline__ void issue_tile(uint32_t stage, i32x4 crs, i32x4 krs, int cts,
                                           int kts, int tstart, int tend, int wave, int lane) {
#pragma unroll
  for (int u = 0; u < C::PER_HI; ++u) {
    const int q = wave + C::NW * u;
    if (q >= C::NI) continue;
    if (q < C::NL) {
      const int row = TAIL ? min(tstart + q, tend - 1) : tstart + q;
      dma16(crs, stage + q * C::RS, (uint32_t)(16 * lane), (uint32_t)(row * cts * 2));
    } else {
      const int r = q - C::NL;
      const int t = r * 8 + (lane >> 3);
      const int lc = (lane & 7) ^ swz_r(t);
      if constexpr (!TAIL) {
        dma16(krs, stage + C::LAT + r * 1024, (uint32_t)(t * kts * 2 + lc * 16),
              (uint32_t)(tstart * kts * 2));
      } else {
        const int row = min(tstart + t, tend - 1);
        dma16(krs, stage + C::LAT + r * 1024, (uint32_t)(row * kts * 2 + lc * 16), 0u);
      }
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
template <class C, int NS>
__device__ __forceinline__ void wait_tiles(int ahead, int wave) {
  if constexpr (C::PER_HI == C::PER_LO) {
    wait_tiles_per<C::PER_HI, NS>(ahead);
  } else {
    if (wave < C::NI % C::NW) wait_tiles_per<C::PER_HI, NS>(ahead);
    else wait_tiles_per<C::PER_LO, NS>(ahead);
  }
}

template <int NBR, int HPW, int NHG, int NS, int HSPLIT>
__global__ __launch_bounds__(64 * NBR * NHG, 1) void decode_branch_kernel(DecodeParams p) {
  using C = BCfg<NBR, HPW, NHG>;
  constexpr int H = C::HWG * HSPLIT;
  constexpr int DC = C::DC;
  __shared__ __attribute__((aligned(1024))) char smem_raw[NS * C::STAGE];
  char LDS_AS* smem = (char LDS_AS*)smem_raw;
  const uint32_t sbase = (uint32_t)(uintptr_t)smem;

  // workgroup -> (item, head group); the head groups of one item share an XCD
  int k, hg;
  if constexpr (HSPLIT == 1) {
    k = blockIdx.x;
    hg = 0;
  } else {
    const int i = blockIdx.x, x = i & 7, jj = i >> 3;
    k = (jj / HSPLIT) * 8 + x;
    hg = jj % HSPLIT;
  }
  const PlanHeader hd = *p.hdr;
  if (k >= hd.n_items) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int j = wave % NBR;          // branch of this wave
  const int g = wave / NBR;          // head group of this wave within the workgroup
  const int l16 = lane & 15, kg = lane >> 4;
  const int head0 = hg * C::HWG + g * HPW;  // first head of this wave

  // Per-lane LDS byte offsets within a stage (the rest are instruction
  // immediates). QK A operand: token row 16 mb + l16, branch columns
  // 32 ks + 8 kg .. +7. RoPE: chunk 4 ks + kg, swizzled by row. PV (transposed
  // reads): token rows 4 kg + (l16 >> 2) (+ 16), columns 16 cb + 4 (l16 & 3) .. +3.
  const int qk_lat = l16 * C::RS + 256 * j + 16 * kg;
  const int qk_rp0 = C::LAT + l16 * 128 + 16 * (kg ^ swz_r(l16));
  const int qk_rp1 = C::LAT + l16 * 128 + 16 * ((4 + kg) ^ swz_r(l16));
  const int pv_lo = (4 * kg + (l16 >> 2)) * C::RS + 256 * j + 8 * (l16 & 3);

  int start = k * hd.chunk;
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

    // earlier stores and loads of this wave done; all waves left the
    // previous segment's LDS tiles
    wait_vm<0>();
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();

    // Q^T as the B operand: lane (head, kg) holds 8 consecutive k of its head
    bf16x8 q[C::KS][C::NBLK];
#pragma unroll
    for (int nb = 0; nb < C::NBLK; ++nb) {
      const __bf16* qrow = p.q_abs + ((int64_t)b * H + head0 + 16 * nb + l16) * (DC + kDR);
#pragma unroll
      for (int ks = 0; ks < C::KL; ++ks)
        q[ks][nb] = *(const bf16x8*)(qrow + kBW * j + 32 * ks + 8 * kg);
#pragma unroll
      for (int ks = C::KL; ks < C::KS; ++ks)
        q[ks][nb] = *(const bf16x8*)(qrow + DC + 32 * (ks - C::KL) + 8 * kg);
    }
    // Q complete before any DMA is in flight: no vmcnt wait for Q is then
    // needed inside the tile loop (it would also drain the DMA)
    wait_vm<0>();
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) {
      if (s < ntiles - 1)
        issue_tile<C, false>(sbase + s * C::STAGE, crs, krs, p.ckv_ts, p.kr_ts, t0 + s * kT, t1,
                             wave, lane);
      else if (s == ntiles - 1)
        issue_tile<C, true>(sbase + s * C::STAGE, crs, krs, p.ckv_ts, p.kr_ts, t0 + s * kT, t1,
                            wave, lane);
    }

    f32x4 o[C::CB][C::NBLK];
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
      for (int nb = 0; nb < C::NBLK; ++nb) o[cb][nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
    float m_run[C::NBLK], l_run[C::NBLK];
#pragma unroll
    for (int nb = 0; nb < C::NBLK; ++nb) {
      m_run[nb] = -INFINITY;
      l_run[nb] = 0.f;
    }

    for (int it = 0; it < ntiles; ++it) {
      const int ahead = min(NS - 2, ntiles - 1 - it);
      wait_tiles<C, NS>(ahead, wave);
      __builtin_amdgcn_s_barrier();
      const int nt = it + NS - 1;  // tile whose DMA goes out now
      if (nt < ntiles - 1)
        issue_tile<C, false>(sbase + (nt % NS) * C::STAGE, crs, krs, p.ckv_ts, p.kr_ts,
                             t0 + nt * kT, t1, wave, lane);
      else if (nt == ntiles - 1)
        issue_tile<C, true>(sbase + (nt % NS) * C::STAGE, crs, krs, p.ckv_ts, p.kr_ts,
                            t0 + nt * kT, t1, wave, lane);
      const char LDS_AS* st = smem + (it % NS) * C::STAGE;
      const int valid = min(kT, t1 - (t0 + it * kT));

      // ---- scores S^T = K Q^T over the branch slice and the RoPE part
      bf16x8 A[2][C::KS];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int ks = 0; ks < C::KL; ++ks)
          A[mb][ks] = *(const bf16x8 LDS_AS*)(st + qk_lat + mb * 16 * C::RS + 64 * ks);
        A[mb][C::KL] = *(const bf16x8 LDS_AS*)(st + qk_rp0 + mb * 2048);
        A[mb][C::KL + 1] = *(const bf16x8 LDS_AS*)(st + qk_rp1 + mb * 2048);
      }
      f32x4 S[2][C::NBLK];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < C::NBLK; ++nb) {
          S[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mb][0], q[0][nb],
                                                              (f32x4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
          for (int ks = 1; ks < C::KS; ++ks)
            S[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mb][ks], q[ks][nb], S[mb][nb],
                                                                0, 0, 0);
        }

      // ---- V^T fragments for PV, read while the softmax runs
      bf16x8 V[C::CB];
#pragma unroll
      for (int cb = 0; cb < C::CB; ++cb) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (i16x4 LDS_AS*)(st + pv_lo + 32 * cb));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (i16x4 LDS_AS*)(st + pv_lo + 16 * C::RS + 32 * cb));
        const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        V[cb] = __builtin_bit_cast(bf16x8, v);
      }

      // ---- online softmax of this branch, per 16-head block
      if (valid < kT) {  // segment's last tile: tokens past its end get -inf
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (16 * mb + 4 * kg + e >= valid)
#pragma unroll
              for (int nb = 0; nb < C::NBLK; ++nb) S[mb][nb][e] = -INFINITY;
      }
      bf16x8 P[C::NBLK];
#pragma unroll
      for (int nb = 0; nb < C::NBLK; ++nb) {
        const float mx = fmaxf(fmaxf(fmaxf(S[0][nb][0], S[0][nb][1]), fmaxf(S[0][nb][2], S[0][nb][3])),
                               fmaxf(fmaxf(S[1][nb][0], S[1][nb][1]), fmaxf(S[1][nb][2], S[1][nb][3])));
        const float mt = max4(mx) * kLog2e;
        // the segment's first tile sets the reference; afterwards it only
        // moves when a tile max exceeds it by more than kRescale (rare)
        m_run[nb] = m_run[nb] == -INFINITY ? mt : m_run[nb];
        const bool need = mt > m_run[nb] + kRescale;
        if (__builtin_expect(__any(need), 0)) {
          const float mn = need ? mt : m_run[nb];
          const float f = __builtin_amdgcn_exp2f(m_run[nb] - mn);
          l_run[nb] *= f;
#pragma unroll
          for (int cb = 0; cb < C::CB; ++cb) o[cb][nb] *= f;
          m_run[nb] = mn;
        }
        float ps = 0.f;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(S[mb][nb][e], kLog2e, -m_run[nb]));
            ps += pe;
            P[nb][4 * mb + e] = (__bf16)pe;
          }
        l_run[nb] += ps;
      }

      // ---- O^T += V^T P^T
#pragma unroll
      for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
        for (int nb = 0; nb < C::NBLK; ++nb)
          o[cb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(V[cb], P[nb], o[cb][nb], 0, 0, 0);
    }

    // partial state of this segment: m, l as [slot][n][H]; acc as
    // [slot][H][d_c] with this branch's 128 columns, 16-byte stores
#pragma unroll
    for (int nb = 0; nb < C::NBLK; ++nb) {
      const int head = head0 + 16 * nb + l16;
      const float lt = sum4(l_run[nb]);
      if (kg == 0) {
        p.m[((int64_t)slot * NBR + j) * H + head] = m_run[nb];
        p.l[((int64_t)slot * NBR + j) * H + head] = lt;
      }
      float* row = p.acc + ((int64_t)slot * H + head) * DC + kBW * j + 4 * kg;
#pragma unroll
      for (int cb = 0; cb < C::CB; ++cb) *(f32x4*)(row + 16 * cb) = o[cb][nb];
    }
    start = seg_end;
    ++b;
  }
}

template <int NBR, int HPW, int NHG, int HSPLIT>
hipError_t launch_b(const Geom& g, const void* q_abs, const void* ckv, const void* krope,
                    const Workspace& ws, int items, hipStream_t s) {
  using C = BCfg<NBR, HPW, NHG>;
  // as many stages as LDS holds (<= 4) and the 6-bit vmcnt can track
  constexpr int NS_LDS = (160 * 1024) / C::STAGE;
  constexpr int NS_VM = 2 * C::PER_HI < 64 ? 4 : 3;
  constexpr int NS = NS_LDS < NS_VM ? NS_LDS : NS_VM;
  static_assert(NS >= 3, "tile ring does not fit LDS");
  DecodeParams p;
  p.q_abs = (const __bf16*)q_abs;
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
  hipLaunchKernelGGL((decode_branch_kernel<NBR, HPW, NHG, NS, HSPLIT>), dim3(grid),
                     dim3(64 * C::NW), 0, s, p);
  return hipGetLastError();
}

}  // namespace

bool decode_branch_supported(const Geom& g) {
  return g.dr == kDR && g.dc == 4 * kBW && g.n == 4 && (g.H == 64 || g.H == 128);
}

// Workgroups per work item (head groups of 64 heads); one workgroup per CU.
int decode_branch_wgs_per_item(const Geom& g) { return g.H / 64; }

hipError_t launch_decode_branch(const Geom& g, const void* q_abs, const void* ckv,
                                const void* krope, const Workspace& ws, int items,
                                hipStream_t s) {
  if (!decode_branch_supported(g)) return hipErrorNotSupported;
  if (g.H == 64) return launch_b<4, 32, 2, 1>(g, q_abs, ckv, krope, ws, items, s);
  return launch_b<4, 32, 2, 2>(g, q_abs, ckv, krope, ws, items, s);
}

}  // namespace mlra
