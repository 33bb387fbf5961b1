// Wide-wave MFMA split-KV decode for a 512-wide latent at 128 heads, gfx950
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
//  * One workgroup per work item, four waves (one per SIMD); wave w owns heads
//    [32 w, 32 w + 32) across the whole 576-wide row. Every byte of a tile in
//    LDS is then read by four waves, each MFMA A fragment (16 tokens x 32
//    columns) feeds two MFMAs (two 16-head blocks): half the LDS reads per
//    HBM byte of a design with 16 heads per wave, whose LDS reads would
//    outrun the tile's HBM time. Q^T (32 heads x 576) stays in VGPRs and
//    O^T (512 x 32 fp32) in AGPRs for the whole segment.
//  * The RoPE score is one pair of k-steps per tile, shared by every branch
//    (the method's flop count); each branch adds its own 512/n latent
//    columns, runs its own softmax and its PV over those columns.
//  * 32-token tiles stream HBM -> LDS by LDS-DMA (device-scope, non-temporal)
//    into a ring of 4 stages of 36 KB; each wave issues 9 of a tile's 36
//    1 KB instructions. One workgroup barrier per tile: after it, every wave
//    has finished the previous tile (whose stage takes the DMA three tiles
//    ahead) and prepared the current one.
//  * F16 (MLA, n = 2): the MFMAs run in fp16. Right after its own DMA of the
//    next tile lands, each lane converts the 16 bytes it loaded from bf16 to
//    fp16 in place (exact for |x| in [2^-14, 65504]: bf16's 8 significant
//    bits fit fp16's 11; round toward zero saturates beyond, flushes the
//    negligible tail below). q~ (its bf16 parts summed in fp32) and P are
//    rounded to fp16, 2^-11 relative, where a bf16 query's 2^-8 alone moves
//    one softmax's output rows by up to ~1.3e-2 at MLA's scales. P is kept
//    <= 2^15 (the reference moves when a tile's max passes it by 15 in log2
//    units), within fp16's range. Without F16 every MFMA runs in bf16 on the
//    cache as stored.
//  * QK: S^T[t][h] on v_mfma_f32_16x16x32_{f16,bf16}, 16 tokens as M and 16
//    heads as N, starting from a per-row bias (0, or -inf past the segment's
//    end). The S^T accumulators (lane = head) are P^T, the B operand of
//    O^T[c][h] += V^T[c][t] P^T[t][h], with V^T read by ds_read_b64_tr_b16
//    from the same LDS tile. The LDS rows are XOR-swizzled in 16-byte chunks
//    (chunk ^ 2 (t & 15) for latent rows, ^ ((t >> 1) & 7) for RoPE rows), as
//    in the head-group kernel, so both read patterns are free of bank
//    conflicts.

#include <hip/hip_ext.h>

#include <type_traits>

#include "device_common.h"

namespace mlra {
namespace {

using namespace dev;

constexpr int kT = 32;                   // tokens per tile
constexpr int kDC = 512;                 // latent width
constexpr int kDR = 64;                  // RoPE width
constexpr int kLat = kT * kDC * 2;       // latent bytes of a stage
constexpr int kStage = kLat + kT * kDR * 2;  // 36 KB
constexpr int kNS = 4;                   // stages (144 KB of LDS)
constexpr int kNW = 4;                   // waves, one per SIMD
constexpr int kHPW = 32;                 // heads per wave
constexpr int kH = kNW * kHPW;           // heads
constexpr int kPer = 9;                  // DMA instructions per wave and tile
constexpr int kKS = kDC / 32;            // latent k-steps
constexpr int kCB = kDC / 16;            // PV output column blocks

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

// bf16 -> fp16 of 8 values in one 16-byte chunk, round toward zero (exact in
// fp16's normal range).
__device__ __forceinline__ i32x4 bf16_to_f16x8(i32x4 x) {
  i32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t v = (uint32_t)x[i];
    const auto h = __builtin_amdgcn_cvt_pkrtz(__builtin_bit_cast(float, v << 16),
                                              __builtin_bit_cast(float, v & 0xFFFF0000u));
    r[i] = __builtin_bit_cast(int, h);
  }
  return r;
}

template <int NB, bool F16>
__global__ __launch_bounds__(64 * kNW, 1) void decode_wide_kernel(DecodeParams p) {
  using O_ = Op<F16>;
  using V = typename O_::V;
  using E = typename O_::E;
  constexpr int KPB = kKS / NB;  // latent k-steps per branch
  constexpr int CPB = kCB / NB;  // PV column blocks per branch
  constexpr float kRescale = F16 ? 15.f : 16.f;
  static_assert(kKS % NB == 0 && kCB % NB == 0, "branches");

  __shared__ __attribute__((aligned(1024))) char smem_raw[kNS * kStage];
  char LDS_AS* smem = (char LDS_AS*)smem_raw;
  const uint32_t sbase = (uint32_t)(uintptr_t)smem;

  const int k = blockIdx.x;
  const PlanHeader hd = *p.hdr;
  if (k >= hd.n_items) return;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int l16 = lane & 15, kg = lane >> 4;

  // DMA: latent instruction u < 8 carries row wave + 4 u (lane l: LDS chunk
  // l, global chunk l ^ swz(row); rows u and u + 4 share a swizzle, and the
  // row offset rides in the scalar offset); instruction 8 carries RoPE rows
  // 8 wave .. 8 wave + 7 (lane l: row 8 wave + l / 8, LDS chunk l % 8,
  // global chunk (l % 8) ^ swz_r(row)).
  uint32_t lat_c[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) lat_c[u] = (uint32_t)(16 * (lane ^ swz(wave + 4 * u)));
  const int rope_t = 8 * wave + (lane >> 3);
  const uint32_t rope_c = (uint32_t)(16 * ((lane & 7) ^ swz_r(rope_t)));
  // LDS byte offset of instruction u within a stage (wave-uniform); the DMA
  // writes lane l's 16 bytes at that offset + 16 l
  auto row_lds = [&](int u) -> uint32_t {
    return u < 8 ? (uint32_t)((wave + 4 * u) * 1024) : (uint32_t)(kLat + wave * 1024);
  };
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
  const int end = min(start + hd.chunk, hd.total);
  int bseq = find_seq(p.prefix, p.B, start);

  while (start < end) {
    while (p.prefix[bseq + 1] <= start) ++bseq;
    const int seg_end = min(end, p.prefix[bseq + 1]);
    const int t0 = start - p.prefix[bseq], t1 = seg_end - p.prefix[bseq];
    const int ntiles = (t1 - t0 + kT - 1) / kT;
    const i32x4 crs = seq_rsrc(p.ckv + (int64_t)bseq * p.ckv_bs, t1, p.ckv_ts);
    const i32x4 krs = seq_rsrc(p.krope + (int64_t)bseq * p.kr_bs, t1, p.kr_ts);
    const int slot = k + bseq;

    // earlier stores and loads of this wave done; all waves left the
    // previous segment's LDS tiles
    wait_vm<0>();
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();

    // Q^T as the B operand: lane (head, kg) holds 8 consecutive k of its
    // head; k-steps 0..15 latent, 16..17 RoPE. The fp16 query is q~'s bf16
    // parts summed in fp32, then rounded once.
    V q[kKS + 2][2];
    // (without a residue in the view the residue loads re-read q~ and are
    // weighted by 0)
    const float wlo = p.q_lo > 0 ? 1.f : 0.f;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const __bf16* qrow =
          p.q_abs + ((int64_t)bseq * kH + kHPW * wave + 16 * nb + l16) * p.q_stride + 8 * kg;
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

    auto issue = [&](int tile) {
      const uint32_t sa = sbase + (uint32_t)((tile & (kNS - 1)) * kStage);
      const int ts0 = t0 + tile * kT;
      if (ts0 + kT <= t1) {
#pragma unroll
        for (int u = 0; u < 8; ++u)
          dma16_stream(crs, sa + row_lds(u), lat_c[u & 3],
                       (uint32_t)((ts0 + wave + 4 * u) * p.ckv_ts * 2));
        dma16_stream(krs, sa + row_lds(8), (uint32_t)(rope_t * p.kr_ts * 2) + rope_c,
                     (uint32_t)(ts0 * p.kr_ts * 2));
      } else {  // the segment's last tile: rows clamped to t1 - 1 (wave-uniform)
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int row = min(ts0 + wave + 4 * u, t1 - 1);
          dma16_stream(crs, sa + row_lds(u), lat_c[u & 3], (uint32_t)(row * p.ckv_ts * 2));
        }
        const int row = min(ts0 + rope_t, t1 - 1);
        dma16_stream(krs, sa + row_lds(8), (uint32_t)(row * p.kr_ts * 2) + rope_c, 0u);
      }
    };
    // wait until this wave's DMA of `tile` has landed, given the tiles
    // issued after it that may stay in flight
    auto wait_own = [&](int tile) {
      const int after = min(tile + 2, ntiles - 1) - tile;  // issued tiles beyond `tile`
      if (after >= 2) wait_vm<2 * kPer>();
      else if (after == 1) wait_vm<kPer>();
      else wait_vm<0>();
      asm volatile("" ::: "memory");
    };
    // this lane's 16-byte chunks of `tile` from bf16 to fp16, in place, three
    // reads in flight at a time
    auto convert = [&](int tile) {
      char LDS_AS* st = smem + (tile & (kNS - 1)) * kStage;
#pragma unroll
      for (int u0 = 0; u0 < kPer; u0 += 3) {
        i32x4 x[3];
#pragma unroll
        for (int u = 0; u < 3; ++u) x[u] = *(const i32x4 LDS_AS*)(st + row_lds(u0 + u) + 16 * lane);
#pragma unroll
        for (int u = 0; u < 3; ++u)
          *(i32x4 LDS_AS*)(st + row_lds(u0 + u) + 16 * lane) = bf16_to_f16x8(x[u]);
      }
    };

#pragma unroll
    for (int s = 0; s < kNS - 1; ++s)
      if (s < ntiles) issue(s);

    f32x4 o[kCB][2];
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) o[cb][nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
    float m_run[NB][2], l_run[NB][2];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        m_run[j][nb] = -INFINITY;
        l_run[j][nb] = 0.f;
      }
    if constexpr (F16) {
      wait_own(0);
      convert(0);
    }

    for (int t = 0; t < ntiles; ++t) {
      if constexpr (!F16) wait_own(t);
      // this wave's LDS writes (the conversion) complete before the barrier:
      // s_barrier does not wait for them
      wait_lgkm0();
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      if (t + kNS - 1 < ntiles) issue(t + kNS - 1);
      const char LDS_AS* st = smem + (t & (kNS - 1)) * kStage;

      // score bias per token row: 0, or -inf past the segment's end
      f32x4 bias[2];
      const int valid = t1 - (t0 + t * kT);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) bias[mb][e] = 16 * mb + 4 * kg + e < valid ? 0.f : -INFINITY;

      // RoPE score, shared by the branches
      f32x4 R[2][2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        V a0 = *(const V LDS_AS*)(st + rp_base + mb * 2048);
        V a1 = *(const V LDS_AS*)((const char LDS_AS*)(((uintptr_t)(st + rp_base + mb * 2048)) ^ 64));
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
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
      // V^T fragment of column block cb
      auto pv_frag = [&](int cb) -> V {
        const int coff = 512 * (cb >> 4) + 16 * ((2 * (cb & 15)) ^ pv_w);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)(st + pv_lo + coff));
        const i16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)(st + pv_lo + 16 * 1024 + coff));
        const i16x8 vv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        return __builtin_bit_cast(V, vv);
      };

#pragma unroll
      for (int j = 0; j < NB; ++j) {
        f32x4 S[2][2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) S[mb][nb] = R[mb][nb];
        // software pipeline: the fragments of k-step ks + 2 are read while
        // k-step ks computes; fences keep the compiler from hoisting every
        // read of the tile (their registers would not fit beside Q and O)
        V A[3][2];
        qk_frag(j * KPB, A[0]);
        if (KPB > 1) qk_frag(j * KPB + 1, A[1]);
#pragma unroll
        for (int kk = 0; kk < KPB; ++kk) {
          const int ks = j * KPB + kk;
          if (kk + 2 < KPB) qk_frag(ks + 2, A[(kk + 2) % 3]);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) S[mb][nb] = O_::mfma(A[kk % 3][mb], q[ks][nb], S[mb][nb]);
          __builtin_amdgcn_sched_barrier(0);
        }
        // the next tile's conversion runs while these MFMAs drain
        if constexpr (F16) {
          if (j == 0 && t + 1 < ntiles) {
            wait_own(t + 1);
            convert(t + 1);
          }
        }
        // branch j's online softmax over the tile, per 16-head block
        V P[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const float mx =
              fmaxf(fmaxf(fmaxf(S[0][nb][0], S[0][nb][1]), fmaxf(S[0][nb][2], S[0][nb][3])),
                    fmaxf(fmaxf(S[1][nb][0], S[1][nb][1]), fmaxf(S[1][nb][2], S[1][nb][3])));
          const float mt = max4(mx) * kLog2e;
          const bool need = mt > m_run[j][nb] + kRescale;
          if (__builtin_expect(__any(need), 0)) {
            const float mn = need ? mt : m_run[j][nb];
            const float f = __builtin_amdgcn_exp2f(m_run[j][nb] - mn);
            l_run[j][nb] *= f;
#pragma unroll
            for (int cb = j * CPB; cb < (j + 1) * CPB; ++cb) o[cb][nb] *= f;
            m_run[j][nb] = mn;
          }
          float ps = 0.f;
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(S[mb][nb][e], kLog2e,
                                                                     -m_run[j][nb]));
              ps += pe;
              P[nb][4 * mb + e] = (E)pe;
            }
          l_run[j][nb] += ps;
        }
        // O^T += V^T P^T over branch j's columns, V^T fragments read three
        // blocks ahead
        V Vf[4];
#pragma unroll
        for (int i = 0; i < 3 && i < CPB; ++i) Vf[i] = pv_frag(j * CPB + i);
#pragma unroll
        for (int c = 0; c < CPB; ++c) {
          const int cb = j * CPB + c;
          if (c + 3 < CPB) Vf[(c + 3) % 4] = pv_frag(cb + 3);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int nb = 0; nb < 2; ++nb) o[cb][nb] = O_::mfma(Vf[c % 4], P[nb], o[cb][nb]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }

    // partial state of this segment: m, l as [slot][n][H]; acc as
    // [slot][H][d_c], 16-byte stores of 4 consecutive latent columns
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int head = kHPW * wave + 16 * nb + l16;
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const float lt = sum4(l_run[j][nb]);
        if (kg == 0) {
          p.m[((int64_t)slot * NB + j) * kH + head] = m_run[j][nb];
          p.l[((int64_t)slot * NB + j) * kH + head] = lt;
        }
      }
      float* row = p.acc + ((int64_t)slot * kH + head) * kDC + 4 * kg;
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) *(f32x4*)(row + 16 * cb) = o[cb][nb];
    }
    start = seg_end;
    ++bseq;
  }
}

template <int NB, bool F16>
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
  hipExtLaunchKernelGGL((decode_wide_kernel<NB, F16>), dim3(items), dim3(64 * kNW), 0, s,
                        t.start, t.stop, 0, p);
  return hipGetLastError();
}

}  // namespace

// MLA: one branch over a 512-wide latent, 64-wide RoPE key, 128 heads. (The
// kernel is written for n branches with a shared RoPE score; only n = 1 is
// built: it needs 400 registers of Q and O per lane, which this compiler
// fits beside the score accumulators only with the MFMAs' results in
// VGPRs, and its pass that moves them to AGPRs fails on the four-branch
// instantiation.)
bool decode_wide_supported(const Geom& g) {
  return g.dc == kDC && g.dr == kDR && g.H == kH && g.n == 1;
}

// fp16 MFMAs on q~ with its residue
bool decode_wide_reads_residue(const Geom&) { return true; }

hipError_t launch_decode_wide(const Geom& g, const QView& q, const void* ckv, const void* krope,
                              const Workspace& ws, int items, hipStream_t s,
                              const KernelTiming& t) {
  if (!decode_wide_supported(g)) return hipErrorNotSupported;
  return launch_w<1, true>(g, q, ckv, krope, ws, items, s, t);
}

}  // namespace mlra
