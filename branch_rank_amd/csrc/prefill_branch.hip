// Causal prefill of MLRA-4 (128-wide branch slices) in one kernel, gfx950
// (MI355X): query absorption, causal latent attention and the W_UV output
// projection, with no intermediate in HBM.
//
// What it computes ("Multi-Head Low-Rank Attention", 核心方法 and 方法步骤详情:
// one softmax per branch over its latent slice plus the shared RoPE key,
// outputs summed and scaled by alpha_kv; "MLA多头潜在注意力机制" 3.3: a key
// after the query's position is masked out): for every position t < L_b of
// sequence b and head h,
//   q~_j  = alpha_q tau W_UK[h][S_j] q^N_t,   rho = tau RoPE(q^R_t, t),
//   o~_j  = sum_{u <= t} softmax_u(q~_j . c_u[S_j] + rho . k^R_u) c_u[S_j],
//   o_t,h = alpha_kv sum_j W_UV[h][S_j]^T o~_j,
// and zeros for L_b <= t < T. This is the decode step's absorbed form with
// one query per position. With d_c' = d_n = d_v = 128 it costs what the
// unabsorbed form costs (192 + 128 multiply-adds per query, key and branch;
// two 128 x 128 projections per position and branch).
//
// Mapping onto CDNA4: a workgroup takes one sequence, one block of 64
// positions and one head; wave (j, g) owns branch j for the 32 positions of
// group g. Keys 0 .. the block's end stream through a ring of four LDS stages
// (32 cached rows, all four branch slices and the RoPE key) by LDS-DMA.
//   prologue  q~_j by MFMA from W_UK rows read straight into the A operand,
//             laid out as the score MFMA's B operand; RoPE of the 64 queries
//             once per workgroup through LDS; the first tiles in flight.
//   loop      S^T = K Q^T (16 keys x 16 queries per v_mfma_f32_16x16x32_bf16),
//             the causal mask as the accumulator start on a wave's diagonal
//             tile, lazily rescaled online softmax per query lane, and
//             O^T += V^T P^T with P kept in its lanes.
//   epilogue  W_UV[h] staged in the ring; out^T = W_UV^T o~^T per branch on
//             MFMA with o~ split into bf16 high and low parts (fp32-accurate
//             product); the four branch partials summed in LDS in a fixed
//             order and stored.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>

#include "device_common.h"

namespace mlra {
namespace {

using namespace dev;

constexpr int kT = 32;                // keys per tile
constexpr int kDC = 512;              // latent width
constexpr int kBW = 128;              // branch width d_c'
constexpr int kDR = 64;               // RoPE width
constexpr int kDN = 128;              // NoPE query width
constexpr int kDV = 128;              // value width
constexpr int kNW = 8;                // waves: 4 branches x 2 position groups
constexpr int kQW = 32;               // positions per wave
constexpr int kQWG = 2 * kQW;         // positions per workgroup
constexpr int kRowB = kDC * 2;        // LDS bytes of a cached latent row
constexpr int kLat = kT * kRowB;      // latent part of a stage
constexpr int kStage = kLat + kT * kDR * 2;
constexpr int kNS = 4;                // ring stages
constexpr int kD = kNS - 1;           // tiles in flight ahead of the one in use
constexpr int kRing = kNS * kStage;
constexpr int kRopeQ = kRing;         // RoPE queries [64][64] bf16
constexpr int kLds = kRing + kQWG * kDR * 2;
constexpr int kWPitch = kDV * 2 + 32; // staged W_UV row (padding spreads the banks)
constexpr int kKL = kBW / 32;         // latent k-steps of a score
constexpr int kKS = kKL + kDR / 32;   // plus the RoPE k-steps
constexpr int kCB = kBW / 16;         // 16-row blocks of a branch's output
constexpr int kNBLK = kQW / 16;       // 16-query blocks per wave
constexpr int kVB = kDV / 16;         // 16-row blocks of the projected output
constexpr float kRescale = 16.f;      // log2 headroom kept when the reference moves
constexpr float kSumLimit = 1048576.f;  // 2^20: per-lane P sum that moves the reference
static_assert(kDC * kWPitch <= kRing, "W_UV fits the ring");
static_assert(kNW * 64 * kVB * kNBLK * 16 <= kRing, "output partials fit the ring");
static_assert(kLds <= 160 * 1024, "LDS");

// 16-byte chunk swizzles: cached latent rows (1 KB) by row & 7, RoPE rows
// (128 B) by (row >> 1) & 7
__device__ __forceinline__ int swz_l(int t) { return 2 * (t & 7); }
__device__ __forceinline__ int swz_r(int t) { return (t >> 1) & 7; }

struct PrefillParams {
  const __bf16* q_nope;  // [B][T][H][d_n]
  const __bf16* q_rope;  // [B][T][H][d_r], unrotated
  const __bf16* w_uk;    // [H][d_c][d_n]
  const __bf16* w_uv;    // [H][d_c][d_v]
  const __bf16* ckv;
  const __bf16* krope;
  int64_t ckv_bs, kr_bs;
  int ckv_ts, kr_ts;     // element strides (host checks the byte ranges fit 31 bits)
  const int32_t* lens;   // [B]
  void* out;             // [B][T][H][d_v]
  int T, H, QB;          // QB: 64-position blocks per sequence
  float scale_n, scale_r;  // query scales, log2(e) folded in: alpha_q tau log2e, tau log2e
  float alpha_kv;
  double omega[kDR / 2];   // rotary frequencies theta^(-2k/d_r)
};

__device__ __forceinline__ void store4(float* p, f32x4 v) { *(f32x4*)p = v; }
__device__ __forceinline__ void store4(__bf16* p, f32x4 v) {
  typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
  *(bf16x4*)p = (bf16x4){(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
}

// Workgroup barrier after this wave's LDS writes have completed; LDS-DMA
// still in flight is not waited for.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <typename TO>
__global__ __launch_bounds__(512, 1) void prefill_kernel(PrefillParams p) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[kLds];
  char LDS_AS* smem = (char LDS_AS*)smem_raw;
  const uint32_t sbase = (uint32_t)(uintptr_t)smem;

  // workgroup -> (sequence, position block, head): the heads of one block
  // are adjacent so that their key tiles meet in L2, and the longest (last)
  // blocks of each sequence are dispatched first
  int i = blockIdx.x;
  const int h = i % p.H;
  i /= p.H;
  const int qb = p.QB - 1 - i % p.QB, b = i / p.QB;
  const int T = p.T;
  const int L = min(max(p.lens[b], 0), T);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = wave & 3, g = wave >> 2;
  const int l16 = lane & 15, kg = lane >> 4;
  const int q0 = qb * kQWG + g * kQW;  // this wave's first position
  const int64_t orow = (int64_t)p.H * kDV;
  TO* out_bh = (TO*)p.out + ((int64_t)b * T * p.H + h) * kDV;  // position t at + t * orow

  if (qb * kQWG >= L) {  // every position of the block lies past the sequence
#pragma unroll
    for (int nb = 0; nb < kNBLK; ++nb) {
      const int t = q0 + 16 * nb + l16;
      if (t >= T) continue;
#pragma unroll
      for (int u = 0; u < 2; ++u)
        store4(out_bh + t * orow + 16 * (2 * j + u) + 4 * kg, (f32x4){0.f, 0.f, 0.f, 0.f});
    }
    return;
  }

  // ---- key tiles: the first kD in flight while the queries are formed ----
  const int kend = min(L, qb * kQWG + kQWG);  // keys of this block: [0, kend)
  const int ntiles = (kend + kT - 1) / kT;
  const i32x4 crs = seq_rsrc(p.ckv + (int64_t)b * p.ckv_bs, kend, p.ckv_ts);
  const i32x4 krs = seq_rsrc(p.krope + (int64_t)b * p.kr_bs, kend, p.kr_ts);
  // wave w fills latent rows w + 8u (u = 0..3) of a tile, all with row & 7 = w
  const uint32_t lat_c = 16u * (uint32_t)(lane ^ swz_l(wave));
  const int rope_t = wave * 8 + (lane >> 3);  // waves 0-3: RoPE rows
  const int rope_c = 16 * ((lane & 7) ^ swz_r(rope_t));
  int dma_off = 0;
  auto issue = [&](int tile) {
    const uint32_t sa = sbase + dma_off;
    dma_off = dma_off + kStage == kRing ? 0 : dma_off + kStage;
    const int ts0 = tile * kT;
    if (ts0 + kT <= kend) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = wave + 8 * u;
        dma16(crs, sa + r * kRowB, lat_c, (uint32_t)((ts0 + r) * p.ckv_ts * 2));
      }
    } else {  // the block's last tile: rows past its keys repeat the last key
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = wave + 8 * u;
        const int row = min(ts0 + r, kend - 1);
        dma16(crs, sa + r * kRowB, (uint32_t)(row * p.ckv_ts * 2) + lat_c, 0u);
      }
    }
    if (wave < 4) {
      const int row = min(ts0 + rope_t, kend - 1);
      dma16(krs, sa + kLat + wave * 1024, (uint32_t)(row * p.kr_ts * 2 + rope_c), 0u);
    }
  };
#pragma unroll
  for (int s = 0; s < kD; ++s)
    if (s < ntiles) issue(s);

  // ---- RoPE queries of the 64 positions, once per workgroup: the angle
  // t * theta^(-2k/d_r) (frequency from the host's table) and its reduction
  // to [-pi, pi] in double precision, sine and cosine of the reduced angle in
  // float ----
  {
    static_assert((64 * kNW) % (kDR / 2) == 0, "one frequency per thread");
    const int k = threadIdx.x % (kDR / 2);
    const double omega = p.omega[k];
    for (int e = threadIdx.x; e < kQWG * (kDR / 2); e += 64 * kNW) {
      const int qi = e / (kDR / 2);
      const int t = min(qb * kQWG + qi, T - 1);
      const __bf16* x = p.q_rope + (((int64_t)b * T + t) * p.H + h) * kDR + 2 * k;
      const double a = (double)t * omega;
      const double r = a - 6.283185307179586 * rint(a * 0.15915494309189535);
      float sn, cs;
      sincosf((float)r, &sn, &cs);
      const float x0 = (float)x[0], x1 = (float)x[1];
      __bf16 LDS_AS* d = (__bf16 LDS_AS*)(smem + kRopeQ + qi * (kDR * 2)) + 2 * k;
      d[0] = (__bf16)(p.scale_r * (x0 * cs - x1 * sn));
      d[1] = (__bf16)(p.scale_r * (x0 * sn + x1 * cs));
    }
  }

  // ---- absorbed queries q~_j of this wave's positions (B operand of the
  // scores: lane (position, kg) holds latent columns 32 ks + 8 kg + 0..7) ----
  bf16x8 q[kKS][kNBLK];
  bf16x8 qlo[kKL][kNBLK];  // low bf16 parts of the latent columns: q~ = q + qlo
  {
    bf16x8 qn[kDN / 32][kNBLK];
#pragma unroll
    for (int nb = 0; nb < kNBLK; ++nb) {
      const int t = min(q0 + 16 * nb + l16, T - 1);
      const __bf16* r = p.q_nope + (((int64_t)b * T + t) * p.H + h) * kDN;
#pragma unroll
      for (int kn = 0; kn < kDN / 32; ++kn) qn[kn][nb] = *(const bf16x8*)(r + 32 * kn + 8 * kg);
    }
    const __bf16* wk = p.w_uk + ((int64_t)h * kDC + kBW * j) * kDN;
#pragma unroll
    for (int ks = 0; ks < kKL; ++ks) {
      // A row l16 of half s is latent column 32 ks + 8 (l16 >> 2) + 4 s +
      // (l16 & 3), so that output row 4 kg + i lands on column 32 ks + 8 kg +
      // 4 s + i of the query lane
      f32x4 acc[2][kNBLK];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int c = 32 * ks + 8 * (l16 >> 2) + 4 * s + (l16 & 3);
        bf16x8 a[kDN / 32];
#pragma unroll
        for (int kn = 0; kn < kDN / 32; ++kn) a[kn] = *(const bf16x8*)(wk + c * kDN + 32 * kn + 8 * kg);
#pragma unroll
        for (int nb = 0; nb < kNBLK; ++nb) {
          acc[s][nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kn = 0; kn < kDN / 32; ++kn)
            acc[s][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[kn], qn[kn][nb], acc[s][nb], 0, 0, 0);
        }
      }
#pragma unroll
      for (int nb = 0; nb < kNBLK; ++nb)
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float v = p.scale_n * acc[s][nb][e];
            const __bf16 hi = (__bf16)v;
            q[ks][nb][4 * s + e] = hi;
            qlo[ks][nb][4 * s + e] = (__bf16)(v - (float)hi);
          }
    }
  }
  lds_barrier();  // RoPE queries staged
#pragma unroll
  for (int nb = 0; nb < kNBLK; ++nb) {
    const int qi = g * kQW + 16 * nb + l16;
#pragma unroll
    for (int kr = 0; kr < kKS - kKL; ++kr)
      q[kKL + kr][nb] = *(const bf16x8 LDS_AS*)(smem + kRopeQ + qi * (kDR * 2) + 64 * kr + 16 * kg);
  }

  // ---- per-lane LDS offsets within a stage ----
  // score A operand (keys l16, l16 + 16): k-step ks at (qk_lat ^ 64 ks)
  const int qk_lat = l16 * kRowB + 16 * ((16 * j + kg) ^ swz_l(l16));
  const int qk_rp = kLat + l16 * 128 + 16 * (kg ^ swz_r(l16));
  // value A operand (V^T, transposed 4 x 16 reads): block cb at (pv_lat ^ 32 cb)
  int pv_lat;
  {
    const int t = 4 * kg + (l16 >> 2), half = l16 & 3;
    pv_lat = t * kRowB + 16 * ((16 * j + (half >> 1)) ^ swz_l(t)) + 8 * (half & 1);
  }

  f32x4 o[kCB][kNBLK];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
    for (int nb = 0; nb < kNBLK; ++nb) o[cb][nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  // scores come out of the MFMA in log2 units relative to the running
  // reference m_run of their position (the accumulators start at -m_run)
  float m_run[kNBLK], l_run[kNBLK];
#pragma unroll
  for (int nb = 0; nb < kNBLK; ++nb) {
    m_run[nb] = 0.f;
    l_run[nb] = 0.f;
  }
  // this wave's diagonal tile (q0 is 32-aligned); a wave whose positions all
  // lie past the sequence computes nothing (its rows come out zero)
  const int last = q0 < L ? q0 / kT : -1;

  int cur_off = 0;
  for (int it = 0; it < ntiles; ++it) {
    // this wave's DMA of tile `it` has landed: waves 0-3 issue 5 loads per
    // tile, waves 4-7 issue 4, and `ahead` later tiles may still be in flight
    {
      const int ahead = min(kD - 1, ntiles - 1 - it);
      if (wave < 4) {
        if (ahead >= 2) wait_vm<10>(); else if (ahead == 1) wait_vm<5>(); else wait_vm<0>();
      } else {
        if (ahead >= 2) wait_vm<8>(); else if (ahead == 1) wait_vm<4>(); else wait_vm<0>();
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    // the stage of tile it + kD last held tile it - 1, which every wave has
    // finished before this barrier
    if (it + kD < ntiles) issue(it + kD);
    const char LDS_AS* st = smem + __builtin_amdgcn_readfirstlane(cur_off);
    cur_off = cur_off + kStage == kRing ? 0 : cur_off + kStage;
    if (it > last) continue;  // keys after all of this wave's positions

    bf16x8 A[2][kKS];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int ks = 0; ks < kKL; ++ks)
        A[mb][ks] = *(const bf16x8 LDS_AS*)((const char LDS_AS*)(((uintptr_t)(st + qk_lat)) ^ (64 * ks)) +
                                            mb * 16 * kRowB);
      A[mb][kKL] = *(const bf16x8 LDS_AS*)(st + qk_rp + mb * 2048);
      A[mb][kKL + 1] =
          *(const bf16x8 LDS_AS*)((const char LDS_AS*)(((uintptr_t)(st + qk_rp)) ^ 64) + mb * 2048);
    }
    bf16x8 V[kCB];
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      const char LDS_AS* a = (const char LDS_AS*)(((uintptr_t)(st + pv_lat)) ^ (32 * cb));
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)a);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)(a + 16 * kRowB));
      const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      V[cb] = __builtin_bit_cast(bf16x8, v);
    }

    // S^T - m_run = K Q^T - m_run (log2 units), the accumulators starting
    // at -m_run of their position, or at -inf where the causal mask of the
    // diagonal tile hides key row 16 mb + 4 kg + e from position column
    // 16 nb + l16. The four (mb, nb) accumulations run interleaved k-step by
    // k-step, so that consecutive MFMAs are independent.
    f32x4 S[2][kNBLK];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < kNBLK; ++nb) {
        S[mb][nb] = (f32x4){-m_run[nb], -m_run[nb], -m_run[nb], -m_run[nb]};
        if (it == last) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (16 * mb + 4 * kg + e > 16 * nb + l16) S[mb][nb][e] = -INFINITY;
        }
      }
#pragma unroll
    for (int ks = 0; ks < kKS; ++ks)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < kNBLK; ++nb) {
          S[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mb][ks], q[ks][nb], S[mb][nb], 0, 0, 0);
          if (ks < kKL)  // the latent part also with the low half of q~
            S[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mb][ks], qlo[ks][nb], S[mb][nb], 0, 0, 0);
        }

    // online softmax per position (lane), lazily rescaled: p = 2^(S - m_run)
    // straight from the accumulators; the exact tile max only on the first
    // tile (no reference yet) or when a lane's sum of P passes 2^20 (or is
    // not finite), then the reference moves to 16 below the max and O, l
    // are rescaled
    bf16x8 P[kNBLK];
    float ps[kNBLK];
    bool need = it == 0;
#pragma unroll
    for (int nb = 0; nb < kNBLK; ++nb) {
      ps[nb] = 0.f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pe = __builtin_amdgcn_exp2f(S[mb][nb][e]);
          ps[nb] += pe;
          P[nb][4 * mb + e] = (__bf16)pe;
        }
      need |= !(ps[nb] <= kSumLimit);
    }
    if (__builtin_expect(__any(need), 0)) {
#pragma unroll
      for (int nb = 0; nb < kNBLK; ++nb) {
        const float mx = fmaxf(fmaxf(fmaxf(S[0][nb][0], S[0][nb][1]), fmaxf(S[0][nb][2], S[0][nb][3])),
                               fmaxf(fmaxf(S[1][nb][0], S[1][nb][1]), fmaxf(S[1][nb][2], S[1][nb][3])));
        const float mt = max4(mx) + m_run[nb];  // the tile max, log2 units
        const float mr = it == 0 ? mt : m_run[nb];
        const float mn = fmaxf(mr, mt - kRescale);
        const float f = __builtin_amdgcn_exp2f(mr - mn);
        l_run[nb] *= f;
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb) o[cb][nb] *= f;
        const float off = m_run[nb] - mn;
        m_run[nb] = mn;
        ps[nb] = 0.f;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float pe = __builtin_amdgcn_exp2f(S[mb][nb][e] + off);
            ps[nb] += pe;
            P[nb][4 * mb + e] = (__bf16)pe;
          }
      }
    }
#pragma unroll
    for (int nb = 0; nb < kNBLK; ++nb) l_run[nb] += ps[nb];

#pragma unroll
    for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
      for (int nb = 0; nb < kNBLK; ++nb)
        o[cb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(V[cb], P[nb], o[cb][nb], 0, 0, 0);
  }

  // ---- o~ normalised per position and split into bf16 high + low parts:
  // B operand of out^T = W_UV^T o~^T, lane (position, kg) holding k index
  // 8 kg + 4 s + i = latent column 32 pp + 16 s + 4 kg + i of the branch ----
  bf16x8 oh[kCB / 2][kNBLK], ol[kCB / 2][kNBLK];
#pragma unroll
  for (int nb = 0; nb < kNBLK; ++nb) {
    const int t = q0 + 16 * nb + l16;
    const float lt = sum4(l_run[nb]);
    const float inv = t < L ? 1.f / lt : 0.f;
#pragma unroll
    for (int pp = 0; pp < kCB / 2; ++pp)
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = o[2 * pp + s][nb][e] * inv;
          const __bf16 hv = (__bf16)v;
          oh[pp][nb][4 * s + e] = hv;
          ol[pp][nb][4 * s + e] = (__bf16)(v - (float)hv);
        }
  }

  // ---- W_UV[h] into the ring as [c][v] rows of kWPitch bytes ----
  lds_barrier();  // every wave is done with the key tiles
  {
    const __bf16* w = p.w_uv + (int64_t)h * kDC * kDV;
    constexpr int NQ = kDC * kDV * 2 / 16 / (64 * kNW);  // 16-byte pieces per thread
    bf16x8 stg[NQ];
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int e = threadIdx.x + 64 * kNW * u, c = e >> 4, ch = e & 15;
      stg[u] = *(const bf16x8*)(w + c * kDV + 8 * ch);
    }
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int e = threadIdx.x + 64 * kNW * u, c = e >> 4, ch = e & 15;
      *(bf16x8 LDS_AS*)(smem + c * kWPitch + 16 * ch) = stg[u];
    }
  }
  lds_barrier();

  // ---- this branch's part of out^T: A = W_UV^T rows v (transposed reads of
  // latent rows 32 pp + 4 kg + 0..3 and + 16), B = o~ high, then low ----
  f32x4 acc[kVB][kNBLK];
  {
    const int r4 = l16 >> 2, q4 = l16 & 3;
#pragma unroll
    for (int vb = 0; vb < kVB; ++vb) {
#pragma unroll
      for (int nb = 0; nb < kNBLK; ++nb) acc[vb][nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int pp = 0; pp < kCB / 2; ++pp) {
        const char LDS_AS* a =
            smem + (kBW * j + 32 * pp + 4 * kg + r4) * kWPitch + 2 * (16 * vb + 4 * q4);
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)a);
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)(a + 16 * kWPitch));
        const i16x8 wv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        const bf16x8 W = __builtin_bit_cast(bf16x8, wv);
#pragma unroll
        for (int nb = 0; nb < kNBLK; ++nb) {
          acc[vb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(W, oh[pp][nb], acc[vb][nb], 0, 0, 0);
          acc[vb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(W, ol[pp][nb], acc[vb][nb], 0, 0, 0);
        }
      }
    }
  }

  // ---- branch partials through LDS, summed j = 0..3 in order, stored ----
  lds_barrier();  // every wave is done with W_UV
  {
    char LDS_AS* mine = smem + wave * (kVB * kNBLK * 1024) + lane * 16;
#pragma unroll
    for (int vb = 0; vb < kVB; ++vb)
#pragma unroll
      for (int nb = 0; nb < kNBLK; ++nb) *(f32x4 LDS_AS*)(mine + (vb * kNBLK + nb) * 1024) = acc[vb][nb];
  }
  lds_barrier();
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int vb = 2 * j + u;
#pragma unroll
    for (int nb = 0; nb < kNBLK; ++nb) {
      f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        sum += *(const f32x4 LDS_AS*)(smem + (4 * g + jj) * (kVB * kNBLK * 1024) +
                                      (vb * kNBLK + nb) * 1024 + lane * 16);
      const int t = q0 + 16 * nb + l16;
      if (t < T) store4(out_bh + t * orow + 16 * vb + 4 * kg, sum * p.alpha_kv);
    }
  }
}

}  // namespace

bool prefill_branch_supported(const Geom& g) {
  return g.dr == kDR && g.dc == kDC && g.n == kDC / kBW && g.dn == kDN && g.dv == kDV;
}

hipError_t launch_prefill_branch(const Geom& g, int T, const void* q_nope, const void* q_rope,
                                 const void* w_uk, const void* w_uv, const void* ckv,
                                 const void* krope, const int32_t* lens, void* out, bool out_bf16,
                                 float tau, float alpha_q, float alpha_kv, float theta,
                                 hipStream_t s, const KernelTiming& t) {
  if (!prefill_branch_supported(g)) return hipErrorNotSupported;
  if (g.B <= 0 || T <= 0) return hipSuccess;
  PrefillParams p;
  p.q_nope = (const __bf16*)q_nope;
  p.q_rope = (const __bf16*)q_rope;
  p.w_uk = (const __bf16*)w_uk;
  p.w_uv = (const __bf16*)w_uv;
  p.ckv = (const __bf16*)ckv;
  p.krope = (const __bf16*)krope;
  p.ckv_bs = g.ckv_bs;
  p.ckv_ts = (int)g.ckv_ts;
  p.kr_bs = g.kr_bs;
  p.kr_ts = (int)g.kr_ts;
  p.lens = lens;
  p.out = out;
  p.T = T;
  p.H = g.H;
  p.QB = (T + kQWG - 1) / kQWG;
  constexpr double kLog2eD = 1.4426950408889634;
  p.scale_n = (float)((double)alpha_q * tau * kLog2eD);
  p.scale_r = (float)((double)tau * kLog2eD);
  p.alpha_kv = alpha_kv;
  const RopeFreqs& fr = rope_freqs(theta, kDR);
  for (int k = 0; k < kDR / 2; ++k) p.omega[k] = fr.w[k];
  const int64_t grid = (int64_t)g.B * p.QB * g.H;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (out_bf16)
    hipExtLaunchKernelGGL(prefill_kernel<__bf16>, dim3((unsigned)grid), dim3(64 * kNW), 0, s,
                          t.start, t.stop, 0, p);
  else
    hipExtLaunchKernelGGL(prefill_kernel<float>, dim3((unsigned)grid), dim3(64 * kNW), 0, s,
                          t.start, t.stop, 0, p);
  return hipGetLastError();
}

}  // namespace mlra
