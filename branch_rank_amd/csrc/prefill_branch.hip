// Causal multi-query latent attention for the prefill of MLRA-n with 128-wide
// branch slices, gfx950 (MI355X).
//
// What it computes ("Multi-Head Low-Rank Attention", 核心方法: one softmax per
// branch over its latent slice plus the shared RoPE key; "vllbc02MLA",
// 苏神思路: the prompt attends causally, every position t to the tokens
// 0..t): for every cached position t < L_b of sequence b, every head h and
// branch j, the branch-normalised latent
//   o~_j[t, h] = sum_{u <= t} softmax_u(q~_j[t, h] . c_u[S_j] + rho[t, h] . k^R_u) c_u[S_j],
// with q~ and rho the absorbed query of position t (absorb_q). With a
// branch width d_c' equal to d_n and d_v (128 at MLRA-4) the absorbed form
// costs what the unabsorbed one does: 192 + 128 multiply-adds per (query,
// key) pair, and a 128 x 128 projection per token and branch on either side.
//
// Mapping onto CDNA4 (the decode's branch-per-wave layout with queries in
// place of heads): a workgroup takes one sequence, one block of 128 query
// positions, one head and one branch pair; wave (b, g) owns branch b of the
// pair for the 32 queries of group g. Keys 0 .. the block's end stream
// through the same LDS-DMA tile ring as the decode (branch_tiles.h). S^T =
// K Q^T on v_mfma_f32_16x16x32_bf16 with 16 keys as M and 16 queries as N;
// the S^T accumulators are the B operand of O^T = V^T P^T, so P stays in its
// lane. The causal mask enters as the accumulators' start on each wave's
// diagonal tile; tiles entirely after a wave's queries are skipped (the
// wave still takes part in the barriers and the loads). The epilogue divides
// by each query's softmax sum and writes the latent rows; positions t >= L_b
// of the block get zeros.

#include <hip/hip_runtime.h>

#include "branch_tiles.h"

namespace mlra {
namespace {

using namespace dev;
using namespace bt;

// Arguments of the prefill kernel (one struct, passed by value).
struct PrefillParams {
  const __bf16* q_abs;  // [B][T][H][d_c + d_r]
  const __bf16* ckv;
  const __bf16* krope;
  int64_t ckv_bs, kr_bs;
  int ckv_ts, kr_ts;
  const int32_t* lens;  // [B]
  float* latent;        // [B][T][H][d_c]
  int B, T, H, QB;      // QB: 128-position query blocks per sequence
};

constexpr int kQW = 32;             // queries per wave
constexpr int kQWG = 4 * kQW;       // queries per workgroup

template <int NS>
__global__ __launch_bounds__(512, 1) void prefill_branch_kernel(PrefillParams p) {
  using C = BCfg<4, 2, kQW, 4>;  // two branches of the pair x four query groups
  constexpr int D = NS - 1;
  constexpr int DC = C::DC;
  __shared__ __attribute__((aligned(1024))) char smem_raw[NS * C::STAGE];
  char LDS_AS* smem = (char LDS_AS*)smem_raw;
  const uint32_t sbase = (uint32_t)(uintptr_t)smem;

  // workgroup -> (sequence, query block, head, branch pair); the pairs and
  // heads of one query block are adjacent, so their K/V tiles meet in L2
  // heads of one query block are adjacent, so their K/V tiles meet in L2;
  // the longest (last) query blocks of each sequence are dispatched first
  int i = blockIdx.x;
  const int hg = i & 1;
  i >>= 1;
  const int h = i % p.H;
  i /= p.H;
  const int qb = p.QB - 1 - i % p.QB, b = i / p.QB;
  const int L = min(max(p.lens[b], 0), p.T);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int bw = wave % C::NBW, g = wave / C::NBW;
  const int j = hg * C::NBW + bw;
  const int l16 = lane & 15, kg = lane >> 4;
  const int q0 = qb * kQWG + g * kQW;  // this wave's first query position
  const int row = DC + kDR;

  if (qb * kQWG >= L) {  // the whole block lies past the sequence: zeros
#pragma unroll
    for (int nb = 0; nb < C::NBLK; ++nb) {
      const int t = q0 + 16 * nb + l16;
      if (t >= p.T) continue;
      float* dst = p.latent + (((int64_t)b * p.T + t) * p.H + h) * DC + kBW * j + 4 * kg;
#pragma unroll
      for (int cb = 0; cb < C::CB; ++cb) *(f32x4*)(dst + 16 * cb) = (f32x4){0.f, 0.f, 0.f, 0.f};
    }
    return;
  }

  // per-lane LDS offsets, as in the decode (branch_tiles.h layout)
  const int qk_lat = l16 * C::ROWB + 16 * ((16 * bw + kg) ^ swz_l(l16));
  const int qk_rp = C::LAT + l16 * 128 + 16 * (kg ^ swz_r(l16));
  int pv_lat;
  {
    const int t = 4 * kg + (l16 >> 2), half = l16 & 3;
    pv_lat = t * C::ROWB + 16 * ((16 * bw + (half >> 1)) ^ swz_l(t)) + 8 * (half & 1);
  }
  const int lat_row = lane / (64 / C::RPI), lat_p = lane % (64 / C::RPI);
  const int lat_c = 16 * (lat_p ^ swz_l(C::RPI * wave + lat_row)) + hg * C::ROWB;
  const int rope_t = wave * 8 + (lane >> 3);
  const int rope_c = 16 * ((lane & 7) ^ swz_r(rope_t));

  const int kend = min(L, qb * kQWG + kQWG);  // keys of this block: [0, kend)
  const int ntiles = (kend + kT - 1) / kT;
  const i32x4 crs = seq_rsrc(p.ckv + (int64_t)b * p.ckv_bs, kend, p.ckv_ts);
  const i32x4 krs = seq_rsrc(p.krope + (int64_t)b * p.kr_bs, kend, p.kr_ts);
  const uint32_t lat_voff = (uint32_t)(lat_row * p.ckv_ts * 2 + lat_c);

  // Q^T of this wave's queries (B operand): lane (query, kg) holds 8
  // consecutive k of its query; positions past the sequence read row L - 1
  bf16x8 q[C::KS][C::NBLK];
#pragma unroll
  for (int nb = 0; nb < C::NBLK; ++nb) {
    const int t = min(q0 + 16 * nb + l16, L - 1);
    const __bf16* qrow = p.q_abs + (((int64_t)b * p.T + t) * p.H + h) * row;
#pragma unroll
    for (int ks = 0; ks < C::KL; ++ks)
      q[ks][nb] = *(const bf16x8*)(qrow + kBW * j + 32 * ks + 8 * kg);
#pragma unroll
    for (int ks = C::KL; ks < C::KS; ++ks)
      q[ks][nb] = *(const bf16x8*)(qrow + DC + 32 * (ks - C::KL) + 8 * kg);
  }
  wait_vm<0>();

  auto next_stage = [](int off) { return off + C::STAGE == NS * C::STAGE ? 0 : off + C::STAGE; };
  int dma_off = 0;
  auto issue = [&](int tile) {
    const uint32_t sa = sbase + dma_off;
    dma_off = next_stage(dma_off);
    const int ts0 = tile * kT;
    if (ts0 + kT <= kend)
      issue_tile<C, false>(sa, crs, krs, p.ckv_ts, p.kr_ts, ts0, kend, wave, lane, lat_voff,
                           lat_c, rope_t, rope_c);
    else
      issue_tile<C, true>(sa, crs, krs, p.ckv_ts, p.kr_ts, ts0, kend, wave, lane, lat_voff, lat_c,
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
  // this wave's diagonal tile (q0 is 32-aligned); a wave whose queries all
  // lie past the sequence computes nothing (its rows are written as zeros)
  const int last = q0 < L ? q0 / kT : -1;

  int cur_off = 0;
  for (int it = 0; it < ntiles; ++it) {
    wait_tiles<C, D - 1>(min(D - 1, ntiles - 1 - it), wave);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    // the stage of tile it + D last held tile it - 1, which every wave has
    // finished before this barrier
    if (it + D < ntiles) issue(it + D);
    const char LDS_AS* st = smem + __builtin_amdgcn_readfirstlane(cur_off);
    cur_off = next_stage(cur_off);
    if (it > last) continue;  // keys after all of this wave's queries

    bf16x8 A[2][C::KS];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int ks = 0; ks < C::KL; ++ks)
        A[mb][ks] = *(const bf16x8 LDS_AS*)((const char LDS_AS*)(((uintptr_t)(st + qk_lat)) ^ (64 * ks)) +
                                            mb * 16 * C::ROWB);
      A[mb][C::KL] = *(const bf16x8 LDS_AS*)(st + qk_rp + mb * 2048);
      A[mb][C::KL + 1] =
          *(const bf16x8 LDS_AS*)((const char LDS_AS*)(((uintptr_t)(st + qk_rp)) ^ 64) + mb * 2048);
    }
    bf16x8 V[C::CB];
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb) {
      const char LDS_AS* a = (const char LDS_AS*)(((uintptr_t)(st + pv_lat)) ^ (32 * cb));
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)a);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)(a + 16 * C::ROWB));
      const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      V[cb] = __builtin_bit_cast(bf16x8, v);
    }

    // S^T = K Q^T, starting from the causal mask on the diagonal tile: key
    // row 16 mb + 4 kg + e of the tile against query column 16 nb + l16
    f32x4 S[2][C::NBLK];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < C::NBLK; ++nb) {
        f32x4 init = {0.f, 0.f, 0.f, 0.f};
        if (it == last) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            init[e] = 16 * mb + 4 * kg + e > 16 * nb + l16 ? -INFINITY : 0.f;
        }
        S[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mb][0], q[0][nb], init, 0, 0, 0);
#pragma unroll
        for (int ks = 1; ks < C::KS; ++ks)
          S[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[mb][ks], q[ks][nb], S[mb][nb], 0, 0, 0);
      }

    // online softmax per query (lane), lazily rescaled as in the decode: P
    // against the running reference, the exact tile max only when a lane's
    // sum of P passes 2^20 or is infinite (no reference yet)
    bf16x8 P[C::NBLK];
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
          P[nb][4 * mb + e] = (__bf16)pe;
        }
    };
#pragma unroll
    for (int nb = 0; nb < C::NBLK; ++nb) {
      probs(nb);
      need |= !(ps[nb] <= kSumLimit);
    }
    if (__builtin_expect(__any(need), 0)) {
#pragma unroll
      for (int nb = 0; nb < C::NBLK; ++nb) {
        const float mx = fmaxf(fmaxf(fmaxf(S[0][nb][0], S[0][nb][1]), fmaxf(S[0][nb][2], S[0][nb][3])),
                               fmaxf(fmaxf(S[1][nb][0], S[1][nb][1]), fmaxf(S[1][nb][2], S[1][nb][3])));
        const float mt = max4(mx) * kLog2e;
        const float mr = m_run[nb] == kNoRef ? mt : m_run[nb];
        const float mn = fmaxf(mr, mt - kRescale);
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

#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb)
#pragma unroll
      for (int nb = 0; nb < C::NBLK; ++nb)
        o[cb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(V[cb], P[nb], o[cb][nb], 0, 0, 0);
  }

  // normalised branch latent of each query; positions past the sequence: 0
#pragma unroll
  for (int nb = 0; nb < C::NBLK; ++nb) {
    const int t = q0 + 16 * nb + l16;
    const float lt = sum4(l_run[nb]);
    if (t >= p.T) continue;
    const float inv = t < L ? 1.f / lt : 0.f;
    float* dst = p.latent + (((int64_t)b * p.T + t) * p.H + h) * DC + kBW * j + 4 * kg;
#pragma unroll
    for (int cb = 0; cb < C::CB; ++cb) *(f32x4*)(dst + 16 * cb) = o[cb][nb] * inv;
  }
}

__global__ void fill_positions(int32_t* pos, int B, int T) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < (int64_t)B * T) pos[i] = (int32_t)(i % T);
}

}  // namespace

hipError_t launch_fill_positions(int32_t* pos, int B, int T, hipStream_t s) {
  const int64_t n = (int64_t)B * T;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_positions, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, pos, B, T);
  return hipGetLastError();
}

bool prefill_branch_supported(const Geom& g) {
  return g.dr == kDR && g.dc == 4 * kBW && g.n == 4;
}

hipError_t launch_prefill_branch(const Geom& g, int T, const void* q_abs, const void* ckv,
                                 const void* krope, const int32_t* lens, float* latent,
                                 hipStream_t s) {
  if (!prefill_branch_supported(g)) return hipErrorNotSupported;
  if (g.B <= 0 || T <= 0) return hipSuccess;
  using C = BCfg<4, 2, kQW, 4>;
  constexpr int NS = (160 * 1024) / C::STAGE < 7 ? (160 * 1024) / C::STAGE : 7;
  PrefillParams p;
  p.q_abs = (const __bf16*)q_abs;
  p.ckv = (const __bf16*)ckv;
  p.krope = (const __bf16*)krope;
  p.ckv_bs = g.ckv_bs;
  p.ckv_ts = (int)g.ckv_ts;
  p.kr_bs = g.kr_bs;
  p.kr_ts = (int)g.kr_ts;
  p.lens = lens;
  p.latent = latent;
  p.B = g.B;
  p.T = T;
  p.H = g.H;
  p.QB = (T + kQWG - 1) / kQWG;
  const int64_t grid = (int64_t)g.B * p.QB * g.H * 2;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((prefill_branch_kernel<NS>), dim3((unsigned)grid), dim3(64 * C::NW), 0, s, p);
  return hipGetLastError();
}

}  // namespace mlra
