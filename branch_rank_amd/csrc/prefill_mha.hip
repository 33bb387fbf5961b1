// Causal prefill of MLA in the unabsorbed (MHA) form, gfx950 (MI355X).
//
// What it computes ("vllbc02MLA", 苏神思路: the prefill is compute-bound and
// runs as ordinary multi-head attention on keys and values up-projected from
// the latent, while decode uses the absorbed form; "MLA多头潜在注意力机制"
// 3.2-3.3: K^N = C W_UK, V = C W_UV per head, the RoPE key shared by all
// heads, a key after the query's position masked out): for every position
// t < L_b of sequence b and head h,
//   s_u   = tau (alpha_q q^N_t . K^N_u + RoPE(q^R_t, t) . k^R_u),  u <= t,
//   o_t,h = alpha_kv sum_u softmax_u(s) V_u,
// and zeros for L_b <= t < T. This is MLA's (one branch's) decode output for
// the cache cut after row t, in the form whose multiply-adds per query and
// key are 192 + 128 instead of the absorbed form's 576 + 512.
//
// Two kernels on the caller's workspace:
//  * kv_up: K^N and V of every head and cached position, a GEMM per head
//    ([positions x 512] x [512 x 256], W_UK and W_UV side by side) on
//    v_mfma_f32_16x16x32_bf16. A workgroup takes 64 positions of one
//    sequence and one head: the 64 latent rows (64 KB) and W's k-steps (32
//    rows of W_UK and W_UV, 16 KB, a ring of four) arrive in LDS by LDS-DMA;
//    W is read transposed (ds_read_b64_tr_b16) as the A operand, so the
//    products come out as [outputs][positions] and every lane stores 4
//    consecutive outputs of one position. K^N is stored pre-scaled by
//    alpha_q tau log2(e) (scores then come out in log2 units) and both as
//    fp16 (2^-11 relative): rounded to bf16, K^N alone moves MLA's output rows
//    by ~1.7e-2 at the pages' scales. The head-0 workgroups also store k^R as
//    fp16.
//  * attn: causal flash attention per (sequence, head, 128 positions), four
//    waves of 32 positions. The keys' rows [K^N || k^R] and values V stream
//    through a ring of four 20 KB LDS stages (32 keys each); S^T = K Q^T and
//    O^T += V^T P^T on v_mfma_f32_16x16x32_f16 with the query and P in the
//    lanes (as the decode kernels), a lazily rescaled online softmax (P kept
//    <= 2^15 for fp16) and the causal mask as the accumulators' start on a
//    wave's diagonal tile.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>

#include "device_common.h"

namespace mlra {
namespace {

using namespace dev;

typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4;

constexpr int kDC = 512, kDN = 128, kDV = 128, kDR = 64;

// ------------------------------------------------------------------ kv_up ----

constexpr int kUT = 64;                // positions per workgroup
constexpr int kUStage = 2 * 32 * 256;  // W_UK and W_UV rows of one k-step (16 KB)
constexpr int kUNS = 4;                // W stages
constexpr int kUC = kUT * kDC * 2;     // latent rows (64 KB)
constexpr int kUKS = kDC / 32;         // k-steps

struct UpParams {
  const __bf16* ckv;    // cache rows, element strides
  const __bf16* krope;
  int64_t ckv_bs, kr_bs;
  int ckv_ts, kr_ts;
  const int32_t* lens;
  const __bf16* w_uk;   // [H][d_c][d_n]
  const __bf16* w_uv;   // [H][d_c][d_v]
  _Float16* kn;         // [B][H][T][d_n]
  _Float16* v;          // [B][H][T][d_v]
  _Float16* kr;         // [B][T][d_r]
  int B, H, T, QB;      // QB: 64-position blocks per sequence
  float kscale;         // alpha_q tau log2(e)
};

// 256-byte rows of a W part: 16-byte chunk c of row t at c ^ 2 (t & 7)
__device__ __forceinline__ int swz_w(int t) { return 2 * (t & 7); }
// 1 KB latent rows: chunk c of row t at c ^ 2 (t & 15)
__device__ __forceinline__ int swz_c(int t) { return 2 * (t & 15); }

__global__ __launch_bounds__(256, 1) void kv_up_kernel(UpParams p) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[kUC + kUNS * kUStage];
  char LDS_AS* smem = (char LDS_AS*)smem_raw;
  char LDS_AS* wring = smem + kUC;
  const uint32_t sbase = (uint32_t)(uintptr_t)smem;
  // workgroup -> (head, sequence, block): the blocks of one head are adjacent
  // so that W_UK[h], W_UV[h] (256 KB) are read from L2 after the first
  int i = blockIdx.x;
  const int h = i / (p.B * p.QB);
  i %= p.B * p.QB;
  const int b = i / p.QB, tb = i % p.QB;
  const int t0 = tb * kUT;
  const int L = min(max(p.lens[b], 0), p.T);
  if (t0 >= L) return;  // no cached row in this block
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, kg = lane >> 4;

  // latent rows t0 .. t0 + 63 (clamped to L - 1): wave w loads rows
  // w + 4 u (u < 16), lane l: LDS chunk l, global chunk l ^ swz_c(row)
  const i32x4 crs = seq_rsrc(p.ckv + (int64_t)b * p.ckv_bs, L, p.ckv_ts);
#pragma unroll
  for (int u = 0; u < kUT / 4; ++u) {
    const int r = wave + 4 * u;
    const int row = min(t0 + r, L - 1);
    dma16(crs, sbase + r * 1024, (uint32_t)(row * p.ckv_ts * 2 + 16 * (lane ^ swz_c(r))), 0u);
  }
  // W k-step ks: rows 32 ks .. + 31 of W_UK[h] (LDS part 0) and W_UV[h]
  // (part 1), 256 bytes each; wave w loads instructions w and w + 4 of each
  // part (4 rows each: lane l LDS row 4 q + l / 16, LDS chunk l % 16, global
  // chunk (l % 16) ^ swz_w(row)). The transposed read gives the lanes of
  // k-group kg the LDS rows 4 kg .. 4 kg + 3 and 16 + 4 kg .. 16 + 4 kg + 3,
  // while the latent operand holds k = 8 kg .. 8 kg + 7 in each lane: so LDS
  // row r holds W row 32 ks + 8 ((r % 16) / 4) + r % 4 + 4 (r / 16).
  const __bf16* wk = p.w_uk + (int64_t)h * kDC * kDN;
  const __bf16* wv = p.w_uv + (int64_t)h * kDC * kDV;
  const i32x4 krs_w = seq_rsrc(wk, kDC, kDN);
  const i32x4 vrs_w = seq_rsrc(wv, kDC, kDV);
  auto issue_w = [&](int ks) {
    const uint32_t sa = sbase + kUC + (ks & (kUNS - 1)) * kUStage;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int q = wave + 4 * u;
      const int row = 4 * q + (lane >> 4);
      const int k = 8 * ((row & 15) >> 2) + (row & 3) + 4 * (row >> 4);
      const uint32_t off = (uint32_t)((32 * ks + k) * 256 + 16 * ((lane & 15) ^ swz_w(row)));
      dma16(krs_w, sa + q * 1024, off, 0u);
      dma16(vrs_w, sa + 8192 + q * 1024, off, 0u);
    }
  };
#pragma unroll
  for (int s = 0; s < kUNS - 1; ++s) issue_w(s);

  // k^R of the block's rows as fp16, once (head 0)
  if (h == 0) {
    for (int e = threadIdx.x; e < kUT * (kDR / 8); e += 256) {
      const int r = e / (kDR / 8), c8 = e % (kDR / 8), t = t0 + r;
      if (t >= L) continue;
      const bf16x8 x = *(const bf16x8*)(p.krope + (int64_t)b * p.kr_bs + (int64_t)t * p.kr_ts + 8 * c8);
      f16x8 y;
#pragma unroll
      for (int k = 0; k < 8; ++k) y[k] = (_Float16)(float)x[k];
      *(f16x8*)(p.kr + ((int64_t)b * p.T + t) * kDR + 8 * c8) = y;
    }
  }

  // wave w: outputs [64 w, 64 w + 64) (waves 0-1: K^N, 2-3: V), 4 blocks of
  // 16, for the 4 blocks of 16 positions
  const int part = wave >> 1;
  const int cb0 = 4 * (wave & 1);  // first 16-column block within the part
  const int pv_t = 4 * kg + (l16 >> 2), half = l16 & 3;
  const int pv = part * 8192 + pv_t * 256 + 16 * ((half >> 1) ^ swz_w(pv_t)) + 8 * (half & 1);
  const int cb_base = l16 * 1024 + 16 * (kg ^ swz_c(l16));
  f32x4 acc[4][4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[c][n] = (f32x4){0.f, 0.f, 0.f, 0.f};

  for (int ks = 0; ks < kUKS; ++ks) {
    // this wave's latent rows and its loads of W k-step ks have landed (4
    // loads per later k-step in flight)
    const int ahead = min(kUNS - 2, kUKS - 1 - ks);
    if (ahead >= 2) wait_vm<8>(); else if (ahead == 1) wait_vm<4>(); else wait_vm<0>();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    // the stage of k-step ks + 3 last held ks - 1, finished before the barrier
    if (ks + kUNS - 1 < kUKS) issue_w(ks + kUNS - 1);
    const char LDS_AS* st = wring + (ks & (kUNS - 1)) * kUStage;
    bf16x8 A[4], Bq[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const char LDS_AS* a = (const char LDS_AS*)(((uintptr_t)(st + pv)) ^ (32 * (cb0 + c)));
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)a);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)(a + 16 * 256));
      const i16x8 vv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      A[c] = __builtin_bit_cast(bf16x8, vv);
    }
#pragma unroll
    for (int n = 0; n < 4; ++n)
      Bq[n] = *(const bf16x8 LDS_AS*)((const char LDS_AS*)(((uintptr_t)(smem + cb_base +
                                                                        n * 16 * 1024)) ^
                                                           (64 * ks)));
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int n = 0; n < 4; ++n)
        acc[c][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[c], Bq[n], acc[c][n], 0, 0, 0);
  }

  // lane (position 16 n + l16, kg) holds outputs 16 (cb0 + c) + 4 kg .. + 3
  _Float16* dst = part == 0 ? p.kn : p.v;
  const float sc = part == 0 ? p.kscale : 1.f;
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int t = t0 + 16 * n + l16;
    if (t >= L) continue;
    _Float16* row = dst + (((int64_t)b * p.H + h) * p.T + t) * 128;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const f16x4 y = {(_Float16)(sc * acc[c][n][0]), (_Float16)(sc * acc[c][n][1]),
                       (_Float16)(sc * acc[c][n][2]), (_Float16)(sc * acc[c][n][3])};
      *(f16x4*)(row + 16 * (cb0 + c) + 4 * kg) = y;
    }
  }
}

// ------------------------------------------------------------------- attn ----

constexpr int kT = 32;               // keys per tile
constexpr int kQW = 32;              // positions per wave
constexpr int kAW = 4;               // waves
constexpr int kQB = kQW * kAW;       // positions per workgroup
constexpr int kAKN = 0, kAKR = 32 * 256, kAV = kAKR + 32 * 128;
constexpr int kAStage = kAV + 32 * 256;  // 20 KB
constexpr int kANS = 4;
constexpr float kRescale = 12.f;     // log2 headroom kept when the reference moves
constexpr float kSumLimit = 32768.f; // per-lane P sum that moves it: every p stays <= 2^15

struct AttnParams {
  const _Float16* kn;   // [B][H][T][d_n], pre-scaled
  const _Float16* v;    // [B][H][T][d_v]
  const _Float16* kr;   // [B][T][d_r]
  const __bf16* q_nope; // [B][T][H][d_n]
  const __bf16* q_rope; // [B][T][H][d_r]
  const int32_t* lens;
  void* out;            // [B][T][H][d_v]
  int B, H, T, QB, grid;
  float rscale;         // tau log2(e), applied to the rotated q^R
  float alpha_kv;
  double omega[kDR / 2];
};

__device__ __forceinline__ int swz_kn(int t) { return t & 15; }
__device__ __forceinline__ int swz_r(int t) { return (t >> 1) & 7; }
__device__ __forceinline__ int swz_v(int t) { return 2 * (t & 7); }

__device__ __forceinline__ void store4(float* p, f32x4 v) { *(f32x4*)p = v; }
__device__ __forceinline__ void store4(__bf16* p, f32x4 v) {
  typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
  *(bf16x4*)p = (bf16x4){(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
}

template <typename TO>
__global__ __launch_bounds__(256, 2) void mha_attn_kernel(AttnParams p) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[kANS * kAStage];
  char LDS_AS* smem = (char LDS_AS*)smem_raw;
  const uint32_t sbase = (uint32_t)(uintptr_t)smem;
  // workgroup -> (sequence, head, block): each XCD (launch order modulo 8)
  // takes a contiguous range, so the blocks of one (sequence, head) share its
  // L2; the last (longest) blocks of a head first
  const int per = p.grid / 8;
  const int j = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (j >= p.B * p.H * p.QB) return;
  const int bh = j / p.QB, qb = p.QB - 1 - j % p.QB;
  const int b = bh / p.H, h = bh % p.H;
  const int T = p.T;
  const int L = min(max(p.lens[b], 0), T);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, kg = lane >> 4;
  const int q0 = qb * kQB + wave * kQW;
  const int64_t orow = (int64_t)p.H * kDV;
  TO* out_bh = (TO*)p.out + ((int64_t)b * T * p.H + h) * kDV;

  if (qb * kQB >= L) {  // every position of the block lies past the sequence
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int t = q0 + 16 * nb + l16;
      if (t >= T) continue;
#pragma unroll
      for (int cb = 0; cb < kDV / 16; ++cb)
        store4(out_bh + t * orow + 16 * cb + 4 * kg, (f32x4){0.f, 0.f, 0.f, 0.f});
    }
    return;
  }

  const int kend = min(L, qb * kQB + kQB);  // keys of this block: [0, kend)
  const int ntiles = (kend + kT - 1) / kT;
  const int64_t hrow = ((int64_t)b * p.H + h) * T;  // row of (b, h, 0)
  const i32x4 knrs = seq_rsrc_bytes(p.kn + hrow * kDN, kend, kDN * 2);
  const i32x4 vrs = seq_rsrc_bytes(p.v + hrow * kDV, kend, kDV * 2);
  const i32x4 krrs = seq_rsrc_bytes(p.kr + (int64_t)b * T * kDR, kend, kDR * 2);
  // wave w loads K^N and V instructions w, w + 4 (rows 4 q + l / 16, LDS
  // chunk l % 16) and RoPE instruction w (rows 8 w + l / 8, chunk l % 8);
  // rows past the block's keys repeat its last key
  int dma_off = 0;
  auto issue = [&](int tile) {
    const uint32_t sa = sbase + dma_off;
    dma_off = dma_off + kAStage == kANS * kAStage ? 0 : dma_off + kAStage;
    const int ts0 = tile * kT;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int q = wave + 4 * u;
      const int r = 4 * q + (lane >> 4), row = min(ts0 + r, kend - 1);
      dma16(knrs, sa + kAKN + q * 1024, (uint32_t)(row * 256 + 16 * ((lane & 15) ^ swz_kn(r))), 0u);
      dma16(vrs, sa + kAV + q * 1024, (uint32_t)(row * 256 + 16 * ((lane & 15) ^ swz_v(r))), 0u);
    }
    const int r = 8 * wave + (lane >> 3), row = min(ts0 + r, kend - 1);
    dma16(krrs, sa + kAKR + wave * 1024, (uint32_t)(row * 128 + 16 * ((lane & 7) ^ swz_r(r))), 0u);
  };
#pragma unroll
  for (int s = 0; s < kANS - 1; ++s)
    if (s < ntiles) issue(s);

  // queries (B operand, lane (position 16 nb + l16, kg) holds k 32 ks + 8 kg
  // .. + 7): q^N as fp16 (bf16 values fit it), then tau log2(e) RoPE(q^R, t)
  // as fp16, the angle t omega_k and its reduction to [-pi, pi] in double,
  // the sine and cosine of the reduced angle in float
  f16x8 q[6][2];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int t = min(q0 + 16 * nb + l16, T - 1);
    const __bf16* qn = p.q_nope + (((int64_t)b * T + t) * p.H + h) * kDN;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const bf16x8 x = *(const bf16x8*)(qn + 32 * ks + 8 * kg);
#pragma unroll
      for (int e = 0; e < 8; ++e) q[ks][nb][e] = (_Float16)(float)x[e];
    }
    const __bf16* qr = p.q_rope + (((int64_t)b * T + t) * p.H + h) * kDR;
#pragma unroll
    for (int kr = 0; kr < 2; ++kr) {
      const bf16x8 x = *(const bf16x8*)(qr + 32 * kr + 8 * kg);
#pragma unroll
      for (int pr = 0; pr < 4; ++pr) {
        const int k = 16 * kr + 4 * kg + pr;  // pair index: elements 2k, 2k + 1
        const double a = (double)t * p.omega[k];
        const double rr = a - 6.283185307179586 * rint(a * 0.15915494309189535);
        float sn, cs;
        sincosf((float)rr, &sn, &cs);
        const float x0 = (float)x[2 * pr], x1 = (float)x[2 * pr + 1];
        q[4 + kr][nb][2 * pr] = (_Float16)(p.rscale * (x0 * cs - x1 * sn));
        q[4 + kr][nb][2 * pr + 1] = (_Float16)(p.rscale * (x0 * sn + x1 * cs));
      }
    }
  }

  // per-lane LDS offsets within a stage (keys l16 and l16 + 16 of the tile)
  const int qk_n = kAKN + l16 * 256 + 16 * (kg ^ swz_kn(l16));  // k-step ks: ^ 64 ks
  const int qk_r = kAKR + l16 * 128 + 16 * (kg ^ swz_r(l16));   // second: ^ 64
  const int pv_t = 4 * kg + (l16 >> 2), half = l16 & 3;
  const int pv = kAV + pv_t * 256 + 16 * ((half >> 1) ^ swz_v(pv_t)) + 8 * (half & 1);

  f32x4 o[8][2];
#pragma unroll
  for (int cb = 0; cb < 8; ++cb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) o[cb][nb] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {0.f, 0.f}, l_run[2] = {0.f, 0.f};
  const int last = q0 < L ? q0 / kT : -1;  // this wave's diagonal tile

  int cur_off = 0;
  for (int it = 0; it < ntiles; ++it) {
    // this wave's 5 loads of tile `it` have landed (later tiles may be in
    // flight)
    {
      const int ahead = min(kANS - 2, ntiles - 1 - it);
      if (ahead >= 2) wait_vm<10>(); else if (ahead == 1) wait_vm<5>(); else wait_vm<0>();
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    // the stage of tile it + 3 last held tile it - 1, finished before the barrier
    if (it + kANS - 1 < ntiles) issue(it + kANS - 1);
    const char LDS_AS* st = smem + __builtin_amdgcn_readfirstlane(cur_off);
    cur_off = cur_off + kAStage == kANS * kAStage ? 0 : cur_off + kAStage;
    if (it > last) continue;  // keys after every position of this wave

    f16x8 A[2][6];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        A[mb][ks] = *(const f16x8 LDS_AS*)((const char LDS_AS*)(((uintptr_t)(st + qk_n +
                                                                             mb * 16 * 256)) ^
                                                                (64 * ks)));
      A[mb][4] = *(const f16x8 LDS_AS*)(st + qk_r + mb * 2048);
      A[mb][5] = *(const f16x8 LDS_AS*)((const char LDS_AS*)(((uintptr_t)(st + qk_r + mb * 2048)) ^ 64));
    }
    f16x8 V[8];
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
      const char LDS_AS* a = (const char LDS_AS*)(((uintptr_t)(st + pv)) ^ (32 * cb));
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)a);
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)(a + 16 * 256));
      const i16x8 vv = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      V[cb] = __builtin_bit_cast(f16x8, vv);
    }

    // S^T - m_run in log2 units, the accumulators starting at -m_run of their
    // position, or at -inf where the diagonal tile's mask hides key row
    // 16 mb + 4 kg + e from position 16 nb + l16
    f32x4 S[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        S[mb][nb] = (f32x4){-m_run[nb], -m_run[nb], -m_run[nb], -m_run[nb]};
        if (it == last) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (16 * mb + 4 * kg + e > 16 * nb + l16) S[mb][nb][e] = -INFINITY;
        }
      }
#pragma unroll
    for (int ks = 0; ks < 6; ++ks)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
          S[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[mb][ks], q[ks][nb], S[mb][nb], 0, 0, 0);

    // online softmax per position (lane), lazily rescaled: p = 2^(S - m_run);
    // the exact tile max on the first tile or when a lane's sum of P passes
    // 2^15 (or is not finite), then the reference moves to 12 below the max
    // and O, l are rescaled, so every p stays <= 2^15 (fp16)
    f16x8 P[2];
    float ps[2];
    bool need = it == 0;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      ps[nb] = 0.f;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pe = __builtin_amdgcn_exp2f(S[mb][nb][e]);
          ps[nb] += pe;
          P[nb][4 * mb + e] = (_Float16)pe;
        }
      need |= !(ps[nb] <= kSumLimit);
    }
    if (__builtin_expect(__any(need), 0)) {
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const float mx = fmaxf(fmaxf(fmaxf(S[0][nb][0], S[0][nb][1]), fmaxf(S[0][nb][2], S[0][nb][3])),
                               fmaxf(fmaxf(S[1][nb][0], S[1][nb][1]), fmaxf(S[1][nb][2], S[1][nb][3])));
        const float mt = max4(mx) + m_run[nb];  // the tile max, log2 units
        const float mr = it == 0 ? mt : m_run[nb];
        const float mn = fmaxf(mr, mt - kRescale);
        const float f = __builtin_amdgcn_exp2f(mr - mn);
        l_run[nb] *= f;
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) o[cb][nb] *= f;
        const float off = m_run[nb] - mn;
        m_run[nb] = mn;
        ps[nb] = 0.f;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float pe = __builtin_amdgcn_exp2f(S[mb][nb][e] + off);
            ps[nb] += pe;
            P[nb][4 * mb + e] = (_Float16)pe;
          }
      }
    }
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) l_run[nb] += ps[nb];
#pragma unroll
    for (int cb = 0; cb < 8; ++cb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        o[cb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(V[cb], P[nb], o[cb][nb], 0, 0, 0);
  }

  // o = alpha_kv O / l per position (lane (position, kg) holds value columns
  // 16 cb + 4 kg .. + 3); positions past the sequence get zeros
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const float lt = sum4(l_run[nb]);
    const int t = q0 + 16 * nb + l16;
    const float sc = t < L && lt > 0.f ? p.alpha_kv / lt : 0.f;
    if (t >= T) continue;
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) store4(out_bh + t * orow + 16 * cb + 4 * kg, sc * o[cb][nb]);
  }
}

}  // namespace

bool prefill_mha_supported(const Geom& g) {
  return g.dc == kDC && g.dr == kDR && g.dn == kDN && g.dv == kDV && g.n == 1;
}

size_t prefill_mha_workspace(const Geom& g, int T) {
  return (size_t)g.B * g.H * T * (kDN + kDV) * 2 + (size_t)g.B * T * kDR * 2;
}

hipError_t launch_prefill_mha(const Geom& g, int T, const void* q_nope, const void* q_rope,
                              const void* w_uk, const void* w_uv, const void* ckv,
                              const void* krope, const int32_t* lens, void* workspace, void* out,
                              bool out_bf16, float tau, float alpha_q, float alpha_kv,
                              float theta, hipStream_t s, const KernelTiming& t) {
  if (!prefill_mha_supported(g)) return hipErrorNotSupported;
  if (g.B <= 0 || T <= 0) return hipSuccess;
  _Float16* kn = static_cast<_Float16*>(workspace);
  _Float16* v = kn + (size_t)g.B * g.H * T * kDN;
  _Float16* kr = v + (size_t)g.B * g.H * T * kDV;
  UpParams u;
  u.ckv = (const __bf16*)ckv;
  u.krope = (const __bf16*)krope;
  u.ckv_bs = g.ckv_bs;
  u.ckv_ts = (int)g.ckv_ts;
  u.kr_bs = g.kr_bs;
  u.kr_ts = (int)g.kr_ts;
  u.lens = lens;
  u.w_uk = (const __bf16*)w_uk;
  u.w_uv = (const __bf16*)w_uv;
  u.kn = kn;
  u.v = v;
  u.kr = kr;
  u.B = g.B;
  u.H = g.H;
  u.T = T;
  u.QB = (T + kUT - 1) / kUT;
  u.kscale = alpha_q * tau * dev::kLog2e;
  hipLaunchKernelGGL(kv_up_kernel, dim3(g.H * g.B * u.QB), dim3(256), 0, s, u);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  AttnParams a;
  a.kn = kn;
  a.v = v;
  a.kr = kr;
  a.q_nope = (const __bf16*)q_nope;
  a.q_rope = (const __bf16*)q_rope;
  a.lens = lens;
  a.out = out;
  a.B = g.B;
  a.H = g.H;
  a.T = T;
  a.QB = (T + kQB - 1) / kQB;
  a.grid = ((g.B * g.H * a.QB + 7) / 8) * 8;
  a.rscale = tau * dev::kLog2e;
  a.alpha_kv = alpha_kv;
  const RopeFreqs& fr = rope_freqs(theta, g.dr);
  for (int k = 0; k < kDR / 2; ++k) a.omega[k] = fr.w[k];
  if (out_bf16)
    hipExtLaunchKernelGGL(mha_attn_kernel<__bf16>, dim3(a.grid), dim3(256), 0, s, t.start, t.stop,
                          0, a);
  else
    hipExtLaunchKernelGGL(mha_attn_kernel<float>, dim3(a.grid), dim3(256), 0, s, t.start, t.stop,
                          0, a);
  return hipGetLastError();
}

}  // namespace mlra
