// Portable kernels: split-KV planning, the partial-softmax combine, and VALU
// versions of query absorption, latent decode and output projection for any
// head count and width, in fp32 or bf16 storage with fp32 arithmetic.
//
// The method (pages cited by title and section):
//   absorb_q  - "Multi-Head Low-Rank Attention", 方法步骤详情 step 1: W_UK is
//               folded into the query; RoPE on the query's rotary part
//               ("从MHA到MLA" 3.2).
//   decode    - 方法步骤详情 step 2: MQA-style attention over [C_KV || K_RoPE]
//               in latent space, one softmax per branch (核心方法).
//   out_proj  - 方法步骤详情 step 3 plus the branch sum of 核心方法.
// The split-KV merge is the standard online-softmax rescaling.

#include <float.h>
#include <hip/hip_ext.h>
#include <math.h>

#include "device_common.h"  // MLRA_DCHECK
#include "internal.h"
#include "plan_device.h"

namespace mlra {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }
// an fp8 cache entry: the E4M3 code's value (exact in fp32)
__device__ __forceinline__ float to_f32(uint8_t x) { return __builtin_amdgcn_cvt_f32_fp8((int)x, 0); }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

__device__ __forceinline__ int clamp_len(int v, int max_len) {
  return v < 0 ? 0 : (v > max_len ? max_len : v);
}

// Block-wide reductions for blockDim.x == 256 (4 waves of 64).
__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ float block_max256(float v, float* red) {
  v = wave_max(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return r;
}
__device__ float block_sum256(float v, float* red) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------- plan ----

__global__ __launch_bounds__(1024) void plan_kernel(PlanArgs a) { plan_block(a); }

// -------------------------------------------------------------- absorb_q ----

constexpr int kQB = 16;  // sequences per absorb / out-proj block

template <typename T>
__global__ __launch_bounds__(256) void absorb_q_generic(Geom g, const T* __restrict__ q_nope,
                                                        const T* __restrict__ q_rope,
                                                        const int32_t* __restrict__ q_pos,
                                                        const int32_t* __restrict__ lens,
                                                        const T* __restrict__ w_uk,
                                                        T* __restrict__ q_abs, int row,
                                                        int lo_off, float lat_scale,
                                                        float rope_scale, RopeFreqs fr) {
  extern __shared__ float sq[];  // [kQB][dn]
  const int h = blockIdx.x, b0 = blockIdx.y * kQB;
  const int nb = min(kQB, g.B - b0);
  for (int i = threadIdx.x; i < nb * g.dn; i += blockDim.x) {
    const int bb = i / g.dn, e = i % g.dn;
    sq[bb * g.dn + e] = to_f32(q_nope[((size_t)(b0 + bb) * g.H + h) * g.dn + e]);
  }
  __syncthreads();
  const float s = lat_scale;
  const double tau = rope_scale;
  const T* w = w_uk + (size_t)h * g.dc * g.dn;
  for (int c = threadIdx.x; c < g.dc; c += blockDim.x) {
    float acc[kQB];
#pragma unroll
    for (int bb = 0; bb < kQB; ++bb) acc[bb] = 0.f;
    for (int e = 0; e < g.dn; ++e) {
      const float wv = to_f32(w[(size_t)c * g.dn + e]);
#pragma unroll
      for (int bb = 0; bb < kQB; ++bb)
        if (bb < nb) acc[bb] += wv * sq[bb * g.dn + e];
    }
    for (int bb = 0; bb < nb; ++bb) {
      // q~ in the storage type and, when asked for, its rounding residue
      const float v = s * acc[bb];
      const T hi = from_f32<T>(v);
      T* qr = q_abs + ((size_t)(b0 + bb) * g.H + h) * row;
      qr[c] = hi;
      if (lo_off > 0) qr[lo_off + c] = from_f32<T>(v - to_f32(hi));
    }
  }
  // RoPE on the query's rotary part, angle in double precision (frequency
  // from the host's table).
  const int half = g.dr / 2;
  for (int i = threadIdx.x; i < nb * half; i += blockDim.x) {
    const int bb = i / half, k = i % half, b = b0 + bb;
    const int p = q_pos ? q_pos[b] : clamp_len(lens[b], g.max_len) - 1;
    double sn, cs;
    sincos((double)p * fr.w[k], &sn, &cs);
    const size_t qi = ((size_t)b * g.H + h) * g.dr + 2 * k;
    const double x0 = to_f32(q_rope[qi]), x1 = to_f32(q_rope[qi + 1]);
    T* o = q_abs + ((size_t)b * g.H + h) * row + g.dc + 2 * k;
    o[0] = from_f32<T>((float)(tau * (x0 * cs - x1 * sn)));
    o[1] = from_f32<T>((float)(tau * (x0 * sn + x1 * cs)));
  }
}

// ---------------------------------------------------------------- decode ----

constexpr int kTok = 256;         // tokens per step of the generic decode
constexpr int kMaxColsPerThr = 4; // d_c <= 1024
constexpr int kMaxBranches = 8;

__device__ __forceinline__ int find_seq(const int32_t* prefix, int B, int pos) {
  // largest b with prefix[b] <= pos (prefix is non-decreasing, prefix[0] = 0)
  int lo = 0, hi = B;  // answer in [0, B)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid] <= pos) lo = mid; else hi = mid;
  }
  return lo;
}

template <typename T, typename TC>
__global__ __launch_bounds__(256) void decode_generic(Geom g, const T* __restrict__ q_abs,
                                                      int q_stride, int q_lo,
                                                      const TC* __restrict__ ckv,
                                                      const TC* __restrict__ krope,
                                                      Workspace ws) {
  extern __shared__ float smem[];
  const int row = g.dc + g.dr;
  float* q = smem;                 // [row]
  float* sc = smem + row;          // [n][kTok]
  __shared__ float red[4];
  const int k = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const PlanHeader hd = *ws.hdr;
  if (k >= hd.n_items) return;
  int start = k * hd.chunk;
  MLRA_DCHECK(ws.hdr, start >= 0 && start < hd.total, 4);
  const int end = min(start + hd.chunk, hd.total);
  int b = find_seq(ws.prefix, g.B, start);
  const int dcp = g.dc / g.n;
  while (start < end) {
    while (ws.prefix[b + 1] <= start) ++b;  // skip empty sequences
    const int seg_end = min(end, ws.prefix[b + 1]);
    const int t0 = start - ws.prefix[b], t1 = seg_end - ws.prefix[b];
    // the query in fp32: q~ (plus its bf16 residue when given) and rho
    const T* qr = q_abs + ((size_t)b * g.H + h) * q_stride;
    for (int i = tid; i < row; i += blockDim.x)
      q[i] = to_f32(qr[i]) + (q_lo > 0 && i < g.dc ? to_f32(qr[q_lo + i]) : 0.f);
    __syncthreads();
    float m[kMaxBranches], l[kMaxBranches], acc[kMaxColsPerThr];
    for (int j = 0; j < kMaxBranches; ++j) { m[j] = -INFINITY; l[j] = 0.f; }
    for (int i = 0; i < kMaxColsPerThr; ++i) acc[i] = 0.f;
    const TC* cb = ckv + (size_t)b * g.ckv_bs;
    const TC* kb = krope + (size_t)b * g.kr_bs;
    for (int tc = t0; tc < t1; tc += kTok) {
      const int nt = min(kTok, t1 - tc);
      if (tid < nt) {
        const TC* crow = cb + (size_t)(tc + tid) * g.ckv_ts;
        const TC* krow = kb + (size_t)(tc + tid) * g.kr_ts;
        float rs = 0.f;
        for (int r = 0; r < g.dr; ++r) rs += q[g.dc + r] * to_f32(krow[r]);
        for (int j = 0; j < g.n; ++j) {
          float s = rs;
          for (int c = j * dcp; c < (j + 1) * dcp; ++c) s += q[c] * to_f32(crow[c]);
          sc[j * kTok + tid] = s * kLog2e;
        }
      }
      __syncthreads();
      float scale[kMaxBranches];
      for (int j = 0; j < g.n; ++j) {
        const float mx = block_max256(tid < nt ? sc[j * kTok + tid] : -INFINITY, red);
        const float mn = fmaxf(m[j], mx);
        scale[j] = exp2f(m[j] - mn);
        const float p = tid < nt ? exp2f(sc[j * kTok + tid] - mn) : 0.f;
        const float ps = block_sum256(p, red);
        if (tid < nt) sc[j * kTok + tid] = p;
        l[j] = l[j] * scale[j] + ps;
        m[j] = mn;
      }
      __syncthreads();
      for (int i = 0; i < kMaxColsPerThr; ++i) {
        const int c = tid + i * 256;
        if (c < g.dc) {
          const int j = c / dcp;
          float a = acc[i] * scale[j];
          const float* pj = sc + j * kTok;
          for (int tt = 0; tt < nt; ++tt) a += pj[tt] * to_f32(cb[(size_t)(tc + tt) * g.ckv_ts + c]);
          acc[i] = a;
        }
      }
      __syncthreads();
    }
    const int slot = k + b;
    MLRA_DCHECK(ws.hdr, b >= 0 && b < g.B, 1);
    MLRA_DCHECK(ws.hdr, t0 >= 0 && t1 > t0 && t1 <= ws.prefix[b + 1] - ws.prefix[b], 2);
    MLRA_DCHECK(ws.hdr, slot >= 0 && slot < hd.n_items + g.B, 3);
    if (tid < g.n) {
      ws.m[((size_t)slot * g.n + tid) * g.H + h] = m[tid];
      ws.l[((size_t)slot * g.n + tid) * g.H + h] = l[tid];
    }
    for (int i = 0; i < kMaxColsPerThr; ++i) {
      const int c = tid + i * 256;
      if (c < g.dc) ws.acc[((size_t)slot * g.dc + c) * g.H + h] = acc[i];
    }
    start = seg_end;
    ++b;
    __syncthreads();
  }
}

// --------------------------------------------------------------- combine ----

constexpr int kCPairs = 16;  // (column, head) pairs per thread: 4096 per block
constexpr int kCSlots = 8;   // slots whose weights are staged at once

// Merge the partials of every work item of sequence b into
// latent_out[b][h][c] = sum_k 2^(m_k - M) acc_k / sum_k 2^(m_k - M) l_k,
// one softmax per branch (the branch of column c is c / (d_c / n)).
__global__ __launch_bounds__(256) void combine_kernel(Geom g, Workspace ws, int cb,
                                                      float* __restrict__ latent_out,
                                                      float out_scale) {
  extern __shared__ float sm[];
  const int H = g.H, n = g.n;
  float* Mx = sm;                       // [n][H]
  float* Li = Mx + n * H;               // [n][H] 1 / L
  float* W = Li + n * H;                // [kCSlots][n][H]
  float* tile = W + kCSlots * n * H;    // [cb][H + 1]
  const int b = blockIdx.x, c0 = blockIdx.y * cb, tid = threadIdx.x;
  const int nc = min(cb, g.dc - c0);
  const PlanHeader hd = *ws.hdr;
  const int p0 = ws.prefix[b], p1 = ws.prefix[b + 1];
  const int dcp = g.dc / n;
  if (p1 <= p0) {
    for (int i = tid; i < H * nc; i += 256) {
      const int hh = i / nc, cl = i % nc;
      latent_out[((size_t)b * H + hh) * g.dc + c0 + cl] = 0.f;
    }
    return;
  }
  const int kf = p0 / hd.chunk, kl = (p1 - 1) / hd.chunk;
  MLRA_DCHECK(ws.hdr, kf >= 0 && kf <= kl && kl < hd.n_items, 5);
  for (int i = tid; i < n * H; i += 256) {
    float M = -INFINITY;
    for (int k = kf; k <= kl; ++k) M = fmaxf(M, ws.m[(size_t)(k + b) * n * H + i]);
    float L = 0.f;
    for (int k = kf; k <= kl; ++k)
      L += exp2f(ws.m[(size_t)(k + b) * n * H + i] - M) * ws.l[(size_t)(k + b) * n * H + i];
    Mx[i] = M;
    Li[i] = 1.f / L;
  }
  float acc[kCPairs];
  const int npair = nc * H;  // <= 256 * kCPairs
#pragma unroll
  for (int i = 0; i < kCPairs; ++i) acc[i] = 0.f;
  for (int ks = kf; ks <= kl; ks += kCSlots) {
    const int kn = min(kCSlots, kl - ks + 1);
    __syncthreads();
    for (int i = tid; i < kn * n * H; i += 256) {
      const int kk = i / (n * H), jh = i % (n * H);
      W[i] = exp2f(ws.m[(size_t)(ks + kk + b) * n * H + jh] - Mx[jh]) * Li[jh];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kCPairs; ++i) {
      const int p = tid + i * 256;
      if (p < npair) {
        const int cl = p / H, hh = p % H, j = (c0 + cl) / dcp;
        float a = acc[i];
        for (int kk = 0; kk < kn; ++kk)
          a += W[(kk * n + j) * H + hh] *
               ws.acc[((size_t)(ks + kk + b) * g.dc + c0 + cl) * H + hh];
        acc[i] = a;
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kCPairs; ++i) {
    const int p = tid + i * 256;
    if (p < npair) tile[(p / H) * (H + 1) + p % H] = acc[i];
  }
  __syncthreads();
  for (int i = tid; i < H * nc; i += 256) {
    const int hh = i / nc, cl = i % nc;
    latent_out[((size_t)b * H + hh) * g.dc + c0 + cl] = out_scale * tile[cl * (H + 1) + hh];
  }
}

// ---------------------------------------------------------------- scale_q ----

// Query rows for an fp8 cache from the caller's bf16 rows: q~ (with its
// residue when the source has one) times lat_scale, rho times rope_scale, in
// fp32, then bf16 (plus the new residue when the destination keeps one).
// grid B * H rows, 256 threads.
__global__ __launch_bounds__(256) void scale_q_kernel(Geom g, const __bf16* __restrict__ src,
                                                      int s_stride, int s_lo,
                                                      __bf16* __restrict__ dst, int d_stride,
                                                      int d_lo, float lat_scale,
                                                      float rope_scale) {
  const int r = blockIdx.x;
  const __bf16* a = src + (size_t)r * s_stride;
  __bf16* o = dst + (size_t)r * d_stride;
  for (int i = threadIdx.x; i < g.dc + g.dr; i += blockDim.x) {
    if (i < g.dc) {
      const float v = lat_scale * ((float)a[i] + (s_lo > 0 ? (float)a[s_lo + i] : 0.f));
      const __bf16 hi = (__bf16)v;
      o[i] = hi;
      if (d_lo > 0) o[d_lo + i] = (__bf16)(v - (float)hi);
    } else {
      o[i] = (__bf16)(rope_scale * (float)a[i]);
    }
  }
}

// -------------------------------------------------------------- out_proj ----

template <typename T, typename TO>
__global__ __launch_bounds__(256) void out_proj_generic(Geom g, const float* __restrict__ latent,
                                                        const T* __restrict__ w_uv,
                                                        TO* __restrict__ out, float alpha_kv,
                                                        int qb) {
  extern __shared__ float sm[];  // [qb][dc] then [256][kQB] partial sums
  float* sl = sm;
  float* part = sm + qb * g.dc;
  const int h = blockIdx.x, b0 = blockIdx.y * qb, tid = threadIdx.x;
  const int nb = min(qb, g.B - b0);
  for (int i = tid; i < nb * g.dc; i += 256) {
    const int bb = i / g.dc, c = i % g.dc;
    sl[bb * g.dc + c] = latent[((size_t)(b0 + bb) * g.H + h) * g.dc + c];
  }
  __syncthreads();
  const T* w = w_uv + (size_t)h * g.dc * g.dv;
  const int vb = min(g.dv, 256);
  const int parts = 256 / vb;
  for (int v0 = 0; v0 < g.dv; v0 += vb) {
    const int v = v0 + tid % vb, cp = tid / vb;
    float acc[kQB];
#pragma unroll
    for (int bb = 0; bb < kQB; ++bb) acc[bb] = 0.f;
    if (cp < parts && v < g.dv) {
      for (int c = cp; c < g.dc; c += parts) {
        const float wv = to_f32(w[(size_t)c * g.dv + v]);
#pragma unroll
        for (int bb = 0; bb < kQB; ++bb)
          if (bb < nb) acc[bb] += wv * sl[bb * g.dc + c];
      }
    }
#pragma unroll
    for (int bb = 0; bb < kQB; ++bb) part[tid * kQB + bb] = acc[bb];
    __syncthreads();
    if (tid < vb && v0 + tid < g.dv) {
      for (int bb = 0; bb < nb; ++bb) {
        float s = 0.f;
        for (int q = 0; q < parts; ++q) s += part[(q * vb + tid) * kQB + bb];
        out[((size_t)(b0 + bb) * g.H + h) * g.dv + v0 + tid] = from_f32<TO>(alpha_kv * s);
      }
    }
    __syncthreads();
  }
}

}  // namespace

// -------------------------------------------------------------- launchers ----

hipError_t launch_plan(const int32_t* lens, int B, int max_len, int target_items,
                       int forced_chunk, const Workspace& ws, hipStream_t s) {
  PlanArgs a;
  a.lens = lens;
  a.B = B;
  a.max_len = max_len;
  a.target_items = target_items;
  a.forced_chunk = forced_chunk;
  a.hdr = ws.hdr;
  a.prefix = ws.prefix;
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(1024), 0, s, a);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_absorb_q_generic(const Geom& g, const T* q_nope, const T* q_rope,
                                   const int32_t* q_pos, const int32_t* lens, const T* w_uk,
                                   T* q_abs, int q_stride, int lo_off, float lat_scale,
                                   float rope_scale, float theta, hipStream_t s) {
  const size_t sh = sizeof(float) * kQB * g.dn;
  hipLaunchKernelGGL(absorb_q_generic<T>, dim3(g.H, (g.B + kQB - 1) / kQB), dim3(256), sh, s, g,
                     q_nope, q_rope, q_pos, lens, w_uk, q_abs, q_stride, lo_off, lat_scale,
                     rope_scale, rope_freqs(theta, g.dr));
  return hipGetLastError();
}

template <typename T, typename TC>
hipError_t launch_decode_generic(const Geom& g, const QView& q, const TC* ckv, const TC* krope,
                                 const Workspace& ws, int grid_items, hipStream_t s,
                                 const KernelTiming& t) {
  const size_t sh = sizeof(float) * (g.dc + g.dr + g.n * kTok);
  hipExtLaunchKernelGGL((decode_generic<T, TC>), dim3(grid_items, g.H), dim3(256), sh, s,
                        t.start, t.stop, 0, g, static_cast<const T*>(q.q), q.stride, q.lo, ckv,
                        krope, ws);
  return hipGetLastError();
}

hipError_t launch_scale_q(const Geom& g, const QView& src, const QView& dst, float lat_scale,
                          float rope_scale, hipStream_t s) {
  if (g.B * g.H == 0) return hipSuccess;
  hipLaunchKernelGGL(scale_q_kernel, dim3(g.B * g.H), dim3(256), 0, s, g,
                     static_cast<const __bf16*>(src.q), src.stride, src.lo,
                     static_cast<__bf16*>(const_cast<void*>(dst.q)), dst.stride, dst.lo,
                     lat_scale, rope_scale);
  return hipGetLastError();
}

hipError_t launch_combine(const Geom& g, const Workspace& ws, float* latent_out, float out_scale,
                          hipStream_t s) {
  int cb = (256 * kCPairs) / g.H;
  if (cb > g.dc) cb = g.dc;
  if (cb < 1) cb = 1;
  const size_t sh = sizeof(float) * (2 * g.n * g.H + kCSlots * g.n * g.H + cb * (g.H + 1));
  hipLaunchKernelGGL(combine_kernel, dim3(g.B, (g.dc + cb - 1) / cb), dim3(256), sh, s, g, ws,
                     cb, latent_out, out_scale);
  return hipGetLastError();
}

template <typename T, typename TO>
hipError_t launch_out_proj_generic(const Geom& g, const float* latent, const T* w_uv, TO* out,
                                   float alpha_kv, hipStream_t s) {
  int qb = 8192 / g.dc;  // keeps the staged latents within 32 KB
  if (qb > kQB) qb = kQB;
  if (qb < 1) qb = 1;
  const size_t sh = sizeof(float) * (qb * g.dc + 256 * kQB);
  hipLaunchKernelGGL((out_proj_generic<T, TO>), dim3(g.H, (g.B + qb - 1) / qb), dim3(256), sh,
                     s, g, latent, w_uv, out, alpha_kv, qb);
  return hipGetLastError();
}

template hipError_t launch_absorb_q_generic<float>(const Geom&, const float*, const float*,
                                                   const int32_t*, const int32_t*, const float*,
                                                   float*, int, int, float, float, float,
                                                   hipStream_t);
template hipError_t launch_absorb_q_generic<__bf16>(const Geom&, const __bf16*, const __bf16*,
                                                    const int32_t*, const int32_t*,
                                                    const __bf16*, __bf16*, int, int, float, float,
                                                    float, hipStream_t);
template hipError_t launch_decode_generic<float, float>(const Geom&, const QView&, const float*,
                                                 const float*, const Workspace&, int,
                                                 hipStream_t, const KernelTiming&);
template hipError_t launch_decode_generic<__bf16, __bf16>(const Geom&, const QView&, const __bf16*,
                                                  const __bf16*, const Workspace&, int,
                                                  hipStream_t, const KernelTiming&);
template hipError_t launch_decode_generic<__bf16, uint8_t>(const Geom&, const QView&, const uint8_t*,
                                                   const uint8_t*, const Workspace&, int,
                                                   hipStream_t, const KernelTiming&);
template hipError_t launch_out_proj_generic<float, float>(const Geom&, const float*,
                                                          const float*, float*, float,
                                                          hipStream_t);
template hipError_t launch_out_proj_generic<float, __bf16>(const Geom&, const float*,
                                                           const float*, __bf16*, float,
                                                           hipStream_t);
template hipError_t launch_out_proj_generic<__bf16, float>(const Geom&, const float*,
                                                           const __bf16*, float*, float,
                                                           hipStream_t);
template hipError_t launch_out_proj_generic<__bf16, __bf16>(const Geom&, const float*,
                                                            const __bf16*, __bf16*, float,
                                                            hipStream_t);

}  // namespace mlra
