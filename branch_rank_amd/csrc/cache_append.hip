// Appending one decoded token per sequence to the latent KV cache, the step
// that precedes the decode attention.
//
// What it computes ("vllbc02MLA", 猛猿大佬思路: the projected row is split into
// the compressed latent and the decoupled RoPE key, the latent is
// RMS-normalised, the RoPE key is rotated by the token's position;
// "从MHA到MLA" 3.2: the cache is updated by writing the new latent at that
// position; "MLA多头潜在注意力机制" 3: only the latent and the RoPE key are
// cached): for sequence b with L_b tokens, row L_b of the cache receives
// [RMSNorm(c) * gain || RoPE(k^R, L_b)] in the cache dtype and L_b becomes
// L_b + 1. A sequence already holding max_len tokens is left unchanged.
// An fp8 cache stores the E4M3 code nearest value / scale (ties to the even
// mantissa, saturating at +-448), one scale per cache tensor
// ("MLA多头潜在注意力机制", 9.2: an 8-bit cache for inference; the format and
// the scale convention are this library's reading).
//
// One workgroup per sequence; the bytes are a few KB per step, so this is a
// latency-bound kernel, not a streaming one.

#include <math.h>

#include "internal.h"

namespace mlra {
namespace {

// E4M3 code of x: round to nearest, ties to the even mantissa, saturating at
// +-448 (NaN gives 0x7F). Below 2^-6 the codes are the multiples of 2^-9;
// above, adding 2^19 - 1 plus the lowest kept bit to the fp32 bits and
// dropping 20 mantissa bits rounds to 3 mantissa bits, a carry moving into
// the exponent, and the exponent's bias moves from 127 to 7.
__device__ __forceinline__ uint8_t e4m3_code(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const uint32_t sign = (u >> 24) & 0x80u;
  if (__builtin_isnan(x)) return 0x7F;
  const float a = fabsf(x);
  uint32_t c;
  if (a < 0.015625f) {
    c = (uint32_t)rintf(a * 512.f);  // exact scaling; rintf rounds half to even
  } else if (a >= 448.f) {
    c = 0x7E;
  } else {
    const uint32_t v = u & 0x7FFFFFFFu;
    const uint32_t r = (v + 0x7FFFFu + ((v >> 20) & 1u)) >> 20;
    c = r - ((127u - 7u) << 3);
    if (c > 0x7Eu) c = 0x7E;
  }
  return (uint8_t)(c | sign);
}

// value v of a cache entry scaled by 1 / scale (fp8 only)
__device__ __forceinline__ void store_as(float* p, float v, float) { *p = v; }
__device__ __forceinline__ void store_as(__bf16* p, float v, float) { *p = (__bf16)v; }
__device__ __forceinline__ void store_as(uint8_t* p, float v, float scale) {
  *p = e4m3_code(v / scale);
}

template <typename T>
__global__ __launch_bounds__(256) void cache_append_kernel(AppendArgs a, RopeFreqs fr) {
  constexpr int kPer = 4;  // latent values per thread (d_c <= 1024)
  __shared__ float red[4];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const float* row = a.rows + (int64_t)b * (a.d_c + a.d_r);
  // every input is loaded up front, together with the length: this thread's
  // latent values and gains, and its RoPE pair (d_r / 2 <= 128 pairs)
  float xv[kPer], gv[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = tid + 256 * u;
    xv[u] = i < a.d_c ? row[i] : 0.f;
    gv[u] = i < a.d_c && a.gain ? a.gain[i] : 1.f;
  }
  const int hp = a.d_r / 2;
  float k0 = 0.f, k1 = 0.f;
  if (tid < hp) {
    k0 = row[a.d_c + 2 * tid];
    k1 = row[a.d_c + 2 * tid + 1];
  }
  const int p = max(a.lens[b], 0);  // position of the new token
  if (p >= a.max_len) return;       // no room: the sequence stays as it is

  // mean of squares over the latent (fp32, two-level tree)
  float ss = 0.f;
#pragma unroll
  for (int u = 0; u < kPer; ++u) ss = fmaf(xv[u], xv[u], ss);
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if (lane == 0) red[wid] = ss;
  __syncthreads();  // also: every thread has read the length
  const float inv = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)a.d_c + a.eps);

  T* c = (T*)a.ckv + (int64_t)b * a.ckv_bs + (int64_t)p * a.ckv_ts;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = tid + 256 * u;
    if (i < a.d_c) store_as(c + i, xv[u] * inv * gv[u], a.ckv_scale);
  }
  // RoPE key rotated to position p: the angle p * theta^(-2i/d_r) (frequency
  // from the host's table), its reduction to [-pi, pi] and its sine and
  // cosine in double precision
  if (tid < hp) {
    T* k = (T*)a.krope + (int64_t)b * a.kr_bs + (int64_t)p * a.kr_ts;
    const double ang = (double)p * fr.w[tid];
    const double r = ang - 6.283185307179586 * rint(ang * 0.15915494309189535);
    double sn, cs;
    sincos(r, &sn, &cs);
    const double x0 = k0, x1 = k1;
    store_as(k + 2 * tid, (float)(x0 * cs - x1 * sn), a.kr_scale);
    store_as(k + 2 * tid + 1, (float)(x0 * sn + x1 * cs), a.kr_scale);
  }
  if (tid == 0) a.lens[b] = p + 1;
}

}  // namespace

hipError_t launch_cache_append(const AppendArgs& a, CacheElt elt, int batch, hipStream_t s) {
  if (batch <= 0) return hipSuccess;
  const RopeFreqs& fr = rope_freqs(a.theta, a.d_r);
  if (elt == CacheElt::kBF16)
    hipLaunchKernelGGL(cache_append_kernel<__bf16>, dim3(batch), dim3(256), 0, s, a, fr);
  else if (elt == CacheElt::kFP8)
    hipLaunchKernelGGL(cache_append_kernel<uint8_t>, dim3(batch), dim3(256), 0, s, a, fr);
  else
    hipLaunchKernelGGL(cache_append_kernel<float>, dim3(batch), dim3(256), 0, s, a, fr);
  return hipGetLastError();
}

}  // namespace mlra
