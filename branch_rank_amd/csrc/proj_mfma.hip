// bf16 MFMA kernels around the split-KV decode on gfx950:
//
//  * absorb_q_mfma - query-side absorption, q~[b][h] = alpha_q tau W_UK[h] q^N[b][h]
//    ("Multi-Head Low-Rank Attention", 方法步骤详情 step 1), one small GEMM per
//    head (M = sequences, N = d_c, K = d_n) on v_mfma_f32_16x16x32_bf16, plus
//    the RoPE rotation of the query's rotary part in double precision.
//  * combine_hc    - merge of the split-KV partials per branch (online-softmax
//    rescaling) into the branch-normalised latent_out [B][H][d_c] fp32.
//  * merge_out     - combine_hc followed by out_proj in one kernel (mlra_decode):
//    the merged latent stays in LDS.
//  * out_proj      - output up-projection and branch sum
//    o[b][h] = alpha_kv W_UV[h]^T concat_j o~_j (方法步骤详情 step 3, 核心方法).
//    The fp32 latent is split into bf16 hi + lo parts so that the MFMA product
//    keeps fp32 accuracy; W_UV[h] is staged in LDS once and read transposed
//    with ds_read_b64_tr_b16.
//
// Partials come from the MFMA decodes: m, l as [slot][n][H] (m in log2
// units) and the accumulator normalised by l, acc / l (a weighted mean of
// cache rows), as fp16 [slot][H][d_c]; sequence b's slots are k + b for the
// work items k that overlap it (see PlanHeader). Slot k's weight in the merge
// of a (branch, head) is 2^(m_k - M) l_k / L with M the largest m_k and
// L = sum_k 2^(m_k - M) l_k.

#include <math.h>

#include "device_common.h"
#include "internal.h"
#include "plan_device.h"

namespace mlra {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8;
#define LDS_AS __attribute__((address_space(3)))

// r[0], r[1] (8 consecutive latent columns) += w times the 8 fp16 values of
// a 16-byte chunk of a partial row
__device__ __forceinline__ void fma_f16x8(f32x4* r, float w, dev::i32x4 x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // the element goes through a scalar first: this compiler's bit_cast of a
    // vector element x[i] reads element 0 whatever i is
    const int xi = x[i];
    const dev::f16x2_t h = __builtin_bit_cast(dev::f16x2_t, xi);
    r[i >> 1][2 * (i & 1)] += w * (float)h[0];
    r[i >> 1][2 * (i & 1) + 1] += w * (float)h[1];
  }
}

__device__ __forceinline__ int clamp_len(int v, int max_len) {
  return v < 0 ? 0 : (v > max_len ? max_len : v);
}

// x if c, else zeros, through a mask the compiler cannot see through: written
// as a select, the load feeding x is put back under a branch and waited for
// at once, which serialises loads meant to be in flight together.
__device__ __forceinline__ bf16x8 keep_if(bf16x8 x, bool c) {
  typedef int i32x4v __attribute__((ext_vector_type(4)));
  int m = c ? -1 : 0;
  asm volatile("" : "+v"(m));
  const i32x4v v = __builtin_bit_cast(i32x4v, x) & m;
  return __builtin_bit_cast(bf16x8, v);
}

// ------------------------------------------------------------- absorb_q ----

// grid (H (+1 when the plan rides along), ceil(B / (16 MBLK)), 2 halves of
// d_c); 4 waves
template <int KSN, int MBLK>
__global__ __launch_bounds__(256) void absorb_q_mfma(Geom g, const __bf16* __restrict__ q_nope,
                                                     const __bf16* __restrict__ q_rope,
                                                     const int32_t* __restrict__ q_pos,
                                                     const int32_t* __restrict__ lens,
                                                     const __bf16* __restrict__ w_uk,
                                                     __bf16* __restrict__ q_abs, int row,
                                                     int lo_off, float scale, float tau,
                                                     RopeFreqs fr, PlanArgs plan) {
  if (blockIdx.x == g.H) {  // the extra column of workgroups: plan (first one only)
    if (blockIdx.y == 0 && blockIdx.z == 0) plan_block(plan);
    return;
  }
  const int h = blockIdx.x, b0 = blockIdx.y * 16 * MBLK, part = blockIdx.z, parts = gridDim.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, kg = lane >> 4;
  const int dn = KSN * 32;
  // Every load below is unconditional (indices clamped into range, values
  // masked afterwards), so that none waits for another: the RoPE inputs of
  // this thread's first (sequence, pair) element, the q^N rows and the W_UK
  // fragments are in flight together.
  const int hp = g.dr / 2, i0 = threadIdx.x + 256 * part;
  int rp;
  float rx0, rx1;
  {
    const int ir = min(i0, max(16 * MBLK * hp - 1, 0));
    const int b = min(b0 + (hp > 0 ? ir / hp : 0), g.B - 1), k = hp > 0 ? ir % hp : 0;
    const int pv = (q_pos ? q_pos : lens)[b];
    rp = q_pos ? pv : clamp_len(pv, g.max_len) - 1;
    const __bf16* xr = hp > 0 ? q_rope + ((size_t)b * g.H + h) * g.dr + 2 * k : q_nope;
    rx0 = (float)xr[0];
    rx1 = (float)xr[hp > 0 ? 1 : 0];
  }
  // A = q^N rows of this block's sequences: lane (b = l16, kg)
  bf16x8 A[MBLK][KSN];
#pragma unroll
  for (int m = 0; m < MBLK; ++m) {
    const int b = b0 + 16 * m + l16, bc = min(b, g.B - 1);
#pragma unroll
    for (int ks = 0; ks < KSN; ++ks) {
      const bf16x8 x = *(const bf16x8*)(q_nope + ((size_t)bc * g.H + h) * dn + 32 * ks + 8 * kg);
      A[m][ks] = keep_if(x, b < g.B);
    }
  }
  // N blocks of 16 latent columns: this part's blocks (of `parts` equal
  // parts), spread over the 4 waves, at most NBW per wave (d_c <= 512 with 2
  // parts); every W_UK fragment of the wave is loaded before the first MFMA,
  // so the loads overlap
  constexpr int NBW = 4;
  const int nblk = g.dc / 16, per_part = nblk / parts;
  const __bf16* w = w_uk + (size_t)h * g.dc * dn;
  const int nu = (per_part - __builtin_amdgcn_readfirstlane(wave) + 3) / 4;  // blocks of this wave
  bf16x8 Bf[NBW][KSN];
#pragma unroll
  for (int u = 0; u < NBW; ++u) {
    if (u >= nu) break;
    const int c = 16 * (part * per_part + wave + 4 * u) + l16;
#pragma unroll
    for (int ks = 0; ks < KSN; ++ks)
      Bf[u][ks] = *(const bf16x8*)(w + (size_t)c * dn + 32 * ks + 8 * kg);
  }
#pragma unroll
  for (int u = 0; u < NBW; ++u) {
    if (u >= nu) break;
    const int c = 16 * (part * per_part + wave + 4 * u) + l16;
#pragma unroll
    for (int m = 0; m < MBLK; ++m) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KSN; ++ks)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[m][ks], Bf[u][ks], acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int b = b0 + 16 * m + 4 * kg + i;
        if (b < g.B) {
          // q~ as bf16 and, when asked for, its rounding residue (QView)
          const float v = scale * acc[i];
          const __bf16 hi = (__bf16)v;
          __bf16* qr = q_abs + ((size_t)b * g.H + h) * row;
          qr[c] = hi;
          if (lo_off > 0) qr[lo_off + c] = (__bf16)(v - (float)hi);
        }
      }
    }
  }

  // RoPE on the query's rotary part, its (sequence, pair) elements spread over
  // the parts' threads: the angle p * theta^(-2k/d_r) (frequency from the
  // host's table) and its reduction to [-pi, pi] in double precision, sine
  // and cosine of the reduced angle in float
  {
    for (int i = i0; i < 16 * MBLK * hp; i += 256 * parts) {
      const int b = b0 + i / hp, k = i % hp;
      if (b >= g.B) continue;
      int p = rp;
      float x0 = rx0, x1 = rx1;
      const size_t qi = ((size_t)b * g.H + h) * g.dr + 2 * k;
      if (i != i0) {  // a later element of this thread (B > 32 or a wide RoPE part)
        p = q_pos ? q_pos[b] : clamp_len(lens[b], g.max_len) - 1;
        x0 = (float)q_rope[qi];
        x1 = (float)q_rope[qi + 1];
      }
      const double a = (double)p * fr.w[k];
      const double r = a - 6.283185307179586 * rint(a * 0.15915494309189535);
      float sn, cs;
      sincosf((float)r, &sn, &cs);
      __bf16* o = q_abs + ((size_t)b * g.H + h) * row + g.dc + 2 * k;
      o[0] = (__bf16)(tau * (x0 * cs - x1 * sn));
      o[1] = (__bf16)(tau * (x0 * sn + x1 * cs));
    }
  }
}

// ----------------------------------------------------------- combine_hc ----

// Merge of the split-KV partials of sequence b into its branch-normalised
// latent, o~_j[h] = sum_k 2^(m_k - M) l_k (acc_k / l_k) / sum_k 2^(m_k - M) l_k
// over the slots k of the sequence (textbook online-softmax merge; one
// softmax per branch, "Multi-Head Low-Rank Attention", 核心方法). grid
// (B, H / kMH); the weights 2^(m_k - M) l_k / L of (slot, branch, head) are
// computed once into LDS, kMS slots at a time, then each thread sums the
// 16-byte fp16 chunks (8 columns) of its partial rows.
constexpr int kMH = 4;    // heads per workgroup
constexpr int kMS = 64;   // slots per weight table
constexpr int kMNB = 8;   // most branches

__global__ __launch_bounds__(256) void combine_hc(Geom g, Workspace ws,
                                                  float* __restrict__ latent_out,
                                                  float out_scale) {
  __shared__ float stat[2 * kMNB * kMH];        // M, 1/L per (branch, head)
  __shared__ float wt[kMS * kMNB * kMH];        // weights of kMS slots
  const int b = blockIdx.x, h0 = blockIdx.y * kMH, tid = threadIdx.x;
  const int H = g.H, DC = g.dc, NB = g.n, C8 = g.dc / 8, NP = NB * kMH;
  const int hn = min(kMH, H - h0);
  const PlanHeader hd = *ws.hdr;
  const int p0 = ws.prefix[b], p1 = ws.prefix[b + 1];
  float* out = latent_out + ((size_t)b * H + h0) * DC;
  if (p1 <= p0) {  // empty sequence: o = 0
    for (int q = tid; q < hn * DC / 4; q += 256) *(f32x4*)(out + 4 * q) = (f32x4){0.f, 0.f, 0.f, 0.f};
    return;
  }
  const int kf = p0 / hd.chunk, kl = (p1 - 1) / hd.chunk;
  MLRA_DCHECK(ws.hdr, kf >= 0 && kf <= kl && kl < hd.n_items, 5);
  // per (branch, head): the max M and 1/L over the sequence's slots
  for (int q = tid; q < NP; q += 256) {
    const int j = q / kMH, hh = q % kMH;
    if (hh < hn) {
      const size_t base = (size_t)j * H + h0 + hh;
      float mx = -INFINITY;
#pragma unroll 8
      for (int k = kf; k <= kl; ++k) mx = fmaxf(mx, ws.m[(size_t)(k + b) * NB * H + base]);
      float L = 0.f;
#pragma unroll 8
      for (int k = kf; k <= kl; ++k) {
        const size_t i = (size_t)(k + b) * NB * H + base;
        L += exp2f(ws.m[i] - mx) * ws.l[i];
      }
      stat[2 * q] = mx;
      stat[2 * q + 1] = 1.f / L;
    }
  }
  // thread -> (head hh, 8 latent columns 8 c8 of branch j); d_c <= 512, so
  // kMH heads take at most 256 threads
  const int per = hn * C8;
  const _Float16* acc16 = reinterpret_cast<const _Float16*>(ws.acc);
  f32x4 r[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  for (int k0 = kf; k0 <= kl; k0 += kMS) {
    const int nk = min(kMS, kl - k0 + 1);
    __syncthreads();  // stats ready / previous table consumed
    for (int q = tid; q < nk * NP; q += 256) {
      const int kk = q / NP, pr = q % NP, j = pr / kMH, hh = pr % kMH;
      float w = 0.f;
      if (hh < hn) {
        const size_t i = ((size_t)(k0 + kk + b) * NB + j) * H + h0 + hh;
        w = exp2f(ws.m[i] - stat[2 * pr]) * ws.l[i] * stat[2 * pr + 1];
      }
      wt[q] = w;
    }
    __syncthreads();
    if (tid < per) {
      const int hh = tid / C8, c8 = tid % C8, j = (8 * c8) / (DC / NB);
      const _Float16* src = acc16 + ((size_t)(k0 + b) * H + h0 + hh) * DC + 8 * c8;
#pragma unroll 8
      for (int kk = 0; kk < nk; ++kk)
        fma_f16x8(r, wt[kk * NP + j * kMH + hh], *(const dev::i32x4*)(src + (size_t)kk * H * DC));
    }
  }
  if (tid < per) {
    *(f32x4*)(out + 8 * tid) = out_scale * r[0];
    *(f32x4*)(out + 8 * tid + 4) = out_scale * r[1];
  }
}

// ------------------------------------------------------------- out_proj ----

// W_UV rows of one v-half staged in LDS: 64 bf16 (128 B) per latent column,
// padded to 160 B so that the transposed reads (4 rows x 32 B per 16 lanes)
// hit distinct banks. Latent rows (bf16 hi and lo) padded by 16 B.
constexpr int kDVH = 64;            // output columns per workgroup
constexpr int kWRow = 160;          // bytes per staged W_UV row
template <int DC>
struct OutLds {
  static constexpr int LROW = (DC + 8) * 2;                 // bytes per latent row
  static constexpr int W_BYTES = DC * kWRow;
  static constexpr int L_BYTES = 16 * LROW;
  static constexpr int TOTAL = W_BYTES + 2 * L_BYTES;
};

// grid H * 2 (the two v-halves of a head share an XCD); 4 waves, wave w owns
// output columns [16 w, 16 w + 16) of its half.
template <int DC, typename TO>
__global__ __launch_bounds__(256) void out_proj(Geom g, const float* __restrict__ latent_in,
                                                const __bf16* __restrict__ w_uv,
                                                TO* __restrict__ out, float alpha_kv) {
  using LD = OutLds<DC>;
  __shared__ __attribute__((aligned(16))) char smem_raw[LD::TOTAL];
  char LDS_AS* smem = (char LDS_AS*)smem_raw;
  char LDS_AS* wl = smem;
  char LDS_AS* lhi = smem + LD::W_BYTES;
  char LDS_AS* llo = lhi + LD::L_BYTES;
  const int i = blockIdx.x, x = i & 7, jj = i >> 3;
  const int h = (jj >> 1) * 8 + x, vh = jj & 1;
  if (h >= g.H) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, kg = lane >> 4;

  // stage W_UV[h][:, 64 vh .. 64 vh + 64): all loads of a thread first
  {
    const __bf16* w = w_uv + (size_t)h * DC * g.dv + kDVH * vh;
    constexpr int NQ = DC * 8 / 256;
    bf16x8 st[NQ];
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int q = tid + 256 * u, c = q >> 3, ch = q & 7;
      st[u] = *(const bf16x8*)(w + (size_t)c * g.dv + 8 * ch);
    }
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int q = tid + 256 * u, c = q >> 3, ch = q & 7;
      *(bf16x8 LDS_AS*)(wl + c * kWRow + 16 * ch) = st[u];
    }
  }
  // per-lane offsets of the transposed W reads (rows 4 r + {0..3}, column quad q)
  const int r4 = l16 >> 2, q4 = l16 & 3;
  const int wcol = 2 * (16 * wave + 4 * q4);

  for (int b0 = 0; b0 < g.B; b0 += 16) {
    __syncthreads();  // W staged / previous block's latent consumed
    // latent rows of sequences b0..b0+15 as bf16 hi + lo
    for (int q = tid; q < 16 * (DC / 4); q += 256) {
      const int bb = q / (DC / 4), c4 = q % (DC / 4), b = b0 + bb;
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (b < g.B) {
        v = *(const f32x4*)(latent_in + ((size_t)b * g.H + h) * DC + 4 * c4);
      }
      __bf16 hi[4], lo[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hi[e] = (__bf16)v[e];
        lo[e] = (__bf16)(v[e] - (float)hi[e]);
      }
      __bf16 LDS_AS* ph = (__bf16 LDS_AS*)(lhi + bb * LD::LROW) + 4 * c4;
      __bf16 LDS_AS* pl = (__bf16 LDS_AS*)(llo + bb * LD::LROW) + 4 * c4;
#pragma unroll
      for (int e = 0; e < 4; ++e) { ph[e] = hi[e]; pl[e] = lo[e]; }
    }
    __syncthreads();
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int ks = 0; ks < DC / 32; ++ks) {
      const int aoff = l16 * LD::LROW + 2 * (32 * ks + 8 * kg);
      const bf16x8 ah = *(const bf16x8 LDS_AS*)(lhi + aoff);
      const bf16x8 al = *(const bf16x8 LDS_AS*)(llo + aoff);
      const int wr = (32 * ks + 8 * kg + r4) * kWRow + wcol;
      const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)(wl + wr));
      const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)(wl + wr + 4 * kWRow));
      const i16x8 wv = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
      const bf16x8 wb = __builtin_bit_cast(bf16x8, wv);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, wb, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, wb, acc, 0, 0, 0);
    }
    // D[b][v]: lane (v = 16 wave + l16 of this half, rows b0 + 4 kg + i)
    const int v = kDVH * vh + 16 * wave + l16;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int b = b0 + 4 * kg + e;
      if (b < g.B) out[((size_t)b * g.H + h) * g.dv + v] = (TO)(alpha_kv * acc[e]);
    }
  }
}

// ------------------------------------------------------------ merge_out ----

// combine_hc and out_proj in one kernel, for mlra_decode: workgroup (head h,
// block of kMSQ sequences) merges head h's partials of each sequence into its
// branch-normalised latent row and projects the rows with W_UV[h]. The
// merged latent never goes to memory and every partial row is read once.
//
// Waves 0-3 bring W_UV[h] (d_c rows of 128 bf16) into LDS by LDS-DMA as soon
// as the workgroup starts; rows are 256 bytes with their 16-byte chunks
// XOR-swizzled by kWSwz, so the transposed reads of the projection hit 64
// distinct banks. Meanwhile waves 4-7 merge: a 16-lane group per (sequence,
// branch) reads the slots' (m, l), reduces them to (M, 1/L) with lane
// shuffles and writes the weights 2^(m_k - M) l_k / L to an LDS table (kMOS
// slots per pass); every thread's first kMKU partial rows (16-byte fp16
// chunks, 8 columns) are already in flight by then. The latent rows go to LDS as bf16 hi + lo (rows 8..15 of
// the MFMA's A operand are zero) and all 8 waves project 16 output columns
// each. The workgroups of a head run on one XCD (8 apart in launch order),
// so W_UV[h] comes from L2 after the first.
constexpr int kMOS = 32;  // slots per weight table pass
constexpr int kMSQ = 8;   // sequences per block
constexpr int kMKU = 8;   // partial rows per (thread, column oct) in flight

__device__ __forceinline__ int kWSwz(int row) { return 2 * ((row & 3) | (((row >> 3) & 1) << 2)); }

template <int DC>
struct MergeLds {
  static constexpr int W_BYTES = DC * 256;       // W_UV[h], 128 columns per row
  static constexpr int LROW = DC * 2 + 16;       // latent row (padded)
  static constexpr int L_BYTES = kMSQ * LROW;
  static constexpr int WT_FLOATS = kMSQ * kMOS * kMNB;  // [sequence][slot][branch]
  static constexpr int TOTAL = W_BYTES + 2 * L_BYTES + 4 * WT_FLOATS + 8 * kMSQ;
};

// (M, L) of an online softmax merged with (m, l); an empty side is M = -inf.
__device__ __forceinline__ void ml_merge(float& M, float& L, float m, float l) {
  if (m == -INFINITY) return;
  if (M == -INFINITY) { M = m; L = l; return; }
  const float mn = fmaxf(M, m);
  L = L * exp2f(M - mn) + l * exp2f(m - mn);
  M = mn;
}

template <int DC, typename TO>
__global__ __launch_bounds__(512) void merge_out(Geom g, Workspace ws,
                                                 const __bf16* __restrict__ w_uv,
                                                 TO* __restrict__ out, float alpha_kv) {
  using MD = MergeLds<DC>;
  static_assert(MD::TOTAL <= 163840, "LDS");
  __shared__ __attribute__((aligned(16))) char smem_raw[MD::TOTAL];
  char LDS_AS* smem = (char LDS_AS*)smem_raw;
  char LDS_AS* wl = smem;
  char LDS_AS* lhi = smem + MD::W_BYTES;
  char LDS_AS* llo = lhi + MD::L_BYTES;
  float LDS_AS* wt = (float LDS_AS*)(llo + MD::L_BYTES);
  int LDS_AS* rng = (int LDS_AS*)(wt + MD::WT_FLOATS);  // kf, kl per sequence of the block
  const int nblk = (g.B + kMSQ - 1) / kMSQ;
  const int i = blockIdx.x, x = i & 7, jj = i >> 3;
  const int h = (jj / nblk) * 8 + x, b0 = (jj % nblk) * kMSQ;
  if (h >= g.H) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, kg = lane >> 4;
  const int NB = g.n, H = g.H, bw = DC / NB;
  constexpr int C8 = DC / 8;
  constexpr int NQ = (kMSQ * C8 + 511) / 512;  // column octs (16-byte fp16 chunks) per thread
  const int nbq = min(kMSQ, g.B - b0);

  if (wave < 4) {
    // W_UV[h] -> LDS: instruction u of wave w carries rows 4 (4 u + w) .. +3
    // (lane: row + lane / 16, LDS chunk lane % 16, read from chunk
    // (lane % 16) ^ kWSwz(row))
    const uint64_t a = reinterpret_cast<uint64_t>(w_uv + (size_t)h * DC * 128);
    dev::i32x4 rs;
    rs.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    rs.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xFFFF);
    rs.z = MD::W_BYTES;
    rs.w = 0x00020000;
    const uint32_t wbase = (uint32_t)reinterpret_cast<uintptr_t>(wl);
#pragma unroll
    for (int u = 0; u < DC / 16; ++u) {
      const int q = 4 * u + wave, row = 4 * q + (lane >> 4);
      dev::dma16(rs, wbase + 1024 * q, (uint32_t)(row * 256 + 16 * ((lane & 15) ^ kWSwz(row))), 0u);
    }
  } else if (tid < 256 + kMSQ) {
    const int bb = tid - 256;
    int kf = 0, kl = -1;
    if (bb < nbq) {
      const int chunk = ws.hdr->chunk;
      const int p0 = ws.prefix[b0 + bb], p1 = ws.prefix[b0 + bb + 1];
      kf = p0 / chunk;
      kl = p1 > p0 ? (p1 - 1) / chunk : kf - 1;
      MLRA_DCHECK(ws.hdr, kf >= 0 && kl < ws.hdr->n_items, 5);
    }
    rng[2 * bb] = kf;
    rng[2 * bb + 1] = kl;
  }
  __syncthreads();
  int maxs = 0;
#pragma unroll
  for (int bb = 0; bb < kMSQ; ++bb) maxs = max(maxs, rng[2 * bb + 1] - rng[2 * bb] + 1);

  // waves 4-7 reduce (m, l): group grp = (tid / 16) % 16 takes (sequence,
  // branch) pairs grp, grp + 16, ...; every thread sums octs q = tid + 512 u
  const int grp = (tid >> 4) & 15;
  constexpr int PPG = kMSQ * kMNB / 16;  // most pairs per group
  float Mp[PPG], Ip[PPG], mk[PPG][2], lk[PPG][2];
  f32x4 r[NQ][2];
  dev::i32x4 v[kMKU][NQ];
  const _Float16* acc16 = reinterpret_cast<const _Float16*>(ws.acc);
  const _Float16* src[NQ];
  int nsq[NQ], wi[NQ];
  // (m, l) of the first 32 slots of each pair: loads on every wave without a
  // branch (slot clamped into the sequence's range, or slot 0 when it has
  // none), so that they stay in flight with the partial rows issued next;
  // only waves 4-7 use them
#pragma unroll
  for (int pj = 0; pj < PPG; ++pj) {
    const int p = grp + 16 * pj, pv = p < kMSQ * NB, bb = pv ? p / NB : 0, j = p % NB;
    const int kf = rng[2 * bb], ns = pv ? rng[2 * bb + 1] - kf + 1 : 0;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int s = l16 + 16 * e;
      const size_t idx =
          ns > 0 ? ((size_t)(kf + min(s, ns - 1) + b0 + bb) * NB + j) * H + h : (size_t)h;
      mk[pj][e] = ws.m[idx];
      lk[pj][e] = ws.l[idx];
    }
  }
  // the first kMKU partial rows of every oct: in flight with the (m, l)
  // loads (and, on waves 0-3, behind the W_UV DMA)
#pragma unroll
  for (int u = 0; u < NQ; ++u) {
    const int q = min(tid + 512 * u, kMSQ * C8 - 1), bb = q / C8, c8 = q % C8;
    const int kf = rng[2 * bb];
    nsq[u] = tid + 512 * u < kMSQ * C8 ? rng[2 * bb + 1] - kf + 1 : 0;
    src[u] = acc16 + ((size_t)(kf + b0 + bb) * H + h) * DC + 8 * c8;
    wi[u] = bb * kMOS * NB + (8 * c8) / bw;
    r[u][0] = r[u][1] = (f32x4){0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int k = 0; k < kMKU; ++k)
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      // no branch: a slot past the sequence re-reads its last one (or slot
      // 0 of the workspace) and is zeroed
      const _Float16* a = nsq[u] > 0 ? src[u] + (size_t)min(k, nsq[u] - 1) * H * DC : acc16;
      const dev::i32x4 x = *(const dev::i32x4*)a;
      v[k][u] = k < nsq[u] ? x : (dev::i32x4){0, 0, 0, 0};
    }
  if (wave >= 4) {
    // (M, 1/L) per pair: online over this lane's slots, then over the 16 lanes
#pragma unroll
    for (int pj = 0; pj < PPG; ++pj) {
      const int p = grp + 16 * pj, pv = p < kMSQ * NB, bb = pv ? p / NB : 0, j = p % NB;
      const int kf = rng[2 * bb], ns = pv ? rng[2 * bb + 1] - kf + 1 : 0;
      float M = -INFINITY, L = 0.f;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        if (l16 + 16 * e >= ns) mk[pj][e] = -INFINITY;
        ml_merge(M, L, mk[pj][e], lk[pj][e]);
      }
      for (int s = l16 + 32; s < ns; s += 16) {  // more than 32 slots: rare
        const size_t idx = ((size_t)(kf + s + b0 + bb) * NB + j) * H + h;
        ml_merge(M, L, ws.m[idx], ws.l[idx]);
      }
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) {
        const float M2 = __shfl_xor(M, o), L2 = __shfl_xor(L, o);
        ml_merge(M, L, M2, L2);
      }
      Mp[pj] = M;
      Ip[pj] = L > 0.f ? 1.f / L : 0.f;  // empty sequence: weights 0, o = 0
    }
  }
  // passes of kMOS slots: weights into the table, then the weighted sum
  for (int s0 = 0; s0 < maxs; s0 += kMOS) {
    if (s0 > 0) __syncthreads();  // the previous pass's table consumed
    if (wave >= 4) {
#pragma unroll
      for (int pj = 0; pj < PPG; ++pj) {
        const int p = grp + 16 * pj, bb = p / NB, j = p % NB;
        if (p >= kMSQ * NB) break;
        const int kf = rng[2 * bb], ns = rng[2 * bb + 1] - kf + 1;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int s = s0 + l16 + 16 * e;
          float m = mk[pj][e], l = lk[pj][e];
          if (s0 > 0 && s < ns) {
            const size_t i = ((size_t)(kf + s + b0 + bb) * NB + j) * H + h;
            m = ws.m[i];
            l = ws.l[i];
          }
          wt[(bb * kMOS + l16 + 16 * e) * NB + j] =
              s < ns && m > -INFINITY ? exp2f(m - Mp[pj]) * l * Ip[pj] : 0.f;
        }
      }
    }
    __syncthreads();
    {
      int kmax = 0;
#pragma unroll
      for (int u = 0; u < NQ; ++u) kmax = max(kmax, min(kMOS, nsq[u] - s0));
      for (int k0 = 0; k0 < kmax; k0 += kMKU) {
        if (s0 + k0 > 0) {
#pragma unroll
          for (int k = 0; k < kMKU; ++k)
#pragma unroll
            for (int u = 0; u < NQ; ++u)
              v[k][u] = s0 + k0 + k < nsq[u] && k0 + k < kMOS
                            ? *(const dev::i32x4*)(src[u] + (size_t)(s0 + k0 + k) * H * DC)
                            : (dev::i32x4){0, 0, 0, 0};
        }
#pragma unroll
        for (int k = 0; k < kMKU; ++k)
#pragma unroll
          for (int u = 0; u < NQ; ++u)
            if (s0 + k0 + k < nsq[u] && k0 + k < kMOS)
              fma_f16x8(r[u], wt[wi[u] + (k0 + k) * NB], v[k][u]);
      }
    }
  }
  {
    // the block's latent rows as bf16 hi + lo
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int q = tid + 512 * u, bb = q / C8, c8 = q % C8;
      if (q >= kMSQ * C8) break;
      bf16x8 hi, lo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = r[u][e >> 2][e & 3];
        hi[e] = (__bf16)x;
        lo[e] = (__bf16)(x - (float)hi[e]);
      }
      *(bf16x8 LDS_AS*)((__bf16 LDS_AS*)(lhi + bb * MD::LROW) + 8 * c8) = hi;
      *(bf16x8 LDS_AS*)((__bf16 LDS_AS*)(llo + bb * MD::LROW) + 8 * c8) = lo;
    }
  }
  if (wave < 4) dev::wait_vm<0>();  // this wave's share of W_UV[h] is in LDS
  __syncthreads();
  // out[b][v] for the 16 columns v = 16 wave + l16: A = latent rows (lane
  // row l16, zero past the block's 8), B = W_UV[h] read transposed
  const int r4 = l16 >> 2, q4 = l16 & 3;
  const int cb = 32 * wave + 8 * q4;  // byte column of this lane's 4 values
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int ks = 0; ks < DC / 32; ++ks) {
    bf16x8 ah = {}, al = {};
    if (l16 < kMSQ) {
      const int aoff = l16 * MD::LROW + 2 * (32 * ks + 8 * kg);
      ah = *(const bf16x8 LDS_AS*)(lhi + aoff);
      al = *(const bf16x8 LDS_AS*)(llo + aoff);
    }
    const int R = 32 * ks + 8 * kg + r4;
    const int o0 = R * 256 + (((cb >> 4) ^ kWSwz(R)) << 4) + (cb & 15);
    const int o1 = (R + 4) * 256 + (((cb >> 4) ^ kWSwz(R + 4)) << 4) + (cb & 15);
    const i16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)(wl + o0));
    const i16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LDS_AS*)(wl + o1));
    const i16x8 wv = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
    const bf16x8 wb = __builtin_bit_cast(bf16x8, wv);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, wb, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, wb, acc, 0, 0, 0);
  }
  // D[row][v]: rows 4 kg + e of the block (only rows < nbq are sequences)
  const int vc = 16 * wave + l16;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int bb = 4 * kg + e;
    if (bb < nbq) out[((size_t)(b0 + bb) * g.H + h) * g.dv + vc] = (TO)(alpha_kv * acc[e]);
  }
}

template <int DC, typename TO>
hipError_t launch_merge_out_t(const Geom& g, const Workspace& ws, const __bf16* w_uv, TO* out,
                              float alpha_kv, hipStream_t s) {
  if (g.dv != 128 || g.n > kMNB || DC % g.n) return hipErrorNotSupported;
  const int64_t grid = (int64_t)((g.H + 7) / 8) * 8 * ((g.B + kMSQ - 1) / kMSQ);
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((merge_out<DC, TO>), dim3((unsigned)grid), dim3(512), 0, s, g, ws, w_uv, out,
                     alpha_kv);
  return hipGetLastError();
}

template <int DC, typename TO>
hipError_t launch_out_t(const Geom& g, const float* lat, const __bf16* w_uv, TO* out,
                        float alpha_kv, hipStream_t s) {
  const int grid = ((g.H + 7) / 8) * 8 * 2;
  hipLaunchKernelGGL((out_proj<DC, TO>), dim3(grid), dim3(256), 0, s, g, lat, w_uv, out, alpha_kv);
  return hipGetLastError();
}

template <int KSN>
hipError_t launch_absorb_k(const Geom& g, const __bf16* qn, const __bf16* qr, const int32_t* qp,
                           const int32_t* lens, const __bf16* w, __bf16* qa, int qs, int lo,
                           float scale, float tau, float theta, const PlanArgs& plan,
                           hipStream_t s) {
  const int gx = g.H + (plan.hdr ? 1 : 0);
  const RopeFreqs& fr = rope_freqs(theta, g.dr);
  // latent column parts per head: the most (<= 8) that split the 16-column
  // blocks evenly, so that more workgroups share the W_UK read (1032 at
  // H = 128, d_c = 512)
  const int nblk = g.dc / 16;
  int parts = 2;
  for (int p = 8; p > 2; p >>= 1)
    if (nblk % p == 0) {
      parts = p;
      break;
    }
  if (g.B > 32) {
    hipLaunchKernelGGL((absorb_q_mfma<KSN, 4>), dim3(gx, (g.B + 63) / 64, parts), dim3(256), 0,
                       s, g, qn, qr, qp, lens, w, qa, qs, lo, scale, tau, fr, plan);
  } else {
    hipLaunchKernelGGL((absorb_q_mfma<KSN, 1>), dim3(gx, (g.B + 15) / 16, parts), dim3(256), 0,
                       s, g, qn, qr, qp, lens, w, qa, qs, lo, scale, tau, fr, plan);
  }
  return hipGetLastError();
}

}  // namespace

bool proj_mfma_supported(const Geom& g) {
  return (g.dc == 128 || g.dc == 256 || g.dc == 512) && g.dv == 2 * kDVH;
}

bool absorb_mfma_supported(const Geom& g) {
  // <= 4 blocks of 16 columns per wave and half: d_c <= 512
  return g.dc % 32 == 0 && g.dc <= 512 && (g.dn == 64 || g.dn == 128 || g.dn == 256);
}

hipError_t launch_absorb_q_mfma(const Geom& g, const __bf16* q_nope, const __bf16* q_rope,
                                const int32_t* q_pos, const int32_t* lens, const __bf16* w_uk,
                                __bf16* q_abs, int q_stride, int lo_off, float lat_scale,
                                float rope_scale, float theta, const PlanArgs& plan,
                                hipStream_t s) {
  const float scale = lat_scale, tau = rope_scale;
  switch (g.dn) {
    case 64:
      return launch_absorb_k<2>(g, q_nope, q_rope, q_pos, lens, w_uk, q_abs, q_stride, lo_off,
                                scale, tau, theta, plan, s);
    case 128:
      return launch_absorb_k<4>(g, q_nope, q_rope, q_pos, lens, w_uk, q_abs, q_stride, lo_off,
                                scale, tau, theta, plan, s);
    case 256:
      return launch_absorb_k<8>(g, q_nope, q_rope, q_pos, lens, w_uk, q_abs, q_stride, lo_off,
                                scale, tau, theta, plan, s);
  }
  return hipErrorNotSupported;
}

hipError_t launch_combine_hc(const Geom& g, const Workspace& ws, float* latent_out,
                             float out_scale, hipStream_t s) {
  // one thread per 8-column chunk of kMH heads: d_c <= 512 (every MFMA decode's)
  if (g.n > kMNB || g.dc > 512 || g.dc % 8) return hipErrorNotSupported;
  hipLaunchKernelGGL(combine_hc, dim3(g.B, (g.H + kMH - 1) / kMH), dim3(256), 0, s, g, ws,
                     latent_out, out_scale);
  return hipGetLastError();
}

template <typename TO>
hipError_t launch_out_proj_mfma(const Geom& g, const float* latent, const __bf16* w_uv, TO* out,
                                float alpha_kv, hipStream_t s) {
  switch (g.dc) {
    case 128: return launch_out_t<128, TO>(g, latent, w_uv, out, alpha_kv, s);
    case 256: return launch_out_t<256, TO>(g, latent, w_uv, out, alpha_kv, s);
    case 512: return launch_out_t<512, TO>(g, latent, w_uv, out, alpha_kv, s);
  }
  return hipErrorNotSupported;
}

template <typename TO>
hipError_t launch_merge_out_proj(const Geom& g, const Workspace& ws, const __bf16* w_uv, TO* out,
                                 float alpha_kv, hipStream_t s) {
  if (g.n > kMNB || g.B <= 0) return g.B <= 0 ? hipSuccess : hipErrorNotSupported;
  switch (g.dc) {
    case 128: return launch_merge_out_t<128, TO>(g, ws, w_uv, out, alpha_kv, s);
    case 256: return launch_merge_out_t<256, TO>(g, ws, w_uv, out, alpha_kv, s);
    case 512: return launch_merge_out_t<512, TO>(g, ws, w_uv, out, alpha_kv, s);
  }
  return hipErrorNotSupported;
}

template hipError_t launch_merge_out_proj<float>(const Geom&, const Workspace&, const __bf16*,
                                                 float*, float, hipStream_t);
template hipError_t launch_merge_out_proj<__bf16>(const Geom&, const Workspace&, const __bf16*,
                                                  __bf16*, float, hipStream_t);

template hipError_t launch_out_proj_mfma<float>(const Geom&, const float*, const __bf16*, float*,
                                                float, hipStream_t);
template hipError_t launch_out_proj_mfma<__bf16>(const Geom&, const float*, const __bf16*,
                                                 __bf16*, float, hipStream_t);

}  // namespace mlra
