// Internal declarations shared by the host API and the kernel translation
// units. Not part of the public C ABI (include/mlra.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mlra {

// Split-KV plan. All cached tokens of the batch form one stream (sequence b
// occupies [prefix[b], prefix[b+1])). The stream is cut into n_items equal
// work items of `chunk` tokens; item k covers [k*chunk, (k+1)*chunk) and may
// span several sequences, one segment per sequence. The segment of item k in
// sequence b writes its softmax partials to slot k + b, which is unique
// because a later sequence never starts in an earlier item.
struct PlanHeader {
  int32_t chunk;
  int32_t n_items;
  int32_t total;
  int32_t bounds_fail;  // debug build: site of the first failed device bounds check, else 0
};

// Arguments of the cache append (cache_append.hip): rows [B][d_c + d_r] fp32
// (latent, then the unrotated RoPE key), written to row L_b of each sequence.
struct AppendArgs {
  const float* rows;
  const float* gain;   // [d_c] or nullptr (1)
  void* ckv;
  void* krope;
  int64_t ckv_bs, ckv_ts, kr_bs, kr_ts;  // element strides
  int32_t* lens;
  int max_len, d_c, d_r;
  float eps, theta;
  float ckv_scale, kr_scale;  // fp8 cache: a value x is stored as the E4M3 code of x / scale
};

// Element type of the cache the append writes.
enum class CacheElt { kF32, kBF16, kFP8 };
hipError_t launch_cache_append(const AppendArgs& a, CacheElt elt, int batch, hipStream_t s);

// Inputs and outputs of the split-KV plan (plan_device.h).
struct PlanArgs {
  const int32_t* lens;  // [B] cache lengths (clamped to [0, max_len])
  int B, max_len;
  int target_items;     // wanted number of work items (automatic chunk)
  int forced_chunk;     // > 0: fixed chunk size in tokens
  PlanHeader* hdr;      // nullptr: no plan to compute
  int32_t* prefix;      // [B + 1]
};

// Partial softmax state per slot: m and l as [slot][n][H] fp32 (m in log2
// units, i.e. max of score*log2(e)). The accumulator region holds, after the
// portable decode, acc as [slot][d_c][H] fp32 (unnormalised); after the MFMA
// decodes, acc / l as fp16 [slot][H][d_c] (half of the region).
struct Workspace {
  PlanHeader* hdr;
  int32_t* prefix;  // [B + 1]
  float* m;         // [slots][n][H]
  float* l;         // [slots][n][H]
  float* acc;       // [slots][d_c][H] fp32, or fp16 [slots][H][d_c] (see above)
  void* q_abs;      // [B][H][d_c + d_r (+ d_c, bf16: q~'s residue)] (mlra_decode only)
  float* latent;    // [B][H][d_c]       (mlra_decode only)
};

// Optional events stamped by the decode dispatch itself at its start and end
// (hipExtLaunchKernel), so that timing adds no packets to the stream.
struct KernelTiming {
  hipEvent_t start = nullptr, stop = nullptr;
};

// Absorbed queries as the decode kernels read them: row (b, h) starts at
// element (b * H + h) * stride of q and holds q~ (d_c) then rho (d_r). With
// lo > 0 (bf16 only), elements [lo, lo + d_c) of the row hold q~'s rounding
// residue bf16(q~ - bf16(q~)), so that the two bf16 parts carry q~ to about
// 16 significant bits; lo = 0 means the query is the bf16 q~ alone.
struct QView {
  const void* q;
  int stride;
  int lo;
};

struct Geom {
  int B, H, dc, dr, dn, dv, n;
  int max_len;
  int64_t ckv_bs, ckv_ts, kr_bs, kr_ts;  // element strides
};

// Causal prefill of MLRA-4 with 128-wide branches (prefill_branch.hip): one
// kernel from the queries q^N, q^R [B][T][H][.] and the cache to the output
// [B][T][H][d_v] (bf16 or fp32), zeros for t >= L_b.
bool prefill_branch_supported(const Geom& g);
hipError_t launch_prefill_branch(const Geom& g, int T, const void* q_nope, const void* q_rope,
                                 const void* w_uk, const void* w_uv, const void* ckv,
                                 const void* krope, const int32_t* lens, void* out, bool out_bf16,
                                 float tau, float alpha_q, float alpha_kv, float theta,
                                 hipStream_t s, const KernelTiming& t);

// Causal prefill of MLA in the unabsorbed (MHA) form (prefill_mha.hip): the
// up-projected keys and values of every head go to `workspace`
// (prefill_mha_workspace bytes), then causal attention writes out
// [B][T][H][d_v].
bool prefill_mha_supported(const Geom& g);
size_t prefill_mha_workspace(const Geom& g, int T);
hipError_t launch_prefill_mha(const Geom& g, int T, const void* q_nope, const void* q_rope,
                              const void* w_uk, const void* w_uv, const void* ckv,
                              const void* krope, const int32_t* lens, void* workspace, void* out,
                              bool out_bf16, float tau, float alpha_q, float alpha_kv,
                              float theta, hipStream_t s, const KernelTiming& t);

// Rotary frequencies omega_k = theta^(-2k / d_r), k < d_r / 2, in double,
// computed on the host once per (theta, d_r) and passed to the kernels by
// value, so that no kernel evaluates pow() per element.
constexpr int kMaxRopePairs = 128;  // d_r <= 256
struct RopeFreqs {
  double w[kMaxRopePairs];
};
const RopeFreqs& rope_freqs(float theta, int dr);

constexpr int kMinChunk = 64;      // smallest automatic work item, tokens
constexpr int kMaxAutoItems = 512; // upper bound on automatic work items

// ---- launchers (return the launch status) ----
hipError_t launch_plan(const int32_t* lens, int B, int max_len, int target_items,
                       int forced_chunk, const Workspace& ws, hipStream_t s);

// Query absorption into rows of q_stride elements; lo_off > 0 (bf16 only)
// also writes q~'s rounding residue at that element of each row (QView).
// lat_scale multiplies W_UK q^N (alpha_q tau, times the cache's latent scale
// for an fp8 cache), rope_scale the rotated q^R (tau, times the RoPE scale).
template <typename T>
hipError_t launch_absorb_q_generic(const Geom& g, const T* q_nope, const T* q_rope,
                                   const int32_t* q_pos, const int32_t* lens, const T* w_uk,
                                   T* q_abs, int q_stride, int lo_off, float lat_scale,
                                   float rope_scale, float theta, hipStream_t s);

// Cache elements T (fp32, bf16) or fp8 E4M3 codes (uint8_t, bf16 queries).
template <typename T, typename TC>
hipError_t launch_decode_generic(const Geom& g, const QView& q, const TC* ckv, const TC* krope,
                                 const Workspace& ws, int grid_items, hipStream_t s,
                                 const KernelTiming& t);

// latent_out = out_scale * the merged latent (out_scale: the fp8 cache's
// latent scale, else 1).
hipError_t launch_combine(const Geom& g, const Workspace& ws, float* latent_out, float out_scale,
                          hipStream_t s);

// Rows of `dst` = the caller's bf16 q_abs rows `src` with q~ times lat_scale
// and rho times rope_scale (q~ taken with its residue when src has one, and
// split again into bf16 parts when dst has one): the query for an fp8 cache.
hipError_t launch_scale_q(const Geom& g, const QView& src, const QView& dst, float lat_scale,
                          float rope_scale, hipStream_t s);

template <typename T, typename TO>
hipError_t launch_out_proj_generic(const Geom& g, const float* latent, const T* w_uv, TO* out,
                                   float alpha_kv, hipStream_t s);

// Fast bf16 MFMA decode. Returns hipErrorNotSupported when the shape has no
// specialisation (the caller then uses the generic kernel).
// fp8: the cache holds E4M3 codes (the kernels convert them exactly after
// LDS); the scales are folded into the query and the merge by the caller.
bool decode_branch_supported(const Geom& g, bool fp8 = false);
int decode_branch_wgs_per_item(const Geom& g);
// whether the branch kernel reads q~'s residue for this geometry, cache type
// and the caller's wish (cfg->q_residue)
bool decode_branch_reads_residue(const Geom& g, bool fp8, bool want);
hipError_t launch_decode_branch(const Geom& g, const QView& q, const void* ckv,
                                const void* krope, const Workspace& ws, int grid_items,
                                hipStream_t s, const KernelTiming& t, bool fp8 = false);

// 16 heads per wave for the scores, 64 latent columns per wave for P V,
// across the whole 576-wide row (decode_wide.hip)
bool decode_wide_supported(const Geom& g, bool fp8 = false);
bool decode_wide_reads_residue(const Geom& g);
hipError_t launch_decode_wide(const Geom& g, const QView& q, const void* ckv, const void* krope,
                              const Workspace& ws, int grid_items, hipStream_t s,
                              const KernelTiming& t, bool fp8 = false);

bool decode_mfma_supported(const Geom& g);
bool decode_mfma_reads_residue(const Geom& g);  // adds q~'s residue when the view has one
int decode_mfma_target_items(const Geom& g, int cus);
hipError_t launch_decode_mfma(const Geom& g, const QView& q, const void* ckv,
                              const void* krope, const Workspace& ws, int grid_items,
                              hipStream_t s, const KernelTiming& t);

// bf16 MFMA projections and the merge for the MFMA decode's partial layout
// ([slot][H][d_c] acc), see proj_mfma.hip.
bool proj_mfma_supported(const Geom& g);   // out projection / fused merge
bool absorb_mfma_supported(const Geom& g);
// With plan.hdr set, one extra workgroup of the launch also computes the
// split-KV plan (as launch_plan would).
hipError_t launch_absorb_q_mfma(const Geom& g, const __bf16* q_nope, const __bf16* q_rope,
                                const int32_t* q_pos, const int32_t* lens, const __bf16* w_uk,
                                __bf16* q_abs, int q_stride, int lo_off, float lat_scale,
                                float rope_scale, float theta, const PlanArgs& plan,
                                hipStream_t s);
hipError_t launch_combine_hc(const Geom& g, const Workspace& ws, float* latent_out,
                             float out_scale, hipStream_t s);
template <typename TO>
hipError_t launch_out_proj_mfma(const Geom& g, const float* latent, const __bf16* w_uv, TO* out,
                                float alpha_kv, hipStream_t s);
// combine_hc followed by launch_out_proj_mfma in one kernel (the merged
// latent stays in LDS); for the MFMA decodes' partial layout.
template <typename TO>
hipError_t launch_merge_out_proj(const Geom& g, const Workspace& ws, const __bf16* w_uv, TO* out,
                                 float alpha_kv, hipStream_t s);

}  // namespace mlra
