// Host side of the C ABI declared in include/mlra.h: argument validation,
// workspace layout, kernel selection and launches on the caller's stream.
// Nothing here allocates device memory or synchronises.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/mlra.h"
#include "internal.h"

using namespace mlra;

// One cached table per thread: the launches of a decode loop share theta and
// d_r, so pow() runs once per thread and configuration.
const RopeFreqs& mlra::rope_freqs(float theta, int dr) {
  thread_local RopeFreqs t;
  thread_local float t_theta = 0.f;
  thread_local int t_dr = -1;
  if (t_theta != theta || t_dr != dr) {
    for (int k = 0; k < dr / 2 && k < kMaxRopePairs; ++k)
      t.w[k] = std::pow((double)theta, -2.0 * (double)k / (double)dr);
    t_theta = theta;
    t_dr = dr;
  }
  return t;
}

namespace {

thread_local std::string g_detail;
thread_local hipEvent_t g_ev_before = nullptr;
thread_local hipEvent_t g_ev_after = nullptr;

mlra_status_t fail(mlra_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_detail = buf;
  return st;
}

mlra_status_t hip_fail(hipError_t e, const char* what) {
  return fail(MLRA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elt_size(mlra_dtype_t t) { return t == MLRA_BF16 ? 2 : 4; }

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Limits of the kernels (see the launchers).
constexpr int kMaxLatent = 1024, kMaxRope = 256, kMaxNope = 512, kMaxBranches = 8;
constexpr int kMaxHeadBranch = 1024;  // num_heads * num_branches

mlra_status_t check_cfg(const mlra_config_t* c) {
  if (!c) return fail(MLRA_ERR_INVALID_ARG, "cfg is NULL");
  if (c->num_heads < 1 || c->d_latent < 1 || c->d_rope < 0 || c->d_nope < 1 || c->d_v < 1)
    return fail(MLRA_ERR_INVALID_ARG, "sizes must be positive (d_rope >= 0)");
  if (c->d_rope % 2) return fail(MLRA_ERR_INVALID_ARG, "d_rope must be even");
  if (c->num_branches < 1 || c->d_latent % c->num_branches)
    return fail(MLRA_ERR_INVALID_ARG, "d_latent (%d) must be a multiple of num_branches (%d)",
                c->d_latent, c->num_branches);
  if (c->dtype != MLRA_BF16 && c->dtype != MLRA_FP32)
    return fail(MLRA_ERR_INVALID_ARG, "unknown dtype %d", (int)c->dtype);
  if (!(c->rope_theta > 0.f)) return fail(MLRA_ERR_INVALID_ARG, "rope_theta must be > 0");
  if (!std::isfinite(c->alpha_q) || !std::isfinite(c->alpha_kv) || !std::isfinite(c->sm_scale))
    return fail(MLRA_ERR_INVALID_ARG, "scales must be finite");
  if (c->kv_chunk < 0) return fail(MLRA_ERR_INVALID_ARG, "kv_chunk must be >= 0");
  if (c->decode_kernel < MLRA_KERNEL_AUTO || c->decode_kernel > MLRA_KERNEL_WIDE)
    return fail(MLRA_ERR_INVALID_ARG, "unknown decode_kernel %d", (int)c->decode_kernel);
  if (c->q_residue != 0 && c->q_residue != 1)
    return fail(MLRA_ERR_INVALID_ARG, "q_residue must be 0 or 1");
  if (c->q_residue && c->dtype != MLRA_BF16)
    return fail(MLRA_ERR_INVALID_ARG, "q_residue needs the bf16 dtype");
  if (c->d_latent > kMaxLatent || c->d_rope > kMaxRope || c->d_nope > kMaxNope ||
      c->num_branches > kMaxBranches || c->num_heads * c->num_branches > kMaxHeadBranch ||
      c->d_v > 4096)
    return fail(MLRA_ERR_UNSUPPORTED,
                "sizes beyond the supported range (d_latent<=%d, d_rope<=%d, d_nope<=%d, "
                "branches<=%d, heads*branches<=%d, d_v<=4096)",
                kMaxLatent, kMaxRope, kMaxNope, kMaxBranches, kMaxHeadBranch);
  return MLRA_OK;
}

float tau_of(const mlra_config_t* c) {
  return c->sm_scale > 0.f ? c->sm_scale : 1.0f / std::sqrt((float)(c->d_nope + c->d_rope));
}

mlra_status_t check_batch(int32_t batch, int32_t max_len) {
  if (batch < 0 || batch > 65535) return fail(MLRA_ERR_INVALID_ARG, "batch must be in [0, 65535]");
  if (max_len < 0) return fail(MLRA_ERR_INVALID_ARG, "max_len must be >= 0");
  if ((int64_t)batch * max_len > 0x7fffffffLL)
    return fail(MLRA_ERR_UNSUPPORTED, "batch * max_len must stay below 2^31 tokens");
  return MLRA_OK;
}

int64_t items_max(const mlra_config_t* c, int32_t batch, int32_t max_len) {
  const int64_t tokens = (int64_t)batch * max_len;
  if (tokens == 0) return 0;
  if (c->kv_chunk > 0) return (tokens + c->kv_chunk - 1) / c->kv_chunk;
  const int64_t by_min = (tokens + kMinChunk - 1) / kMinChunk;
  return by_min < kMaxAutoItems ? by_min : kMaxAutoItems;
}

// Elements per absorbed-query row in the workspace: q~ and rho, plus (bf16)
// the bf16 residue of q~ after them (QView), which the head-group and
// portable decodes add to their scores.
size_t q_row(const mlra_config_t* c) {
  return (size_t)c->d_latent + c->d_rope + (c->dtype == MLRA_BF16 ? c->d_latent : 0);
}

// The workspace's query rows for the decode kernel `kern`: the residue is
// written and read only where that kernel adds it to its scores.
// The caller's q_abs rows (mla_absorb_q, mla_decode_attn).
QView user_qview(const mlra_config_t* c, const void* q) {
  QView v;
  v.q = q;
  v.stride = c->d_latent + c->d_rope + (c->q_residue ? c->d_latent : 0);
  v.lo = c->q_residue ? c->d_latent + c->d_rope : 0;
  return v;
}

QView ws_qview(const mlra_config_t* c, const Geom& g, mlra_kernel_t kern, const void* q,
               bool fp8) {
  const bool lo = c->dtype == MLRA_BF16 &&
                  (kern == MLRA_KERNEL_PORTABLE ||
                   (kern == MLRA_KERNEL_HEAD_GROUP && decode_mfma_reads_residue(g)) ||
                   (kern == MLRA_KERNEL_BRANCH &&
                    decode_branch_reads_residue(g, fp8, c->q_residue != 0)) ||
                   (kern == MLRA_KERNEL_WIDE && decode_wide_reads_residue(g)));
  QView v;
  v.q = q;
  v.stride = (int)q_row(c);
  v.lo = lo ? c->d_latent + c->d_rope : 0;
  return v;
}

struct Layout {
  size_t hdr, prefix, m, l, acc, q_abs, latent, total;
  int64_t slots;
};

// Workspace layout for up to `items` work items (default: the most any plan
// for this batch and max_len can make).
Layout layout(const mlra_config_t* c, int32_t batch, int32_t max_len, int64_t items = -1) {
  Layout L;
  const size_t H = c->num_heads, n = c->num_branches, dc = c->d_latent, dr = c->d_rope;
  L.slots = (items >= 0 ? items : items_max(c, batch, max_len)) + batch;
  size_t off = 0;
  L.hdr = off;    off = round_up(off + sizeof(PlanHeader), 256);
  L.prefix = off; off = round_up(off + 4 * (size_t)(batch + 1), 256);
  L.m = off;      off = round_up(off + 4 * (size_t)L.slots * n * H, 256);
  L.l = off;      off = round_up(off + 4 * (size_t)L.slots * n * H, 256);
  L.acc = off;    off = round_up(off + 4 * (size_t)L.slots * dc * H, 256);
  L.q_abs = off;  off = round_up(off + elt_size(c->dtype) * (size_t)batch * H * q_row(c), 256);
  L.latent = off; off = round_up(off + 4 * (size_t)batch * H * dc, 256);
  L.total = off;
  return L;
}

Workspace carve(const Layout& L, void* base) {
  char* p = static_cast<char*>(base);
  Workspace w;
  w.hdr = reinterpret_cast<PlanHeader*>(p + L.hdr);
  w.prefix = reinterpret_cast<int32_t*>(p + L.prefix);
  w.m = reinterpret_cast<float*>(p + L.m);
  w.l = reinterpret_cast<float*>(p + L.l);
  w.acc = reinterpret_cast<float*>(p + L.acc);
  w.q_abs = p + L.q_abs;
  w.latent = reinterpret_cast<float*>(p + L.latent);
  return w;
}

constexpr int kMaxPrefillRows = 1 << 22;

// ---- per-device properties, filled once per device ----
constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
int g_cu_count[kMaxDevices];

mlra_status_t current_device(int* dev, int* cus) {
  int count = 0;
  hipError_t e = hipGetDeviceCount(&count);
  if (e != hipSuccess || count <= 0) {
    (void)hipGetLastError();
    return fail(MLRA_ERR_NO_DEVICE, "no HIP device available (%s)",
                e == hipSuccess ? "count is 0" : hipGetErrorString(e));
  }
  e = hipGetDevice(dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (*dev < 0 || *dev >= kMaxDevices) return fail(MLRA_ERR_UNSUPPORTED, "device id too large");
  hipError_t ae = hipSuccess;
  std::call_once(g_dev_once[*dev], [&] {
    int v = 0;
    ae = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, *dev);
    g_cu_count[*dev] = v > 0 ? v : 1;
  });
  if (ae != hipSuccess) return hip_fail(ae, "hipDeviceGetAttribute");
  *cus = g_cu_count[*dev];
  return MLRA_OK;
}

Geom make_geom(const mlra_config_t* c, int32_t batch, const mlra_cache_t* cache) {
  Geom g;
  g.B = batch;
  g.H = c->num_heads;
  g.dc = c->d_latent;
  g.dr = c->d_rope;
  g.dn = c->d_nope;
  g.dv = c->d_v;
  g.n = c->num_branches;
  g.max_len = cache ? cache->max_len : 0;
  g.ckv_bs = cache ? cache->ckv_batch_stride : 0;
  g.ckv_ts = cache ? cache->ckv_token_stride : 0;
  g.kr_bs = cache ? cache->krope_batch_stride : 0;
  g.kr_ts = cache ? cache->krope_token_stride : 0;
  return g;
}

#define TRY(x)                          \
  do {                                  \
    mlra_status_t st_ = (x);            \
    if (st_ != MLRA_OK) return st_;     \
  } while (0)

// fp8 cache scales: finite and within [2^-32, 2^32], so that their products
// with the query and output scales stay far from fp32's range limits
mlra_status_t check_fp8_scales(float sc, float sr) {
  auto ok = [](float v) { return std::isfinite(v) && v >= 0x1p-32f && v <= 0x1p32f; };
  if (!ok(sc) || !ok(sr))
    return fail(MLRA_ERR_INVALID_ARG, "fp8 cache scales must be finite and in [2^-32, 2^32]");
  return MLRA_OK;
}

// Multipliers that the decode folds into q~, rho and the merged latent: the
// fp8 cache's scales, else 1.
float lat_mul(const mlra_cache_t* k) { return k && k->fp8 ? k->ckv_scale : 1.f; }
float rope_mul(const mlra_cache_t* k) { return k && k->fp8 ? k->krope_scale : 1.f; }

mlra_status_t check_cache(const mlra_config_t* c, const mlra_cache_t* k, int32_t batch) {
  if (!k) return fail(MLRA_ERR_INVALID_ARG, "cache is NULL");
  mlra_status_t st = check_batch(batch, k->max_len);
  if (st != MLRA_OK) return st;
  if (batch == 0) return MLRA_OK;
  if (!k->cache_lens) return fail(MLRA_ERR_INVALID_ARG, "cache_lens is NULL");
  if (k->max_len == 0) return MLRA_OK;
  if (!k->ckv || (c->d_rope > 0 && !k->krope))
    return fail(MLRA_ERR_INVALID_ARG, "cache pointers are NULL");
  if (!aligned16(k->ckv) || (c->d_rope > 0 && !aligned16(k->krope)))
    return fail(MLRA_ERR_INVALID_ARG, "cache base pointers must be 16-byte aligned");
  if (k->fp8 != 0 && k->fp8 != 1) return fail(MLRA_ERR_INVALID_ARG, "cache fp8 must be 0 or 1");
  if (k->fp8) {
    if (c->dtype != MLRA_BF16)
      return fail(MLRA_ERR_INVALID_ARG, "an fp8 cache needs the bf16 dtype");
    TRY(check_fp8_scales(k->ckv_scale, k->krope_scale));
  }
  const int64_t e = k->fp8 ? 1 : (int64_t)elt_size(c->dtype);
  if (k->ckv_token_stride < 1 || k->ckv_batch_stride < 0 ||
      (c->d_rope > 0 && (k->krope_token_stride < 1 || k->krope_batch_stride < 0)))
    return fail(MLRA_ERR_INVALID_ARG, "cache strides: token stride >= 1, batch stride >= 0");
  // a row must fit its token stride: the MFMA kernels bound each sequence's
  // rows by max_len * token stride bytes, the portable kernel reads whole rows
  if (k->ckv_token_stride < c->d_latent || (c->d_rope > 0 && k->krope_token_stride < c->d_rope))
    return fail(MLRA_ERR_INVALID_ARG, "cache token strides must be >= the row widths (%d, %d)",
                c->d_latent, c->d_rope);
  if ((k->ckv_token_stride * e) % 16 || (k->ckv_batch_stride * e) % 16 ||
      (c->d_rope > 0 && ((k->krope_token_stride * e) % 16 || (k->krope_batch_stride * e) % 16)))
    return fail(MLRA_ERR_INVALID_ARG, "cache strides must be multiples of 16 bytes");
  return MLRA_OK;
}

mlra_status_t check_ptr(const void* p, const char* name) {
  if (!p) return fail(MLRA_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(MLRA_ERR_INVALID_ARG, "%s must be 16-byte aligned", name);
  return MLRA_OK;
}

#define TRY_HIP(x, what)                       \
  do {                                         \
    hipError_t e_ = (x);                       \
    if (e_ != hipSuccess) return hip_fail(e_, what); \
  } while (0)

// ---- launches (arguments already validated) ----

// Query absorption. When `plan` is given and the MFMA kernel runs, the split-KV
// plan rides along in that launch and *plan_done is set.
// Query absorption into rows described by `q` (stride, residue offset).
// lat_m and rope_m multiply q~ and rho on top of alpha_q tau and tau (an fp8
// cache's scales).
mlra_status_t run_absorb(const mlra_config_t* c, const Geom& g, const void* q_nope,
                         const void* q_rope, const int32_t* q_pos, const int32_t* lens,
                         const void* w_uk, const QView& q, hipStream_t s,
                         const PlanArgs* plan = nullptr, bool* plan_done = nullptr,
                         float lat_m = 1.f, float rope_m = 1.f) {
  const float tau = tau_of(c);
  const float lat_scale = c->alpha_q * tau * lat_m, rope_scale = tau * rope_m;
  void* q_abs = const_cast<void*>(q.q);
  hipError_t e;
  if (c->dtype == MLRA_BF16 && absorb_mfma_supported(g)) {
    PlanArgs none{};
    e = launch_absorb_q_mfma(g, (const __bf16*)q_nope, (const __bf16*)q_rope, q_pos, lens,
                             (const __bf16*)w_uk, (__bf16*)q_abs, q.stride, q.lo, lat_scale,
                             rope_scale, c->rope_theta, plan ? *plan : none, s);
    if (plan && plan_done) *plan_done = true;
  } else if (c->dtype == MLRA_BF16)
    e = launch_absorb_q_generic<__bf16>(g, (const __bf16*)q_nope, (const __bf16*)q_rope, q_pos,
                                        lens, (const __bf16*)w_uk, (__bf16*)q_abs, q.stride, q.lo,
                                        lat_scale, rope_scale, c->rope_theta, s);
  else
    e = launch_absorb_q_generic<float>(g, (const float*)q_nope, (const float*)q_rope, q_pos, lens,
                                       (const float*)w_uk, (float*)q_abs, q.stride, 0, lat_scale,
                                       rope_scale, c->rope_theta, s);
  TRY_HIP(e, "absorb_q launch");
  return MLRA_OK;
}

// The decode kernel that runs for this configuration and cache view.
mlra_status_t select_kernel(const mlra_config_t* c, const Geom& g, const mlra_cache_t* k,
                            mlra_kernel_t* out) {
  // the MFMA kernels address one sequence's rows through 31-bit buffer offsets
  const bool mfma_ok = c->dtype == MLRA_BF16 &&
                       (int64_t)k->max_len * k->ckv_token_stride * 2 < 0x7fffffffLL &&
                       (int64_t)k->max_len * k->krope_token_stride * 2 < 0x7fffffffLL;
  const bool fp8 = k->fp8 != 0;
  const bool branch_ok = mfma_ok && decode_branch_supported(g, fp8);
  const bool group_ok = mfma_ok && !fp8 && decode_mfma_supported(g);
  const bool wide_ok = mfma_ok && decode_wide_supported(g, fp8);
  mlra_kernel_t kern = c->decode_kernel;
  if (kern == MLRA_KERNEL_AUTO)
    kern = branch_ok ? MLRA_KERNEL_BRANCH
         : wide_ok   ? MLRA_KERNEL_WIDE
         : group_ok  ? MLRA_KERNEL_HEAD_GROUP
                     : MLRA_KERNEL_PORTABLE;
  if ((kern == MLRA_KERNEL_BRANCH && !branch_ok) || (kern == MLRA_KERNEL_HEAD_GROUP && !group_ok) ||
      (kern == MLRA_KERNEL_WIDE && !wide_ok))
    return fail(MLRA_ERR_UNSUPPORTED, "decode_kernel %d does not support this configuration",
                (int)kern);
  *out = kern;
  return MLRA_OK;
}

// Work items the automatic plan aims for with decode kernel `kern`: enough
// workgroups for every CU.
int target_items(const Geom& g, int cus, mlra_kernel_t kern) {
  int target;
  if (kern == MLRA_KERNEL_BRANCH)
    target = cus / decode_branch_wgs_per_item(g);
  else if (kern == MLRA_KERNEL_WIDE)
    target = cus;  // one workgroup (all heads) per item and CU
  else if (kern == MLRA_KERNEL_HEAD_GROUP)
    target = decode_mfma_target_items(g, cus);
  else
    target = cus * 4 / g.H;
  if (target < 1) target = 1;
  if (target > kMaxAutoItems) target = kMaxAutoItems;
  return target;
}

// The split-KV plan for this decode: kernel choice and work-item target.
mlra_status_t plan_for(const mlra_config_t* c, const Geom& g, int cus, const mlra_cache_t* k,
                       const Workspace& ws, const Layout& L, mlra_kernel_t* kern, PlanArgs* a) {
  const int64_t imax = L.slots - g.B;
  TRY(select_kernel(c, g, k, kern));
  int target = target_items(g, cus, *kern);
  if (target > imax && imax > 0) target = (int)imax;
  a->lens = k->cache_lens;
  a->B = g.B;
  a->max_len = g.max_len;
  a->target_items = target;
  a->forced_chunk = c->kv_chunk;
  a->hdr = ws.hdr;
  a->prefix = ws.prefix;
  return MLRA_OK;
}

// Split-KV decode into the workspace partials, after the plan (launched here
// unless plan_done). *fast tells which kind of decode ran: an MFMA kernel
// (partials acc / l as fp16 [slot][H][d_c]) or the portable one (acc as fp32
// [slot][d_c][H]); the merge must match.
mlra_status_t run_decode(const mlra_config_t* c, const Geom& g, const QView& q,
                         const mlra_cache_t* k, const Workspace& ws, const Layout& L,
                         mlra_kernel_t kern, const PlanArgs& plan, bool plan_done, bool* fast_out,
                         hipStream_t s) {
  const int64_t imax = L.slots - g.B;
  if (!plan_done)
    TRY_HIP(launch_plan(plan.lens, plan.B, plan.max_len, plan.target_items, plan.forced_chunk, ws,
                        s),
            "plan launch");
  if (imax > 0) {
    KernelTiming t;
    t.start = g_ev_before;
    t.stop = g_ev_after;
    hipError_t e;
    const bool fp8 = k->fp8 != 0;
    if (kern == MLRA_KERNEL_BRANCH)
      e = launch_decode_branch(g, q, k->ckv, k->krope, ws, (int)imax, s, t, fp8);
    else if (kern == MLRA_KERNEL_HEAD_GROUP)
      e = launch_decode_mfma(g, q, k->ckv, k->krope, ws, (int)imax, s, t);
    else if (kern == MLRA_KERNEL_WIDE)
      e = launch_decode_wide(g, q, k->ckv, k->krope, ws, (int)imax, s, t, fp8);
    else if (fp8)
      e = launch_decode_generic<__bf16, uint8_t>(g, q, (const uint8_t*)k->ckv,
                                                 (const uint8_t*)k->krope, ws, (int)imax, s, t);
    else if (c->dtype == MLRA_BF16)
      e = launch_decode_generic<__bf16, __bf16>(g, q, (const __bf16*)k->ckv,
                                                (const __bf16*)k->krope, ws, (int)imax, s, t);
    else
      e = launch_decode_generic<float, float>(g, q, (const float*)k->ckv, (const float*)k->krope,
                                              ws, (int)imax, s, t);
    TRY_HIP(e, "decode launch");
  }
  *fast_out = kern != MLRA_KERNEL_PORTABLE;
  return MLRA_OK;
}

mlra_status_t run_merge(const Geom& g, const Workspace& ws, bool fast, float* latent_out,
                        float out_scale, hipStream_t s) {
  TRY_HIP(fast ? launch_combine_hc(g, ws, latent_out, out_scale, s)
               : launch_combine(g, ws, latent_out, out_scale, s),
          "combine launch");
  return MLRA_OK;
}

mlra_status_t run_out_proj(const mlra_config_t* c, const Geom& g, const float* latent,
                           const void* w_uv, void* out, mlra_dtype_t od, hipStream_t s) {
  hipError_t e;
  if (c->dtype == MLRA_BF16 && proj_mfma_supported(g)) {
    if (od == MLRA_BF16)
      e = launch_out_proj_mfma<__bf16>(g, latent, (const __bf16*)w_uv, (__bf16*)out, c->alpha_kv, s);
    else
      e = launch_out_proj_mfma<float>(g, latent, (const __bf16*)w_uv, (float*)out, c->alpha_kv, s);
  } else if (c->dtype == MLRA_BF16) {
    if (od == MLRA_BF16)
      e = launch_out_proj_generic<__bf16, __bf16>(g, latent, (const __bf16*)w_uv, (__bf16*)out,
                                                  c->alpha_kv, s);
    else
      e = launch_out_proj_generic<__bf16, float>(g, latent, (const __bf16*)w_uv, (float*)out,
                                                 c->alpha_kv, s);
  } else {
    if (od == MLRA_BF16)
      e = launch_out_proj_generic<float, __bf16>(g, latent, (const float*)w_uv, (__bf16*)out,
                                                 c->alpha_kv, s);
    else
      e = launch_out_proj_generic<float, float>(g, latent, (const float*)w_uv, (float*)out,
                                                c->alpha_kv, s);
  }
  TRY_HIP(e, "out_proj launch");
  return MLRA_OK;
}

// Debug build (MLRA_DEBUG_BOUNDS): the plan header's bounds word after the
// call, where every device bounds check that failed left its site; the
// release build checks nothing and waits for nothing.
mlra_status_t debug_bounds(const Workspace& ws, hipStream_t s) {
#ifdef MLRA_DEBUG_BOUNDS
  PlanHeader h;
  TRY_HIP(hipMemcpyAsync(&h, ws.hdr, sizeof h, hipMemcpyDeviceToHost, s), "bounds word copy");
  TRY_HIP(hipStreamSynchronize(s), "bounds word sync");
  if (h.bounds_fail != 0)
    return fail(MLRA_ERR_BOUNDS, "device bounds check failed (site %d)", h.bounds_fail);
#else
  (void)ws;
  (void)s;
#endif
  return MLRA_OK;
}

// The whole decode step on a carved workspace: plan (inside absorb_q's
// launch when the MFMA absorption runs), absorb_q, split-KV decode, then the
// fused merge + output projection (or combine and out_proj).
mlra_status_t run_step_body(const mlra_config_t* cfg, int32_t batch, int cus, const void* q_nope,
                       const void* q_rope, const int32_t* q_pos, const void* w_uk,
                       const void* w_uv, const mlra_cache_t* cache, const Layout& L,
                       const Workspace& ws, void* out, mlra_dtype_t out_dtype, hipStream_t s) {
  const Geom g = make_geom(cfg, batch, cache);
  mlra_kernel_t kern;
  PlanArgs plan;
  TRY(plan_for(cfg, g, cus, cache, ws, L, &kern, &plan));
  bool plan_done = false;
  const QView qv = ws_qview(cfg, g, kern, ws.q_abs, cache->fp8 != 0);
  // an fp8 cache's scales go into q~, rho and the merged latent
  const float sc = lat_mul(cache), sr = rope_mul(cache);
  TRY(run_absorb(cfg, g, q_nope, q_rope, q_pos, cache->cache_lens, w_uk, qv, s, &plan,
                 &plan_done, sc, sr));
  bool fast = false;
  TRY(run_decode(cfg, g, qv, cache, ws, L, kern, plan, plan_done, &fast, s));
  if (fast && cfg->dtype == MLRA_BF16 && proj_mfma_supported(g)) {
    // merge and out projection in one kernel: the latent stays on chip
    const __bf16* wv = static_cast<const __bf16*>(w_uv);
    const float akv = cfg->alpha_kv * sc;
    TRY_HIP(out_dtype == MLRA_BF16
                ? launch_merge_out_proj<__bf16>(g, ws, wv, static_cast<__bf16*>(out), akv, s)
                : launch_merge_out_proj<float>(g, ws, wv, static_cast<float*>(out), akv, s),
            "merge_out launch");
    return MLRA_OK;
  }
  TRY(run_merge(g, ws, fast, ws.latent, sc, s));
  return run_out_proj(cfg, g, ws.latent, w_uv, out, out_dtype, s);
}

mlra_status_t run_step(const mlra_config_t* cfg, int32_t batch, int cus, const void* q_nope,
                       const void* q_rope, const int32_t* q_pos, const void* w_uk,
                       const void* w_uv, const mlra_cache_t* cache, const Layout& L,
                       const Workspace& ws, void* out, mlra_dtype_t out_dtype, hipStream_t s) {
  TRY(run_step_body(cfg, batch, cus, q_nope, q_rope, q_pos, w_uk, w_uv, cache, L, ws, out,
                    out_dtype, s));
  return debug_bounds(ws, s);
}

// ---- the scratch of mlra_decode_noalloc ----
// A file-scope device array: each GPU the library runs on holds its own copy
// (allocated when the code object loads there, kept until the process ends).
// In host code `scratch` names a host-side stand-in, not a device address:
// every use goes through the per-device address from hipGetSymbolAddress,
// taken once per device with that device current. Every call on a GPU shares
// that GPU's copy; nothing in it needs to start at zero (the plan and the
// partials are written before they are read), and calls that overlap on one
// GPU race.
constexpr size_t kScratchBytes = size_t(128) << 20;
__device__ __attribute__((aligned(256))) char scratch[kScratchBytes];
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

mlra_status_t scratch_base(int dev, void** base) {
  std::call_once(g_scratch_once[dev], [&] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess) return hip_fail(g_scratch_err[dev], "hipGetSymbolAddress");
  if (!g_scratch_ptr[dev] || (reinterpret_cast<uintptr_t>(g_scratch_ptr[dev]) & 255u))
    return fail(MLRA_ERR_HIP, "scratch address missing or misaligned");
  *base = g_scratch_ptr[dev];
  return MLRA_OK;
}

}  // namespace

extern "C" {

const char* mlra_status_string(mlra_status_t s) {
  switch (s) {
    case MLRA_OK: return "MLRA_OK";
    case MLRA_ERR_INVALID_ARG: return "MLRA_ERR_INVALID_ARG";
    case MLRA_ERR_UNSUPPORTED: return "MLRA_ERR_UNSUPPORTED";
    case MLRA_ERR_WORKSPACE: return "MLRA_ERR_WORKSPACE";
    case MLRA_ERR_NO_DEVICE: return "MLRA_ERR_NO_DEVICE";
    case MLRA_ERR_HIP: return "MLRA_ERR_HIP";
    case MLRA_ERR_BOUNDS: return "MLRA_ERR_BOUNDS";
  }
  return "MLRA_ERR_UNKNOWN";
}

const char* mlra_last_error_detail(void) { return g_detail.c_str(); }

int mlra_bounds_checks(void) {
#ifdef MLRA_DEBUG_BOUNDS
  return 1;
#else
  return 0;
#endif
}

mlra_status_t mlra_set_kernel_timing(void* before, void* after) {
  if ((before == nullptr) != (after == nullptr))
    return fail(MLRA_ERR_INVALID_ARG, "give both events or neither");
  g_ev_before = static_cast<hipEvent_t>(before);
  g_ev_after = static_cast<hipEvent_t>(after);
  return MLRA_OK;
}

mlra_status_t mlra_workspace_size(const mlra_config_t* cfg, int32_t batch, int32_t max_len,
                                  size_t* bytes) {
  g_detail.clear();
  TRY(check_cfg(cfg));
  TRY(check_batch(batch, max_len));
  if (!bytes) return fail(MLRA_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = layout(cfg, batch, max_len).total;
  return MLRA_OK;
}

mlra_status_t mla_absorb_q(const mlra_config_t* cfg, int32_t batch, const void* q_nope,
                           const void* q_rope, const int32_t* q_pos, const int32_t* cache_lens,
                           const void* w_uk, void* q_abs, void* stream) {
  g_detail.clear();
  TRY(check_cfg(cfg));
  TRY(check_batch(batch, 0));
  if (batch == 0) return MLRA_OK;
  TRY(check_ptr(q_nope, "q_nope"));
  if (cfg->d_rope > 0) TRY(check_ptr(q_rope, "q_rope"));
  TRY(check_ptr(w_uk, "w_uk"));
  TRY(check_ptr(q_abs, "q_abs"));
  if (!q_pos && !cache_lens) return fail(MLRA_ERR_INVALID_ARG, "need q_pos or cache_lens");
  int dev, cus;
  TRY(current_device(&dev, &cus));
  Geom g = make_geom(cfg, batch, nullptr);
  g.max_len = 0x7fffffff;  // cache_lens - 1 is used as given (clamped below by 0)
  const QView qv = user_qview(cfg, q_abs);
  return run_absorb(cfg, g, q_nope, q_rope, q_pos, cache_lens, w_uk, qv,
                    static_cast<hipStream_t>(stream));
}

mlra_status_t mla_decode_attn(const mlra_config_t* cfg, int32_t batch, const void* q_abs,
                              const mlra_cache_t* cache, void* workspace, size_t ws_bytes,
                              float* latent_out, void* stream) {
  g_detail.clear();
  TRY(check_cfg(cfg));
  TRY(check_cache(cfg, cache, batch));
  if (batch == 0) return MLRA_OK;
  TRY(check_ptr(q_abs, "q_abs"));
  TRY(check_ptr(latent_out, "latent_out"));
  const Layout L = layout(cfg, batch, cache->max_len);
  if (!workspace || ws_bytes < L.total)
    return fail(MLRA_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", L.total, ws_bytes);
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(MLRA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  int dev, cus;
  TRY(current_device(&dev, &cus));
  const Geom g = make_geom(cfg, batch, cache);
  const Workspace ws = carve(L, workspace);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  mlra_kernel_t kern;
  PlanArgs plan;
  TRY(plan_for(cfg, g, cus, cache, ws, L, &kern, &plan));
  bool fast = false;
  QView qv = user_qview(cfg, q_abs);
  if (cache->fp8) {
    // the cache's scales go into a copy of the query in the workspace
    const QView scaled = ws_qview(cfg, g, kern, ws.q_abs, true);
    TRY_HIP(launch_scale_q(g, qv, scaled, lat_mul(cache), rope_mul(cache), s), "scale_q launch");
    qv = scaled;
  }
  TRY(run_decode(cfg, g, qv, cache, ws, L, kern, plan, false, &fast, s));
  TRY(run_merge(g, ws, fast, latent_out, lat_mul(cache), s));
  return debug_bounds(ws, s);
}

}  // extern "C"

namespace {

mlra_status_t append_impl(const mlra_config_t* cfg, int32_t batch, const float* new_rows,
                          const float* gain, float eps, void* ckv, void* krope,
                          int64_t ckv_batch_stride, int64_t ckv_token_stride,
                          int64_t krope_batch_stride, int64_t krope_token_stride,
                          int32_t* cache_lens, int32_t max_len, bool fp8, float ckv_scale,
                          float krope_scale, void* stream) {
  g_detail.clear();
  TRY(check_cfg(cfg));
  TRY(check_batch(batch, max_len));
  if (fp8) {
    if (cfg->dtype != MLRA_BF16)
      return fail(MLRA_ERR_INVALID_ARG, "an fp8 cache needs the bf16 dtype");
    TRY(check_fp8_scales(ckv_scale, krope_scale));
  }
  if (batch == 0 || max_len == 0) return MLRA_OK;
  if (!new_rows || !cache_lens || !ckv || (cfg->d_rope > 0 && !krope))
    return fail(MLRA_ERR_INVALID_ARG, "new_rows, cache_lens and the cache pointers must be set");
  if (!std::isfinite(eps) || eps < 0.f) return fail(MLRA_ERR_INVALID_ARG, "eps must be >= 0");
  if (ckv_token_stride < cfg->d_latent || ckv_batch_stride < 0 ||
      (cfg->d_rope > 0 && (krope_token_stride < cfg->d_rope || krope_batch_stride < 0)))
    return fail(MLRA_ERR_INVALID_ARG,
                "cache strides: token stride >= the row width, batch stride >= 0");
  int dev, cus;
  TRY(current_device(&dev, &cus));
  AppendArgs a;
  a.rows = new_rows;
  a.gain = gain;
  a.ckv = ckv;
  a.krope = krope;
  a.ckv_bs = ckv_batch_stride;
  a.ckv_ts = ckv_token_stride;
  a.kr_bs = krope_batch_stride;
  a.kr_ts = krope_token_stride;
  a.lens = cache_lens;
  a.max_len = max_len;
  a.d_c = cfg->d_latent;
  a.d_r = cfg->d_rope;
  a.eps = eps;
  a.theta = cfg->rope_theta;
  a.ckv_scale = fp8 ? ckv_scale : 1.f;
  a.kr_scale = fp8 ? krope_scale : 1.f;
  const CacheElt elt = fp8 ? CacheElt::kFP8
                     : cfg->dtype == MLRA_BF16 ? CacheElt::kBF16 : CacheElt::kF32;
  TRY_HIP(launch_cache_append(a, elt, batch, static_cast<hipStream_t>(stream)),
          "cache_append launch");
  return MLRA_OK;
}

}  // namespace

extern "C" {

mlra_status_t mlra_cache_append(const mlra_config_t* cfg, int32_t batch, const float* new_rows,
                                const float* gain, float eps, void* ckv, void* krope,
                                int64_t ckv_batch_stride, int64_t ckv_token_stride,
                                int64_t krope_batch_stride, int64_t krope_token_stride,
                                int32_t* cache_lens, int32_t max_len, void* stream) {
  return append_impl(cfg, batch, new_rows, gain, eps, ckv, krope, ckv_batch_stride,
                     ckv_token_stride, krope_batch_stride, krope_token_stride, cache_lens,
                     max_len, false, 1.f, 1.f, stream);
}

mlra_status_t mlra_cache_append_fp8(const mlra_config_t* cfg, int32_t batch,
                                    const float* new_rows, const float* gain, float eps,
                                    void* ckv, void* krope, int64_t ckv_batch_stride,
                                    int64_t ckv_token_stride, int64_t krope_batch_stride,
                                    int64_t krope_token_stride, int32_t* cache_lens,
                                    int32_t max_len, float ckv_scale, float krope_scale,
                                    void* stream) {
  return append_impl(cfg, batch, new_rows, gain, eps, ckv, krope, ckv_batch_stride,
                     ckv_token_stride, krope_batch_stride, krope_token_stride, cache_lens,
                     max_len, true, ckv_scale, krope_scale, stream);
}

mlra_status_t mlra_prefill(const mlra_config_t* cfg_in, int32_t num_branches, int32_t batch,
                           const void* q_nope, const void* q_rope, const void* w_uk,
                           const void* w_uv, const mlra_cache_t* cache, void* out,
                           mlra_dtype_t out_dtype, void* stream) {
  g_detail.clear();
  if (!cfg_in) return fail(MLRA_ERR_INVALID_ARG, "cfg is NULL");
  mlra_config_t cfg = *cfg_in;
  cfg.num_branches = num_branches;
  TRY(check_cfg(&cfg));
  TRY(check_cache(&cfg, cache, batch));
  if (out_dtype != MLRA_BF16 && out_dtype != MLRA_FP32)
    return fail(MLRA_ERR_INVALID_ARG, "unknown out_dtype");
  if (cache->fp8) return fail(MLRA_ERR_UNSUPPORTED, "the prefill reads bf16 caches only");
  if (batch == 0 || cache->max_len == 0) return MLRA_OK;
  TRY(check_ptr(q_nope, "q_nope"));
  if (cfg.d_rope > 0) TRY(check_ptr(q_rope, "q_rope"));
  TRY(check_ptr(w_uk, "w_uk"));
  TRY(check_ptr(w_uv, "w_uv"));
  TRY(check_ptr(out, "out"));
  const Geom g = make_geom(&cfg, batch, cache);
  const bool ranges_ok = (int64_t)cache->max_len * cache->ckv_token_stride * 2 < 0x7fffffffLL &&
                         (int64_t)cache->max_len * cache->krope_token_stride * 2 < 0x7fffffffLL;
  if (cfg.dtype != MLRA_BF16 || !prefill_branch_supported(g) || !ranges_ok)
    return fail(MLRA_ERR_UNSUPPORTED,
                "prefill supports bf16 MLRA-4 at d_latent 512, d_rope 64, d_nope 128, d_v 128 "
                "and per-sequence byte ranges below 2^31");
  if ((int64_t)batch * cache->max_len > kMaxPrefillRows)
    return fail(MLRA_ERR_UNSUPPORTED, "batch * max_len must stay at or below %d prompt rows",
                kMaxPrefillRows);
  int dev, cus;
  TRY(current_device(&dev, &cus));
  KernelTiming timing;
  timing.start = g_ev_before;
  timing.stop = g_ev_after;
  TRY_HIP(launch_prefill_branch(g, cache->max_len, q_nope, q_rope, w_uk, w_uv, cache->ckv,
                                cache->krope, cache->cache_lens, out, out_dtype == MLRA_BF16,
                                tau_of(&cfg), cfg.alpha_q, cfg.alpha_kv, cfg.rope_theta, static_cast<hipStream_t>(stream),
                                timing),
          "prefill launch");
  return MLRA_OK;
}

mlra_status_t mla_prefill_workspace_size(const mlra_config_t* cfg, int32_t batch,
                                         int32_t max_len, size_t* bytes) {
  g_detail.clear();
  TRY(check_cfg(cfg));
  TRY(check_batch(batch, max_len));
  if (!bytes) return fail(MLRA_ERR_INVALID_ARG, "bytes is NULL");
  mlra_config_t c = *cfg;
  c.num_branches = 1;
  *bytes = round_up(prefill_mha_workspace(make_geom(&c, batch, nullptr), max_len), 256);
  return MLRA_OK;
}

mlra_status_t mla_prefill(const mlra_config_t* cfg_in, int32_t batch, const void* q_nope,
                          const void* q_rope, const void* w_uk, const void* w_uv,
                          const mlra_cache_t* cache, void* workspace, size_t ws_bytes, void* out,
                          mlra_dtype_t out_dtype, void* stream) {
  g_detail.clear();
  if (!cfg_in) return fail(MLRA_ERR_INVALID_ARG, "cfg is NULL");
  mlra_config_t cfg = *cfg_in;
  cfg.num_branches = 1;
  TRY(check_cfg(&cfg));
  TRY(check_cache(&cfg, cache, batch));
  if (out_dtype != MLRA_BF16 && out_dtype != MLRA_FP32)
    return fail(MLRA_ERR_INVALID_ARG, "unknown out_dtype");
  if (cache->fp8) return fail(MLRA_ERR_UNSUPPORTED, "the prefill reads bf16 caches only");
  const Geom g = make_geom(&cfg, batch, cache);
  const bool ranges_ok = (int64_t)cache->max_len * cache->ckv_token_stride * 2 < 0x7fffffffLL &&
                         (int64_t)cache->max_len * cache->krope_token_stride * 2 < 0x7fffffffLL &&
                         (int64_t)cache->max_len * 256 < 0x7fffffffLL;
  if (cfg.dtype != MLRA_BF16 || !prefill_mha_supported(g) || !ranges_ok)
    return fail(MLRA_ERR_UNSUPPORTED,
                "mla_prefill supports bf16 MLA at d_latent 512, d_rope 64, d_nope 128, d_v 128 "
                "and per-sequence byte ranges below 2^31");
  if ((int64_t)batch * cache->max_len > kMaxPrefillRows)
    return fail(MLRA_ERR_UNSUPPORTED, "batch * max_len must stay at or below %d prompt rows",
                kMaxPrefillRows);
  if (batch == 0 || cache->max_len == 0) return MLRA_OK;
  TRY(check_ptr(q_nope, "q_nope"));
  TRY(check_ptr(q_rope, "q_rope"));
  TRY(check_ptr(w_uk, "w_uk"));
  TRY(check_ptr(w_uv, "w_uv"));
  TRY(check_ptr(out, "out"));
  const size_t need = round_up(prefill_mha_workspace(g, cache->max_len), 256);
  if (!workspace || ws_bytes < need)
    return fail(MLRA_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need, ws_bytes);
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(MLRA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  int dev, cus;
  TRY(current_device(&dev, &cus));
  KernelTiming timing;
  timing.start = g_ev_before;
  timing.stop = g_ev_after;
  TRY_HIP(launch_prefill_mha(g, cache->max_len, q_nope, q_rope, w_uk, w_uv, cache->ckv,
                             cache->krope, cache->cache_lens, workspace, out,
                             out_dtype == MLRA_BF16, tau_of(&cfg), cfg.alpha_q, cfg.alpha_kv,
                             cfg.rope_theta, static_cast<hipStream_t>(stream), timing),
          "mla_prefill launch");
  return MLRA_OK;
}

mlra_status_t mlra_select_decode_kernel(const mlra_config_t* cfg, int32_t batch,
                                        const mlra_cache_t* cache, mlra_kernel_t* kernel) {
  g_detail.clear();
  TRY(check_cfg(cfg));
  TRY(check_cache(cfg, cache, batch));
  if (!kernel) return fail(MLRA_ERR_INVALID_ARG, "kernel is NULL");
  return select_kernel(cfg, make_geom(cfg, batch, cache), cache, kernel);
}

mlra_status_t mla_out_proj(const mlra_config_t* cfg, int32_t batch, const float* latent_out,
                           const void* w_uv, void* out, mlra_dtype_t out_dtype, void* stream) {
  g_detail.clear();
  TRY(check_cfg(cfg));
  TRY(check_batch(batch, 0));
  if (out_dtype != MLRA_BF16 && out_dtype != MLRA_FP32)
    return fail(MLRA_ERR_INVALID_ARG, "unknown out_dtype");
  if (batch == 0) return MLRA_OK;
  TRY(check_ptr(latent_out, "latent_out"));
  TRY(check_ptr(w_uv, "w_uv"));
  TRY(check_ptr(out, "out"));
  int dev, cus;
  TRY(current_device(&dev, &cus));
  return run_out_proj(cfg, make_geom(cfg, batch, nullptr), latent_out, w_uv, out, out_dtype,
                      static_cast<hipStream_t>(stream));
}

mlra_status_t mlra_decode(const mlra_config_t* cfg_in, int32_t num_branches, int32_t batch,
                          const void* q_nope, const void* q_rope, const int32_t* q_pos,
                          const void* w_uk, const void* w_uv, const mlra_cache_t* cache,
                          void* workspace, size_t ws_bytes, void* out, mlra_dtype_t out_dtype,
                          void* stream) {
  g_detail.clear();
  if (!cfg_in) return fail(MLRA_ERR_INVALID_ARG, "cfg is NULL");
  mlra_config_t cfg = *cfg_in;
  cfg.num_branches = num_branches;
  TRY(check_cfg(&cfg));
  TRY(check_cache(&cfg, cache, batch));
  if (out_dtype != MLRA_BF16 && out_dtype != MLRA_FP32)
    return fail(MLRA_ERR_INVALID_ARG, "unknown out_dtype");
  if (batch == 0) return MLRA_OK;
  TRY(check_ptr(q_nope, "q_nope"));
  if (cfg.d_rope > 0) TRY(check_ptr(q_rope, "q_rope"));
  TRY(check_ptr(w_uk, "w_uk"));
  TRY(check_ptr(w_uv, "w_uv"));
  TRY(check_ptr(out, "out"));
  const Layout L = layout(&cfg, batch, cache->max_len);
  if (!workspace || ws_bytes < L.total)
    return fail(MLRA_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", L.total, ws_bytes);
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(MLRA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  int dev, cus;
  TRY(current_device(&dev, &cus));
  return run_step(&cfg, batch, cus, q_nope, q_rope, q_pos, w_uk, w_uv, cache, L,
                  carve(L, workspace), out, out_dtype, static_cast<hipStream_t>(stream));
}

mlra_status_t mlra_decode_noalloc(const mlra_config_t* cfg_in, int32_t num_branches,
                                  int32_t batch, const void* q_nope, const void* q_rope,
                                  const int32_t* q_pos, const void* w_uk, const void* w_uv,
                                  const mlra_cache_t* cache, void* out, mlra_dtype_t out_dtype,
                                  void* stream) {
  g_detail.clear();
  if (!cfg_in) return fail(MLRA_ERR_INVALID_ARG, "cfg is NULL");
  mlra_config_t cfg = *cfg_in;
  cfg.num_branches = num_branches;
  TRY(check_cfg(&cfg));
  TRY(check_cache(&cfg, cache, batch));
  if (out_dtype != MLRA_BF16 && out_dtype != MLRA_FP32)
    return fail(MLRA_ERR_INVALID_ARG, "unknown out_dtype");
  if (batch == 0) return MLRA_OK;
  TRY(check_ptr(q_nope, "q_nope"));
  if (cfg.d_rope > 0) TRY(check_ptr(q_rope, "q_rope"));
  TRY(check_ptr(w_uk, "w_uk"));
  TRY(check_ptr(w_uv, "w_uv"));
  TRY(check_ptr(out, "out"));
  int dev, cus;
  TRY(current_device(&dev, &cus));
  void* base = nullptr;
  TRY(scratch_base(dev, &base));
  // Sized for the work items this call's plan can make: with kv_chunk = 0
  // the plan makes at most target_items() items, else at most items_max().
  const Geom g = make_geom(&cfg, batch, cache);
  mlra_kernel_t kern;
  TRY(select_kernel(&cfg, g, cache, &kern));
  int64_t items = items_max(&cfg, batch, cache->max_len);
  if (cfg.kv_chunk == 0 && target_items(g, cus, kern) < items) items = target_items(g, cus, kern);
  const Layout L = layout(&cfg, batch, cache->max_len, items);
  if (L.total > kScratchBytes)
    return fail(MLRA_ERR_WORKSPACE,
                "mlra_decode_noalloc needs %zu bytes of scratch for this batch and cache; the "
                "library's scratch holds %zu (use mlra_decode with a workspace)",
                L.total, kScratchBytes);
  return run_step(&cfg, batch, cus, q_nope, q_rope, q_pos, w_uk, w_uv, cache, L, carve(L, base),
                  out, out_dtype, static_cast<hipStream_t>(stream));
}

}  // extern "C"
