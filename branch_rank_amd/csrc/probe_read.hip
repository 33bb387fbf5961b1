// HBM read-bandwidth probe (include/mlra_probe.h): every byte of a buffer is
// read once, either into VGPRs or by LDS-DMA into a ring in LDS, the two
// load paths a split-KV decode kernel can stream its cache through. Used by
// the benchmark for the measured read ceiling; not part of libmlra.

#include <hip/hip_runtime.h>

#include "../../include/mlra_probe.h"
#include "device_common.h"

namespace {

using namespace mlra::dev;

// Mode 0: grid-strided 16-byte non-temporal loads, D of them in flight per
// lane before their values are combined.
template <int D>
__global__ __launch_bounds__(1024) void read_vgpr(const i32x4* __restrict__ p, size_t n16,
                                                   int32_t* sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  i32x4 acc = {0, 0, 0, 0};
  for (; i + (D - 1) * stride < n16; i += D * stride) {
    i32x4 v[D];
#pragma unroll
    for (int u = 0; u < D; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < D; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(p + i);
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x5A5A5A5A) sink[0] = 1;
}

// Mode 1: workgroup k streams bytes [k * per, (k + 1) * per) through LDS-DMA,
// wave w issuing the 1 KB pieces w, w + waves, ... into its own four 1 KB
// slots of a ring (the data is never read back: only the load path is
// measured); after each issue a wave waits until at most W of its pieces are
// still in flight. The loads are volatile asm, so nothing removes them.
template <int W>
__global__ __launch_bounds__(1024) void read_lds_dma(const char* base, uint32_t per) {
  __shared__ __attribute__((aligned(1024))) char ring[16 * 4 * 1024];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, nw = blockDim.x >> 6;
  const char* p = base + (size_t)blockIdx.x * per;
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  i32x4 rs;
  rs.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  rs.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xFFFF);
  rs.z = __builtin_amdgcn_readfirstlane((int)per);
  rs.w = 0x00020000;
  const uint32_t slot0 = (uint32_t)(uintptr_t)ring + (uint32_t)wave * 4 * 1024;
  int u = 0;
  for (uint32_t off = (uint32_t)wave * 1024; off < per; off += (uint32_t)nw * 1024, ++u) {
    dma16_stream(rs, slot0 + (uint32_t)(u & 3) * 1024, (uint32_t)lane * 16, off);
    wait_vm<W>();
  }
  wait_vm<0>();
}

}  // namespace

extern "C" int mlra_probe_read(const void* buf, size_t bytes, int mode, int workgroups,
                               int waves, int depth, int32_t* sink, void* stream) {
  if (!buf || !sink || (reinterpret_cast<uintptr_t>(buf) & 15) || workgroups < 1 ||
      workgroups > 65536 || waves < 1 || waves > 16 || bytes == 0 ||
      bytes % (1024 * (size_t)workgroups))
    return -1;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(workgroups), block(64 * waves);
  if (mode == 0) {
    const i32x4* p = static_cast<const i32x4*>(buf);
    const size_t n16 = bytes / 16;
    switch (depth) {
      case 1: hipLaunchKernelGGL(read_vgpr<1>, grid, block, 0, s, p, n16, sink); break;
      case 2: hipLaunchKernelGGL(read_vgpr<2>, grid, block, 0, s, p, n16, sink); break;
      case 4: hipLaunchKernelGGL(read_vgpr<4>, grid, block, 0, s, p, n16, sink); break;
      case 8: hipLaunchKernelGGL(read_vgpr<8>, grid, block, 0, s, p, n16, sink); break;
      default: return -1;
    }
  } else if (mode == 1) {
    const size_t per = bytes / workgroups;
    if (per > 0x7fffffffULL) return -1;
    const char* p = static_cast<const char*>(buf);
    const uint32_t pr = (uint32_t)per;
    switch (depth) {
      case 1: hipLaunchKernelGGL(read_lds_dma<0>, grid, block, 0, s, p, pr); break;
      case 2: hipLaunchKernelGGL(read_lds_dma<1>, grid, block, 0, s, p, pr); break;
      case 4: hipLaunchKernelGGL(read_lds_dma<3>, grid, block, 0, s, p, pr); break;
      case 8: hipLaunchKernelGGL(read_lds_dma<7>, grid, block, 0, s, p, pr); break;
      case 12: hipLaunchKernelGGL(read_lds_dma<11>, grid, block, 0, s, p, pr); break;
      case 16: hipLaunchKernelGGL(read_lds_dma<15>, grid, block, 0, s, p, pr); break;
      default: return -1;
    }
  } else {
    return -1;
  }
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? 0 : (int)e;
}
