/*
 * mlra_probe.h - HBM read-bandwidth probe for the benchmark (libmlra_probe.so).
 *
 * Not part of the decode library: it measures the read ceiling that the
 * split-KV decode kernels stream against on this GPU, so that their
 * achieved cache bandwidth can be reported as a fraction of a measured
 * ceiling as well as of the published peak. The decode's cost is set by
 * streaming the cache from HBM ("Multi-Head Low-Rank Attention", 研究动机),
 * which is what both modes do: read every byte of a buffer once.
 *
 *   buf         device buffer of `bytes` bytes (16-byte aligned), read only
 *   bytes       bytes to read; must be a multiple of 1024 * workgroups
 *   mode        0: loads into VGPRs (16 bytes per lane and load, `depth`
 *                  loads in flight per lane, non-temporal), grid-strided;
 *               1: LDS-DMA loads (buffer_load_dwordx4 ... lds, device-scope
 *                  non-temporal, as the decode kernels' cache tiles), each
 *                  workgroup streaming its own contiguous bytes / workgroups
 *                  slice into a ring in LDS with `depth` loads in flight
 *                  per wave
 *   workgroups  grid size (1 .. 65536)
 *   waves       waves per workgroup (1 .. 16)
 *   depth       loads in flight per lane (mode 0: 1, 2, 4 or 8) or per
 *               wave (mode 1: 1, 2, 4, 8, 12 or 16)
 *   sink        device int32 buffer of >= 1 element; mode 0 writes it only
 *               when the read data takes a value it practically never
 *               takes, which keeps the loads from being removed
 *   stream      hipStream_t (NULL = legacy default stream)
 *
 * Returns 0 when the launch was enqueued, -1 on invalid arguments (nothing
 * launched), or the HIP error code of the launch. Allocates nothing and
 * does not synchronise; the caller times the launch with events.
 */
#ifndef MLRA_PROBE_H_
#define MLRA_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define MLRA_PROBE_API __attribute__((visibility("default")))
#else
#define MLRA_PROBE_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

MLRA_PROBE_API int mlra_probe_read(const void* buf, size_t bytes, int mode, int workgroups,
                                   int waves, int depth, int32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLRA_PROBE_H_ */
