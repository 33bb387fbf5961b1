// Tile machinery of the branch-per-wave split-KV decode (gfx950): 32-token
// tiles of the latent cache, one or two 128-column branch slices plus the
// shared RoPE key per workgroup, streamed HBM -> LDS by LDS-DMA into a ring of
// stages with XOR-swizzled 16-byte chunks.
#pragma once

#include <hip/hip_runtime.h>

#include "device_common.h"

namespace mlra {
namespace bt {

using namespace dev;

constexpr int kT = 32;    // tokens per tile
constexpr int kDR = 64;   // RoPE width
constexpr int kBW = 128;  // latent width of one branch
constexpr float kRescale = 16.f;  // log2 headroom kept when the reference moves
constexpr float kSumLimit = 1048576.f;  // 2^20: per-lane P sum that moves the reference
// "no reference yet": finite, so that masked scores (-inf) still give p = 0,
// while every real score overflows to p = inf and forces the exact path
constexpr float kNoRef = -3.0e38f;

template <int NBR, int NSPLIT, int HPW, int NHG>
struct BCfg {
  static constexpr int DC = NBR * kBW;            // total latent width
  static constexpr int NBW = NBR / NSPLIT;        // branches per workgroup
  static constexpr int NW = NBW * NHG;            // waves per workgroup
  static constexpr int H = HPW * NHG;             // heads (every workgroup has all)
  static constexpr int NBLK = HPW / 16;           // MFMA N blocks (16 heads) per wave
  static constexpr int ROWB = NBW * kBW * 2;      // latent bytes of a row in LDS
  static constexpr int LAT = kT * ROWB;           // latent part of a stage
  static constexpr int STAGE = LAT + kT * kDR * 2;
  static constexpr int RPI = 1024 / ROWB;         // latent rows per DMA instruction
  static constexpr int NL = kT / RPI;             // latent DMA instructions per tile
  static constexpr int NR = kT * kDR * 2 / 1024;  // RoPE DMA instructions per tile (8 rows each)
  static constexpr int KL = kBW / 32;             // latent k-steps of a branch score
  static constexpr int KS = KL + kDR / 32;        // plus the RoPE k-steps
  static constexpr int CB = kBW / 16;             // PV output row blocks of a branch
  static_assert(NBR % NSPLIT == 0 && (ROWB == 512 || ROWB == 256),
                "one or two 128-column branches per workgroup");
  static_assert(HPW % 16 == 0 && NW <= 16, "wave shape");
  static_assert(NL % NW == 0 && NR <= NW, "DMA assignment");
};

// Chunk swizzles: latent rows of ROWB bytes (16-byte chunk index ^ 2 * (row &
// (ROWB / 32 - 1)), which stays inside the row: row & 15 for two branches,
// row & 7 for one); RoPE rows of 128 bytes (chunk ^ ((row >> 1) & 7)).
template <int ROWB>
__device__ __forceinline__ int swz_l(int t) { return 2 * (t & (ROWB / 32 - 1)); }
__device__ __forceinline__ int swz_r(int t) { return (t >> 1) & 7; }

// DMA of one tile into the stage at LDS byte address `stage` (streaming
// loads, dma16_stream). Wave w issues
// latent instructions q = w, w + NW, ... (rows RPI*q .. +RPI-1; lat_voff is
// this lane's offset within such a row group, the tile row in soffset) and,
// if w < NR, RoPE instruction w (8 rows; rope_t and rope_c are this lane's row
// in it and its swizzled 16-byte chunk offset). The segment's last tile
// (TAIL) clamps every row to tend - 1 per lane, so no load passes the
// sequence's rows.
template <class C, bool TAIL>
__device__ __forceinline__ void issue_tile(uint32_t stage, i32x4 crs, i32x4 krs, int cts,
                                           int kts, int tstart, int tend, int wave, int lane,
                                           uint32_t lat_voff, int lat_c, int rope_t, int rope_c) {
#pragma unroll
  for (int u = 0; u < C::NL / C::NW; ++u) {
    const int q = wave + C::NW * u;
    if constexpr (!TAIL) {
      dma16_stream(crs, stage + q * 1024, lat_voff, (uint32_t)((tstart + C::RPI * q) * cts * 2));
    } else {
      const int row = min(tstart + C::RPI * q + lane / (64 / C::RPI), tend - 1);
      dma16_stream(crs, stage + q * 1024, (uint32_t)(row * cts * 2 + lat_c), 0u);
    }
  }
  if (wave < C::NR) {
    const int row = min(tstart + rope_t, tend - 1);
    dma16_stream(krs, stage + C::LAT + wave * 1024, (uint32_t)(row * kts * 2 + rope_c), 0u);
  }
}

// Wait until at most `ahead` (<= MAXA) tiles of this wave's DMA, PER
// instructions per tile, are still in flight.
template <int PER, int MAXA>
__device__ __forceinline__ void wait_tiles_per(int ahead) {
  static_assert(MAXA * PER < 64, "vmcnt range");
  if constexpr (MAXA >= 5) if (ahead >= 5) { wait_vm<5 * PER>(); return; }
  if constexpr (MAXA >= 4) if (ahead == 4) { wait_vm<4 * PER>(); return; }
  if constexpr (MAXA >= 3) if (ahead == 3) { wait_vm<3 * PER>(); return; }
  if constexpr (MAXA >= 2) if (ahead == 2) { wait_vm<2 * PER>(); return; }
  if (ahead == 1) { wait_vm<PER>(); return; }
  wait_vm<0>();
}
template <class C, int MAXA>
__device__ __forceinline__ void wait_tiles(int ahead, int wave) {
  if (wave < C::NR) wait_tiles_per<C::NL / C::NW + 1, MAXA>(ahead);
  else wait_tiles_per<C::NL / C::NW, MAXA>(ahead);
}

}  // namespace bt
}  // namespace mlra
