// Device helpers shared by the gfx950 split-KV decode kernels: vector types,
// hand-placed wait counts, raw buffer descriptors, the LDS-DMA load, the
// sequence lookup of a token position and the 4-lane reductions.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.h"

namespace mlra {
namespace dev {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8;
typedef int i32x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;

// Device bounds checks of the debug build (-DMLRA_DEBUG_BOUNDS): a failed
// check records its site in the plan header (the first failure wins, by a
// vector compare-and-swap) and the kernel goes on with the values it has,
// which every access clamps; the debug library's host side reads the word
// after the call and fails the call. Without the define the checks compile
// to nothing. Sites: 1 sequence index, 2 token range of a segment, 3 slot of
// the partial state, 4 work item past the plan, 5 merge slot range.
#ifdef MLRA_DEBUG_BOUNDS
#define MLRA_DCHECK(hdr, cond, site)                                                     \
  do {                                                                                   \
    if (!(cond)) atomicCAS(const_cast<int*>(&(hdr)->bounds_fail), 0, (site));           \
  } while (0)
#else
#define MLRA_DCHECK(hdr, cond, site) \
  do {                               \
  } while (0)
#endif

// Arguments of the split-KV decode kernels (one struct, passed by value).
struct DecodeParams {
  const __bf16* q_abs;  // row (b, h) at q_abs + (b * H + h) * q_stride: q~ (d_c), rho (d_r)
  int q_stride;         // elements per query row
  int q_lo;             // > 0: the row's bf16 residue of q~ starts at this element
  const __bf16* ckv;
  const __bf16* krope;
  int64_t ckv_bs, kr_bs;
  int ckv_ts, kr_ts;  // token strides in elements (host checks the byte ranges fit 31 bits)
  const PlanHeader* hdr;
  const int32_t* prefix;
  float* m;
  float* l;
  float* acc;
  int B;
};

// s_waitcnt vmcnt(N), leaving lgkmcnt/expcnt alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Raw buffer descriptor (gfx9 layout: base, stride 0, byte range, word 3)
// over one sequence's rows [0, rows).
__device__ __forceinline__ i32x4 seq_rsrc_bytes(const void* base, int rows, int ts_bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;  // wave-uniform values, made explicit for the SGPR operands
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xFFFF);
  r.z = __builtin_amdgcn_readfirstlane(rows * ts_bytes);
  r.w = 0x00020000;
  return r;
}
// the same for bf16 rows of ts elements
__device__ __forceinline__ i32x4 seq_rsrc(const __bf16* base, int rows, int ts) {
  return seq_rsrc_bytes(base, rows, ts * 2);
}

// bf16 -> fp16 of the 8 values in a 16-byte chunk, rounded toward zero:
// exact for |x| in fp16's normal range [2^-14, 65504] (bf16's 8 significant
// bits fit fp16's 11); larger magnitudes saturate to 65504 and the tail below
// 2^-14 keeps fp16's subnormal precision.
__device__ __forceinline__ i32x4 bf16_to_f16x8(i32x4 x) {
  i32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t v = (uint32_t)x[i];
    const auto h = __builtin_amdgcn_cvt_pkrtz(__builtin_bit_cast(float, v << 16),
                                              __builtin_bit_cast(float, v & 0xFFFF0000u));
    r[i] = __builtin_bit_cast(int, h);
  }
  return r;
}

// Four fp32 values as fp16 (round to nearest even) in one 8-byte store; a
// value beyond fp16's range saturates at +-65504 instead of becoming inf (a
// NaN stays NaN).
__device__ __forceinline__ void store_f16x4_sat(_Float16* dst, f32x4 v) {
  typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
  u16x4 b;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    unsigned short x = __builtin_bit_cast(unsigned short, (_Float16)v[i]);
    if ((x & 0x7fff) == 0x7c00) x = (unsigned short)((x & 0x8000) | 0x7bff);
    b[i] = x;
  }
  *(u16x4*)dst = b;
}

// 16 FP8 E4M3 codes (16 bytes, element i in byte i) to 16 exact fp16 values
// (two 16-byte halves: elements 0-7, then 8-15): v_cvt_scalef32_pk_f16_fp8
// with scale 1 turns two codes into two fp16 values. E4M3's range and its 3
// mantissa bits fit fp16's normals and subnormals, so nothing rounds.
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void fp8x16_to_f16(i32x4 x, i32x4& lo, i32x4& hi) {
  int r[8];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const f16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)x[w], 1.0f, false);
    const f16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)x[w], 1.0f, true);
    r[2 * w] = __builtin_bit_cast(int, a);
    r[2 * w + 1] = __builtin_bit_cast(int, b);
  }
  lo = (i32x4){r[0], r[1], r[2], r[3]};
  hi = (i32x4){r[4], r[5], r[6], r[7]};
}
// the same to bf16 (E4M3 fits bf16 exactly as well)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void fp8x16_to_bf16(i32x4 x, i32x4& lo, i32x4& hi) {
  int r[8];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)x[w], 1.0f, false);
    const bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)x[w], 1.0f, true);
    r[2 * w] = __builtin_bit_cast(int, a);
    r[2 * w + 1] = __builtin_bit_cast(int, b);
  }
  lo = (i32x4){r[0], r[1], r[2], r[3]};
  hi = (i32x4){r[4], r[5], r[6], r[7]};
}

// One LDS-DMA instruction: 16 bytes per lane from rsrc + voff + soff into
// LDS at lds_base + 16 * lane. Issued from asm so that the compiler does not
// add its own (conservative) vmcnt waits before later LDS reads; every wait
// for this data is placed by hand. No output registers.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t lds_base, uint32_t voff,
                                      uint32_t soff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(rsrc),
        "s"(__builtin_amdgcn_readfirstlane(soff))
      : "memory");
}

// The same load for data that streams through once, the decode's cache
// tiles: device scope (sc1: not kept in the CU's vector cache) and
// non-temporal (nt: evicted first from L2 and the Infinity Cache), so that
// the step's weights and split-KV partials stay cached while hundreds of MB of
// cache pass by. The second workgroup of an item still finds the shared RoPE
// rows in L2 (fetched bytes past L2 are unchanged).
__device__ __forceinline__ void dma16_stream(i32x4 rsrc, uint32_t lds_base, uint32_t voff,
                                             uint32_t soff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen sc1 nt lds"
      :
      : "s"(__builtin_amdgcn_readfirstlane(lds_base)), "v"(voff), "s"(rsrc),
        "s"(__builtin_amdgcn_readfirstlane(soff))
      : "memory");
}

// Sequence holding token position pos of the batch-wide token stream.
__device__ __forceinline__ int find_seq(const int32_t* prefix, int B, int pos) {
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (prefix[mid] <= pos) lo = mid; else hi = mid;
  }
  return lo;
}

// Reductions over the four lanes l16 + 16 kg (kg = 0..3) with the gfx950
// lane swaps (VALU, no LDS): v_permlane16_swap exchanges the odd 16-lane rows
// of its first operand with the even rows of its second, so with both
// operands equal to x the pair holds x of this lane and of lane ^ 16;
// v_permlane32_swap likewise for lane ^ 32. The swaps are issued from asm with
// both registers as in/out operands: this compiler's permlane*_swap builtins
// return the first result for both halves of the pair. s_nop 1 on either side
// covers the VALU -> permlane and permlane -> VALU operand hazards.
__device__ __forceinline__ void swap16(float x, float& lo, float& hi) {
  float y = x;
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(x), "+v"(y));
  lo = x;
  hi = y;
}
__device__ __forceinline__ void swap32(float x, float& lo, float& hi) {
  float y = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(x), "+v"(y));
  lo = x;
  hi = y;
}
__device__ __forceinline__ float max4(float x) {
  float a, b;
  swap16(x, a, b);
  swap32(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float sum4(float x) {
  float a, b;
  swap16(x, a, b);
  swap32(a + b, a, b);
  return a + b;
}

}  // namespace dev
}  // namespace mlra
