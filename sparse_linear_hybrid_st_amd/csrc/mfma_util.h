// MFMA-tile helpers shared by the bf16 attention kernels (forward and
// backward): operand types, the 32x32x16 bf16 MFMA, the LDS swizzle of
// 64 x 128 bf16 tiles, a fence-free workgroup barrier and the XCD-aware
// workgroup order.
#pragma once

#include "common.h"

namespace salad {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernels, d = 128.
// ---------------------------------------------------------------------------
constexpr int kD = 128;   // head dim
constexpr int kBN = 64;   // keys per tile

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Workgroup barrier without the memory fence of __syncthreads(), whose
// release half waits for every DMA in flight.  The barrier intrinsic by
// itself does not order memory accesses in the compiler, so the empty asm
// statements with a memory clobber pin every access (LDS reads, DMA issues)
// to its side of the barrier, and the lgkmcnt wait makes this wave's LDS
// reads complete before any wave passes.  DMA completion is waited for
// explicitly (vmcnt) by the callers.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt: no wait
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// K and V tiles are stored row-major ([key][d], 256-byte rows) in LDS.  The
// 16-byte unit u of row j sits at u ^ kv_swz(j).  kv_swz is a bijection on
// the low 4 bits of j that swaps its two 2-bit halves, so
//   * the K operand reads (16 consecutive keys, one unit) hit 16 distinct
//     units, and
//   * the transposing V reads (4 consecutive keys x one 64-byte segment)
//     hit 4 distinct segments.
__device__ __forceinline__ int kv_swz(int j) { return ((j & 3) << 2) | ((j >> 2) & 3); }

// Workgroups are dispatched round-robin over the 8 XCDs; renumber them so
// that each XCD walks a contiguous range of query tiles (neighbouring tiles
// share most of their key window, which then stays in that XCD's L2).
__device__ __forceinline__ int xcd_order(int bid, int T) {
  const int q = T >> 3, r = T & 7, x = bid & 7, k = bid >> 3;
  return x < r ? x * (q + 1) + k : r * (q + 1) + (x - r) * q + k;
}

}  // namespace salad
