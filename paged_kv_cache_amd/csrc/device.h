// device.h -- shared device helpers of the gfx950 kernels: page geometry,
// bf16 bit handling, MFMA operand types, error flags.  Device code only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedattn.h"

namespace pa {

// 16 tokens per page; K block first, V block V_OFFSET bytes later
// (tiny-vllm part 6, "Block contents: K in front, V after V_OFFSET").
constexpr int kPageTokens = 16;

// Read-only view of a global array through the constant address space: a
// wave-uniform load from it always goes to the scalar unit, whatever else the
// kernel writes.  Only for memory that no thread writes during the launch.
typedef const __attribute__((address_space(4))) int32_t *const_i32_ptr;
__device__ inline const_i32_ptr as_const(const int32_t *p) { return (const_i32_ptr)p; }

// 16 bytes per lane from global memory straight into LDS, no registers in
// between: lane L reads base + off (base wave-uniform, off this lane's) and
// its bytes land at dst + 16*L (dst wave-uniform).  The transfer counts on
// vmcnt like any vector load and the caller waits for it explicitly: the
// compiler does not see it as a load, so it neither waits on it nor treats
// its registers as in use.  NT=1 adds the non-temporal hint.
template <int NT = 0>
__device__ __forceinline__ void dma16(const uint8_t *base, uint32_t off, void *dst_lds) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)dst_lds;
  if constexpr (NT)
    asm volatile("global_load_lds_dwordx4 %0, %1 nt" ::"v"(off), "s"(base), "{m0}"(m0) : "memory");
  else
    asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(m0) : "memory");
}

// s_waitcnt vmcnt(N) lgkmcnt(0) (gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt 6:4 left at its maximum, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
// native 16-byte vector (HIP's uint4 is a struct of unions that the compiler
// may copy through private memory)
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

__device__ __forceinline__ float bf16_to_f32(uint16_t bits) {
  return __uint_as_float((uint32_t)bits << 16);
}

// Round-to-nearest-even float -> bf16 bits (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ void raise_err(int32_t *err, int bits) {
  if (err) atomicOr(err, bits);
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The value of lane 0 in a scalar register: for values that are the same in
// every lane but that the compiler cannot prove uniform (e.g. after a branch
// on the lane id), so that addresses built from them use scalar loads.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Block-table view of one (slot, layer): physical page of each logical block.
struct PageTable {
  const uint8_t *pool;
  const int32_t *row;  // block_table + (slot * n_layers + layer) * mbps
  int64_t n_pages;
  int64_t page_bytes;
  int64_t v_offset;
  int mbps;

  // Physical page of logical block blk, or -1 when the entry is missing or
  // outside the pool.
  __device__ __forceinline__ int64_t page(int blk) const {
    if (blk < 0 || blk >= mbps) return -1;
    int32_t p = row[blk];
    return (p < 0 || (int64_t)p >= n_pages) ? -1 : (int64_t)p;
  }
};

}  // namespace pa
