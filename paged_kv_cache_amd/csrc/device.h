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

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
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
