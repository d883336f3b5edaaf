// common.h -- device helpers shared by the libmoe kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define MOE_WAVE 64

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

// 16-byte global load (the caller guarantees alignment and bounds).
__device__ __forceinline__ u32x4 ldg16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// SiLU with the hardware reciprocal (about 1 ulp); -0 for very negative g
__device__ __forceinline__ float silu_f32(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// Completion count of a launch whose last workgroup to finish does the rest
// of its work.  The workgroup barrier orders every wave's stores before it
// (they are in this CU's L2); then one wave releases them at device scope
// (one L2 write-back per workgroup, not one per wave) and counts.  The last
// workgroup acquires every other's stores the same way (one wave's
// invalidate, then the barrier) and resets the counter for the next launch.
// True in every thread of the last workgroup.  *flag: a __shared__ int.
__device__ __forceinline__ bool last_workgroup(int32_t* counter, int* flag) {
  __syncthreads();
  if (threadIdx.x < 64) {
    __threadfence();  // release, at device scope
    if (threadIdx.x == 0) *flag = (atomicAdd(counter, 1) == (int)gridDim.x - 1);
  }
  __syncthreads();
  if (!*flag) return false;
  if (threadIdx.x < 64) __threadfence();  // acquire, at device scope
  if (threadIdx.x == 0) *counter = 0;     // every workgroup has counted
  __syncthreads();
  return true;
}

// The chip has 8 XCDs, each with its own L2; consecutive workgroup ids are
// dealt round-robin over them.  Renumber so that blocks sharing data (same
// logical neighbourhood) land on the same XCD: physical id i -> logical id
// (i % 8) * (n / 8) + i / 8, for n a multiple of 8.
__device__ __forceinline__ uint32_t xcd_logical_id(uint32_t i, uint32_t n) {
  return (i & 7u) * (n >> 3) + (i >> 3);
}

// Largest index e with off[e] <= v, for off ascending with off[0] == 0.
__device__ __forceinline__ int upper_segment(const int32_t* off, int n_seg, int v) {
  int lo = 0, hi = n_seg;  // answer in [lo, hi)
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (off[mid] <= v) lo = mid; else hi = mid;
  }
  return lo;
}
