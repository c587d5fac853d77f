// Wave64 / workgroup primitives for gfx950 (64-lane wavefronts).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace igc {

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63u); }

// Orders this wave's LDS accesses before and after the call (no other wave takes part).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ uint64_t shfl64(uint64_t v, int src) {
  const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)v, src, 64);
  const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(v >> 32), src, 64);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m, 64);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t wave_or64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v |= shfl_xor64(v, m);
  return v;
}

__device__ __forceinline__ uint64_t wave_and64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v &= shfl_xor64(v, m);
  return v;
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t t = (uint32_t)__shfl_up((int)v, d, 64);
    if (lane >= d) v += t;
  }
  return v;
}

__device__ __forceinline__ uint64_t wave_incl_scan64(uint64_t v) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t lo = (uint32_t)__shfl_up((int)(uint32_t)v, d, 64);
    const uint32_t hi = (uint32_t)__shfl_up((int)(uint32_t)(v >> 32), d, 64);
    if (lane >= d) v += ((uint64_t)hi << 32) | lo;
  }
  return v;
}

// Exclusive prefix sum over a workgroup of NT threads (NT a multiple of 64, at most 1024).
// s_tmp holds NT/64 values. Returns the exclusive prefix; *total gets the sum.
template <int NT>
__device__ __forceinline__ uint64_t block_excl_scan64(uint64_t v, uint64_t* s_tmp, uint64_t* total) {
  const int lane = lane_id();
  const int wave = (int)(threadIdx.x >> 6);
  const uint64_t inc = wave_incl_scan64(v);
  if (lane == 63) s_tmp[wave] = inc;
  __syncthreads();
  uint64_t wave_base = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const uint64_t t = s_tmp[w];
    if (w < wave) wave_base += t;
    sum += t;
  }
  __syncthreads();
  if (total) *total = sum;
  return wave_base + inc - v;
}

}  // namespace igc
