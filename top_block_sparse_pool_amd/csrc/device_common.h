// Device-side helpers shared by the HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tbs {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

#define TBS_LDS __attribute__((address_space(3)))

constexpr int kWave = 64;

// Value held by the lane 32 positions away (lanes l and l^32 exchange).
__device__ __forceinline__ float xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  // After the swap, r[0] holds the lower half's value in the upper lanes and
  // r[1] the upper half's value in the lower lanes.
  unsigned lane = __lane_id();
  return __uint_as_float(lane < 32 ? r[1] : r[0]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wave-wide sums and maxima in a fixed order (deterministic).
__device__ __forceinline__ double wave_sum_f64(double x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}
__device__ __forceinline__ double wave_max_f64(double x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmax(x, __shfl_xor(x, off, kWave));
  return x;
}
__device__ __forceinline__ int wave_sum_i32(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  unsigned lane = __lane_id();
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maxima), as the
// builtin so that the compiler's own wait bookkeeping sees it.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

}  // namespace tbs
