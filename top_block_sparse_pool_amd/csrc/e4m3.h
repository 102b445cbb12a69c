// E4M3 quantisation steps shared by the quantising kernels (gfx950).
//
// Source: ParaAttention/HunyuanVideo post (WaveSpeed), section on FP8 dynamic
// quantisation.  Format and groups are readings: OCP E4M3 (largest magnitude
// 448); for a group with largest magnitude a:
//   inv = 448 / a;  code = E4M3(clamp(x * inv, -448, 448)), round to nearest
//   even;  scale = a / 448;  a = 0 gives inv = scale = 0 (codes +-0).
// Every step is a correctly rounded fp32 operation.
#pragma once

#include "device_common.h"

namespace tbs {

constexpr float kE4M3Max = 448.0f;

// Eight bf16 values of a 16-byte chunk, exactly, as fp32.
__device__ __forceinline__ void bf16x8_to_f32(const u32x4& w, float* out) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    out[2 * j] = __uint_as_float(w[j] << 16);
    out[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
  }
}

// Eight codes of x * inv, packed little-endian (element 0 in the low byte).
// v_cvt_pk_fp8_f32 rounds to nearest even; the clamp keeps every input in
// the finite E4M3 range.
__device__ __forceinline__ u32x2 e4m3_encode8(const float* x, float inv) {
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = fminf(fmaxf(x[e] * inv, -kE4M3Max), kE4M3Max);
  u32x2 r;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    int v = 0;
    v = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * w], y[4 * w + 1], v, false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * w + 2], y[4 * w + 3], v, true);
    r[w] = static_cast<unsigned>(v);
  }
  return r;
}

__device__ __forceinline__ float e4m3_group_inv(float a) { return a > 0.f ? __fdiv_rn(kE4M3Max, a) : 0.f; }
__device__ __forceinline__ float e4m3_group_scale(float a) { return a > 0.f ? __fdiv_rn(a, kE4M3Max) : 0.f; }

}  // namespace tbs
