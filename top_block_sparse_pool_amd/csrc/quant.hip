// FP8 (E4M3) dynamic quantisation of Q and K for the fp8 attention path.
//
// Source: ParaAttention/HunyuanVideo post (WaveSpeed), section on FP8
// dynamic quantisation: activations are quantised to FP8 at run time so the
// products run on 8-bit matrix units.  Format and groups are readings: OCP
// E4M3 (largest magnitude 448), one scale per query token and one per
// 64-token tile of keys of a (batch, head).  Each decision is a correctly
// rounded fp32 step:
//
//   a = max |x| over the group;  inv = 448 / a;  y = x * inv;
//   code = E4M3(clamp(y, -448, 448)), round to nearest even;  scale = a / 448
//
// and a group with a = 0 gets inv = scale = 0 (all codes +-0).
//
// bf16 inputs with head_dim 128.  One workgroup of 256 threads per (b, h,
// 64-token tile) quantises both the Q
// rows and the K rows of the tile: it reads each bf16 element once and
// writes one byte, so the kernel is HBM-bound (3 bytes moved per element of
// Q and of K).  A thread holds 16-byte chunks (8 elements) of tile rows; the
// per-token maxima reduce over the row's lanes with shuffles, the tile
// maximum over the workgroup through LDS.
#include "device_common.h"
#include "e4m3.h"
#include "launch.h"

namespace tbs {
namespace {

constexpr int kQuantThreads = 256;
constexpr int kQuantTile = 64;

__device__ __forceinline__ void load_bf16x8(const unsigned short* src, float* out) {
  bf16x8_to_f32(*reinterpret_cast<const u32x4*>(src), out);
}

template <int D>
__global__ __launch_bounds__(kQuantThreads) void quant_qk_kernel(
    const unsigned short* __restrict__ q, const unsigned short* __restrict__ k, unsigned char* __restrict__ q8,
    float* __restrict__ q_scale, unsigned char* __restrict__ k8, float* __restrict__ k_scale, int N, int nkt) {
  constexpr int C = D / 8;                        // 16-byte chunks per row
  constexpr int RP = kQuantThreads / C;           // rows per pass
  constexpr int PASSES = kQuantTile / RP;
  __shared__ float red[kQuantThreads / kWave];

  const int tile = blockIdx.x % nkt;
  const long long bh = blockIdx.x / nkt;
  const int tid = threadIdx.x;
  const int c = tid % C;
  const int r0 = tid / C;
  const int lo = tile * kQuantTile;
  const long long base = bh * N;

  // Q: every row is its own group.
#pragma unroll
  for (int pass = 0; pass < PASSES; ++pass) {
    const int row = lo + r0 + pass * RP;
    const bool valid = row < N;
    float x[8];
    if (valid) {
      load_bf16x8(q + (base + row) * D + c * 8, x);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.f;
    }
    float a = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(x[e]));
#pragma unroll
    for (int off = 1; off < C; off <<= 1) a = fmaxf(a, __shfl_xor(a, off, kWave));
    if (valid) {
      *reinterpret_cast<u32x2*>(q8 + (base + row) * D + c * 8) = e4m3_encode8(x, e4m3_group_inv(a));
      if (c == 0) q_scale[base + row] = e4m3_group_scale(a);
    }
  }

  // K: one group per tile.
  float xk[PASSES][8];
  float a = 0.f;
#pragma unroll
  for (int pass = 0; pass < PASSES; ++pass) {
    const int row = lo + r0 + pass * RP;
    if (row < N) {
      load_bf16x8(k + (base + row) * D + c * 8, xk[pass]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) xk[pass][e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(xk[pass][e]));
  }
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) a = fmaxf(a, __shfl_xor(a, off, kWave));
  if ((tid & (kWave - 1)) == 0) red[tid / kWave] = a;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kQuantThreads / kWave; ++w) a = fmaxf(a, red[w]);
  const float inv = e4m3_group_inv(a);
#pragma unroll
  for (int pass = 0; pass < PASSES; ++pass) {
    const int row = lo + r0 + pass * RP;
    if (row < N) *reinterpret_cast<u32x2*>(k8 + (base + row) * D + c * 8) = e4m3_encode8(xk[pass], inv);
  }
  if (tid == 0) k_scale[bh * nkt + tile] = e4m3_group_scale(a);
}

}  // namespace

int quant_tiles(const Shape& s) { return (s.N + kQuantTile - 1) / kQuantTile; }

hipError_t launch_quantize_qk(const Shape& s, const void* q, const void* k, uint8_t* q8, float* q_scale, uint8_t* k8,
                              float* k_scale, hipStream_t stream) {
  const int nkt = quant_tiles(s);
  const long long grid = static_cast<long long>(s.B) * s.H * nkt;
  hipLaunchKernelGGL(quant_qk_kernel<128>, dim3(static_cast<unsigned>(grid)), dim3(kQuantThreads), 0, stream,
                     static_cast<const unsigned short*>(q), static_cast<const unsigned short*>(k), q8, q_scale, k8,
                     k_scale, s.N, nkt);
  return hipGetLastError();
}

}  // namespace tbs
