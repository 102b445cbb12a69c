// Top-p block router for gfx950.
//
// Source: FVAttn review page, section 1 (Key Terms, "Top-p routing") and
// section 3 (Method): every query block keeps the key blocks whose
// cumulative probability, taken in order of importance, first reaches p.
// The block importance is the scaled dot product of block-mean-pooled Q and
// K with a softmax over key blocks.  Everything that decides the mask is in
// fp64 so the selection matches exact arithmetic up to fp64 rounding.
//
// Kernels:
//   pool_kernel    one workgroup per (tensor, b, h, block): block means in fp64
//                  (HBM-bound: reads Q and K once).
//   select_kernel  one workgroup per (b, h, R query blocks): fp64 scores for R
//                  rows against all key blocks (pooled K read transposed so
//                  that lanes read consecutive key blocks), then per row a
//                  max/sum softmax, an LDS bitonic sort by (P desc, index asc),
//                  a fixed-order prefix sum to find the cut, and the outputs.
#include <math.h>

#include "device_common.h"
#include "launch.h"

namespace tbs {
namespace {

constexpr int kPoolThreads = 256;
constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / kWave;

template <typename T>
__device__ __forceinline__ void load_chunk_f64(const T* src, double* out);

template <>
__device__ __forceinline__ void load_chunk_f64<unsigned short>(const unsigned short* src, double* out) {
  u32x4 w = *reinterpret_cast<const u32x4*>(src);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    out[2 * e] = static_cast<double>(__uint_as_float(w[e] << 16));
    out[2 * e + 1] = static_cast<double>(__uint_as_float(w[e] & 0xffff0000u));
  }
}

template <>
__device__ __forceinline__ void load_chunk_f64<float>(const float* src, double* out) {
  f32x4 w = *reinterpret_cast<const f32x4*>(src);
#pragma unroll
  for (int e = 0; e < 4; ++e) out[e] = static_cast<double>(w[e]);
}

// Block mean of Q (tensor 0) or K (tensor 1) over the valid tokens of block i.
template <typename T, int D>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(
    const T* __restrict__ q, const T* __restrict__ k, double* __restrict__ qbar,
    double* __restrict__ kbar_t, int32_t* __restrict__ head_cnt, int BH, int N, int nb, int block) {
  constexpr int E = 16 / sizeof(T);           // elements per 16-byte chunk
  constexpr int C = D / E;                    // chunks per token row
  constexpr int R = kPoolThreads / C;         // token rows per pass
  __shared__ double red[R][D];

  const long long wg = blockIdx.x;
  const int i = static_cast<int>(wg % nb);
  const long long tb = wg / nb;
  const int bh = static_cast<int>(tb % BH);
  const int tensor = static_cast<int>(tb / BH);
  const T* x = (tensor == 0 ? q : k) + static_cast<long long>(bh) * N * D;
  const int lo = i * block;
  const int n = min(block, N - lo);
  const int tid = threadIdx.x;
  const int r0 = tid / C;
  const int c = tid % C;

  double acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.0;
  for (int r = r0; r < n; r += R) {
    double v[E];
    load_chunk_f64<T>(x + static_cast<long long>(lo + r) * D + c * E, v);
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] += v[e];
  }
#pragma unroll
  for (int e = 0; e < E; ++e) red[r0][c * E + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    double s = 0.0;
#pragma unroll
    for (int r = 0; r < R; ++r) s += red[r][tid];
    const double mean = s / static_cast<double>(n);
    if (tensor == 0)
      qbar[(static_cast<long long>(bh) * nb + i) * D + tid] = mean;
    else
      kbar_t[(static_cast<long long>(bh) * D + tid) * nb + i] = mean;
  }
  if (wg == 0)
    for (int x2 = tid; x2 < BH; x2 += kPoolThreads) head_cnt[x2] = 0;
}

struct SelectSmem {
  double* z;         // [R][NP] scores, then probabilities (bit patterns sort as uint64)
  int* sidx;         // [NP] key-block index travelling with each key
  unsigned char* flag;  // [NP] selected flags by key-block index
  double* tot;       // [kSelThreads] chunk sums
  double* tot2;      // [kSelThreads] exclusive chunk prefixes
  int* itot;         // [kSelThreads]
  int* itot2;        // [kSelThreads]
  double* red;       // [kSelWaves]
  int* kfirst;       // [1]
};

__device__ double block_max(double x, double* red) {
  x = wave_max_f64(x);
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) red[wave] = x;
  __syncthreads();
  double r = red[0];
#pragma unroll
  for (int w = 1; w < kSelWaves; ++w) r = fmax(r, red[w]);
  __syncthreads();
  return r;
}

__device__ double block_sum(double x, double* red) {
  x = wave_sum_f64(x);
  const int wave = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) red[wave] = x;
  __syncthreads();
  double r = red[0];
#pragma unroll
  for (int w = 1; w < kSelWaves; ++w) r += red[w];
  __syncthreads();
  return r;
}

// Exclusive prefix of in[0..256) into out[0..256), fixed summation order.
// Called by wave 0 only.
template <typename V>
__device__ void wave0_exclusive_scan256(const V* in, V* out) {
  const int lane = threadIdx.x & (kWave - 1);
  const V a0 = in[4 * lane], a1 = in[4 * lane + 1], a2 = in[4 * lane + 2], a3 = in[4 * lane + 3];
  const V s = ((a0 + a1) + a2) + a3;
  V incl = s;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const V y = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += y;
  }
  V excl = __shfl_up(incl, 1, kWave);
  if (lane == 0) excl = V(0);
  out[4 * lane] = excl;
  out[4 * lane + 1] = excl + a0;
  out[4 * lane + 2] = (excl + a0) + a1;
  out[4 * lane + 3] = ((excl + a0) + a1) + a2;
}

template <int D, int R>
__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const double* __restrict__ qbar, const double* __restrict__ kbar_t, double scale, double top_p,
    int nb, int NP, int tiles_per_head, uint8_t* __restrict__ mask, int32_t* __restrict__ row_cnt,
    int32_t* __restrict__ row_idx, int32_t* __restrict__ head_cnt, double* __restrict__ block_prob) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  SelectSmem sm;
  {
    unsigned char* p = smem_raw;
    sm.z = reinterpret_cast<double*>(p);            p += sizeof(double) * R * NP;
    sm.tot = reinterpret_cast<double*>(p);          p += sizeof(double) * kSelThreads;
    sm.tot2 = reinterpret_cast<double*>(p);         p += sizeof(double) * kSelThreads;
    sm.red = reinterpret_cast<double*>(p);          p += sizeof(double) * kSelWaves;
    sm.sidx = reinterpret_cast<int*>(p);            p += sizeof(int) * NP;
    sm.itot = reinterpret_cast<int*>(p);            p += sizeof(int) * kSelThreads;
    sm.itot2 = reinterpret_cast<int*>(p);           p += sizeof(int) * kSelThreads;
    sm.kfirst = reinterpret_cast<int*>(p);          p += sizeof(int) * 4;
    sm.flag = p;
  }
  const int tid = threadIdx.x;
  const int bh = blockIdx.x / tiles_per_head;
  const int i0 = (blockIdx.x % tiles_per_head) * R;
  const int rows = min(R, nb - i0);

  // Phase 1: Z[r][j] = scale * <Qbar_{i0+r}, Kbar_j> in fp64.
  const double* kt = kbar_t + static_cast<long long>(bh) * D * nb;
  const double* qb = qbar + static_cast<long long>(bh) * nb * D;
  for (int j = tid; j < NP; j += kSelThreads) {
    double acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0;
    if (j < nb) {
      for (int c = 0; c < D; ++c) {
        const double kv = kt[static_cast<long long>(c) * nb + j];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int ir = min(i0 + r, nb - 1);
          acc[r] = fma(qb[static_cast<long long>(ir) * D + c], kv, acc[r]);
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) sm.z[r * NP + j] = scale * acc[r];
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r) sm.z[r * NP + j] = -INFINITY;
    }
  }
  __syncthreads();

  for (int r = 0; r < rows; ++r) {
    const int i = i0 + r;
    const long long row = static_cast<long long>(bh) * nb + i;
    double* zr = sm.z + r * NP;

    // Softmax over key blocks.
    double m = -INFINITY;
    for (int j = tid; j < nb; j += kSelThreads) m = fmax(m, zr[j]);
    m = block_max(m, sm.red);
    double s = 0.0;
    for (int j = tid; j < nb; j += kSelThreads) {
      const double e = exp(zr[j] - m);
      zr[j] = e;
      s += e;
    }
    s = block_sum(s, sm.red);
    for (int j = tid; j < NP; j += kSelThreads) {
      double pj = 0.0;
      if (j < nb) {
        pj = zr[j] / s;
        if (block_prob) block_prob[row * nb + j] = pj;
      }
      zr[j] = pj;
      sm.sidx[j] = j;
    }
    if (tid == 0) sm.kfirst[0] = NP;
    __syncthreads();

    // Bitonic sort: "a before b" iff P_a > P_b, or P_a == P_b and a < b.
    // Non-negative doubles order like their bit patterns; padding (P = 0,
    // index >= nb) sorts after every real block.
    unsigned long long* key = reinterpret_cast<unsigned long long*>(zr);
    for (int kk = 2; kk <= NP; kk <<= 1) {
      for (int jj = kk >> 1; jj > 0; jj >>= 1) {
        for (int e = tid; e < (NP >> 1); e += kSelThreads) {
          const int a = ((e & ~(jj - 1)) << 1) | (e & (jj - 1));
          const int b = a | jj;
          const bool up = (a & kk) == 0;
          const unsigned long long ka = key[a], kb = key[b];
          const int ia = sm.sidx[a], ib = sm.sidx[b];
          const bool b_first = (kb > ka) || (kb == ka && ib < ia);
          if (b_first == up) {
            key[a] = kb; key[b] = ka;
            sm.sidx[a] = ib; sm.sidx[b] = ia;
          }
        }
        __syncthreads();
      }
    }

    // Inclusive prefix sums of the ranked probabilities; first rank reaching p.
    const int per = NP >= kSelThreads ? NP / kSelThreads : 1;
    const int beg = tid * per;
    double loc = 0.0;
    for (int e = 0; e < per; ++e)
      if (beg + e < NP) loc += zr[beg + e];
    sm.tot[tid] = loc;
    __syncthreads();
    if (tid < kWave) wave0_exclusive_scan256<double>(sm.tot, sm.tot2);
    __syncthreads();
    {
      double run = sm.tot2[tid];
      for (int e = 0; e < per; ++e) {
        const int pos = beg + e;
        if (pos >= nb) break;
        run += zr[pos];
        if (run >= top_p) {
          atomicMin(sm.kfirst, pos);
          break;
        }
      }
    }
    for (int j = tid; j < NP; j += kSelThreads) sm.flag[j] = 0;
    __syncthreads();
    const int kf = sm.kfirst[0];
    const int kcnt = (top_p >= 1.0 || kf >= nb) ? nb : kf + 1;
    for (int e = tid; e < kcnt; e += kSelThreads) sm.flag[sm.sidx[e]] = 1;
    __syncthreads();

    // Mask row, ascending index list, counts.
    uint8_t* mrow = mask + row * nb;
    for (int j = tid; j < nb; j += kSelThreads) mrow[j] = sm.flag[j];
    const int per2 = (nb + kSelThreads - 1) / kSelThreads;
    const int beg2 = tid * per2;
    int cnt = 0;
    for (int e = 0; e < per2; ++e)
      if (beg2 + e < nb) cnt += sm.flag[beg2 + e];
    sm.itot[tid] = cnt;
    __syncthreads();
    if (tid < kWave) wave0_exclusive_scan256<int>(sm.itot, sm.itot2);
    __syncthreads();
    {
      int pos = sm.itot2[tid];
      int32_t* ridx = row_idx + row * nb;
      for (int e = 0; e < per2; ++e) {
        const int j = beg2 + e;
        if (j < nb && sm.flag[j]) ridx[pos++] = j;
      }
    }
    if (tid == 0) {
      row_cnt[row] = kcnt;
      atomicAdd(head_cnt + bh, kcnt);
    }
    __syncthreads();
  }
}

int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

template <int D, int R>
hipError_t launch_select_t(const Shape& s, const double* qbar, const double* kbar_t, double top_p,
                           uint8_t* mask, int32_t* row_cnt, int32_t* row_idx, int32_t* head_cnt,
                           double* block_prob, hipStream_t stream) {
  const int NP = next_pow2(s.nb);
  const size_t smem = sizeof(double) * (static_cast<size_t>(R) * NP + 2 * kSelThreads + kSelWaves) +
                      sizeof(int) * (NP + 2 * kSelThreads + 4) + NP;
  auto kern = select_kernel<D, R>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
  if (e != hipSuccess) return e;
  const int tiles = (s.nb + R - 1) / R;
  const long long grid = static_cast<long long>(s.B) * s.H * tiles;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(kSelThreads), smem, stream, qbar,
                     kbar_t, s.scale, top_p, s.nb, NP, tiles, mask, row_cnt, row_idx, head_cnt,
                     block_prob);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pool(const Shape& s, const void* q, const void* k, double* qbar, double* kbar_t,
                       int32_t* head_cnt, hipStream_t stream) {
  const int BH = s.B * s.H;
  const long long grid = 2LL * BH * s.nb;
  dim3 g(static_cast<unsigned>(grid)), b(kPoolThreads);
  if (s.dtype == 0) {
    auto qq = static_cast<const unsigned short*>(q);
    auto kk = static_cast<const unsigned short*>(k);
    if (s.d == 128)
      hipLaunchKernelGGL((pool_kernel<unsigned short, 128>), g, b, 0, stream, qq, kk, qbar, kbar_t,
                         head_cnt, BH, s.N, s.nb, s.block);
    else
      hipLaunchKernelGGL((pool_kernel<unsigned short, 64>), g, b, 0, stream, qq, kk, qbar, kbar_t,
                         head_cnt, BH, s.N, s.nb, s.block);
  } else {
    auto qq = static_cast<const float*>(q);
    auto kk = static_cast<const float*>(k);
    if (s.d == 128)
      hipLaunchKernelGGL((pool_kernel<float, 128>), g, b, 0, stream, qq, kk, qbar, kbar_t, head_cnt,
                         BH, s.N, s.nb, s.block);
    else
      hipLaunchKernelGGL((pool_kernel<float, 64>), g, b, 0, stream, qq, kk, qbar, kbar_t, head_cnt,
                         BH, s.N, s.nb, s.block);
  }
  return hipGetLastError();
}

hipError_t launch_select(const Shape& s, const double* qbar, const double* kbar_t, double top_p,
                         uint8_t* mask, int32_t* row_cnt, int32_t* row_idx, int32_t* head_cnt,
                         double* block_prob, hipStream_t stream) {
  const bool big = next_pow2(s.nb) > 512;
  if (s.d == 128)
    return big ? launch_select_t<128, 8>(s, qbar, kbar_t, top_p, mask, row_cnt, row_idx, head_cnt,
                                         block_prob, stream)
               : launch_select_t<128, 16>(s, qbar, kbar_t, top_p, mask, row_cnt, row_idx, head_cnt,
                                          block_prob, stream);
  return big ? launch_select_t<64, 8>(s, qbar, kbar_t, top_p, mask, row_cnt, row_idx, head_cnt,
                                      block_prob, stream)
             : launch_select_t<64, 16>(s, qbar, kbar_t, top_p, mask, row_cnt, row_idx, head_cnt,
                                       block_prob, stream);
}

}  // namespace tbs
