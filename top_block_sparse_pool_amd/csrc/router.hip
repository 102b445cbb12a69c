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
//   select_kernel  one workgroup per (b, h, R = 8 query blocks): fp64 scores
//                  for R rows against all key blocks (the R pooled query rows
//                  staged in LDS and read as broadcasts, pooled K read
//                  transposed so that lanes read consecutive key blocks, each
//                  thread holding all of its key blocks' sums); then one wave per
//                  row: a max/sum softmax, a register bitonic sort by
//                  (P desc, index asc), a fixed-order prefix sum to find the
//                  cut, and the outputs -- no workgroup barriers per row.
//
// Causal routing (decoder models): row i only considers key blocks j <= i.
// They are cut before the softmax, so the probabilities of row i are a
// softmax over its i+1 eligible scores, and p >= 1 (or a cumulative sum that
// never reaches p) selects those i+1 blocks.  The pages state top-p routing
// for full attention only; this block-level cut is the reading taken here.
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

// Block mean of Q over the valid tokens of query block i (workgroups
// 0 .. BH*nbq-1) or of K over key block j (the next BH*nbk workgroups).
template <typename T, int D>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(
    const T* __restrict__ q, const T* __restrict__ k, double* __restrict__ qbar,
    double* __restrict__ kbar_t, int32_t* __restrict__ head_cnt, int BH, int N, int nbq, int bq, int nbk,
    int bk) {
  constexpr int E = 16 / sizeof(T);           // elements per 16-byte chunk
  constexpr int C = D / E;                    // chunks per token row
  constexpr int R = kPoolThreads / C;         // token rows per pass
  __shared__ double red[R][D];

  const long long wg = blockIdx.x;
  const long long nq = static_cast<long long>(BH) * nbq;
  const int tensor = wg < nq ? 0 : 1;
  const long long wl = tensor == 0 ? wg : wg - nq;
  const int nb = tensor == 0 ? nbq : nbk;
  const int block = tensor == 0 ? bq : bk;
  const int i = static_cast<int>(wl % nb);
  const int bh = static_cast<int>(wl / nb);
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

// "a before b" in the ranking: larger probability first, then smaller index.
// Probabilities are non-negative doubles, which order like their bit
// patterns; padding elements (P = 0, index >= nb) rank after every real block.
__device__ __forceinline__ bool ranks_before(unsigned long long ka, int ia, unsigned long long kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

// Row phase of the selection, run by one wave per query-block row: E
// elements per lane in blocked order (position = lane*E + i).  Key blocks
// nv..nb-1 are not eligible (nv = nb except under causal routing): they get
// P = 0, rank after every eligible block and are never selected.
template <int E>
__device__ void select_row(const double* __restrict__ zr, int nb, int nv, double top_p, long long row, int bh,
                           unsigned char* __restrict__ flag, uint8_t* __restrict__ mask,
                           int32_t* __restrict__ row_cnt, int32_t* __restrict__ row_idx,
                           int32_t* __restrict__ head_cnt, double* __restrict__ block_prob) {
  constexpr int NP = 64 * E;
  const int lane = threadIdx.x & (kWave - 1);
  const int base = lane * E;

  // Softmax over key blocks (fp64), reductions in a fixed order.
  double v[E];
  double m = -INFINITY;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    v[i] = (base + i < nv) ? zr[base + i] : -INFINITY;
    m = fmax(m, v[i]);
  }
  m = wave_max_f64(m);
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    v[i] = (base + i < nv) ? exp(v[i] - m) : 0.0;
    s += v[i];
  }
  s = wave_sum_f64(s);
  unsigned long long key[E];
  int idx[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const double pj = v[i] / s;
    if (block_prob && base + i < nb) block_prob[row * nb + base + i] = pj;
    key[i] = __double_as_longlong(pj);
    idx[i] = base + i;
  }

  // Bitonic sort into ranking order.
#pragma unroll
  for (int k = 2; k <= NP; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j < E) {
#pragma unroll
        for (int i = 0; i < E; ++i) {
          if (i & j) continue;
          const int b = i | j;
          const bool up = ((base + i) & k) == 0;
          const bool b_first = ranks_before(key[b], idx[b], key[i], idx[i]);
          if (b_first == up) {
            const unsigned long long tk = key[i]; key[i] = key[b]; key[b] = tk;
            const int ti = idx[i]; idx[i] = idx[b]; idx[b] = ti;
          }
        }
      } else {
        const int lx = j / E;   // partner lane distance
#pragma unroll
        for (int i = 0; i < E; ++i) {
          const unsigned long long ok = __shfl_xor(key[i], lx, kWave);
          const int oi = __shfl_xor(idx[i], lx, kWave);
          const int pos = base + i;
          const bool lower = (pos & j) == 0;
          const bool up = (pos & k) == 0;
          const bool mine_first = ranks_before(key[i], idx[i], ok, oi);
          const bool keep = (lower == up) ? mine_first : !mine_first;
          if (!keep) { key[i] = ok; idx[i] = oi; }
        }
      }
    }
  }

  // Inclusive prefix of the ranked probabilities; first rank reaching top_p.
  double c[E];
  double run = 0.0;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    run += __longlong_as_double(key[i]);
    c[i] = run;
  }
  double incl = run;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const double y = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += y;
  }
  double excl = __shfl_up(incl, 1, kWave);
  if (lane == 0) excl = 0.0;
  int first = NP;
#pragma unroll
  for (int i = E - 1; i >= 0; --i)
    if (base + i < nv && excl + c[i] >= top_p) first = base + i;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) first = min(first, __shfl_xor(first, off, kWave));
  const int kcnt = (top_p >= 1.0 || first >= nv) ? nv : first + 1;

  // Flags by key-block index (this wave's LDS strip), then the outputs.
#pragma unroll
  for (int i = 0; i < E; ++i) flag[base + i] = 0;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int i = 0; i < E; ++i)
    if (base + i < kcnt) flag[idx[i]] = 1;
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
  int cnt = 0;
  unsigned char f[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    f[i] = flag[base + i];
    cnt += f[i];
  }
  uint8_t* mrow = mask + row * nb;
#pragma unroll
  for (int i = 0; i < E; ++i)
    if (base + i < nb) mrow[base + i] = f[i];
  int ic = cnt;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(ic, off, kWave);
    if (lane >= off) ic += y;
  }
  int pos = ic - cnt;
  int32_t* ridx = row_idx + row * nb;
#pragma unroll
  for (int i = 0; i < E; ++i)
    if (f[i]) ridx[pos++] = base + i;
  // After the selected blocks: the unselected eligible blocks in rank order
  // (rank positions kcnt .. nv-1), for slack-aware augmentation.
#pragma unroll
  for (int i = 0; i < E; ++i)
    if (base + i >= kcnt && base + i < nv) ridx[base + i] = idx[i];
  if (lane == 0) {
    row_cnt[row] = kcnt;
    atomicAdd(head_cnt + bh, kcnt);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

template <int D, int R, int E>
__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const double* __restrict__ qbar, const double* __restrict__ kbar_t, double scale, double top_p,
    int nbq, int nbk, int bq, int bk, int causal, int tiles_per_head, uint8_t* __restrict__ mask,
    int32_t* __restrict__ row_cnt,
    int32_t* __restrict__ row_idx, int32_t* __restrict__ head_cnt, double* __restrict__ block_prob) {
  constexpr int NP = 64 * E;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  double* z = reinterpret_cast<double*>(smem_raw);                           // [R][NP]
  double* qs = z + R * NP;                                                   // [R][D]
  unsigned char* flags = reinterpret_cast<unsigned char*>(qs + R * D);       // [waves][NP]
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int bh = blockIdx.x / tiles_per_head;
  const int i0 = (blockIdx.x % tiles_per_head) * R;
  const int rows = min(R, nbq - i0);

  // Phase 1: Z[r][j] = scale * <Qbar_{i0+r}, Kbar_j> in fp64.
  const double* kt = kbar_t + static_cast<long long>(bh) * D * nbk;
  const double* qb = qbar + static_cast<long long>(bh) * nbq * D;
  // The workgroup's R pooled query rows in LDS (read back as broadcasts).
  for (int x = tid; x < R * D; x += kSelThreads) qs[x] = qb[static_cast<long long>(min(i0 + x / D, nbq - 1)) * D + x % D];
  __syncthreads();
  // Each thread accumulates all J of its key blocks (j = tid + u * threads)
  // at once, so every broadcast read of a pooled query value feeds J FMAs;
  // the sum over the head dimension runs in increasing order.
  constexpr int CU = NP > 2 * kSelThreads ? 4 : 8;   // head-dimension steps per batch of pooled-K loads
  constexpr int J = NP > kSelThreads ? NP / kSelThreads : 1;
  if (tid < NP) {
    double acc[J][R];
    bool live[J];
#pragma unroll
    for (int u = 0; u < J; ++u) {
      live[u] = tid + u * kSelThreads < nbk;
#pragma unroll
      for (int r = 0; r < R; ++r) acc[u][r] = 0.0;
    }
    for (int c0 = 0; c0 < D; c0 += CU) {
      double kv[J][CU];
#pragma unroll
      for (int u = 0; u < J; ++u)
#pragma unroll
        for (int c = 0; c < CU; ++c)
          kv[u][c] = live[u] ? kt[static_cast<long long>(c0 + c) * nbk + tid + u * kSelThreads] : 0.0;
#pragma unroll
      for (int c = 0; c < CU; ++c)
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const double qv = qs[r * D + c0 + c];
#pragma unroll
          for (int u = 0; u < J; ++u) acc[u][r] = fma(qv, kv[u][c], acc[u][r]);
        }
    }
#pragma unroll
    for (int u = 0; u < J; ++u)
#pragma unroll
      for (int r = 0; r < R; ++r) z[r * NP + tid + u * kSelThreads] = live[u] ? scale * acc[u][r] : -INFINITY;
  }
  __syncthreads();

  // Phase 2: one wave per row.
  for (int r = wave; r < rows; r += kSelWaves) {
    const long long row = static_cast<long long>(bh) * nbq + i0 + r;
    // Causal routing: key blocks that start at or before the query block's last token.
    const int nv = causal ? min(nbk, ((i0 + r + 1) * bq - 1) / bk + 1) : nbk;
    select_row<E>(z + r * NP, nbk, nv, top_p, row, bh, flags + wave * NP, mask, row_cnt, row_idx, head_cnt,
                  block_prob);
  }
}

int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

template <int D, int R, int E>
hipError_t launch_select_t(const Shape& s, const double* qbar, const double* kbar_t, double top_p,
                           uint8_t* mask, int32_t* row_cnt, int32_t* row_idx, int32_t* head_cnt,
                           double* block_prob, hipStream_t stream) {
  constexpr int NP = 64 * E;
  const size_t smem = sizeof(double) * static_cast<size_t>(R) * (NP + D) + static_cast<size_t>(kSelWaves) * NP;
  auto kern = select_kernel<D, R, E>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
  if (e != hipSuccess) return e;
  const int tiles = (s.nb + R - 1) / R;   // query-block rows per head, R per workgroup
  const long long grid = static_cast<long long>(s.B) * s.H * tiles;
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(grid)), dim3(kSelThreads), smem, stream, qbar, kbar_t,
                     s.scale, top_p, s.nb, s.nbk, s.block, s.kb, s.causal ? 1 : 0, tiles, mask, row_cnt, row_idx, head_cnt, block_prob);
  return hipGetLastError();
}

template <int D>
hipError_t launch_select_d(const Shape& s, const double* qbar, const double* kbar_t, double top_p,
                           uint8_t* mask, int32_t* row_cnt, int32_t* row_idx, int32_t* head_cnt,
                           double* block_prob, hipStream_t stream) {
  const int np = next_pow2(s.nbk < 64 ? 64 : s.nbk);
  switch (np) {
    case 64: return launch_select_t<D, 8, 1>(s, qbar, kbar_t, top_p, mask, row_cnt, row_idx, head_cnt, block_prob, stream);
    case 128: return launch_select_t<D, 8, 2>(s, qbar, kbar_t, top_p, mask, row_cnt, row_idx, head_cnt, block_prob, stream);
    case 256: return launch_select_t<D, 8, 4>(s, qbar, kbar_t, top_p, mask, row_cnt, row_idx, head_cnt, block_prob, stream);
    case 512: return launch_select_t<D, 8, 8>(s, qbar, kbar_t, top_p, mask, row_cnt, row_idx, head_cnt, block_prob, stream);
    default: return launch_select_t<D, 8, 16>(s, qbar, kbar_t, top_p, mask, row_cnt, row_idx, head_cnt, block_prob, stream);
  }
}

}  // namespace

hipError_t launch_pool(const Shape& s, const void* q, const void* k, double* qbar, double* kbar_t,
                       int32_t* head_cnt, hipStream_t stream) {
  const int BH = s.B * s.H;
  const long long grid = static_cast<long long>(BH) * (s.nb + s.nbk);
  dim3 g(static_cast<unsigned>(grid)), b(kPoolThreads);
  if (s.dtype == 0) {
    auto qq = static_cast<const unsigned short*>(q);
    auto kk = static_cast<const unsigned short*>(k);
    if (s.d == 128)
      hipLaunchKernelGGL((pool_kernel<unsigned short, 128>), g, b, 0, stream, qq, kk, qbar, kbar_t,
                         head_cnt, BH, s.N, s.nb, s.block, s.nbk, s.kb);
    else
      hipLaunchKernelGGL((pool_kernel<unsigned short, 64>), g, b, 0, stream, qq, kk, qbar, kbar_t,
                         head_cnt, BH, s.N, s.nb, s.block, s.nbk, s.kb);
  } else {
    auto qq = static_cast<const float*>(q);
    auto kk = static_cast<const float*>(k);
    if (s.d == 128)
      hipLaunchKernelGGL((pool_kernel<float, 128>), g, b, 0, stream, qq, kk, qbar, kbar_t, head_cnt,
                         BH, s.N, s.nb, s.block, s.nbk, s.kb);
    else
      hipLaunchKernelGGL((pool_kernel<float, 64>), g, b, 0, stream, qq, kk, qbar, kbar_t, head_cnt,
                         BH, s.N, s.nb, s.block, s.nbk, s.kb);
  }
  return hipGetLastError();
}

hipError_t launch_select(const Shape& s, const double* qbar, const double* kbar_t, double top_p,
                         uint8_t* mask, int32_t* row_cnt, int32_t* row_idx, int32_t* head_cnt,
                         double* block_prob, hipStream_t stream) {
  if (s.d == 128)
    return launch_select_d<128>(s, qbar, kbar_t, top_p, mask, row_cnt, row_idx, head_cnt, block_prob, stream);
  return launch_select_d<64>(s, qbar, kbar_t, top_p, mask, row_cnt, row_idx, head_cnt, block_prob, stream);
}

}  // namespace tbs
