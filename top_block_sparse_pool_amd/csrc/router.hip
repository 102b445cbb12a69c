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
//   pool_qk_kernel one workgroup per (b, h, span of 64 or 128 tokens) of bf16
//                  Q and K: block means in fp64 (HBM-bound: reads Q and K
//                  once, every load of a thread in flight at once), and for
//                  the fp8 path the E4M3 codes and scales of the same rows.
//   pool_kernel    the same means for fp32 inputs, one workgroup per
//                  (tensor, b, h, block).
//   select_kernel  one workgroup per (b, h, R = 8 query blocks): fp64 scores
//                  for R rows against all key blocks (the R pooled query rows
//                  staged in LDS and read as broadcasts, pooled K read
//                  transposed so that lanes read consecutive key blocks, each
//                  thread holding all of its key blocks' sums); then one wave per
//                  row: a max/sum softmax, a register bitonic sort of one
//                  64-bit key per block (P's high bits, then the index;
//                  rows of more than 512 blocks keep the stage loop rolled),
//                  an exact fix-up of runs with equal high bits, a
//                  fixed-order prefix sum to find the cut, and the outputs --
//                  no workgroup barriers per row.  The pooled query rows
//                  share LDS with the score tile, which they precede.
//
// Causal routing (decoder models): row i only considers key blocks j <= i.
// They are cut before the softmax, so the probabilities of row i are a
// softmax over its i+1 eligible scores, and p >= 1 (or a cumulative sum that
// never reaches p) selects those i+1 blocks.  The pages state top-p routing
// for full attention only; this block-level cut is the reading taken here.
#include <math.h>

#include "device_common.h"
#include "e4m3.h"
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

// Block means of bf16 Q and K over one span of SPAN tokens of one (b, h) per
// workgroup (SPAN = the larger of the query and key block sizes, so every
// block lies in one span), and with QUANT the E4M3 codes and scales of the
// same rows (one scale per query token, one per 64-token key tile), from one
// read of each element.
//
// Summation order (fp64, fixed): per 64-token tile, a thread adds its rows
// r0, r0 + RP, ... of one 16-byte column chunk; the row groups of a wave
// combine by xor shuffles (the same sum in every lane, fp64 addition being
// commutative); the four waves add in wave order; a 128-token block adds its
// two tiles in order.  The mean divides by the block's valid tokens.
template <int D, int SPAN, bool QUANT>
__global__ __launch_bounds__(kPoolThreads) void pool_qk_kernel(
    const unsigned short* __restrict__ q, const unsigned short* __restrict__ k, double* __restrict__ qbar,
    double* __restrict__ kbar_t, int32_t* __restrict__ head_cnt, uint8_t* __restrict__ q8,
    float* __restrict__ q_scale, uint8_t* __restrict__ k8, float* __restrict__ k_scale, int BH, int N, int nbq,
    int bq, int nbk, int bk, int nspan, int nkt) {
  constexpr int C = D / 8;                    // 16-byte chunks per token row
  constexpr int RP = kPoolThreads / C;        // rows per pass (16 for d = 128, 32 for d = 64)
  constexpr int P = 64 / RP;                  // passes per 64-token tile
  constexpr int T = SPAN / 64;                // tiles per span
  constexpr int NW = kPoolThreads / kWave;
  static_assert(!QUANT || D == 128, "the fp8 path takes head_dim 128");
  __shared__ double red[NW][2][T][D];
  __shared__ float kmax_s[NW][T];

  // Heads in reverse order: the first heads that the selection (and then
  // the attention) reads are the ones pooled last, still in the caches.
  const int bh = BH - 1 - static_cast<int>(blockIdx.x) / nspan;
  const int t0 = (blockIdx.x % nspan) * SPAN;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int c = tid % C;
  const int r0 = tid / C;
  const long long base = static_cast<long long>(bh) * N;

  // Every load first: P rows of each tile, Q and K.
  u32x4 xq[T][P], xk[T][P];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int pp = 0; pp < P; ++pp) {
      const int row = t0 + 64 * t + r0 + RP * pp;
      const bool valid = row < N;
      const long long off = (base + (valid ? row : 0)) * D + c * 8;
      xq[t][pp] = valid ? *reinterpret_cast<const u32x4*>(q + off) : u32x4{0u, 0u, 0u, 0u};
      xk[t][pp] = valid ? *reinterpret_cast<const u32x4*>(k + off) : u32x4{0u, 0u, 0u, 0u};
    }

  // Column sums of each tile: over the thread's rows, then the wave's row
  // groups; lanes of the first row group write their chunk.
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int ten = 0; ten < 2; ++ten) {
      double acc[8];
#pragma unroll
      for (int pp = 0; pp < P; ++pp) {
        float x[8];
        bf16x8_to_f32(ten == 0 ? xq[t][pp] : xk[t][pp], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = pp == 0 ? static_cast<double>(x[e]) : acc[e] + static_cast<double>(x[e]);
      }
#pragma unroll
      for (int off = C; off < kWave; off <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], off, kWave);
      if (lane < C)
#pragma unroll
        for (int e = 0; e < 8; ++e) red[wave][ten][t][c * 8 + e] = acc[e];
    }

  if constexpr (QUANT) {
    // E4M3: a scale per query row (over the row's C lanes), one per K tile.
#pragma unroll
    for (int t = 0; t < T; ++t) {
      float km = 0.f;
#pragma unroll
      for (int pp = 0; pp < P; ++pp) {
        const int row = t0 + 64 * t + r0 + RP * pp;
        float x[8];
        bf16x8_to_f32(xq[t][pp], x);
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(x[e]));
#pragma unroll
        for (int off = 1; off < C; off <<= 1) a = fmaxf(a, __shfl_xor(a, off, kWave));
        if (row < N) {
          *reinterpret_cast<u32x2*>(q8 + (base + row) * D + c * 8) = e4m3_encode8(x, e4m3_group_inv(a));
          if (c == 0) q_scale[base + row] = e4m3_group_scale(a);
        }
        bf16x8_to_f32(xk[t][pp], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) km = fmaxf(km, fabsf(x[e]));
      }
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) km = fmaxf(km, __shfl_xor(km, off, kWave));
      if (lane == 0) kmax_s[wave][t] = km;
    }
  }
  __syncthreads();

  if constexpr (QUANT) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int tile = (t0 + 64 * t) / 64;
      if (tile >= nkt) continue;
      float a = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) a = fmaxf(a, kmax_s[w][t]);
      const float inv = e4m3_group_inv(a);
#pragma unroll
      for (int pp = 0; pp < P; ++pp) {
        const int row = t0 + 64 * t + r0 + RP * pp;
        if (row < N) {
          float x[8];
          bf16x8_to_f32(xk[t][pp], x);
          *reinterpret_cast<u32x2*>(k8 + (base + row) * D + c * 8) = e4m3_encode8(x, inv);
        }
      }
      if (tid == 0) k_scale[static_cast<long long>(bh) * nkt + tile] = e4m3_group_scale(a);
    }
  }

  // Block means: tile sums over the waves in order, blocks of 128 tokens
  // adding their two tiles.
  if (tid < 2 * D) {
    const int ten = tid / D;
    const int col = tid % D;
    double ts[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
      double s = red[0][ten][t][col];
#pragma unroll
      for (int w = 1; w < NW; ++w) s += red[w][ten][t][col];
      ts[t] = s;
    }
    const int blk = ten == 0 ? bq : bk;
    const int nb = ten == 0 ? nbq : nbk;
    if (blk == 64) {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int i = (t0 + 64 * t) / 64;
        if (i >= nb) continue;
        const double mean = ts[t] / static_cast<double>(min(64, N - 64 * i));
        if (ten == 0)
          qbar[(static_cast<long long>(bh) * nb + i) * D + col] = mean;
        else
          kbar_t[(static_cast<long long>(bh) * D + col) * nb + i] = mean;
      }
    } else {
      const int i = t0 / 128;
      double s = ts[0];
#pragma unroll
      for (int t = 1; t < T; ++t) s += ts[t];
      const double mean = s / static_cast<double>(min(128, N - 128 * i));
      if (ten == 0)
        qbar[(static_cast<long long>(bh) * nb + i) * D + col] = mean;
      else
        kbar_t[(static_cast<long long>(bh) * D + col) * nb + i] = mean;
    }
  }
  if (blockIdx.x == 0)
    for (int x2 = tid; x2 < BH; x2 += kPoolThreads) head_cnt[x2] = 0;
}

// Value of lane (lane ^ LX) for a 32-bit register, with VALU lane moves instead
// of an LDS permute: DPP quad permutations (1, 2), a quad reversal followed by
// a half-row mirror (4), a row rotation by half a row (8), and the gfx950 row
// swaps (16, 32).
template <int LX>
__device__ __forceinline__ unsigned xor_lane(unsigned v) {
  const unsigned lane = __lane_id();
  if constexpr (LX == 1) {
    return __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  } else if constexpr (LX == 2) {
    return __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  } else if constexpr (LX == 4) {
    // quad reversal (l ^ 3) then the half-row mirror (7 - l within 8 lanes):
    // lane l reads lane (7 - l) ^ 3 = l ^ 4
    const unsigned r = __builtin_amdgcn_update_dpp(v, v, 0x1B, 0xF, 0xF, false);    // quad_perm [3,2,1,0]
    return __builtin_amdgcn_update_dpp(r, r, 0x141, 0xF, 0xF, false);               // row_half_mirror
  } else if constexpr (LX == 8) {
    return __builtin_amdgcn_update_dpp(v, v, 0x128, 0xF, 0xF, false);  // row_ror:8
  } else if constexpr (LX == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (lane & 16) ? r[0] : r[1];
  } else {
    static_assert(LX == 32, "lane distance");
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (lane & 32) ? r[0] : r[1];
  }
}

template <int LX>
__device__ __forceinline__ unsigned long long xor_lane64(unsigned long long v) {
  const unsigned lo = xor_lane<LX>(static_cast<unsigned>(v));
  const unsigned hi = xor_lane<LX>(static_cast<unsigned>(v >> 32));
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}

// Sort keys: the top 32 bits of P's bit pattern (non-negative doubles order
// like their bits, so this is monotone in P), then the key-block index
// inverted, so that a larger key ranks first and equal high bits rank the
// smaller index first.  Equal high bits do not mean equal P: such runs are
// put in exact order afterwards.
__device__ __forceinline__ unsigned long long rank_key(double p, int idx) {
  const unsigned hi = static_cast<unsigned>(static_cast<unsigned long long>(__double_as_longlong(p)) >> 31);
  return (static_cast<unsigned long long>(hi) << 32) | (0xffffffffu - static_cast<unsigned>(idx));
}
__device__ __forceinline__ int key_index(unsigned long long key) {
  return static_cast<int>(0xffffffffu - static_cast<unsigned>(key));
}
// Exact ranking of two keys with equal high bits: larger P (read by index from
// the row's probabilities p) first, then the smaller index.
__device__ __forceinline__ bool exact_before(const TBS_LDS double* p, unsigned long long a, unsigned long long b) {
  const int ia = key_index(a), ib = key_index(b);
  const double pa = p[ia], pb = p[ib];
  return pa > pb || (pa == pb && ia < ib);
}
__device__ __forceinline__ bool same_run(unsigned long long a, unsigned long long b) { return (a >> 32) == (b >> 32); }

// Row phase of the selection, run by one wave per query-block row: E
// elements per lane in blocked order (position = lane*E + i).  Key blocks
// nv..nb-1 are not eligible (nv = nb except under causal routing): they get
// P = 0, rank after every eligible block and are never selected.  zr holds
// the row's scores on entry and its probabilities (by key-block index) after.
template <int E>
__device__ void select_row(TBS_LDS double* __restrict__ zr, int nb, int nv, double top_p, long long row, int bh,
                           TBS_LDS unsigned char* __restrict__ flag, uint8_t* __restrict__ mask,
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
  const double inv = 1.0 / s;
  unsigned long long key[E];
#pragma unroll
  for (int i = 0; i < E; ++i) {
    const double pj = v[i] * inv;
    if (block_prob && base + i < nb) block_prob[row * nb + base + i] = pj;
    zr[base + i] = pj;
    key[i] = rank_key(pj, base + i);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();

  // Bitonic sort by key, larger first.
  if constexpr (E >= 16) {
    // Rows of more than 512 blocks: the same stages with the stage loop kept
    // rolled and cross-lane partners read with a lane permute at a run-time
    // distance, so the code (and with it the register need) stays small.
    for (int k = 2; k <= NP; k <<= 1) {
      for (int j = k >> 1; j >= E; j >>= 1) {
        const int lx = j / E;   // partner lane distance
#pragma unroll
        for (int i = 0; i < E; ++i) {
          const unsigned long long ok = __shfl_xor(key[i], lx, kWave);
          const int pos = base + i;
          const bool lower = (pos & j) == 0;
          const bool up = (pos & k) == 0;
          const bool mine_first = key[i] > ok;
          key[i] = (lower == up) != mine_first ? ok : key[i];
        }
      }
#pragma unroll
      for (int j = E >> 1; j > 0; j >>= 1) {
        if (j >= k) continue;
#pragma unroll
        for (int i = 0; i < E; ++i) {
          if (i & j) continue;
          const int b = i | j;
          const bool up = ((base + i) & k) == 0;
          const bool sw = (key[b] > key[i]) == up;
          const unsigned long long ki = key[i], kb = key[b];
          key[i] = sw ? kb : ki;
          key[b] = sw ? ki : kb;
        }
      }
    }
  } else {
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
            const bool sw = (key[b] > key[i]) == up;
            const unsigned long long ki = key[i], kb = key[b];
            key[i] = sw ? kb : ki;
            key[b] = sw ? ki : kb;
          }
        } else {
          const int lx = j / E;   // partner lane distance
#pragma unroll
          for (int i = 0; i < E; ++i) {
            unsigned long long ok;
            switch (lx) {
              case 1: ok = xor_lane64<1>(key[i]); break;
              case 2: ok = xor_lane64<2>(key[i]); break;
              case 4: ok = xor_lane64<4>(key[i]); break;
              case 8: ok = xor_lane64<8>(key[i]); break;
              case 16: ok = xor_lane64<16>(key[i]); break;
              default: ok = xor_lane64<32>(key[i]); break;
            }
            const int pos = base + i;
            const bool lower = (pos & j) == 0;
            const bool up = (pos & k) == 0;
            const bool mine_first = key[i] > ok;
            key[i] = (lower == up) != mine_first ? ok : key[i];
          }
        }
      }
    }
  }

  // Exact order inside runs of equal high bits: odd-even transposition over
  // neighbouring positions, comparing P itself, until a pass swaps nothing
  // (usually at once: such runs need P equal to about 2^-21 relative).
  for (;;) {
    bool swapped = false;
#pragma unroll
    for (int phase = 0; phase < 2; ++phase) {
      if constexpr (E == 1) {
        // positions are lanes: partner lane^1 (phase 0) or the odd pair (phase 1)
        const bool left = phase == 0 ? (lane & 1) == 0 : (lane & 1) == 1;
        const int partner = left ? lane + 1 : lane - 1;
        const unsigned long long ok = __shfl(key[0], partner & (kWave - 1), kWave);
        const bool valid = partner >= 0 && partner < kWave;
        if (valid && same_run(key[0], ok)) {
          const bool in_order = left ? exact_before(zr, key[0], ok) : exact_before(zr, ok, key[0]);
          if (!in_order) {
            key[0] = ok;
            swapped = true;
          }
        }
      } else {
        // in-lane pairs (i, i + 1) with i = phase, phase + 2, ...
#pragma unroll
        for (int i = phase; i + 1 < E; i += 2) {
          if (same_run(key[i], key[i + 1]) && !exact_before(zr, key[i], key[i + 1])) {
            const unsigned long long t = key[i];
            key[i] = key[i + 1];
            key[i + 1] = t;
            swapped = true;
          }
        }
        if (phase == 1) {
          // across lanes: this lane's last element and the next lane's first
          const unsigned long long right = __shfl_down(key[0], 1, kWave);
          const unsigned long long left = __shfl_up(key[E - 1], 1, kWave);
          const unsigned long long my_last = key[E - 1], my_first = key[0];
          if (lane < kWave - 1 && same_run(my_last, right) && !exact_before(zr, my_last, right)) {
            key[E - 1] = right;
            swapped = true;
          }
          if (lane > 0 && same_run(left, my_first) && !exact_before(zr, left, my_first)) {
            key[0] = left;
            swapped = true;
          }
        }
      }
    }
    if (!__any(swapped)) break;
  }
  int idx[E];
#pragma unroll
  for (int i = 0; i < E; ++i) idx[i] = key_index(key[i]);

  // Inclusive prefix of the ranked probabilities; first rank reaching top_p.
  double c[E];
  double run = 0.0;
#pragma unroll
  for (int i = 0; i < E; ++i) {
    run += zr[idx[i]];
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
  // The pooled query rows are read only before the scores are stored, so
  // they share the score tile's memory.
  constexpr int ZQ = NP > D ? NP : D;                                        // doubles per row of that memory
  TBS_LDS double* z = (TBS_LDS double*)smem_raw;                             // [R][NP]
  TBS_LDS double* qs = z;                                                    // [R][D]
  TBS_LDS unsigned char* flags = (TBS_LDS unsigned char*)(z + R * ZQ);       // [waves][NP]
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
  double acc[J][R];
  bool live[J];
#pragma unroll
  for (int u = 0; u < J; ++u) {
    live[u] = tid + u * kSelThreads < nbk;
#pragma unroll
    for (int r = 0; r < R; ++r) acc[u][r] = 0.0;
  }
  if (tid < NP) {
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
  }
  __syncthreads();   // every read of the pooled query rows is done
  if (tid < NP) {
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
  const size_t smem = sizeof(double) * static_cast<size_t>(R) * (NP > D ? NP : D) + static_cast<size_t>(kSelWaves) * NP;
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

namespace {
template <int D, int SPAN, bool QUANT>
void launch_pool_qk_t(const Shape& s, const unsigned short* q, const unsigned short* k, double* qbar, double* kbar_t,
                      int32_t* head_cnt, uint8_t* q8, float* q_scale, uint8_t* k8, float* k_scale,
                      hipStream_t stream) {
  const int BH = s.B * s.H;
  const int nspan = (s.N + SPAN - 1) / SPAN;
  const int nkt = (s.N + 63) / 64;
  const long long grid = static_cast<long long>(BH) * nspan;
  hipLaunchKernelGGL((pool_qk_kernel<D, SPAN, QUANT>), dim3(static_cast<unsigned>(grid)), dim3(kPoolThreads), 0,
                     stream, q, k, qbar, kbar_t, head_cnt, q8, q_scale, k8, k_scale, BH, s.N, s.nb, s.block, s.nbk,
                     s.kb, nspan, nkt);
}
}  // namespace

hipError_t launch_pool_quant(const Shape& s, const void* q, const void* k, double* qbar, double* kbar_t,
                             int32_t* head_cnt, uint8_t* q8, float* q_scale, uint8_t* k8, float* k_scale,
                             hipStream_t stream) {
  auto qq = static_cast<const unsigned short*>(q);
  auto kk = static_cast<const unsigned short*>(k);
  if (s.dtype != 0 || s.d != 128) return hipErrorInvalidValue;
  if (s.block == 128 || s.kb == 128)
    launch_pool_qk_t<128, 128, true>(s, qq, kk, qbar, kbar_t, head_cnt, q8, q_scale, k8, k_scale, stream);
  else
    launch_pool_qk_t<128, 64, true>(s, qq, kk, qbar, kbar_t, head_cnt, q8, q_scale, k8, k_scale, stream);
  return hipGetLastError();
}

hipError_t launch_pool(const Shape& s, const void* q, const void* k, double* qbar, double* kbar_t,
                       int32_t* head_cnt, hipStream_t stream) {
  const int BH = s.B * s.H;
  const long long grid = static_cast<long long>(BH) * (s.nb + s.nbk);
  dim3 g(static_cast<unsigned>(grid)), b(kPoolThreads);
  if (s.dtype == 0) {
    auto qq = static_cast<const unsigned short*>(q);
    auto kk = static_cast<const unsigned short*>(k);
    const bool wide = s.block == 128 || s.kb == 128;
    if (s.d == 128) {
      // 64-token blocks too go two to a workgroup (half as many workgroups,
      // 64 KB read by each; the same per-block sums)
      launch_pool_qk_t<128, 128, false>(s, qq, kk, qbar, kbar_t, head_cnt, nullptr, nullptr, nullptr, nullptr, stream);
    } else {
      if (wide)
        launch_pool_qk_t<64, 128, false>(s, qq, kk, qbar, kbar_t, head_cnt, nullptr, nullptr, nullptr, nullptr, stream);
      else
        launch_pool_qk_t<64, 64, false>(s, qq, kk, qbar, kbar_t, head_cnt, nullptr, nullptr, nullptr, nullptr, stream);
    }
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
