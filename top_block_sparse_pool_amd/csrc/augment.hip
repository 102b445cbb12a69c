// Slack-aware sparse augmentation on one GPU (gfx950).
//
// Source: FVAttn review page, section 1 (Key Terms, "Slack-Aware Sparse
// Augmentation (SASA)"): after load balancing, ranks left with slack receive
// additional high-value sparse blocks; section 3 (Method & Key Results): SASA
// spends each rank's idle time after load balancing on extra blocks.
//
// On one GPU the ranks are the W workers of the longest-first LPT model: the
// slack of worker w is s_w = M - L_w (M the largest load), and w adds the
// first min(s_w, #candidates) of its candidates -- the eligible unselected
// key blocks of the query blocks of its work items -- in the order
// (P desc, unit asc, key block asc).  Inside one row that is the routing rank
// order, which the router leaves in row_idx after the selected blocks, so a
// row's additions are the next entries of that ranked tail.
//
// Kernels:
//   aug_csr_kernel     one workgroup: the query-block rows of every worker as
//                      one array segmented by worker (counts, scan, fill).
//   aug_merge_kernel   one wave per worker: a merge of its rows' ranked tails
//                      by (P desc, unit asc); every row keeps its next 16
//                      candidates cached (LDS, or workspace memory for a
//                      worker with more than 512 rows), so a pick costs a
//                      scan of the winning lane's rows and one wave argmax,
//                      and a row's cache is refilled every 16 picks.
//   aug_rebuild_kernel one wave per row that gained blocks: the ascending
//                      list of the new selection, mask bits, counts.
//   aug_union_kernel   slack inside a work item (attn_augment_union): one
//                      workgroup per item, one wave per member row.  The
//                      attention kernel runs an item as the union of its rows'
//                      key tiles and a wave idles on the tiles its row did not
//                      select; every row takes the eligible blocks of the
//                      union, so the item's tiles, and its time, stay the same.
#include "device_common.h"
#include "launch.h"

namespace tbs {
namespace {

constexpr int kCsrThreads = 1024;
constexpr int kAugCache = 16;        // cached candidates per row
constexpr int kAugLdsRows = 512;     // rows per worker whose state fits LDS (104 KB)

struct AugRow {
  int u;       // unit id (b*H + h)*nb + i
  int k;       // selected blocks before augmentation
  int rem;     // eligible unselected blocks (length of the ranked tail)
  int a;       // blocks added so far
  double cp[kAugCache];   // P and index of ranked-tail entries a - a % kAugCache .. + kAugCache - 1
  int cj[kAugCache];
};

__device__ __forceinline__ int unit_group_size(int g, int nb, int G, int ng) {
  const int i0 = (g % ng) * G;
  return min(G, nb - i0);
}

// Rows of every worker, grouped by worker: off[w] .. off[w+1] in rows[].
__global__ __launch_bounds__(kCsrThreads) void aug_csr_kernel(const int32_t* __restrict__ worker_of, int items,
                                                              int nb, int G, int ng, int W,
                                                              int32_t* __restrict__ off,
                                                              int32_t* __restrict__ rows) {
  __shared__ int cnt[4096];
  __shared__ int part[kCsrThreads];
  const int tid = threadIdx.x;
  for (int w = tid; w < W; w += kCsrThreads) cnt[w] = 0;
  __syncthreads();
  for (int g = tid; g < items; g += kCsrThreads) {
    const int w = min(max(worker_of[g], 0), W - 1);
    atomicAdd(&cnt[w], unit_group_size(g, nb, G, ng));
  }
  __syncthreads();
  // Exclusive scan over workers: each thread sums a run of consecutive workers.
  const int per = (W + kCsrThreads - 1) / kCsrThreads;
  const int w0 = min(W, tid * per);
  const int w1 = min(W, w0 + per);
  int run = 0;
  for (int w = w0; w < w1; ++w) run += cnt[w];
  part[tid] = run;
  __syncthreads();
  for (int d = 1; d < kCsrThreads; d <<= 1) {
    const int y = tid >= d ? part[tid - d] : 0;
    __syncthreads();
    part[tid] += y;
    __syncthreads();
  }
  int acc = part[tid] - run;
  for (int w = w0; w < w1; ++w) {
    const int c = cnt[w];
    off[w] = acc;
    cnt[w] = acc;   // becomes the fill cursor
    acc += c;
  }
  if (tid == kCsrThreads - 1) off[W] = part[tid];
  __syncthreads();
  for (int g = tid; g < items; g += kCsrThreads) {
    const int w = min(max(worker_of[g], 0), W - 1);
    const int gs = unit_group_size(g, nb, G, ng);
    const int p = atomicAdd(&cnt[w], gs);
    const int u0 = (g / ng) * nb + (g % ng) * G;
    for (int m = 0; m < gs; ++m) rows[p + m] = u0 + m;
  }
}

// Candidates a .. a + kAugCache - 1 of a row's ranked tail into its cache
// (rows of nbk key-block entries).
__device__ __forceinline__ void aug_refill(AugRow* st, const int32_t* __restrict__ row_idx,
                                           const double* __restrict__ block_prob, int nbk) {
  const long long rb = static_cast<long long>(st->u) * nbk;
  const int a = st->a, k = st->k, rem = st->rem;
  // All index loads, then all probability loads, then the stores: the state
  // may live in global memory, so stores between loads would serialise them.
  int jv[kAugCache];
#pragma unroll
  for (int c = 0; c < kAugCache; ++c) jv[c] = a + c < rem ? min(max(row_idx[rb + k + a + c], 0), nbk - 1) : 0;
  double pv[kAugCache];
#pragma unroll
  for (int c = 0; c < kAugCache; ++c) pv[c] = a + c < rem ? block_prob[rb + jv[c]] : 0.0;
#pragma unroll
  for (int c = 0; c < kAugCache; ++c) {
    st->cj[c] = jv[c];
    st->cp[c] = pv[c];
  }
}

// Ordering key of a row's next candidate: P's bits (P >= 0 orders like its
// bits), -1 once the tail is used up.
__device__ __forceinline__ long long aug_head(const AugRow* st) {
  if (st->a >= st->rem) return -1;
  return __double_as_longlong(st->cp[st->a % kAugCache]);
}

__global__ __launch_bounds__(kWave) void aug_merge_kernel(const double* __restrict__ block_prob,
                                                          const int32_t* __restrict__ row_cnt,
                                                          const int32_t* __restrict__ row_idx,
                                                          const int64_t* __restrict__ worker_load, int W, int nb,
                                                          int nbk, int bq, int bk, int causal,
                                                          const int32_t* __restrict__ off,
                                                          const int32_t* __restrict__ rows,
                                                          AugRow* __restrict__ gstate,
                                                          int32_t* __restrict__ aug_add,
                                                          int32_t* __restrict__ added) {
  __shared__ AugRow lstate[kAugLdsRows];
  const int lane = threadIdx.x;
  const int w = blockIdx.x;

  long long mx = 0;
  for (int x = lane; x < W; x += kWave) mx = max(mx, static_cast<long long>(worker_load[x]));
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = max(mx, __shfl_xor(mx, o, kWave));
  const long long slack = mx - static_cast<long long>(worker_load[w]);

  const int r0 = off[w];
  const int nr = off[w + 1] - r0;
  AugRow* st = nr <= kAugLdsRows ? lstate : gstate + r0;

  long long total = 0;
  for (int r = lane; r < nr; r += kWave) {
    AugRow* s = st + r;
    const int u = rows[r0 + r];
    const int i = u % nb;
    // Causal routing: key blocks that start at or before the query block's last token.
    const int nv = causal ? min(nbk, ((i + 1) * bq - 1) / bk + 1) : nbk;
    s->u = u;
    s->k = min(max(row_cnt[u], 0), nv);
    s->rem = nv - s->k;
    s->a = 0;
    total += s->rem;
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) total += __shfl_xor(total, o, kWave);

  long long picks = 0;
  if (slack >= total) {
    // Every candidate fits in the slack.
    for (int r = lane; r < nr; r += kWave) st[r].a = st[r].rem;
    picks = total;
  } else if (slack > 0) {
    for (int r = lane; r < nr; r += kWave) aug_refill(st + r, row_idx, block_prob, nbk);
    // Best head among this lane's rows; only the lane that owned the last
    // winner rescans.
    long long bk = -1;
    int bu = 0x7fffffff, br = -1;
    auto rescan = [&]() {
      bk = -1;
      bu = 0x7fffffff;
      br = -1;
      for (int r = lane; r < nr; r += kWave) {
        const long long k = aug_head(st + r);
        const int u = st[r].u;
        if (k > bk || (k == bk && k >= 0 && u < bu)) {
          bk = k;
          bu = u;
          br = r;
        }
      }
    };
    rescan();
    for (; picks < slack; ++picks) {
      long long k = bk;
      int u = bu;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const long long ok = __shfl_xor(k, o, kWave);
        const int ou = __shfl_xor(u, o, kWave);
        if (ok > k || (ok == k && ou < u)) {
          k = ok;
          u = ou;
        }
      }
      if (k < 0) break;   // no candidate left (cannot happen while picks < total)
      if (bk == k && bu == u) {
        AugRow* s = st + br;
        s->a += 1;
        if (s->a % kAugCache == 0 && s->a < s->rem) aug_refill(s, row_idx, block_prob, nbk);
        rescan();
      }
    }
  }
  for (int r = lane; r < nr; r += kWave) aug_add[st[r].u] = st[r].a;
  if (lane == 0 && added) added[w] = static_cast<int32_t>(picks);
}

// A row that gained `a` blocks: its first k + a row_idx entries (the old
// ascending list, then the added blocks in rank order) become one ascending
// list; mask bits, row count and head count follow.  The ranked tail after
// them is unchanged.
constexpr int kRebuildWaves = 4;
__global__ __launch_bounds__(kRebuildWaves * kWave) void aug_rebuild_kernel(const int32_t* __restrict__ aug_add,
                                                                            int U, int nb, int nbk,
                                                                            uint8_t* __restrict__ mask,
                                                                            int32_t* __restrict__ row_cnt,
                                                                            int32_t* __restrict__ row_idx,
                                                                            int32_t* __restrict__ head_cnt) {
  __shared__ unsigned bits[kRebuildWaves][32];   // nbk <= 1024
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int u = blockIdx.x * kRebuildWaves + wave;
  if (u >= U) return;
  const int a = aug_add[u];
  if (a <= 0) return;
  const int k = row_cnt[u];
  const int n = k + a;
  unsigned* bw = bits[wave];
  if (lane < 32) bw[lane] = 0u;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  int32_t* ri = row_idx + static_cast<long long>(u) * nbk;
  uint8_t* mr = mask + static_cast<long long>(u) * nbk;
  for (int x = lane; x < n; x += kWave) {
    const int j = min(max(ri[x], 0), nbk - 1);
    atomicOr(&bw[j >> 5], 1u << (j & 31));
    if (x >= k) mr[j] = 1;
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  __builtin_amdgcn_wave_barrier();
  const unsigned word = lane < 32 ? bw[lane] : 0u;
  const int c = __popc(word);
  int incl = c;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  int pos = incl - c;
  unsigned wv = word;
  while (wv) {
    const int b = __ffs(wv) - 1;
    wv &= wv - 1;
    ri[pos++] = lane * 32 + b;
  }
  if (lane == 0) {
    row_cnt[u] = n;
    atomicAdd(head_cnt + u / nb, a);
  }
}

// Row of one member: old entries (selected blocks ascending, then the ranked
// tail) are read into registers first, the item's union is built in LDS,
// then the row is rewritten: union blocks below the row's eligible count in
// ascending order, then the old tail without them (rank order kept).
constexpr int kUnionPerLane = 16;   // nbk <= 1024
__global__ __launch_bounds__(4 * kWave) void aug_union_kernel(uint8_t* __restrict__ mask,
                                                              int32_t* __restrict__ row_cnt,
                                                              int32_t* __restrict__ row_idx,
                                                              int32_t* __restrict__ head_cnt, int nb, int nbk,
                                                              int bq, int bk, int causal, int G, int ng) {
  __shared__ unsigned uni[32];
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int g = blockIdx.x;
  const int bh = g / ng;
  const int i0 = (g - bh * ng) * G;
  const int gsz = min(G, nb - i0);
  const bool active = wave < gsz;
  const int i = i0 + wave;
  const long long u = static_cast<long long>(bh) * nb + i;
  if (threadIdx.x < 32) uni[threadIdx.x] = 0u;
  __syncthreads();
  int k = 0, nv = 0;
  int ent[kUnionPerLane];
  if (active) {
    nv = causal ? min(nbk, ((i + 1) * bq - 1) / bk + 1) : nbk;
    k = min(max(row_cnt[u], 0), nv);
#pragma unroll
    for (int e = 0; e < kUnionPerLane; ++e) {
      const int pos = lane * kUnionPerLane + e;
      ent[e] = pos < nv ? min(max(row_idx[u * nbk + pos], 0), nbk - 1) : 0;
      if (pos < k) atomicOr(&uni[ent[e] >> 5], 1u << (ent[e] & 31));
    }
  }
  __syncthreads();
  if (!active) return;
  // New selection: union blocks j < nv, ascending (lane w < 32 owns word w).
  unsigned word = lane < 32 ? uni[lane] : 0u;
  const int lo = lane * 32;
  if (lo >= nv) word = 0u;
  else if (nv - lo < 32) word &= (1u << (nv - lo)) - 1u;
  const int c = __popc(word);
  int incl = c;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  const int kn = __shfl(incl, kWave - 1, kWave);
  // Old tail entries that stay unselected, counted per lane (blocked layout).
  int keep = 0;
#pragma unroll
  for (int e = 0; e < kUnionPerLane; ++e) {
    const int pos = lane * kUnionPerLane + e;
    const int j = ent[e];
    if (pos >= k && pos < nv && !((uni[j >> 5] >> (j & 31)) & 1u)) ++keep;
  }
  int kincl = keep;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(kincl, o, kWave);
    if (lane >= o) kincl += y;
  }
  int32_t* ri = row_idx + u * nbk;
  uint8_t* mr = mask + u * nbk;
  int pos = incl - c;
  unsigned wv = word;
  while (wv) {
    const int b = __ffs(wv) - 1;
    wv &= wv - 1;
    ri[pos++] = lo + b;
    mr[lo + b] = 1;
  }
  int tp = kn + kincl - keep;
#pragma unroll
  for (int e = 0; e < kUnionPerLane; ++e) {
    const int p2 = lane * kUnionPerLane + e;
    const int j = ent[e];
    if (p2 >= k && p2 < nv && !((uni[j >> 5] >> (j & 31)) & 1u)) ri[tp++] = j;
  }
  if (lane == 0) {
    row_cnt[u] = kn;
    atomicAdd(head_cnt + bh, kn - k);
  }
}

}  // namespace

hipError_t launch_augment_union(const Shape& s, uint8_t* mask, int32_t* row_cnt, int32_t* row_idx,
                                int32_t* head_cnt, hipStream_t stream) {
  const int G = group_size(s);
  const int ng = (s.nb + G - 1) / G;
  const long long items = static_cast<long long>(s.B) * s.H * ng;
  if (G < 1 || G > 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL(aug_union_kernel, dim3(static_cast<unsigned>(items)), dim3(G * kWave), 0, stream, mask,
                     row_cnt, row_idx, head_cnt, s.nb, s.nbk, s.block, s.kb, s.causal ? 1 : 0, G, ng);
  return hipGetLastError();
}

size_t augment_ws_bytes(const Shape& s, int num_workers) {
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  const size_t U = static_cast<size_t>(s.units());
  return kCtrlBytes + up(sizeof(int32_t) * (num_workers + 1)) + up(sizeof(int32_t) * U) * 2 + up(sizeof(AugRow) * U);
}

hipError_t launch_augment(const Shape& s, const double* block_prob, const int32_t* worker_of,
                          const int64_t* worker_load, int num_workers, uint8_t* mask, int32_t* row_cnt,
                          int32_t* row_idx, int32_t* head_cnt, int32_t* added, void* ws, hipStream_t stream) {
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  const int G = group_size(s);
  const int ng = (s.nb + G - 1) / G;
  const int items = s.B * s.H * ng;
  const long long U = s.units();
  unsigned char* p = static_cast<unsigned char*>(ws) + kCtrlBytes;
  auto* off = reinterpret_cast<int32_t*>(p);
  p += up(sizeof(int32_t) * (num_workers + 1));
  auto* rows = reinterpret_cast<int32_t*>(p);
  p += up(sizeof(int32_t) * U);
  auto* aug_add = reinterpret_cast<int32_t*>(p);
  p += up(sizeof(int32_t) * U);
  auto* gstate = reinterpret_cast<AugRow*>(p);
  hipLaunchKernelGGL(aug_csr_kernel, dim3(1), dim3(kCsrThreads), 0, stream, worker_of, items, s.nb, G, ng,
                     num_workers, off, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(aug_merge_kernel, dim3(num_workers), dim3(kWave), 0, stream, block_prob, row_cnt, row_idx,
                     worker_load, num_workers, s.nb, s.nbk, s.block, s.kb, s.causal ? 1 : 0, off, rows, gstate,
                     aug_add, added);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned blocks = static_cast<unsigned>((U + kRebuildWaves - 1) / kRebuildWaves);
  hipLaunchKernelGGL(aug_rebuild_kernel, dim3(blocks), dim3(kRebuildWaves * kWave), 0, stream, aug_add,
                     static_cast<int>(U), s.nb, s.nbk, mask, row_cnt, row_idx, head_cnt);
  return hipGetLastError();
}

}  // namespace tbs
