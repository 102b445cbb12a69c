// Slack-aware sparse augmentation on one GPU (gfx950).
//
// Source: FVAttn review page, section 1 (Key Terms, "Slack-Aware Sparse
// Augmentation (SASA)"): after load balancing, ranks left with slack receive
// additional high-value sparse blocks; section 3 (Method & Key Results): SASA
// spends each rank's idle time after load balancing on extra blocks.
//
// Priced in what the attention kernel runs, in row-tiles (one query row
// block computing one 64-key tile): a work item (G query blocks of one head)
// runs the union of its rows' key blocks as tiles, each tile with a fixed
// part of F row-tiles (staging, the softmax pipeline) plus one row-tile per
// row that selected it, so an item costs F * (union tiles) + (row tiles).
// The ranks are the W workers of a batched longest-first assignment of the
// items in work-list order; worker w has slack s_w = M - L_w (M the largest
// load) and spends it on its last item, where extra cost changes no other
// choice of the assignment.  Its candidates are the (row, block) pairs of
// that item with the block eligible for the row and not selected by it, in
// the order (P desc, row asc, block asc); a pair costs the block's tiles,
// plus F times them when its block is in neither the union nor an earlier
// pair; the worker buys the longest prefix of the order that fits s_w.
//
// Kernels (after item_union_kernel and lpt_batched_kernel of the scheduler):
//   aug_buy_kernel     one workgroup per worker: the candidate pairs of its
//                      last item as 64-bit keys (P's bits + 1) compacted in
//                      LDS, a bitonic sort by (key desc, slot asc), the first
//                      position of every block, the pairs' costs, a prefix
//                      sum, and the pairs within the slack into per-row
//                      bitmaps.
//   aug_rows_kernel    one wave per member row of an item: the row's new
//                      selection from an LDS bitmap -- the item's union
//                      (attn_augment_union) or the row's own blocks plus the
//                      pairs it bought (attn_augment, only the last items
//                      of workers that bought) -- written as an ascending
//                      list followed by the old ranked tail without the new
//                      blocks.
#include <climits>

#include "device_common.h"
#include "launch.h"

namespace tbs {
namespace {

constexpr int kBuyThreads = 1024;
constexpr int kBuyMaxRows = 4;                    // G <= 4
constexpr int kBuyMaxBlocks = 1024;               // nbk <= 1024
constexpr int kBuyMax = kBuyMaxRows * kBuyMaxBlocks;
constexpr int kBuyWords = kBuyMaxBlocks / 32;

// Causal routing: key blocks that start at or before query block i's last
// token; otherwise every key block.
__device__ __forceinline__ int eligible_blocks(int i, int nbk, int bq, int bk, int causal) {
  return causal ? min(nbk, ((i + 1) * bq - 1) / bk + 1) : nbk;
}

// Pair order: larger key first, equal keys by the smaller slot (row, block).
__device__ __forceinline__ bool buy_before(unsigned long long ka, int sa, unsigned long long kb, int sb) {
  return ka > kb || (ka == kb && sa < sb);
}

__global__ __launch_bounds__(kBuyThreads) void aug_buy_kernel(
    const double* __restrict__ block_prob, const int32_t* __restrict__ row_cnt, const int32_t* __restrict__ row_idx,
    const int64_t* __restrict__ worker_load, const int32_t* __restrict__ last_item,
    const int64_t* __restrict__ makespan, const unsigned* __restrict__ ubits, int nb, int nbk, int N, int bq, int bk,
    int causal, int G, int ng, int tile_fixed, int buy, unsigned* __restrict__ addbits, int32_t* __restrict__ paid) {
  __shared__ unsigned long long s_key[kBuyMax];
  __shared__ unsigned short s_slot[kBuyMax];
  __shared__ unsigned s_sel[kBuyMaxRows][kBuyWords];
  __shared__ unsigned s_add[kBuyMaxRows][kBuyWords];
  __shared__ unsigned s_u[kBuyWords];
  __shared__ int s_first[kBuyMaxBlocks];
  __shared__ int s_part[kBuyThreads / kWave];
  __shared__ int s_cnt[kBuyThreads / kWave];
  const int w = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int g = last_item[w];
  const long long slack = g < 0 || !buy ? 0 : makespan[0] - worker_load[w];
  // uniform over the workgroup: no barrier has been passed yet
  if (slack <= 0) {
    if (tid == 0) paid[w] = 0;
    return;
  }
  const int nwords = (nbk + 31) / 32;
  const int bh = g / ng;
  const int i0 = (g - bh * ng) * G;
  const int gsz = min(G, nb - i0);
  for (int x = tid; x < kBuyMaxRows * kBuyWords; x += kBuyThreads) {
    (&s_sel[0][0])[x] = 0u;
    (&s_add[0][0])[x] = 0u;
  }
  for (int x = tid; x < nbk; x += kBuyThreads) s_first[x] = INT_MAX;
  if (tid < kBuyWords) s_u[tid] = tid < nwords ? ubits[static_cast<long long>(g) * nwords + tid] : 0u;
  __syncthreads();
  for (int m = 0; m < gsz; ++m) {
    const long long u = static_cast<long long>(bh) * nb + i0 + m;
    const int cnt = min(max(row_cnt[u], 0), nbk);
    for (int x = tid; x < cnt; x += kBuyThreads) {
      const int j = min(max(row_idx[u * nbk + x], 0), nbk - 1);
      atomicOr(&s_sel[m][j >> 5], 1u << (j & 31));
    }
  }
  __syncthreads();
  // Slot x = m * nbk + j is pair (row m, block j).  Every thread keys a run
  // of consecutive slots; the candidates are compacted to the front, and the
  // sort runs over the next power of two, padded with keys of 0.
  const int n = G * nbk;
  const int run_len = (n + kBuyThreads - 1) / kBuyThreads;   // <= kBuyMax / kBuyThreads
  unsigned long long kk[kBuyMax / kBuyThreads];
  int nmine = 0;
#pragma unroll
  for (int r = 0; r < kBuyMax / kBuyThreads; ++r) {
    const int x = tid * run_len + r;
    const int m = x / nbk;
    const int j = x - m * nbk;
    unsigned long long key = 0;
    if (r < run_len && x < n && m < gsz && j < eligible_blocks(i0 + m, nbk, bq, bk, causal) &&
        !((s_sel[m][j >> 5] >> (j & 31)) & 1u))
      key = static_cast<unsigned long long>(
                __double_as_longlong(block_prob[(static_cast<long long>(bh) * nb + i0 + m) * nbk + j])) + 1ull;
    kk[r] = key;
    nmine += key != 0;
  }
  int cincl = nmine;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(cincl, o, kWave);
    if (lane >= o) cincl += y;
  }
  if (lane == kWave - 1) s_cnt[wv] = cincl;
  __syncthreads();
  int at = cincl - nmine, nc = 0;
  for (int x = 0; x < kBuyThreads / kWave; ++x) {
    if (x < wv) at += s_cnt[x];
    nc += s_cnt[x];
  }
#pragma unroll
  for (int r = 0; r < kBuyMax / kBuyThreads; ++r) {
    if (kk[r] != 0) {
      s_key[at] = kk[r];
      s_slot[at] = static_cast<unsigned short>(tid * run_len + r);
      ++at;
    }
  }
  int S = 64;
  while (S < nc) S <<= 1;
  for (int x = nc + tid; x < S; x += kBuyThreads) {
    s_key[x] = 0;
    s_slot[x] = 0xffff;
  }
  __syncthreads();
  for (int k = 2; k <= S; k <<= 1) {
    for (int h = k >> 1; h > 0; h >>= 1) {
      for (int x = tid; x < S; x += kBuyThreads) {
        const int y = x ^ h;
        if (y > x) {
          const unsigned long long kx = s_key[x], ky = s_key[y];
          const int sx = s_slot[x], sy = s_slot[y];
          const bool xb = buy_before(kx, sx, ky, sy);
          if (((x & k) == 0) != xb) {
            s_key[x] = ky;
            s_key[y] = kx;
            s_slot[x] = static_cast<unsigned short>(sy);
            s_slot[y] = static_cast<unsigned short>(sx);
          }
        }
      }
      __syncthreads();
    }
  }
  // First position of every block in the order.
  for (int e = tid; e < S; e += kBuyThreads)
    if (s_key[e] != 0) atomicMin(&s_first[s_slot[e] % nbk], e);
  __syncthreads();
  // Costs over a run of R consecutive positions per thread, then a prefix sum.
  const int spb = bk / 64;
  const int t_last = (N - (nbk - 1) * bk + 63) / 64;
  const int R = S / kBuyThreads > 0 ? S / kBuyThreads : 1;
  const int e0 = tid * R;
  int cost[kBuyMax / kBuyThreads];
  int run = 0;
#pragma unroll
  for (int r = 0; r < kBuyMax / kBuyThreads; ++r) {
    const int e = e0 + r;
    int c = 0;
    if (r < R && e < S && s_key[e] != 0) {
      const int j = s_slot[e] % nbk;
      const int t = j == nbk - 1 ? t_last : spb;
      const bool opens = !((s_u[j >> 5] >> (j & 31)) & 1u) && s_first[j] == e;
      c = t * (1 + (opens ? tile_fixed : 0));
    }
    cost[r] = c;
    run += c;
  }
  int incl = run;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += y;
  }
  if (lane == kWave - 1) s_part[wv] = incl;
  __syncthreads();
  int before = incl - run;
  for (int x = 0; x < wv; ++x) before += s_part[x];
  int taken = 0;
  int pre = before;
#pragma unroll
  for (int r = 0; r < kBuyMax / kBuyThreads; ++r) {
    const int e = e0 + r;
    pre += cost[r];
    if (r < R && e < S && s_key[e] != 0 && pre <= slack) {
      const int x = s_slot[e];
      const int m = x / nbk;
      const int j = x - m * nbk;
      atomicOr(&s_add[m][j >> 5], 1u << (j & 31));
      ++taken;
    }
  }
  taken = wave_sum_i32(taken);
  if (lane == 0) s_cnt[wv] = taken;
  __syncthreads();
  for (int x = tid; x < kBuyMaxRows * kBuyWords; x += kBuyThreads)
    addbits[static_cast<long long>(w) * kBuyMaxRows * kBuyWords + x] = (&s_add[0][0])[x];
  if (tid == 0) {
    int all = 0;
    for (int x = 0; x < kBuyThreads / kWave; ++x) all += s_cnt[x];
    paid[w] = all;
  }
}

// Row of one member: old entries (selected blocks ascending, then the ranked
// tail) are read into registers first, the row's new selection is built as
// an LDS bitmap, then the row is rewritten: the bitmap's blocks below the
// row's eligible count in ascending order, then the old tail without them
// (rank order kept).  ADD = false: the bitmap is the item's union, one
// workgroup per item.  ADD = true: one workgroup per worker, the item is the
// worker's last one and the bitmap is the row's own blocks plus the pairs it
// bought; workers that bought nothing return at once.
constexpr int kUnionPerLane = 16;   // nbk <= 1024
template <bool ADD>
__global__ __launch_bounds__(4 * kWave) void aug_rows_kernel(uint8_t* __restrict__ mask,
                                                             int32_t* __restrict__ row_cnt,
                                                             int32_t* __restrict__ row_idx,
                                                             int32_t* __restrict__ head_cnt, int nb, int nbk,
                                                             int bq, int bk, int causal, int G, int ng,
                                                             const int32_t* __restrict__ last_item,
                                                             const int32_t* __restrict__ paid,
                                                             const unsigned* __restrict__ addbits) {
  __shared__ unsigned bits[ADD ? kBuyMaxRows : 1][kBuyWords];
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  int g = blockIdx.x;
  if (ADD) {
    g = last_item[blockIdx.x];
    if (g < 0 || paid[blockIdx.x] <= 0) return;   // uniform over the workgroup
  }
  const int bh = g / ng;
  const int i0 = (g - bh * ng) * G;
  const int gsz = min(G, nb - i0);
  const bool active = wave < gsz;
  const int i = i0 + wave;
  const long long u = static_cast<long long>(bh) * nb + i;
  unsigned* mine = bits[ADD ? wave : 0];
  if (ADD) {
    if (lane < kBuyWords)
      mine[lane] = addbits[(static_cast<long long>(blockIdx.x) * kBuyMaxRows + wave) * kBuyWords + lane];
  } else if (threadIdx.x < kBuyWords) {
    bits[0][threadIdx.x] = 0u;
  }
  __syncthreads();
  int k = 0, nv = 0;
  int ent[kUnionPerLane];
  if (active) {
    nv = eligible_blocks(i, nbk, bq, bk, causal);
    k = min(max(row_cnt[u], 0), nv);
#pragma unroll
    for (int e = 0; e < kUnionPerLane; ++e) {
      const int pos = lane * kUnionPerLane + e;
      ent[e] = pos < nv ? min(max(row_idx[u * nbk + pos], 0), nbk - 1) : 0;
      if (pos < k) atomicOr(&mine[ent[e] >> 5], 1u << (ent[e] & 31));
    }
  }
  __syncthreads();
  if (!active) return;
  // New selection: bitmap blocks j < nv, ascending (lane w < 32 owns word w).
  unsigned word = lane < 32 ? mine[lane] : 0u;
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
    if (pos >= k && pos < nv && !((mine[j >> 5] >> (j & 31)) & 1u)) ++keep;
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
    if (p2 >= k && p2 < nv && !((mine[j >> 5] >> (j & 31)) & 1u)) ri[tp++] = j;
  }
  if (lane == 0) {
    row_cnt[u] = kn;
    if (kn != k) atomicAdd(head_cnt + bh, kn - k);
  }
}

}  // namespace

hipError_t launch_augment_union(const Shape& s, uint8_t* mask, int32_t* row_cnt, int32_t* row_idx,
                                int32_t* head_cnt, hipStream_t stream) {
  const int G = group_size(s);
  const int ng = (s.nb + G - 1) / G;
  const long long items = static_cast<long long>(s.B) * s.H * ng;
  if (G < 1 || G > kBuyMaxRows || s.nbk > kBuyMaxBlocks) return hipErrorInvalidValue;
  hipLaunchKernelGGL(aug_rows_kernel<false>, dim3(static_cast<unsigned>(items)), dim3(G * kWave), 0, stream, mask,
                     row_cnt, row_idx, head_cnt, s.nb, s.nbk, s.block, s.kb, s.causal ? 1 : 0, G, ng,
                     static_cast<const int32_t*>(nullptr), static_cast<const int32_t*>(nullptr),
                     static_cast<const unsigned*>(nullptr));
  return hipGetLastError();
}

namespace {
// Workspace of attn_augment after the control block: item bitmaps, item
// tiles and costs, per worker the last item and the bought pairs' bitmaps,
// then the worker of every item, the loads, the pairs bought (used when the
// caller passes no array of its own) and the makespan.
struct AugLayout {
  size_t ubits, tiles, cost, last, addbits, worker_of, load, paid, makespan, total;
};
AugLayout augment_layout(const Shape& s, int num_workers) {
  auto up = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  const int G = group_size(s);
  const size_t items = static_cast<size_t>(s.B) * s.H * ((s.nb + G - 1) / G);
  const size_t nwords = (static_cast<size_t>(s.nbk) + 31) / 32;
  const size_t W = static_cast<size_t>(num_workers);
  AugLayout l;
  l.ubits = kCtrlBytes;
  l.tiles = l.ubits + up(items * nwords * sizeof(unsigned));
  l.cost = l.tiles + up(items * sizeof(int));
  l.last = l.cost + up(items * sizeof(int));
  l.addbits = l.last + up(W * sizeof(int32_t));
  l.worker_of = l.addbits + up(W * kBuyMaxRows * kBuyWords * sizeof(unsigned));
  l.load = l.worker_of + up(items * sizeof(int32_t));
  l.paid = l.load + up(W * sizeof(int64_t));
  l.makespan = l.paid + up(W * sizeof(int32_t));
  l.total = l.makespan + 256;
  return l;
}
}  // namespace

size_t augment_ws_bytes(const Shape& s, int num_workers) { return augment_layout(s, num_workers).total; }

hipError_t launch_augment(const Shape& s, const double* block_prob, const int32_t* work_list, int num_workers,
                          uint8_t* mask, int32_t* row_cnt, int32_t* row_idx, int32_t* head_cnt,
                          int32_t* worker_of, int64_t* worker_load, int32_t* paid, void* ws, hipStream_t stream,
                          int tile_fixed) {
  // A forward that splits its items runs them in equal shares of their
  // tiles, not in the order the assignment models: nothing is bought then.
  const int buy = sparse_split(s, s.causal ? kSparseCausal : kSparse) ? 0 : 1;
  const int G = group_size(s);
  const int ng = (s.nb + G - 1) / G;
  if (G < 1 || G > kBuyMaxRows || s.nbk > kBuyMaxBlocks || num_workers < 1 || num_workers > kMaxLptWorkers ||
      tile_fixed < 0)
    return hipErrorInvalidValue;
  const AugLayout l = augment_layout(s, num_workers);
  auto* base = static_cast<unsigned char*>(ws);
  auto* ubits = reinterpret_cast<unsigned*>(base + l.ubits);
  auto* tiles = reinterpret_cast<int*>(base + l.tiles);
  auto* cost = reinterpret_cast<int*>(base + l.cost);
  auto* last = reinterpret_cast<int32_t*>(base + l.last);
  auto* addbits = reinterpret_cast<unsigned*>(base + l.addbits);
  auto* makespan = reinterpret_cast<int64_t*>(base + l.makespan);
  if (!worker_of) worker_of = reinterpret_cast<int32_t*>(base + l.worker_of);
  if (!worker_load) worker_load = reinterpret_cast<int64_t*>(base + l.load);
  if (!paid) paid = reinterpret_cast<int32_t*>(base + l.paid);
  hipError_t e = launch_item_union(s, row_cnt, row_idx, tiles, ubits, stream, tile_fixed, cost);
  if (e != hipSuccess) return e;
  e = launch_lpt_batched(s, cost, work_list, num_workers, worker_of, worker_load, last, makespan, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(aug_buy_kernel, dim3(num_workers), dim3(kBuyThreads), 0, stream, block_prob, row_cnt, row_idx,
                     worker_load, last, makespan, ubits, s.nb, s.nbk, s.N, s.block, s.kb, s.causal ? 1 : 0, G, ng,
                     tile_fixed, buy, addbits, paid);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(aug_rows_kernel<true>, dim3(num_workers), dim3(G * kWave), 0, stream, mask, row_cnt, row_idx,
                     head_cnt, s.nb, s.nbk, s.block, s.kb, s.causal ? 1 : 0, G, ng, static_cast<const int32_t*>(last),
                     static_cast<const int32_t*>(paid), static_cast<const unsigned*>(addbits));
  return hipGetLastError();
}

}  // namespace tbs
