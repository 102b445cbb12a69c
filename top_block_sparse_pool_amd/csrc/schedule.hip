// Longest-first work list for the persistent attention kernel (gfx950).
//
// Source: FVAttn review page, section 1 (Key Terms, "Runtime Load
// Balancing"): once the sparse mask is fixed, the real per-head workload is
// profiled and work is redistributed to shorten the critical path; section 2
// (Motivation): predicted or history-based layouts fail because the load
// changes between steps, so the order is rebuilt on every call.  On one GPU
// the workers are the compute units and the work items are (b, h, query
// block) units costing row_cnt key blocks; a persistent kernel that takes
// units in longest-first order performs greedy list scheduling.
//
// Head windows: the (b, h) pairs are cut into windows of `head_window`
// consecutive heads and the list runs window by window, longest first inside
// each window.  Query blocks running at the same time then share the K/V of a
// few heads, which stay cache-resident, instead of streaming every head's K/V
// from HBM; the dynamic queue still balances the load, because a workgroup
// that finishes early simply takes the next unit, from the next window.
//
// Work items: the persistent kernel processes groups of G consecutive query
// blocks of one head (256 query rows: G = 4 for 64-row blocks, 2 for 128-row
// blocks), so the list orders groups; a group costs the summed
// selected-block counts of its blocks.
//
// schedule_kernel: one workgroup per window, a stable counting sort by cost
//   descending.  Each wave owns a contiguous slice of the window's unit ids
//   and counts costs into its own LDS histogram; a prefix over (cost
//   descending, wave ascending) gives every (wave, cost) pair its first output
//   slot; each wave then walks its slice in order, ranking equal costs inside
//   a 64-unit batch with ballots over the cost bits, so equal costs keep
//   ascending unit ids.
// lpt_kernel: greedy longest-processing-time model of the same order over W
//   workers (the worker of every item and every worker's load), for
//   reporting load balance.
// item_union_kernel: the union of every work item's rows' key blocks (a
//   bitmap per item, optional) and the 64-key tiles it holds -- what the
//   attention kernel runs for the item -- and, optionally, the item's cost
//   in row-tiles: F * (union tiles) + the tiles of every row's blocks.
// lpt_batched_kernel: longest-first assignment of the items in list order,
//   W list positions at a time: before each batch the workers are ranked by
//   (load, id) and take the batch's items in that order, one each, so each
//   batch is one parallel step (used by slack-aware augmentation, with items
//   priced in row-tiles).
#include "device_common.h"
#include "launch.h"

namespace tbs {
namespace {

constexpr int kSchedThreads = 256;
constexpr int kSchedWaves = kSchedThreads / kWave;
constexpr int kMaxCost = 4096;  // a work item holds at most 4 blocks of <= 1024 key blocks
constexpr int kCostBits = 13;   // costs are in [0, 4096]
// LDS histogram: one row of G * nbk + 1 counters per wave.
constexpr size_t sched_lds_bytes(int maxc) { return sizeof(int) * kSchedWaves * (maxc + 1); }

// Cost of work item g: the summed selected-key-block counts of its query
// blocks (nb query blocks and nbk key blocks per head).
__device__ __forceinline__ int item_cost(const int32_t* __restrict__ row_cnt, int g, int nb, int nbk, int G,
                                         int ng) {
  const int bh = g / ng;
  const int i0 = (g - bh * ng) * G;
  const int gsz = min(G, nb - i0);
  int c = 0;
  for (int m = 0; m < gsz; ++m) c += min(max(row_cnt[static_cast<long long>(bh) * nb + i0 + m], 0), nbk);
  return c;
}

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(const int32_t* __restrict__ row_cnt,
                                                                 int items, int nb, int nbk, int G, int ng,
                                                                 int window_items,
                                                                 int32_t* __restrict__ work_list,
                                                                 uint32_t* __restrict__ ctrl) {
  extern __shared__ int sched_hist[];   // [kSchedWaves][ncost]
  __shared__ int ctot[kSchedThreads];
  __shared__ int cexc[kSchedThreads];
  __shared__ int wtot[kSchedWaves];
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid & (kWave - 1);
  const int maxc = G * nbk;
  const int ncost = maxc + 1;   // cost values 0..maxc
  auto cnt = [&](int w, int c) -> int& { return sched_hist[w * ncost + c]; };

  for (int x = tid; x < kSchedWaves * ncost; x += kSchedThreads) sched_hist[x] = 0;
  __syncthreads();

  // This workgroup's window: item ids [w0, w1); output slots start at w0.
  const int w0 = blockIdx.x * window_items;
  const int w1 = min(items, w0 + window_items);
  const int chunk = (w1 - w0 + kSchedWaves - 1) / kSchedWaves;
  const int ubeg = min(w1, w0 + wave * chunk);
  const int uend = min(w1, ubeg + chunk);
  for (int u = ubeg + lane; u < uend; u += kWave) atomicAdd(&cnt(wave, item_cost(row_cnt, u, nb, nbk, G, ng)), 1);
  __syncthreads();

  // Position x = 0..ncost-1 enumerates costs in descending order (c = maxc - x).
  // Each thread owns a contiguous run of positions; exclusive prefix over runs.
  const int per = (ncost + kSchedThreads - 1) / kSchedThreads;
  const int xbeg = tid * per;
  int run = 0;
  for (int e = 0; e < per; ++e) {
    const int x = xbeg + e;
    if (x < ncost) {
      const int c = maxc - x;
      for (int w = 0; w < kSchedWaves; ++w) run += cnt(w, c);
    }
  }
  ctot[tid] = run;
  __syncthreads();
  {
    const int v = ctot[tid];
    int incl = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int y = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += y;
    }
    if (lane == kWave - 1) wtot[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += wtot[w];
    cexc[tid] = w0 + base + incl - v;
  }
  __syncthreads();
  {
    int off = cexc[tid];
    for (int e = 0; e < per; ++e) {
      const int x = xbeg + e;
      if (x < ncost) {
        const int c = maxc - x;
        for (int w = 0; w < kSchedWaves; ++w) {
          const int t = cnt(w, c);
          cnt(w, c) = off;
          off += t;
        }
      }
    }
  }
  __syncthreads();

  // Stable placement: rank among equal costs inside each 64-item batch.
  const uint64_t lt = lanemask_lt();
  for (int base = ubeg; base < uend; base += kWave) {
    const int u = base + lane;
    const bool valid = u < uend;
    const int c = valid ? item_cost(row_cnt, u, nb, nbk, G, ng) : 0;
    uint64_t same = __ballot(valid);
#pragma unroll
    for (int b = 0; b < kCostBits; ++b) {
      const bool bit = (c >> b) & 1;
      const uint64_t ones = __ballot(bit);
      same &= bit ? ones : ~ones;
    }
    int slot = 0;
    if (valid) slot = cnt(wave, c);
    if (valid) work_list[slot + __popcll(same & lt)] = u;
    const bool last_of_group = valid && ((same >> lane) >> 1) == 0;
    if (last_of_group) cnt(wave, c) = slot + __popcll(same);
    __builtin_amdgcn_wave_barrier();
  }
  if (blockIdx.x == 0 && tid < static_cast<int>(kCtrlBytes / sizeof(uint32_t))) ctrl[tid] = 0u;
}

// Minimum of a uniform-free value over the wave, returned in every lane:
// butterflies inside each row of 16 lanes (DPP), then the four row minima.
__device__ __forceinline__ unsigned wave_min_u32(unsigned v) {
  v = min(v, static_cast<unsigned>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), 0xB1, 0xF,
                                                               0xF, false)));   // quad_perm 1,0,3,2
  v = min(v, static_cast<unsigned>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), 0x4E, 0xF,
                                                               0xF, false)));   // quad_perm 2,3,0,1
  v = min(v, static_cast<unsigned>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), 0x141, 0xF,
                                                               0xF, false)));   // row_half_mirror
  v = min(v, static_cast<unsigned>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), 0x140, 0xF,
                                                               0xF, false)));   // row_mirror
  const unsigned r0 = __builtin_amdgcn_readlane(static_cast<int>(v), 0);
  const unsigned r1 = __builtin_amdgcn_readlane(static_cast<int>(v), 16);
  const unsigned r2 = __builtin_amdgcn_readlane(static_cast<int>(v), 32);
  const unsigned r3 = __builtin_amdgcn_readlane(static_cast<int>(v), 48);
  return min(min(r0, r1), min(r2, r3));
}

constexpr int kLptThreads = 1024;
constexpr int kLptChunk = 8192;   // work-list entries staged in LDS per round

// Greedy LPT in list order: every item goes to the worker with the least load
// so far, equal loads to the lowest worker id.  All workgroup threads stage
// the item costs of a chunk of the list in LDS; wave 0 then runs the
// sequential greedy with the loads in registers (worker w = 64 s + lane in
// slot s).  A worker is compared through the key (load - base) << 12 | w,
// where base is the previous minimum: every load is at least base, and loads
// never spread by more than the largest item cost (<= 4096), so the key fits
// 32 bits and its minimum is the least load with the lowest id.
template <int R>
__global__ __launch_bounds__(kLptThreads) void lpt_kernel(const int32_t* __restrict__ row_cnt,
                                                          const int32_t* __restrict__ work_list, int items, int nb,
                                                          int nbk, int G, int ng, int W, int32_t* __restrict__ worker_of,
                                                          int64_t* __restrict__ worker_load) {
  __shared__ unsigned short s_cost[kLptChunk];
  __shared__ int s_id[kLptChunk];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  unsigned key[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int w = kWave * r + lane;
    key[r] = w < W ? static_cast<unsigned>(w) : 0xffffffffu;
  }
  unsigned long long base = 0;
  for (int c0 = 0; c0 < items; c0 += kLptChunk) {
    const int n = min(kLptChunk, items - c0);
    __syncthreads();
    for (int x = tid; x < n; x += kLptThreads) {
      const int u = min(max(work_list[c0 + x], 0), items - 1);
      s_id[x] = u;
      s_cost[x] = static_cast<unsigned short>(item_cost(row_cnt, u, nb, nbk, G, ng));
    }
    __syncthreads();
    if (wave != 0) continue;
    for (int b = 0; b < n; b += kWave) {
      const int m = min(kWave, n - b);
      const int my_cost = lane < m ? s_cost[b + lane] : 0;
      const int my_id = lane < m ? s_id[b + lane] : 0;
      int my_w = 0;
      for (int e = 0; e < m; ++e) {
        const unsigned c = static_cast<unsigned>(__builtin_amdgcn_readlane(my_cost, e));
        unsigned k = key[0];
#pragma unroll
        for (int r = 1; r < R; ++r) k = min(k, key[r]);
        const unsigned kmin = wave_min_u32(k);
        const unsigned wmin = kmin & 0xfffu;
        const unsigned shift = kmin & ~0xfffu;   // the new base, relative to the old one
        base += kmin >> 12;
        const int slot = static_cast<int>(wmin) / kWave;
        const bool mine = lane == static_cast<int>(wmin) % kWave;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          if (key[r] != 0xffffffffu) key[r] -= shift;
          if (r == slot && mine) key[r] += c << 12;
        }
        if (lane == e) my_w = static_cast<int>(wmin);
      }
      if (lane < m && worker_of) worker_of[my_id] = my_w;
    }
  }
  if (wave == 0 && worker_load) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int w = kWave * r + lane;
      if (w < W) worker_load[w] = static_cast<int64_t>(base + (key[r] >> 12));
    }
  }
}

// One workgroup per work item: the rows' lists OR'ed into an LDS bitmap;
// the union's key blocks hold kb/64 tiles each, the last block only the
// tiles its keys reach.  Row tiles: every listed entry holds kb/64 tiles,
// less for the entries naming the last block.
constexpr int kUnionThreads = 256;
constexpr int kTileKeys = 64;   // keys per tile of the attention kernel
__global__ __launch_bounds__(kUnionThreads) void item_union_kernel(const int32_t* __restrict__ row_cnt,
                                                                   const int32_t* __restrict__ row_idx, int nb,
                                                                   int nbk, int kb, int N, int ng, int G,
                                                                   int* __restrict__ item_tiles,
                                                                   unsigned* __restrict__ ubits, int tile_fixed,
                                                                   int* __restrict__ item_cost) {
  __shared__ unsigned bm[kItemWords];
  __shared__ int s_entries, s_last;
  const int g = blockIdx.x;
  const int bh = g / ng;
  const int i0 = (g - bh * ng) * G;
  const int gsz = min(G, nb - i0);
  const int nwords = (nbk + 31) / 32;
  const int tid = threadIdx.x;
  for (int x = tid; x < nwords; x += kUnionThreads) bm[x] = 0u;
  if (tid == 0) {
    s_entries = 0;
    s_last = 0;
  }
  __syncthreads();
  int last_hits = 0;
  for (int m = 0; m < gsz; ++m) {
    const long long u = static_cast<long long>(bh) * nb + i0 + m;
    const int cnt = min(max(row_cnt[u], 0), nbk);
    if (tid == 0) s_entries += cnt;
    const int32_t* lst = row_idx + u * nbk;
    for (int x = tid; x < cnt; x += kUnionThreads) {
      const int j = min(max(lst[x], 0), nbk - 1);
      atomicOr(&bm[j >> 5], 1u << (j & 31));
      last_hits += j == nbk - 1;
    }
  }
  if (item_cost && last_hits) atomicAdd(&s_last, last_hits);
  __syncthreads();
  if (ubits)
    for (int x = tid; x < nwords; x += kUnionThreads) ubits[static_cast<long long>(g) * nwords + x] = bm[x];
  if (tid < kWave) {
    int c = 0;
    for (int x = tid; x < nwords; x += kWave) c += __popc(bm[x]);
    c = wave_sum_i32(c);
    if (tid == 0) {
      const int spb = kb / kTileKeys;
      const int t_last = (N - (nbk - 1) * kb + kTileKeys - 1) / kTileKeys;
      int tiles = c * spb;
      if (c > 0 && ((bm[(nbk - 1) >> 5] >> ((nbk - 1) & 31)) & 1u)) tiles = (c - 1) * spb + t_last;
      item_tiles[g] = tiles;
      if (item_cost) item_cost[g] = tile_fixed * tiles + s_entries * spb - s_last * (spb - t_last);
    }
  }
}

// Batched longest-first assignment (one workgroup, dynamic LDS of
// lpt_batched_lds(W) bytes).  Worker w's key is load << 12 | w (W <= 4096,
// so keys are distinct and equal loads order by id); its rank in a batch is
// the number of smaller keys.  With W <= 1024 the 1024 threads count in
// floor(1024 / W) slices of the other workers and add their counts in LDS;
// with more workers each thread counts for up to four workers.  The worker
// of rank r < m takes the batch's r-th item.  Loads run ahead of use: while a
// batch is counted, the next batch's costs (its items are known) and the
// items of the batch after it are in flight.
constexpr int kLptBThreads = 1024;
constexpr int kLptBPer = kMaxLptWorkers / kLptBThreads;
size_t lpt_batched_lds(int W) { return static_cast<size_t>(W) * (sizeof(unsigned long long) + 3 * sizeof(int)); }

__global__ __launch_bounds__(kLptBThreads) void lpt_batched_kernel(const int* __restrict__ cost,
                                                                   const int32_t* __restrict__ work_list,
                                                                   int items, int W,
                                                                   int32_t* __restrict__ worker_of,
                                                                   int64_t* __restrict__ worker_load,
                                                                   int32_t* __restrict__ last_item,
                                                                   int64_t* __restrict__ makespan) {
  extern __shared__ unsigned long long s_dyn[];
  unsigned long long* s_key = s_dyn;                              // [W], by worker
  int* s_rank = reinterpret_cast<int*>(s_key + W);                // [W], by worker
  int* s_g = s_rank + W;                                          // [W], by batch position
  int* s_c = s_g + W;                                             // [W], by batch position
  __shared__ unsigned long long s_max[kLptBThreads / kWave];
  const int tid = threadIdx.x;
  const int slices = W <= kLptBThreads ? kLptBThreads / W : 1;
  const int mine = W <= kLptBThreads ? (tid < slices * W ? 1 : 0) : kLptBPer;
  const int w0 = W <= kLptBThreads ? tid % W : tid;
  const int slice = W <= kLptBThreads ? tid / W : 0;
  const int v_lo = W <= kLptBThreads ? slice * W / slices : 0;
  const int v_hi = W <= kLptBThreads ? (slice + 1) * W / slices : W;
  const bool owner = W <= kLptBThreads ? tid < W : true;
  unsigned long long load[kLptBPer];
#pragma unroll
  for (int q = 0; q < kLptBPer; ++q) {
    load[q] = 0;
    const int w = tid + q * kLptBThreads;
    if (w < W) {
      s_key[w] = static_cast<unsigned long long>(w);
      last_item[w] = -1;
    }
  }
  // item at list position p (-1 past the end) and its cost
  auto item_at = [&](int p) { return p < items ? (work_list ? min(max(work_list[p], 0), items - 1) : p) : -1; };
  int g_cur[kLptBPer], c_cur[kLptBPer], g_nxt[kLptBPer];
#pragma unroll
  for (int q = 0; q < kLptBPer; ++q) {
    const int r = tid + q * kLptBThreads;
    g_cur[q] = r < W ? item_at(r) : -1;
    g_nxt[q] = r < W ? item_at(W + r) : -1;
    c_cur[q] = g_cur[q] >= 0 ? cost[g_cur[q]] : 0;
  }
  for (int b = 0; b < items; b += W) {
    const int m = min(W, items - b);
    int c_nxt[kLptBPer], g_aft[kLptBPer];
#pragma unroll
    for (int q = 0; q < kLptBPer; ++q) {
      const int r = tid + q * kLptBThreads;
      if (r < W) {
        s_g[r] = g_cur[q];
        s_c[r] = c_cur[q];
        s_rank[r] = 0;
      }
      c_nxt[q] = g_nxt[q] >= 0 ? cost[g_nxt[q]] : 0;
      g_aft[q] = r < W ? item_at(b + 2 * W + r) : -1;
    }
    __syncthreads();
    // ranks: smaller keys among the workers of this thread's slice
    for (int q = 0; q < mine; ++q) {
      const int w = w0 + q * kLptBThreads;
      if (w >= W) break;
      const unsigned long long kw = s_key[w];
      int c = 0;
      int v = v_lo;
      // eight independent LDS reads in flight per step
      for (; v + 8 <= v_hi; v += 8) {
        unsigned long long kv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) kv[e] = s_key[v + e];
#pragma unroll
        for (int e = 0; e < 8; ++e) c += kv[e] < kw;
      }
      for (; v < v_hi; ++v) c += s_key[v] < kw;
      if (c) atomicAdd(&s_rank[w], c);
    }
    __syncthreads();
    if (owner) {
#pragma unroll
      for (int q = 0; q < kLptBPer; ++q) {
        const int w = tid + q * kLptBThreads;
        if (w < W) {
          const int rank = s_rank[w];
          if (rank < m) {
            const int g = s_g[rank];
            load[q] += static_cast<unsigned long long>(s_c[rank]);
            s_key[w] = (load[q] << 12) | static_cast<unsigned>(w);
            worker_of[g] = w;
            last_item[w] = g;
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kLptBPer; ++q) {
      g_cur[q] = g_nxt[q];
      c_cur[q] = c_nxt[q];
      g_nxt[q] = g_aft[q];
    }
    __syncthreads();
  }
  unsigned long long mx = 0;
#pragma unroll
  for (int q = 0; q < kLptBPer; ++q) {
    const int w = tid + q * kLptBThreads;
    if (owner && w < W) {
      worker_load[w] = static_cast<int64_t>(load[q]);
      mx = max(mx, load[q]);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = max(mx, static_cast<unsigned long long>(__shfl_xor(mx, o, kWave)));
  if ((tid & (kWave - 1)) == 0) s_max[tid / kWave] = mx;
  __syncthreads();
  if (tid == 0) {
    unsigned long long all = 0;
    for (int x = 0; x < kLptBThreads / kWave; ++x) all = max(all, s_max[x]);
    makespan[0] = static_cast<int64_t>(all);
  }
}

}  // namespace

hipError_t launch_item_union(const Shape& s, const int32_t* row_cnt, const int32_t* row_idx, int* item_tiles,
                             unsigned* ubits, hipStream_t stream, int tile_fixed, int* item_cost) {
  const int G = group_size(s);
  const int ng = (s.nb + G - 1) / G;
  const long long items = static_cast<long long>(s.B) * s.H * ng;
  if (s.nbk > kItemWords * 32 || items < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(item_union_kernel, dim3(static_cast<unsigned>(items)), dim3(kUnionThreads), 0, stream, row_cnt,
                     row_idx, s.nb, s.nbk, s.kb, s.N, ng, G, item_tiles, ubits, tile_fixed, item_cost);
  return hipGetLastError();
}

hipError_t launch_lpt_batched(const Shape& s, const int* cost, const int32_t* work_list, int num_workers,
                              int32_t* worker_of, int64_t* worker_load, int32_t* last_item, int64_t* makespan,
                              hipStream_t stream) {
  const int G = group_size(s);
  const int ng = (s.nb + G - 1) / G;
  const long long items = static_cast<long long>(s.B) * s.H * ng;
  if (num_workers < 1 || num_workers > kMaxLptWorkers) return hipErrorInvalidValue;
  const size_t lds = lpt_batched_lds(num_workers);
  const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(lpt_batched_kernel),
                                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(lpt_batched_kernel, dim3(1), dim3(kLptBThreads), lds, stream, cost, work_list,
                     static_cast<int>(items), num_workers, worker_of, worker_load, last_item, makespan);
  return hipGetLastError();
}

hipError_t launch_schedule(const Shape& s, const int32_t* row_cnt, int head_window, int32_t* work_list,
                           uint32_t* ctrl, hipStream_t stream) {
  const int G = group_size(s);
  const int ng = (s.nb + G - 1) / G;
  const int BH = s.B * s.H;
  const int items = BH * ng;
  const int hw = (head_window <= 0 || head_window > BH) ? BH : head_window;
  const int windows = (BH + hw - 1) / hw;
  const int maxc = G * s.nbk;
  if (maxc > kMaxCost) return hipErrorInvalidValue;
  const size_t lds = sched_lds_bytes(maxc);
  const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(schedule_kernel),
                                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL(schedule_kernel, dim3(windows), dim3(kSchedThreads), lds, stream, row_cnt, items, s.nb, s.nbk,
                     G, ng,
                     hw * ng, work_list, ctrl);
  return hipGetLastError();
}

hipError_t launch_lpt(const Shape& s, const int32_t* row_cnt, const int32_t* work_list, int num_workers,
                      int32_t* worker_of, int64_t* worker_load, hipStream_t stream) {
  const int G = group_size(s);
  const int ng = (s.nb + G - 1) / G;
  const int items = s.B * s.H * ng;
  auto kern = num_workers <= 64 ? lpt_kernel<1>
             : num_workers <= 256 ? lpt_kernel<4>
             : num_workers <= 1024 ? lpt_kernel<16> : lpt_kernel<64>;
  hipLaunchKernelGGL(kern, dim3(1), dim3(kLptThreads), 0, stream, row_cnt, work_list, items, s.nb, s.nbk, G, ng,
                     num_workers, worker_of, worker_load);
  return hipGetLastError();
}

}  // namespace tbs
