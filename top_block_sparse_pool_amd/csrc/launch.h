// Internal launchers behind the C ABI.  Host-side declarations only; every
// launcher enqueues on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tbs {

struct Shape {
  int B, H, N, d, block, nb;   // query blocks: size and count
  int kb, nbk;                 // key blocks: size and count
  int dtype;      // 0 bf16, 1 f32
  int causal;
  int flags;
  double scale;   // resolved (never 0)
  long long units() const { return static_cast<long long>(B) * H * nb; }
  // Key blocks eligible for query block i under causal routing: those that
  // start at or before the query block's last token.
  int causal_valid(int i) const {
    const long long e = (static_cast<long long>(i + 1) * block - 1) / kb + 1;
    return e < nbk ? static_cast<int>(e) : nbk;
  }
};

// Forward modes: a per-row block list (sparse), all keys (dense), all keys
// up to the query (causal), or a per-row block list of blocks j <= i with
// keys after the query masked (sparse causal).
enum FwdMode { kSparse = 0, kDense = 1, kCausal = 2, kSparseCausal = 3 };
constexpr bool fwd_listed(int m) { return m == kSparse || m == kSparseCausal; }
constexpr bool fwd_causal(int m) { return m == kCausal || m == kSparseCausal; }

// Problem flag: run every work item whole (no split along the keys).
constexpr int kFlagNoSplit = 2;

// Control block at workspace offset 0 (bytes [0, 256)): queue counters.
constexpr size_t kCtrlBytes = 256;

// Router: block means (Qbar row-major [B,H,nb,d], Kbar transposed [B,H,d,nb]),
// zeroes head_cnt; then scores, softmax, top-p cut and outputs.
hipError_t launch_pool(const Shape& s, const void* q, const void* k, double* qbar, double* kbar_t,
                       int32_t* head_cnt, hipStream_t stream);
// Pooling of bf16 Q and K (head_dim 128) fused with their E4M3 quantisation
// (the same codes and scales as launch_quantize_qk, the same means as
// launch_pool), reading each element once.
hipError_t launch_pool_quant(const Shape& s, const void* q, const void* k, double* qbar, double* kbar_t,
                             int32_t* head_cnt, uint8_t* q8, float* q_scale, uint8_t* k8, float* k_scale,
                             hipStream_t stream);
hipError_t launch_select(const Shape& s, const double* qbar, const double* kbar_t, double top_p,
                         uint8_t* mask, int32_t* row_cnt, int32_t* row_idx, int32_t* head_cnt,
                         double* block_prob, hipStream_t stream);

// Scheduler: longest-first work list; zeroes the control block.
hipError_t launch_schedule(const Shape& s, const int32_t* row_cnt, int head_window, int32_t* work_list,
                           uint32_t* ctrl, hipStream_t stream);
hipError_t launch_lpt(const Shape& s, const int32_t* row_cnt, const int32_t* work_list,
                      int num_workers, int32_t* worker_of, int64_t* worker_load, hipStream_t stream);

// Union of every work item's rows' key blocks: its 64-key tiles (item_tiles,
// [items]) and, when ubits is given, the bitmap ([items, ceil(nbk/32)]
// words); when item_cost is given, the item's cost in row-tiles,
// tile_fixed * (union tiles) + (the tiles of every row's listed blocks).
// nbk <= kItemWords * 32.
constexpr int kItemWords = 64;
hipError_t launch_item_union(const Shape& s, const int32_t* row_cnt, const int32_t* row_idx, int* item_tiles,
                             unsigned* ubits, hipStream_t stream, int tile_fixed = 0, int* item_cost = nullptr);
// Longest-first assignment of the items (cost [items]) in work-list order
// (natural order if work_list is null), W positions per batch, workers
// ranked by (load, id) before each batch.  Writes worker_of [items],
// worker_load [W], last_item [W] (-1: none) and makespan [1].
constexpr int kMaxLptWorkers = 4096;
hipError_t launch_lpt_batched(const Shape& s, const int* cost, const int32_t* work_list, int num_workers,
                              int32_t* worker_of, int64_t* worker_load, int32_t* last_item, int64_t* makespan,
                              hipStream_t stream);

// Slack-aware augmentation priced in row-tiles: item unions and costs, the
// batched assignment, each worker's purchase of (row, block) pairs for its
// last item, then the rows that bought pairs are rewritten.  Workspace bytes
// (control block included) for num_workers workers.
size_t augment_ws_bytes(const Shape& s, int num_workers);
// Work-item slack: every row takes the eligible blocks of its item's union.
hipError_t launch_augment_union(const Shape& s, uint8_t* mask, int32_t* row_cnt, int32_t* row_idx,
                                int32_t* head_cnt, hipStream_t stream);
hipError_t launch_augment(const Shape& s, const double* block_prob, const int32_t* work_list, int num_workers,
                          uint8_t* mask, int32_t* row_cnt, int32_t* row_idx, int32_t* head_cnt,
                          int32_t* worker_of, int64_t* worker_load, int32_t* paid, void* ws, hipStream_t stream,
                          int tile_fixed);

// FP8 (E4M3) quantisation of Q (per token) and K (per 64-token tile) for
// the fp8 attention path; bf16 inputs, head_dim 128.
int quant_tiles(const Shape& s);
hipError_t launch_quantize_qk(const Shape& s, const void* q, const void* k, uint8_t* q8, float* q_scale, uint8_t* k8,
                              float* k_scale, hipStream_t stream);

// Attention forward.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* row_cnt;
  const int32_t* row_idx;
  const int32_t* work_list;
  uint32_t* ctrl;
  uint64_t* prof;
  // fp8 path: q and k hold E4M3 codes ([B,H,N,d] bytes) with per-token Q
  // scales [B,H,N] and per-64-key-tile K scales [B,H,ceil(N/64)].
  bool fp8 = false;
  const float* q_scale = nullptr;
  const float* k_scale = nullptr;
  // Split items (dense causal or sparse): causal_split_bytes(s, mode) bytes
  // of workspace, any contents on entry (per-item part counters, zeroed by
  // the call, the sparse plan, then the parts' partial results).
  void* split_ws = nullptr;
};
// Query blocks per work item (G) and number of work items B*H*ceil(nb/G).
int group_size(const Shape& s);
long long work_items(const Shape& s);
int fwd_workers(const Shape& s, int mode, bool fp8 = false);
// Dense causal work items split along the keys: parts of at most this many
// 64-key tiles (0: no split).  Items are split when the problem holds fewer
// than four per compute unit and its longest item is longer than half the
// mean work per compute unit (at least 16 tiles), which is then the part
// length, so that the items of the last query blocks do not set the makespan.
int causal_split_tiles(const Shape& s, int mode);
// Queue entries of the split problem (parts of every item).
long long causal_split_entries(const Shape& s, int split_tiles);
// Sparse (listed) bf16 problems with fewer than 4 work items per compute
// unit (and at most 1024) run as equal shares of their union tiles: the
// items laid end to end in item order, cut into one chunk per persistent
// workgroup (planned on the device from the routed lists), items crossing a
// cut merged like the dense causal parts.  kFlagNoSplit turns both splits
// off.
bool sparse_split(const Shape& s, int mode);
// Workspace bytes a split needs (0 without a split).
size_t causal_split_bytes(const Shape& s, int mode);
hipError_t launch_fwd(const Shape& s, int mode, const FwdArgs& a, hipStream_t stream);

int device_cu_count();

// Allocation-free sparse attention: the device address of this device's
// file-scope scratch array (looked up once per device), its size, and a fill
// kernel that zeroes it on `stream`.
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void** out);
hipError_t noalloc_clear(void* ptr, size_t bytes, hipStream_t stream);

}  // namespace tbs
