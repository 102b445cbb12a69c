// C ABI of the top-p block-sparse attention library: argument validation,
// workspace layout and dispatch to the HIP launchers.  Every argument is
// checked before the first HIP call; failures return a status code and set
// a per-thread message.  No exception crosses the interface.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/attn_tbs.h"
#include "launch.h"

#define TBS_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

int32_t fail(int32_t code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int32_t fail(int32_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int32_t ok() {
  g_last_error.clear();
  return ATTN_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

constexpr size_t kProfileBytes = 16 * 4096;   // per-worker stamps, at most 4096 workers
constexpr int kMaxRouteBlocks = 1024;
constexpr int kMaxSparseBlocks = 2048;
constexpr int kMaxWorkers = 4096;

// Validates the problem descriptor and resolves it into a Shape.
int32_t check_problem(const attn_problem* pr, tbs::Shape* s) {
  if (!pr) return fail(ATTN_E_INVALID, "problem is NULL");
  if (pr->batch < 1 || pr->heads < 1 || pr->seq_len < 1)
    return fail(ATTN_E_INVALID, "batch, heads and seq_len must be >= 1 (got %d, %d, %d)", pr->batch,
                pr->heads, pr->seq_len);
  if (pr->head_dim < 1 || pr->block < 1)
    return fail(ATTN_E_INVALID, "head_dim and block must be >= 1 (got %d, %d)", pr->head_dim, pr->block);
  if (pr->dtype != ATTN_DTYPE_BF16 && pr->dtype != ATTN_DTYPE_F32)
    return fail(ATTN_E_INVALID, "dtype must be ATTN_DTYPE_BF16 or ATTN_DTYPE_F32 (got %d)", pr->dtype);
  if (pr->causal != 0 && pr->causal != 1) return fail(ATTN_E_INVALID, "causal must be 0 or 1");
  if (pr->flags & ~(ATTN_FLAG_PROFILE_WORKERS | ATTN_FLAG_NO_SPLIT))
    return fail(ATTN_E_INVALID, "unknown flag bits 0x%x", pr->flags);
  if (!(pr->scale >= 0.0) || !std::isfinite(pr->scale))
    return fail(ATTN_E_INVALID, "scale must be finite and >= 0 (0 selects 1/sqrt(head_dim))");
  if (pr->head_dim != 64 && pr->head_dim != 128)
    return fail(ATTN_E_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", pr->head_dim);
  if (pr->block != 64 && pr->block != 128)
    return fail(ATTN_E_UNSUPPORTED, "block %d unsupported (64 or 128)", pr->block);
  if (pr->key_block < 0 || pr->reserved != 0)
    return fail(ATTN_E_INVALID, "key_block must be >= 0 and reserved 0 (got %d, %d)", pr->key_block, pr->reserved);
  const int kb = pr->key_block ? pr->key_block : pr->block;
  if (kb != 64 && kb != 128) return fail(ATTN_E_UNSUPPORTED, "key_block %d unsupported (64 or 128)", kb);
  const long long nb = (static_cast<long long>(pr->seq_len) + pr->block - 1) / pr->block;
  const long long units = static_cast<long long>(pr->batch) * pr->heads * nb;
  if (units > 0x3fffffffLL) return fail(ATTN_E_UNSUPPORTED, "batch*heads*blocks = %lld too large", units);
  const long long elems = static_cast<long long>(pr->batch) * pr->heads * pr->seq_len * pr->head_dim;
  if (elems > (1LL << 40)) return fail(ATTN_E_UNSUPPORTED, "tensor of %lld elements too large", elems);
  s->B = pr->batch;
  s->H = pr->heads;
  s->N = pr->seq_len;
  s->d = pr->head_dim;
  s->block = pr->block;
  s->nb = static_cast<int>(nb);
  s->kb = kb;
  s->nbk = (pr->seq_len + kb - 1) / kb;
  s->dtype = pr->dtype;
  s->causal = pr->causal;
  s->flags = pr->flags;
  s->scale = pr->scale > 0.0 ? pr->scale : 1.0 / std::sqrt(static_cast<double>(pr->head_dim));
  return ATTN_OK;
}

size_t route_bytes(const tbs::Shape& s) {
  return tbs::kCtrlBytes + sizeof(double) * static_cast<size_t>(s.B) * s.H * (s.nb + s.nbk) * s.d;
}

// Control block, optional worker stamps, then (dense causal with split
// items) the part counters and partial results, 256-byte aligned.
size_t fwd_split_offset(const tbs::Shape& s) {
  return tbs::kCtrlBytes + ((s.flags & ATTN_FLAG_PROFILE_WORKERS) ? kProfileBytes : 0);
}

size_t fwd_bytes(const tbs::Shape& s, int mode) { return fwd_split_offset(s) + tbs::causal_split_bytes(s, mode); }

int32_t check_tensor(const void* p, const char* name) {
  if (!p) return fail(ATTN_E_INVALID, "%s is NULL", name);
  if (!aligned(p, 16)) return fail(ATTN_E_INVALID, "%s is not 16-byte aligned", name);
  return ATTN_OK;
}

int32_t check_i32(const void* p, const char* name, bool nullable) {
  if (!p) return nullable ? ATTN_OK : fail(ATTN_E_INVALID, "%s is NULL", name);
  if (!aligned(p, 4)) return fail(ATTN_E_INVALID, "%s is not 4-byte aligned", name);
  return ATTN_OK;
}

int32_t check_ws(const void* ws, size_t have, size_t need) {
  if (need == 0) return ATTN_OK;
  if (!ws) return fail(ATTN_E_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (!aligned(ws, 16)) return fail(ATTN_E_WORKSPACE, "workspace is not 16-byte aligned");
  if (have < need) return fail(ATTN_E_WORKSPACE, "workspace holds %zu bytes, %zu needed", have, need);
  return ATTN_OK;
}

int32_t device_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(ATTN_E_DEVICE, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

std::mutex g_cu_mutex;
int g_cu_count[64] = {0};

}  // namespace

namespace tbs {
int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
  std::lock_guard<std::mutex> lock(g_cu_mutex);
  if (g_cu_count[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 1;
    g_cu_count[dev] = n;
  }
  return g_cu_count[dev];
}
}  // namespace tbs

TBS_EXPORT int32_t attn_abi_version(void) { return ATTN_TBS_ABI_VERSION; }

TBS_EXPORT const char* attn_last_error(void) { return g_last_error.c_str(); }

TBS_EXPORT size_t attn_workspace_bytes(const attn_problem* problem, int32_t op) {
  tbs::Shape s;
  if (check_problem(problem, &s) != ATTN_OK) return 0;
  switch (op) {
    case ATTN_OP_ROUTE: return route_bytes(s);
    case ATTN_OP_SCHEDULE: return tbs::kCtrlBytes;
    case ATTN_OP_SPARSE_FWD: return fwd_bytes(s, s.causal ? tbs::kSparseCausal : tbs::kSparse);
    case ATTN_OP_DENSE_FWD: return fwd_bytes(s, s.causal ? tbs::kCausal : tbs::kDense);
    case ATTN_OP_AUGMENT: return tbs::augment_ws_bytes(s, kMaxWorkers);
    default: fail(ATTN_E_INVALID, "unknown op %d", op); return 0;
  }
}

TBS_EXPORT int32_t attn_group_size(const attn_problem* problem) {
  tbs::Shape s;
  if (check_problem(problem, &s) != ATTN_OK) return 0;
  return tbs::group_size(s);
}

TBS_EXPORT int32_t attn_num_workers(const attn_problem* problem, int32_t op) {
  tbs::Shape s;
  if (check_problem(problem, &s) != ATTN_OK) return 0;
  if (op != ATTN_OP_SPARSE_FWD && op != ATTN_OP_DENSE_FWD) {
    fail(ATTN_E_INVALID, "attn_num_workers: op must be a fwd op");
    return 0;
  }
  const int mode = op == ATTN_OP_SPARSE_FWD ? (s.causal ? tbs::kSparseCausal : tbs::kSparse)
                                            : (s.causal ? tbs::kCausal : tbs::kDense);
  return tbs::fwd_workers(s, mode);
}

TBS_EXPORT int32_t attn_route(const attn_problem* problem, const void* q, const void* k, double top_p,
                              uint8_t* mask, int32_t* row_cnt, int32_t* row_idx, int32_t* head_cnt,
                              double* block_prob, void* ws, size_t ws_bytes, void* stream) {
  tbs::Shape s;
  int32_t st = check_problem(problem, &s);
  if (st != ATTN_OK) return st;
  if (s.nbk > kMaxRouteBlocks)
    return fail(ATTN_E_UNSUPPORTED, "attn_route: %d key blocks per sequence exceed %d", s.nbk, kMaxRouteBlocks);
  if (!(top_p > 0.0 && top_p <= 1.0)) return fail(ATTN_E_INVALID, "top_p must be in (0, 1] (got %g)", top_p);
  if ((st = check_tensor(q, "q")) || (st = check_tensor(k, "k"))) return st;
  if (!mask) return fail(ATTN_E_INVALID, "mask is NULL");
  if ((st = check_i32(row_cnt, "row_cnt", false)) || (st = check_i32(row_idx, "row_idx", false)) ||
      (st = check_i32(head_cnt, "head_cnt", false)))
    return st;
  if (block_prob && !aligned(block_prob, 8)) return fail(ATTN_E_INVALID, "block_prob is not 8-byte aligned");
  if ((st = check_ws(ws, ws_bytes, route_bytes(s)))) return st;

  auto* base = static_cast<unsigned char*>(ws) + tbs::kCtrlBytes;
  auto* qbar = reinterpret_cast<double*>(base);
  auto* kbar_t = qbar + static_cast<size_t>(s.B) * s.H * s.nb * s.d;   // [B,H,d,nbk]
  auto strm = static_cast<hipStream_t>(stream);
  hipError_t e = tbs::launch_pool(s, q, k, qbar, kbar_t, head_cnt, strm);
  if (e != hipSuccess) return device_status(e, "attn_route pool launch");
  e = tbs::launch_select(s, qbar, kbar_t, top_p, mask, row_cnt, row_idx, head_cnt, block_prob, strm);
  return device_status(e, "attn_route select launch");
}

TBS_EXPORT int32_t attn_schedule(const attn_problem* problem, const int32_t* row_cnt, int32_t head_window,
                                 int32_t num_workers, int32_t* work_list, int32_t* worker_of,
                                 int64_t* worker_load, void* ws, size_t ws_bytes, void* stream) {
  tbs::Shape s;
  int32_t st = check_problem(problem, &s);
  if (st != ATTN_OK) return st;
  if (s.nbk > kMaxRouteBlocks)
    return fail(ATTN_E_UNSUPPORTED, "attn_schedule: %d key blocks per sequence exceed %d", s.nbk, kMaxRouteBlocks);
  if (head_window < 0) return fail(ATTN_E_INVALID, "head_window must be >= 0 (got %d)", head_window);
  if (num_workers < 0 || num_workers > kMaxWorkers)
    return fail(ATTN_E_INVALID, "num_workers must be in [0, %d] (got %d)", kMaxWorkers, num_workers);
  if ((st = check_i32(row_cnt, "row_cnt", false)) || (st = check_i32(work_list, "work_list", false)) ||
      (st = check_i32(worker_of, "worker_of", true)))
    return st;
  if (worker_load && !aligned(worker_load, 8)) return fail(ATTN_E_INVALID, "worker_load is not 8-byte aligned");
  if ((st = check_ws(ws, ws_bytes, tbs::kCtrlBytes))) return st;
  auto strm = static_cast<hipStream_t>(stream);
  hipError_t e = tbs::launch_schedule(s, row_cnt, head_window, work_list, static_cast<uint32_t*>(ws), strm);
  if (e != hipSuccess) return device_status(e, "attn_schedule launch");
  if (worker_of || worker_load) {
    const int W = num_workers > 0 ? num_workers : tbs::device_cu_count();
    if (W > 4096) return fail(ATTN_E_UNSUPPORTED, "attn_schedule: %d workers exceed 4096", W);
    e = tbs::launch_lpt(s, row_cnt, work_list, W, worker_of, worker_load, strm);
    if (e != hipSuccess) return device_status(e, "attn_schedule lpt launch");
  }
  return ok();
}

TBS_EXPORT int32_t attn_augment(const attn_problem* problem, const double* block_prob, const int32_t* work_list,
                                int32_t num_workers, uint8_t* mask, int32_t* row_cnt, int32_t* row_idx,
                                int32_t* head_cnt, int32_t* worker_of, int64_t* worker_load, int32_t* paid, void* ws,
                                size_t ws_bytes, void* stream) {
  tbs::Shape s;
  int32_t st = check_problem(problem, &s);
  if (st != ATTN_OK) return st;
  if (s.nbk > kMaxRouteBlocks)
    return fail(ATTN_E_UNSUPPORTED, "attn_augment: %d key blocks per sequence exceed %d", s.nbk, kMaxRouteBlocks);
  if (num_workers < 1 || num_workers > kMaxWorkers)
    return fail(ATTN_E_INVALID, "num_workers must be in [1, %d] (got %d)", kMaxWorkers, num_workers);
  if (!block_prob || !aligned(block_prob, 8)) return fail(ATTN_E_INVALID, "block_prob is NULL or not 8-byte aligned");
  if (worker_load && !aligned(worker_load, 8)) return fail(ATTN_E_INVALID, "worker_load is not 8-byte aligned");
  if (!mask) return fail(ATTN_E_INVALID, "mask is NULL");
  if ((st = check_i32(work_list, "work_list", true)) || (st = check_i32(row_cnt, "row_cnt", false)) ||
      (st = check_i32(row_idx, "row_idx", false)) || (st = check_i32(head_cnt, "head_cnt", false)) ||
      (st = check_i32(worker_of, "worker_of", true)) || (st = check_i32(paid, "paid", true)))
    return st;
  if ((st = check_ws(ws, ws_bytes, tbs::augment_ws_bytes(s, num_workers)))) return st;
  hipError_t e = tbs::launch_augment(s, block_prob, work_list, num_workers, mask, row_cnt, row_idx, head_cnt,
                                     worker_of, worker_load, paid, ws, static_cast<hipStream_t>(stream),
                                     ATTN_SASA_TILE_FIXED);
  return device_status(e, "attn_augment launch");
}

TBS_EXPORT int32_t attn_augment_union(const attn_problem* problem, uint8_t* mask, int32_t* row_cnt,
                                      int32_t* row_idx, int32_t* head_cnt, void* stream) {
  tbs::Shape s;
  int32_t st = check_problem(problem, &s);
  if (st != ATTN_OK) return st;
  if (s.nbk > kMaxRouteBlocks)
    return fail(ATTN_E_UNSUPPORTED, "attn_augment_union: %d key blocks per sequence exceed %d", s.nbk,
                kMaxRouteBlocks);
  if (!mask) return fail(ATTN_E_INVALID, "mask is NULL");
  if ((st = check_i32(row_cnt, "row_cnt", false)) || (st = check_i32(row_idx, "row_idx", false)) ||
      (st = check_i32(head_cnt, "head_cnt", false)))
    return st;
  hipError_t e = tbs::launch_augment_union(s, mask, row_cnt, row_idx, head_cnt, static_cast<hipStream_t>(stream));
  return device_status(e, "attn_augment_union launch");
}

namespace {
int32_t run_fwd(const tbs::Shape& s, int mode, const void* q, const void* k, const void* v,
                const int32_t* row_cnt, const int32_t* row_idx, const int32_t* work_list, void* o, float* lse,
                void* ws, size_t ws_bytes, void* stream, const float* q_scale = nullptr,
                const float* k_scale = nullptr) {
  int32_t st;
  const bool fp8 = q_scale != nullptr;
  if ((st = check_tensor(q, fp8 ? "q8" : "q")) || (st = check_tensor(k, fp8 ? "k8" : "k")) ||
      (st = check_tensor(v, "v")) || (st = check_tensor(o, "o")))
    return st;
  if (lse && !aligned(lse, 4)) return fail(ATTN_E_INVALID, "lse is not 4-byte aligned");
  if ((st = check_ws(ws, ws_bytes, fwd_bytes(s, mode)))) return st;
  tbs::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.row_cnt = row_cnt;
  a.row_idx = row_idx;
  a.work_list = work_list;
  a.ctrl = static_cast<uint32_t*>(ws);
  a.prof = (s.flags & ATTN_FLAG_PROFILE_WORKERS)
               ? reinterpret_cast<uint64_t*>(static_cast<unsigned char*>(ws) + tbs::kCtrlBytes)
               : nullptr;
  a.fp8 = fp8;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.split_ws = static_cast<unsigned char*>(ws) + fwd_split_offset(s);
  if (a.prof && tbs::fwd_workers(s, mode, fp8) > 4096)
    return fail(ATTN_E_UNSUPPORTED, "worker profiling supports at most 4096 workers");
  hipError_t e = tbs::launch_fwd(s, mode, a, static_cast<hipStream_t>(stream));
  return device_status(e, "attention kernel launch");
}
}  // namespace

TBS_EXPORT int32_t attn_sparse_fwd(const attn_problem* problem, const void* q, const void* k, const void* v,
                                   const int32_t* row_cnt, const int32_t* row_idx, const int32_t* work_list,
                                   void* o, float* lse, void* ws, size_t ws_bytes, void* stream) {
  tbs::Shape s;
  int32_t st = check_problem(problem, &s);
  if (st != ATTN_OK) return st;
  if (s.nbk > kMaxSparseBlocks)
    return fail(ATTN_E_UNSUPPORTED, "attn_sparse_fwd: %d key blocks per sequence exceed %d", s.nbk, kMaxSparseBlocks);
  if ((st = check_i32(row_cnt, "row_cnt", false)) || (st = check_i32(row_idx, "row_idx", false)) ||
      (st = check_i32(work_list, "work_list", true)))
    return st;
  return run_fwd(s, s.causal ? tbs::kSparseCausal : tbs::kSparse, q, k, v, row_cnt, row_idx, work_list, o, lse,
                 ws, ws_bytes, stream);
}

TBS_EXPORT int32_t attn_sparse_fwd_noalloc(const attn_problem* problem, const void* q, const void* k, const void* v,
                                           const int32_t* row_cnt, const int32_t* row_idx, const int32_t* work_list,
                                           void* o, float* lse, void* stream) {
  tbs::Shape s;
  int32_t st = check_problem(problem, &s);
  if (st != ATTN_OK) return st;
  s.flags |= ATTN_FLAG_NO_SPLIT;   // every work item runs whole: no parts to keep
  if (s.nbk > kMaxSparseBlocks)
    return fail(ATTN_E_UNSUPPORTED, "attn_sparse_fwd_noalloc: %d key blocks per sequence exceed %d", s.nbk,
                kMaxSparseBlocks);
  if ((st = check_i32(row_cnt, "row_cnt", false)) || (st = check_i32(row_idx, "row_idx", false)) ||
      (st = check_i32(work_list, "work_list", true)))
    return st;
  const int mode = s.causal ? tbs::kSparseCausal : tbs::kSparse;
  const size_t need = fwd_bytes(s, mode);
  if (need > tbs::noalloc_scratch_bytes())
    return fail(ATTN_E_WORKSPACE,
                "attn_sparse_fwd_noalloc: the call needs %zu bytes of scratch, the static array holds %zu "
                "(ATTN_FLAG_PROFILE_WORKERS needs a workspace: use attn_sparse_fwd)",
                need, tbs::noalloc_scratch_bytes());
  if ((st = check_tensor(q, "q")) || (st = check_tensor(k, "k")) || (st = check_tensor(v, "v")) ||
      (st = check_tensor(o, "o")))
    return st;
  if (lse && !aligned(lse, 4)) return fail(ATTN_E_INVALID, "lse is not 4-byte aligned");
  void* scratch = nullptr;
  hipError_t e = tbs::noalloc_scratch(&scratch);
  if (e != hipSuccess) return device_status(e, "attn_sparse_fwd_noalloc scratch lookup");
  auto strm = static_cast<hipStream_t>(stream);
  // The queue counters must be zero when the attention kernel starts.
  e = tbs::noalloc_clear(scratch, tbs::noalloc_scratch_bytes(), strm);
  if (e != hipSuccess) return device_status(e, "attn_sparse_fwd_noalloc scratch clear");
  return run_fwd(s, mode, q, k, v, row_cnt, row_idx, work_list, o, lse, scratch, tbs::noalloc_scratch_bytes(),
                 stream);
}

TBS_EXPORT int32_t attn_dense_fwd(const attn_problem* problem, const void* q, const void* k, const void* v,
                                  void* o, float* lse, void* ws, size_t ws_bytes, void* stream) {
  tbs::Shape s;
  int32_t st = check_problem(problem, &s);
  if (st != ATTN_OK) return st;
  return run_fwd(s, s.causal ? tbs::kCausal : tbs::kDense, q, k, v, nullptr, nullptr, nullptr, o, lse, ws,
                 ws_bytes, stream);
}

namespace {
// The fp8 calls take bf16 problems with head_dim 128.
int32_t check_fp8_problem(const tbs::Shape& s, const char* who) {
  if (s.dtype != ATTN_DTYPE_BF16) return fail(ATTN_E_UNSUPPORTED, "%s: dtype must be ATTN_DTYPE_BF16", who);
  if (s.d != 128) return fail(ATTN_E_UNSUPPORTED, "%s: head_dim %d unsupported (128)", who, s.d);
  return ATTN_OK;
}

int32_t check_scales(const float* q_scale, const float* k_scale) {
  if (!q_scale || !aligned(q_scale, 4)) return fail(ATTN_E_INVALID, "q_scale is NULL or not 4-byte aligned");
  if (!k_scale || !aligned(k_scale, 4)) return fail(ATTN_E_INVALID, "k_scale is NULL or not 4-byte aligned");
  return ATTN_OK;
}
}  // namespace

TBS_EXPORT int32_t attn_quantize_qk_fp8(const attn_problem* problem, const void* q, const void* k, uint8_t* q8,
                                        float* q_scale, uint8_t* k8, float* k_scale, void* stream) {
  tbs::Shape s;
  int32_t st = check_problem(problem, &s);
  if (st != ATTN_OK) return st;
  if ((st = check_fp8_problem(s, "attn_quantize_qk_fp8"))) return st;
  if ((st = check_tensor(q, "q")) || (st = check_tensor(k, "k")) || (st = check_tensor(q8, "q8")) ||
      (st = check_tensor(k8, "k8")) || (st = check_scales(q_scale, k_scale)))
    return st;
  hipError_t e = tbs::launch_quantize_qk(s, q, k, q8, q_scale, k8, k_scale, static_cast<hipStream_t>(stream));
  return device_status(e, "attn_quantize_qk_fp8 launch");
}

TBS_EXPORT int32_t attn_route_fp8(const attn_problem* problem, const void* q, const void* k, double top_p,
                                  uint8_t* mask, int32_t* row_cnt, int32_t* row_idx, int32_t* head_cnt,
                                  double* block_prob, uint8_t* q8, float* q_scale, uint8_t* k8, float* k_scale,
                                  void* ws, size_t ws_bytes, void* stream) {
  tbs::Shape s;
  int32_t st = check_problem(problem, &s);
  if (st != ATTN_OK) return st;
  if ((st = check_fp8_problem(s, "attn_route_fp8"))) return st;
  if (s.nbk > kMaxRouteBlocks)
    return fail(ATTN_E_UNSUPPORTED, "attn_route_fp8: %d key blocks per sequence exceed %d", s.nbk, kMaxRouteBlocks);
  if (!(top_p > 0.0 && top_p <= 1.0)) return fail(ATTN_E_INVALID, "top_p must be in (0, 1] (got %g)", top_p);
  if ((st = check_tensor(q, "q")) || (st = check_tensor(k, "k")) || (st = check_tensor(q8, "q8")) ||
      (st = check_tensor(k8, "k8")) || (st = check_scales(q_scale, k_scale)))
    return st;
  if (!mask) return fail(ATTN_E_INVALID, "mask is NULL");
  if ((st = check_i32(row_cnt, "row_cnt", false)) || (st = check_i32(row_idx, "row_idx", false)) ||
      (st = check_i32(head_cnt, "head_cnt", false)))
    return st;
  if (block_prob && !aligned(block_prob, 8)) return fail(ATTN_E_INVALID, "block_prob is not 8-byte aligned");
  if ((st = check_ws(ws, ws_bytes, route_bytes(s)))) return st;
  auto* base = static_cast<unsigned char*>(ws) + tbs::kCtrlBytes;
  auto* qbar = reinterpret_cast<double*>(base);
  auto* kbar_t = qbar + static_cast<size_t>(s.B) * s.H * s.nb * s.d;
  auto strm = static_cast<hipStream_t>(stream);
  hipError_t e = tbs::launch_pool_quant(s, q, k, qbar, kbar_t, head_cnt, q8, q_scale, k8, k_scale, strm);
  if (e != hipSuccess) return device_status(e, "attn_route_fp8 pool launch");
  e = tbs::launch_select(s, qbar, kbar_t, top_p, mask, row_cnt, row_idx, head_cnt, block_prob, strm);
  return device_status(e, "attn_route_fp8 select launch");
}

TBS_EXPORT int32_t attn_sparse_fwd_fp8(const attn_problem* problem, const uint8_t* q8, const float* q_scale,
                                       const uint8_t* k8, const float* k_scale, const void* v,
                                       const int32_t* row_cnt, const int32_t* row_idx, const int32_t* work_list,
                                       void* o, float* lse, void* ws, size_t ws_bytes, void* stream) {
  tbs::Shape s;
  int32_t st = check_problem(problem, &s);
  if (st != ATTN_OK) return st;
  if ((st = check_fp8_problem(s, "attn_sparse_fwd_fp8"))) return st;
  if (s.nbk > kMaxSparseBlocks)
    return fail(ATTN_E_UNSUPPORTED, "attn_sparse_fwd_fp8: %d key blocks per sequence exceed %d", s.nbk,
                kMaxSparseBlocks);
  if ((st = check_scales(q_scale, k_scale)) || (st = check_i32(row_cnt, "row_cnt", false)) ||
      (st = check_i32(row_idx, "row_idx", false)) || (st = check_i32(work_list, "work_list", true)))
    return st;
  return run_fwd(s, s.causal ? tbs::kSparseCausal : tbs::kSparse, q8, k8, v, row_cnt, row_idx, work_list, o, lse,
                 ws, ws_bytes, stream, q_scale, k_scale);
}

TBS_EXPORT int32_t attn_dense_fwd_fp8(const attn_problem* problem, const uint8_t* q8, const float* q_scale,
                                      const uint8_t* k8, const float* k_scale, const void* v, void* o, float* lse,
                                      void* ws, size_t ws_bytes, void* stream) {
  tbs::Shape s;
  int32_t st = check_problem(problem, &s);
  if (st != ATTN_OK) return st;
  if ((st = check_fp8_problem(s, "attn_dense_fwd_fp8")) || (st = check_scales(q_scale, k_scale))) return st;
  return run_fwd(s, s.causal ? tbs::kCausal : tbs::kDense, q8, k8, v, nullptr, nullptr, nullptr, o, lse, ws,
                 ws_bytes, stream, q_scale, k_scale);
}

static_assert(ATTN_FLAG_NO_SPLIT == tbs::kFlagNoSplit, "flag values of the header and the launchers agree");
