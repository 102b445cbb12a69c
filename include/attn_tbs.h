/*
 * attn_tbs.h -- top-p block-sparse attention forward for AMD MI355X (gfx950).
 *
 * The path, in call order on one stream:
 *
 *   attn_route       block mean-pooling of Q and K, block scores, a softmax
 *                    over key blocks and the top-p cut, giving a block mask,
 *                    per-row index lists and per-row / per-head work counts.
 *   attn_schedule    turns the per-row counts into a longest-first work list
 *                    that a persistent kernel dequeues, so heavily loaded
 *                    heads do not straggle.
 *   attn_sparse_fwd  exact softmax attention of every query block over the
 *                    tokens of its selected key blocks (tiled, online
 *                    softmax, one kernel launch).
 *   attn_dense_fwd   the same kernel over every key block (optionally
 *                    causal): dense attention is the p = 1 case.
 *
 * With causal == 1 (decoder models) every call keeps to the causal order:
 * routing considers only the key blocks that start at or before the last
 * token of query block i (j <= i when key_block == block), and the attention
 * calls keep only keys s <= t for query token t.
 *
 * Sources.  Top-p routing: FVAttn review page, section 1 (Key Terms, "Top-p
 * routing") and section 3 (Method): per query block, key blocks are taken by
 * importance until their cumulative probability reaches p.  Runtime load
 * balancing: same page, section 1 ("Runtime Load Balancing") and section 2:
 * the work is profiled after the mask is fixed and redistributed so no
 * worker straggles.  Exact fused tiled attention: FlashAttention review page,
 * Introduction (exact attention), Model (one fused GPU call; tiling of the
 * matrix products and of the softmax) and Background [3] (S = QK^T,
 * P = softmax(S), O = PV, with S and P never written to memory).
 *
 * Conventions shared by every call
 * --------------------------------
 * - All pointers except `problem` are device pointers (HBM) unless stated.
 *   The caller owns every buffer; the library allocates no memory and keeps
 *   no state between calls other than cached device properties.
 * - Tensors are contiguous, row-major.  q, k, v, o: [B, H, N, d], element
 *   type `dtype` (bf16 or fp32), 16-byte aligned.  Query block i of a
 *   sequence covers tokens [i*block, min((i+1)*block, N)); nb = ceil(N /
 *   block); the last block may hold fewer than `block` tokens.  Key blocks
 *   are the same with key_block (default: block): nbk = ceil(N / key_block).
 *   Unit u = (b*H + h)*nb + i names query block i of head h of batch b;
 *   U = B*H*nb units.  Per-row outputs (mask, row_idx, block_prob) have nbk
 *   entries per unit.
 * - All work is enqueued on `stream` (a hipStream_t; NULL is the default
 *   stream) and the calls return before it completes.  No call synchronises
 *   with the host; route -> schedule -> sparse_fwd on one stream need no
 *   synchronisation because every count stays on the device.
 * - Errors: arguments are validated on the host before any HIP call; a
 *   failed validation enqueues nothing and returns ATTN_E_INVALID,
 *   ATTN_E_UNSUPPORTED or ATTN_E_WORKSPACE.  ATTN_E_DEVICE reports a HIP
 *   error at launch.  attn_last_error() then describes the failure (per
 *   thread).  No C++ exception crosses this interface.
 * - Results are bitwise reproducible for identical inputs: each unit is
 *   computed by one workgroup in a fixed key order, whichever workgroup
 *   takes it.
 * - Calls that share one workspace must not overlap in time (for example on
 *   two streams without ordering between them).
 */
#ifndef ATTN_TBS_H
#define ATTN_TBS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_TBS_ABI_VERSION 8

/* Status codes. */
#define ATTN_OK            0
#define ATTN_E_INVALID     1  /* bad dimension, pointer, alignment or top_p */
#define ATTN_E_UNSUPPORTED 2  /* valid but unsupported combination (d, block, dtype, nb) */
#define ATTN_E_WORKSPACE   3  /* workspace missing or smaller than attn_workspace_bytes() */
#define ATTN_E_DEVICE      4  /* HIP error reported at launch */

/* Element types of q, k, v and o. */
#define ATTN_DTYPE_BF16 0
#define ATTN_DTYPE_F32  1

/* Operations, for attn_workspace_bytes() and attn_num_workers(). */
#define ATTN_OP_ROUTE      0
#define ATTN_OP_SCHEDULE   1
#define ATTN_OP_SPARSE_FWD 2
#define ATTN_OP_DENSE_FWD  3
#define ATTN_OP_AUGMENT    4

/* Problem flags. */
#define ATTN_FLAG_PROFILE_WORKERS 1  /* fwd calls record per-worker start/end
                                        times in the workspace (see below) */
#define ATTN_FLAG_NO_SPLIT        2  /* fwd calls run every work item whole,
                                        never as parts along the keys: results
                                        then do not depend on the number of
                                        compute units (see attn_sparse_fwd) */

typedef struct attn_problem {
  int32_t batch;     /* B >= 1 */
  int32_t heads;     /* H >= 1 */
  int32_t seq_len;   /* N >= 1 */
  int32_t head_dim;  /* d: 64 or 128 */
  int32_t block;     /* query block size (routing rows, query tiles): 64 or 128 */
  int32_t dtype;     /* ATTN_DTYPE_BF16 or ATTN_DTYPE_F32 */
  int32_t causal;    /* 0 or 1: causal routing and causal attention (keys s <= t) */
  int32_t flags;     /* ATTN_FLAG_* bits, 0 for none */
  double scale;      /* softmax scale; 0 selects 1/sqrt(head_dim) */
  int32_t key_block; /* key block size (routing columns, selection unit): 64 or 128; 0 selects block */
  int32_t reserved;  /* must be 0 */
} attn_problem;

/* ABI version of the loaded library (ATTN_TBS_ABI_VERSION when it was built). */
int32_t attn_abi_version(void);

/* Message for the last failed call on this thread ("" if none).  The string
 * stays valid until the next call on the same thread. */
const char* attn_last_error(void);

/* Bytes of workspace `op` needs for `problem` (0 if the problem is invalid).
 * Workspaces must be 16-byte aligned.  Its first 256 bytes are a control
 * block (the persistent kernel's queue counters): they must be zero when
 * attn_sparse_fwd or attn_dense_fwd starts.  A zero-filled workspace
 * satisfies this, and attn_schedule and every fwd call leave them zero when
 * they complete, so one zero fill at allocation is enough (attn_route and
 * attn_augment use only the bytes after it).  One workspace of the largest
 * size serves every operation.  For ATTN_OP_DENSE_FWD of a causal problem
 * with few work items (see attn_dense_fwd) the size includes per-item part
 * counters, which the call zeroes itself, and the parts' partial results:
 * (256 * head_dim + 1024) * 4 bytes per part, at most (work items + 2 *
 * compute units) parts, which depends on the current device. */
size_t attn_workspace_bytes(const attn_problem* problem, int32_t op);

/* Query blocks per work item, G.  The persistent fwd kernel processes a work
 * item -- G consecutive query blocks of one (b, h) -- in one workgroup: every
 * K/V tile in the union of the G blocks' selected key blocks is loaded once and
 * each block's waves compute only the tiles that block selected (adjacent
 * query blocks select largely the same key blocks).  For bf16 a work item
 * holds 256 query rows: G = 4 with block 64, G = 2 with block 128; G = 1 for
 * fp32.  Work item g = (b*H + h)*ceil(nb/G) + i/G covers query
 * blocks G*(i/G) .. min(G*(i/G) + G, nb) - 1; there are B*H*ceil(nb/G) items.
 * Returns 0 if the problem is invalid. */
int32_t attn_group_size(const attn_problem* problem);

/* Number of persistent workgroups ("workers") the fwd kernel of `op`
 * launches on the current device for `problem` (0 if invalid).  With
 * ATTN_FLAG_PROFILE_WORKERS, worker w writes two uint64 values at workspace
 * byte offset 256 + 16*w: its first and last s_memrealtime stamp (100 MHz). */
int32_t attn_num_workers(const attn_problem* problem, int32_t op);

/* Top-p block routing.
 *
 * Per (b, h): Qbar_i = mean of q over the valid tokens of query block i,
 * Kbar_j = mean of k over the valid tokens of key block j (key_block tokens);
 * Z_ij = scale * <Qbar_i, Kbar_j>; P_i. = softmax_j(Z_i.) over the nbk key
 * blocks.  Key blocks are ranked by P descending, equal P by smaller index;
 * row i keeps the shortest ranked prefix whose cumulative probability is
 * >= top_p (all nbk blocks when top_p >= 1).  Pooling, scores, softmax and the cut are
 * evaluated in fp64, so the decisions are those of exact arithmetic up to
 * fp64 rounding.
 *
 * Causal routing (causal == 1): row i only considers the eligible key
 * blocks, those with j * key_block <= (i+1) * block - 1 (the blocks j <= i
 * when key_block == block); there are e_i = min(nbk, ((i+1)*block - 1) /
 * key_block + 1) of them.  The others are cut before the softmax (Z_ij =
 * -inf, P_ij = 0), so P_i. is a softmax over the e_i eligible scores, the
 * ranking and the cut run over those blocks only, and top_p >= 1 selects
 * all of them.  The routing
 * pages state top-p routing for full attention; cutting the future blocks
 * before the softmax is the reading this library takes for decoders.
 *
 *   q, k      [B,H,N,d] dtype, read only.
 *   top_p     in (0, 1].
 *   mask      [B,H,nb,nbk] uint8 out: 1 where key block j is selected for row i.
 *   row_cnt   [B,H,nb] int32 out: k_i, number of selected key blocks (>= 1).
 *   row_idx   [B,H,nb,nbk] int32 out: the first row_cnt entries of each row are
 *             the selected key blocks in ascending order; the next entries,
 *             up to the number of eligible blocks (nbk, or e_i under causal
 *             routing), are the unselected eligible blocks in rank order
 *             (P descending, equal P by smaller index), which attn_augment
 *             reads; entries after those are not written.
 *   head_cnt  [B,H] int32 out: sum over i of row_cnt (overwritten, not added to).
 *   block_prob [B,H,nb,nbk] double out, nullable: the block probabilities P
 *             (0 for key blocks cut by causal routing).
 *   ws        workspace of attn_workspace_bytes(problem, ATTN_OP_ROUTE) bytes.
 * Requires nbk <= 1024. */
int32_t attn_route(const attn_problem* problem, const void* q, const void* k, double top_p,
                   uint8_t* mask, int32_t* row_cnt, int32_t* row_idx, int32_t* head_cnt,
                   double* block_prob, void* ws, size_t ws_bytes, void* stream);

/* Longest-first work list, in head windows.
 *
 * Work item g (see attn_group_size) costs the summed row_cnt of its query
 * blocks.  The (b, h) pairs are cut into windows of `head_window` consecutive
 * pairs (window of item g = (g / ceil(nb/G)) / head_window); work_list
 * receives every item id once, sorted by window ascending, then cost
 * descending, then id ascending.  The persistent fwd kernel takes items from
 * this list in order, each workgroup taking the next one when it becomes free
 * (dynamic list scheduling): longest-first keeps heavy items from straggling
 * at the end, and the windows keep the items that run at the same time on the
 * K/V of a few heads, so that K/V is read from cache instead of HBM.
 * head_window = 0 (or >= B*H) gives one window: a pure longest-first list.
 * Also zeroes the workspace control block.
 *
 *   row_cnt      [B*H*nb] int32 in, each in [0, nb].
 *   head_window  >= 0, see above.
 *   num_workers  workers for the optional static model; 0 selects the number
 *                of compute units of the current device.
 *   work_list    [B*H*ceil(nb/G)] int32 out.
 *   worker_of    [B*H*ceil(nb/G)] int32 out, nullable: greedy
 *                longest-processing-time assignment in work-list order (each
 *                item to the least-loaded worker, ties to the lowest id).  Only
 *                computed when worker_of or worker_load is given: the greedy
 *                is sequential (one wavefront, loads in registers), so it
 *                costs time proportional to the number of work items; it
 *                serves load-balance reports.
 *   worker_load  [num_workers] int64 out, nullable: summed cost per worker
 *                under that assignment.
 * Requires nbk <= 1024 and num_workers <= 4096. */
int32_t attn_schedule(const attn_problem* problem, const int32_t* row_cnt, int32_t head_window,
                      int32_t num_workers, int32_t* work_list, int32_t* worker_of, int64_t* worker_load,
                      void* ws, size_t ws_bytes, void* stream);

/* Fixed cost of one 64-key tile of the attention kernel, in row-tiles (one
 * query block computing one tile): staging the tile and running the softmax
 * pipeline cost about as much as three rows' products.  Measured: giving
 * every row of the video-32k and skewed-32k problems the blocks of its work
 * item's union added 18% / 12% row-tiles and 1.1% / 0.9% tiles and took 10.3%
 * / 7.2% more time, which fits F = 2.4 to 3.0. */
#define ATTN_SASA_TILE_FIXED 3

/* Slack-aware sparse augmentation (SASA) on one GPU, priced in row-tiles.
 *
 * Source: FVAttn review page, section 1 (Key Terms, "Slack-Aware Sparse
 * Augmentation") and section 3 (Method): after load balancing, ranks with
 * slack compute extra high-value blocks.  A work item (attn_group_size query
 * blocks of one head) runs the union of its rows' key blocks as 64-key tiles
 * (key_block/64 per block, the last block only the tiles its keys reach); a
 * tile costs F = ATTN_SASA_TILE_FIXED row-tiles plus one per row that
 * selected it, so an item costs F * (union tiles) + (row tiles).  The ranks
 * are num_workers workers that take the items in work_list order W positions
 * at a time: before each batch the workers are ranked by (load, id) and the
 * r-th ranked worker takes the batch's r-th item.  With M the largest load,
 * worker w has slack M - load[w] and spends it on its last item (the one of
 * the latest batch that reached it), where extra cost changes no other choice
 * of the assignment.  Its candidates are the (row, key block) pairs of that
 * item whose block is eligible for the row and not selected by it, ordered
 * by the row's block probability descending, then row, then block; a pair
 * costs the block's tiles, plus F times them when its block is in neither
 * the item's union nor an earlier pair; the worker buys the longest prefix of
 * that order whose cost fits its slack.  No worker's load exceeds M.  mask,
 * row_cnt, row_idx and head_cnt are updated in place (only rows that bought
 * pairs change); row_idx keeps the new selection ascending, then the row's
 * remaining eligible blocks in their routing rank order.  Run the forward on
 * the same work_list: its items then run in the order the assignment assumed.
 * A problem whose attn_sparse_fwd splits its items along their keys (bf16,
 * fewer than 4 items per compute unit, no ATTN_FLAG_NO_SPLIT) runs in equal
 * shares of its tiles instead, with no modelled idle time: attn_augment then
 * changes nothing (paid = 0; worker_of and worker_load are still written).
 *
 *   block_prob   [B,H,nb,nbk] double, from attn_route (block_prob output).
 *   work_list    [B*H*ceil(nb/G)] int32, a permutation of the items (from
 *                attn_schedule over the same routing), nullable: item order.
 *   num_workers  1 .. 4096 (the fwd kernel's workgroups: attn_num_workers).
 *   mask, row_cnt, row_idx, head_cnt   attn_route's outputs, updated in
 *                place; row_idx must hold the ranked tail attn_route writes
 *                after the selected blocks.
 *   worker_of    [B*H*ceil(nb/G)] int32 out, nullable: the worker of every item.
 *   worker_load  [num_workers] int64 out, nullable: cost per worker (row-tiles)
 *                before augmentation.
 *   paid         [num_workers] int32 out, nullable: pairs bought per worker.
 *   ws           attn_workspace_bytes(problem, ATTN_OP_AUGMENT) bytes; the
 *                control block is not touched.
 * Honours causal (the eligible blocks of routing).  Requires nbk <= 1024. */
int32_t attn_augment(const attn_problem* problem, const double* block_prob, const int32_t* work_list,
                     int32_t num_workers, uint8_t* mask, int32_t* row_cnt, int32_t* row_idx, int32_t* head_cnt,
                     int32_t* worker_of, int64_t* worker_load, int32_t* paid, void* ws, size_t ws_bytes,
                     void* stream);

/* Slack-aware augmentation inside work items.
 *
 * The attention kernel runs a work item (G query blocks, see
 * attn_group_size) as one sequence of key tiles, the union of the G rows'
 * selections; a wave whose row did not select a tile idles through that
 * step.  That idle time is slack inside the item (FVAttn review page,
 * section 1, "Slack-Aware Sparse Augmentation": extra high-value blocks in
 * the slack).  This call fills it: every row selects every block of its
 * item's union that is eligible for it (all blocks, or those allowed by
 * causal routing).  The union of every item, and so the attention kernel's
 * tiles, stay the same.  mask, row_cnt, row_idx and head_cnt are updated in
 * place: row_idx keeps the new selection ascending, followed by the row's
 * remaining eligible blocks in their routing rank order.  row_idx must hold
 * attn_route's ranked tail.  No workspace.  With G = 1 (fp32) it changes
 * nothing.  Requires nbk <= 1024. */
int32_t attn_augment_union(const attn_problem* problem, uint8_t* mask, int32_t* row_cnt, int32_t* row_idx,
                           int32_t* head_cnt, void* stream);

/* Block-sparse attention forward, one persistent kernel launch.
 *
 * For each unit (b, h, i) and each query token t of block i, over the key
 * tokens s of the key blocks row_idx[u][0..row_cnt[u]):
 *   O_t = sum_s exp(l_s - mu) V_s / sum_s exp(l_s - mu),  l_s = scale*<Q_t, K_s>,
 *   LSE_t = mu + ln sum_s exp(l_s - mu)   (natural log), mu = max_s l_s.
 * Products in MFMA with fp32 accumulation (bf16 operands for bf16 inputs;
 * softmax weights are rounded to bf16 before the P*V product), online
 * softmax in fp32; o is written in dtype (bf16 round-to-nearest-even).
 *
 *   q, k, v    [B,H,N,d] dtype.
 *   row_cnt    [U] int32, row_idx [U, nbk] int32 as written by attn_route
 *              (key-block indices in [0, nbk); the library clamps
 *              out-of-range values).
 *   work_list  [B*H*ceil(nb/G)] int32, nullable: work-item order (from
 *              attn_schedule); NULL processes items in natural order.
 *   o          [B,H,N,d] dtype out.  A unit whose row_cnt is 0 gets o = 0.
 *   lse        [B,H,N] float out, nullable (-inf for a unit with no keys).
 *   ws         attn_workspace_bytes(problem, ATTN_OP_SPARSE_FWD) bytes, control
 *              block zero on entry (see attn_workspace_bytes).
 * With causal == 1, only keys s <= t enter the sums for query token t (the
 * lists come from causal routing, so they hold eligible blocks; a listed
 * block entirely after the query block contributes no keys, and a unit left
 * with no keys gets o = 0 and lse = -inf).
 *
 * Problems with few work items (bf16, fewer than 4 items of 256 query rows
 * per compute unit and at most 1024 items, e.g. one GPU's share of a few
 * heads) run as equal shares of their union key tiles: two small kernels on
 * `stream` count each item's union tiles from the lists, lay the items end
 * to end in item order and cut the sequence into one chunk of equal length
 * (within a tile) per persistent workgroup, so an item crossing a cut runs
 * as parts on several workgroups.  Each part's running maximum, sum and
 * unnormalised O are merged in part order by the item's last part to finish
 * (FlashAttention review, Tiling Softmax).  The result is deterministic,
 * independent of work_list, and equal to the unsplit one up to fp32
 * rounding; attn_workspace_bytes accounts for the parts (work_items +
 * 2 * CUs slots of partial results).  ATTN_FLAG_NO_SPLIT
 * runs every item whole (then an all-ones mask gives attn_dense_fwd's bits).
 * Requires nbk <= 2048. */
int32_t attn_sparse_fwd(const attn_problem* problem, const void* q, const void* k, const void* v,
                        const int32_t* row_cnt, const int32_t* row_idx, const int32_t* work_list,
                        void* o, float* lse, void* ws, size_t ws_bytes, void* stream);

/* attn_sparse_fwd without a workspace argument, for callers that cannot
 * allocate device memory or hand one over: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Same arguments
 * (minus ws / ws_bytes), arithmetic and results as attn_sparse_fwd, bit for
 * bit, except that every work item runs whole: where attn_sparse_fwd splits
 * the items of a small problem along the keys, the results agree up to fp32
 * rounding.  Its only scratch -- the persistent queue's control block, 256 bytes
 * -- lives in a file-scope device array of the library, one per GPU, held
 * until the process ends; each call zeroes it with a fill kernel on `stream`
 * before the attention kernel.  The call allocates nothing and needs no prior
 * attn_schedule to reset a control block.  Every call on one GPU shares that
 * GPU's array: calls that overlap in time on one GPU (for example on two
 * streams without ordering between them) race and must not be issued.
 * Problems whose attn_sparse_fwd workspace would exceed the array (the
 * ATTN_FLAG_PROFILE_WORKERS flag) are rejected with ATTN_E_WORKSPACE before
 * any HIP call.  Requires nbk <= 2048. */
int32_t attn_sparse_fwd_noalloc(const attn_problem* problem, const void* q, const void* k, const void* v,
                                const int32_t* row_cnt, const int32_t* row_idx, const int32_t* work_list,
                                void* o, float* lse, void* stream);

/* Dense attention forward (every key block; causal keeps keys s <= t).
 * Same arithmetic, layouts and workspace rules as attn_sparse_fwd; with
 * causal the query blocks with the most keys are processed first.  Equals,
 * bit for bit, attn_sparse_fwd with every block selected (causal == 0) or
 * with every eligible block selected (causal == 1), for any key_block, when
 * neither call splits its work items (ATTN_FLAG_NO_SPLIT on both calls makes
 * sure of it), and up to fp32 rounding otherwise.  The key block size does
 * not enter the dense result.
 *
 * Causal bf16 problems (unless ATTN_FLAG_NO_SPLIT) with fewer than 4 work
 * items per compute unit whose
 * last item holds more than half the mean work per compute unit (at least
 * 16 key tiles of 64 keys) run their longer items as equal parts along the
 * keys, each part's running maximum, sum and unnormalised O merged in part
 * order by the item's last part to finish (FlashAttention review, Tiling
 * Softmax: partial softmax results combine exactly).  The result is then
 * deterministic and equal to the unsplit one up to fp32 rounding, not bit
 * for bit; attn_num_workers and attn_workspace_bytes account for the parts. */
int32_t attn_dense_fwd(const attn_problem* problem, const void* q, const void* k, const void* v,
                       void* o, float* lse, void* ws, size_t ws_bytes, void* stream);

/* FP8 (E4M3) path
 * ---------------
 * Source: ParaAttention/HunyuanVideo post (WaveSpeed), section on FP8 dynamic
 * quantisation: activations are quantised to FP8 at run time so that the
 * products run on 8-bit matrix units.  The post fixes neither format nor
 * granularity; this library takes OCP E4M3 (largest magnitude 448, round to
 * nearest even), one scale per query token and one per 64-token tile of keys,
 * and quantises only Q and K: the S = Q K^T product runs on gfx950's fp8
 * matrix instructions while V, the softmax weights (bf16) and O stay as in
 * attn_sparse_fwd.  The result is, up to fp32 rounding, exact attention on
 * the dequantised Q and K: q_t = code * q_scale[t], k_s = code * k_scale[s/64].
 * These calls take bf16 problems with head_dim 128 (ATTN_E_UNSUPPORTED
 * otherwise); routing keeps reading the bf16 Q and K (attn_route, or
 * attn_route_fp8, which also quantises them in the same pass). */

/* Dynamic E4M3 quantisation of Q and K.  For each group (a query token's d
 * values; the d values of up to 64 tokens of keys, tile tau holding tokens
 * 64 tau .. min(64 tau + 64, N) - 1 of a (b, h)) with largest magnitude a,
 * in correctly rounded fp32: inv = 448 / a, code = E4M3(clamp(x * inv, -448,
 * 448)) rounded to nearest even (the sign bit kept, so a negative value that
 * rounds to zero gives 0x80), scale = a / 448; a = 0 gives scale 0 and zero
 * codes.
 *
 *   q, k     [B,H,N,128] bf16, read only.
 *   q8, k8   [B,H,N,128] uint8 out: E4M3 codes, 16-byte aligned.
 *   q_scale  [B,H,N] float out: per-token Q scales.
 *   k_scale  [B,H,ceil(N/64)] float out: per-tile K scales.
 * One kernel launch; reads Q and K once. */
int32_t attn_quantize_qk_fp8(const attn_problem* problem, const void* q, const void* k, uint8_t* q8,
                             float* q_scale, uint8_t* k8, float* k_scale, void* stream);

/* attn_route and attn_quantize_qk_fp8 in one pass over Q and K: the block
 * means, scores, softmax and top-p cut of attn_route (the same mask, lists,
 * counts and block probabilities, bit for bit) and the E4M3 codes and scales
 * of attn_quantize_qk_fp8 (bit for bit), with each element of Q and K read
 * from HBM once by a kernel that pools and quantises the same registers.
 * Arguments as in the two calls; bf16 problems with head_dim 128
 * (ATTN_E_UNSUPPORTED otherwise); ws as for attn_route. */
int32_t attn_route_fp8(const attn_problem* problem, const void* q, const void* k, double top_p, uint8_t* mask,
                       int32_t* row_cnt, int32_t* row_idx, int32_t* head_cnt, double* block_prob, uint8_t* q8,
                       float* q_scale, uint8_t* k8, float* k_scale, void* ws, size_t ws_bytes, void* stream);

/* attn_sparse_fwd with Q and K as E4M3 codes and scales (from
 * attn_quantize_qk_fp8).  The logit of query t and key s is
 * scale * q_scale[t] * k_scale[s/64] * sum_c code_q[t][c] * code_k[s][c], the
 * sum of code products accumulated in fp32 by the matrix unit; everything
 * else (lists, work list, masks, causal rule, outputs, workspace) is as in
 * attn_sparse_fwd.  v and o are bf16. */
int32_t attn_sparse_fwd_fp8(const attn_problem* problem, const uint8_t* q8, const float* q_scale,
                            const uint8_t* k8, const float* k_scale, const void* v, const int32_t* row_cnt,
                            const int32_t* row_idx, const int32_t* work_list, void* o, float* lse, void* ws,
                            size_t ws_bytes, void* stream);

/* attn_dense_fwd with fp8 Q and K (same logits as attn_sparse_fwd_fp8); equals
 * attn_sparse_fwd_fp8 with every (eligible) block selected, bit for bit, when
 * neither call splits its work items (see attn_dense_fwd). */
int32_t attn_dense_fwd_fp8(const attn_problem* problem, const uint8_t* q8, const float* q_scale,
                           const uint8_t* k8, const float* k_scale, const void* v, void* o, float* lse, void* ws,
                           size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_TBS_H */
