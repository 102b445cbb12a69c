// Persistent tiled attention forward with online softmax for gfx950.
//
// Source: FlashAttention review page, Model ("fuse O = Attn(Q,K,V) into one
// GPU call"; tile the matrix products; tile the softmax because it works
// row by row) and Tiling Softmax (compute the softmax block by block from
// on-chip tiles and combine the partial results), Introduction (the result
// is exact attention); FVAttn review page, section 1 ("Top-p routing": each
// query block attends only to its selected key blocks).
//
// Work item: 256 consecutive query rows of one (b, h) (for fp32: one query
// block).  Workgroups are persistent: each takes the next item from a queue
// (the longest-first work list, or natural order) with one atomic, so a heavy
// item never waits behind a fixed grid assignment.
//
// bf16 kernel (8 waves, each owning 32 query rows; details at the kernel):
//   * Key tiles of 64 keys.  K and V tiles are copied HBM -> LDS with
//     buffer_load ... lds (16 bytes per lane, no VGPR staging), two stages
//     each, two steps ahead of their use.  Rows are stored with an XOR
//     swizzle of their 16-byte chunks so the MFMA operand reads hit distinct
//     LDS banks.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: K (A operand) from LDS, Q^T
//     (B operand) held in registers for the whole item.  Computing S
//     transposed puts one query per lane (lanes l and l^32 share it), so the
//     running max and sum of the online softmax are lane-local plus one
//     permlane32 swap.
//   * A-operand rows of K are permuted (bits 2 and 3 of the row swapped) so
//     each lane's 16 accumulator values are 2 runs of 8 consecutive keys:
//     exactly the B operand (P^T) the next product needs, with no shuffle.
//   * O^T += V^T P^T on the same MFMA: V^T (A operand) comes straight from the
//     row-major V tile through ds_read_b64_tr_b16 transposed reads.
//   * Online softmax in fp32 with exp2 (scale*log2 e folded in); a row's
//     reference maximum only moves when a tile's maximum exceeds it by more
//     than 2^8 in weight (the result is exact for any reference maximum; the
//     bound keeps every weight <= 256).  Weights are rounded to bf16 for the
//     P V product.
//   * The two waves of each SIMD alternate: one issues the MFMA part of a
//     tile while the other runs the softmax of another.
//   * Epilogue: O / l in fp32 -> bf16 (round to nearest even), LSE = m + ln l.
//   * Dense causal problems with few items per compute unit run their long
//     items as parts along the keys: each part keeps its own running
//     maximum, sum and unnormalised O and writes them to the workspace; the
//     item's last part to finish combines the parts (the partial results of
//     Tiling Softmax) and writes O and LSE.
//
// fp32 kernel: same unit/tile/queue structure and the same transposed
// formulation on v_mfma_f32_32x32x2_f32, operands read from padded LDS
// tiles; weights stay fp32.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace tbs {
namespace {

constexpr int kKeyTile = 64;

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* row_cnt;
  const int32_t* row_idx;
  const int32_t* work_list;
  uint32_t* ctrl;
  unsigned long long* prof;
  const float* q_scale;   // fp8 path: per-token Q scales [BH, N]
  const float* k_scale;   // fp8 path: per-64-key-tile K scales [BH, nkt]
  int nkt;                // fp8 path: 64-key tiles per (b, h)
  int BH;
  int N;
  int nb;             // query blocks per (b, h)
  int nbk;            // key blocks per (b, h): entries of a row_idx row
  int U;              // work items in the queue (query-block groups)
  int G;              // query blocks per work item
  int ng;             // work items per (b, h) = ceil(nb / G)
  float scale;        // softmax scale
  float scale_log2;   // scale * log2(e)
  // Dense causal, split items (split_tiles > 0): the queue holds U parts of
  // at most split_tiles key tiles; part_buf holds each part's unnormalised O,
  // running maximum and sum, part_cnt the parts finished per item.
  int split_tiles;
  uint32_t* part_cnt;
  float* part_buf;
  // Listed modes with split items: the entries written by the planning
  // kernels ({item, part, parts, first tile | end tile << 16}), their number,
  // and the first entry of every workgroup (workgroup w runs entries
  // starts[w] .. starts[w + 1] - 1 in order; no shared queue).
  const int4* entries;
  const int* n_entries;
  const int* starts;
};

// Unit bookkeeping of the fp32 kernel: query blocks of BQ rows, listed key
// blocks of BK keys.
template <int BQ, int BK, int MODE>
struct UnitInfo {
  int bh, i, ntiles;
  const int32_t* list;

  __device__ __forceinline__ void decode(const FwdParams& p, int qpos) {
    int u;
    if (MODE == kCausal) {
      // Longest first: the last query blocks of every head have the most keys.
      i = p.nb - 1 - qpos / p.BH;
      bh = qpos % p.BH;
      u = bh * p.nb + i;
    } else {
      u = qpos;
      if (fwd_listed(MODE) && p.work_list) u = min(max(p.work_list[qpos], 0), p.U - 1);
      bh = u / p.nb;
      i = u - bh * p.nb;
    }
    constexpr int SPB = BK / kKeyTile;   // key tiles per key block
    if (fwd_listed(MODE)) {
      const int cnt = min(max(p.row_cnt[u], 0), p.nbk);
      list = p.row_idx + static_cast<long long>(u) * p.nbk;
      ntiles = cnt * SPB;
      if (SPB > 1 && cnt > 0 && list[cnt - 1] >= p.nbk - 1) {
        const int tail = p.N - (p.nbk - 1) * BK;
        ntiles = (cnt - 1) * SPB + (tail + kKeyTile - 1) / kKeyTile;
      }
    } else if (MODE == kDense) {
      list = nullptr;
      ntiles = (p.N + kKeyTile - 1) / kKeyTile;
    } else {
      list = nullptr;
      ntiles = (min(p.N, (i + 1) * BQ) + kKeyTile - 1) / kKeyTile;
    }
  }

  __device__ __forceinline__ int key0(const FwdParams& p, int t) const {
    if (fwd_listed(MODE)) {
      constexpr int SPB = BK / kKeyTile;
      const int jb = min(max(list[t / SPB], 0), p.nbk - 1);
      return jb * BK + (t % SPB) * kKeyTile;
    }
    return t * kKeyTile;
  }
};

// max of three floats in one v_max3_f32 (operands are never NaN here: logits
// are finite or -inf).
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// MFMA A-operand fragments are read this many products ahead through a
// register ring; TBS_KPF_PIN pins the read/MFMA interleave for the scheduler.
#ifndef TBS_KPF
#define TBS_KPF 4
#endif
#ifndef TBS_KPF_PIN
#define TBS_KPF_PIN 1
#endif

template <int S>
struct Stage {
  static constexpr int value = S;
};

__device__ __forceinline__ int swap_bits23(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// 16-byte-chunk XOR swizzle of an LDS tile row (see the operand reads).
template <int D>
__device__ __forceinline__ int chunk_swz(int row) {
  if (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  // 128-byte rows: two rows share a line of the 64 four-byte banks, so the
  // rows of a 16-lane read group must differ in (row parity, chunk).
  return (row >> 1) & 7;
}

// Copies a 64-key tile of K or V (rows key0 .. key0+63 of one head) from HBM
// into LDS with buffer_load ... lds: each instruction writes 1 KB of LDS (16
// bytes per lane, lane-contiguous); the lane picks the global chunk whose
// swizzled position is its LDS slot.  The buffer resource starts at row key0
// and holds the rows left in the sequence, so chunks past the end read as
// zero (their logits are masked) without a separate tail path.
//
// Wave w of NW copies the PER_WAVE consecutive 1 KB slices w*PER_WAVE ..
// +PER_WAVE-1 of a tile.  The instruction offset (j * 1 KB) is added to both
// the LDS and the global address, so one M0 value (the LDS base operand of
// the copy) serves all of a wave's instructions for a tile: M0 is written
// once per tile instead of once per instruction.
constexpr int kRsrcWord3 = 0x00020000;   // raw dword buffer

template <int D, int NW>
struct TileLoader {
  static constexpr int ROWB = D * 2;
  static constexpr int TILEB = kKeyTile * ROWB;
  static constexpr int PER_WAVE = TILEB / 1024 / NW;
  static_assert(PER_WAVE == 1 || PER_WAVE == 2 || PER_WAVE == 4, "copy slices per wave");
  // Global byte offset, minus the instruction offset j * 1 KB, of this lane's
  // chunk for the wave's slice j.
  unsigned voff[PER_WAVE];
  unsigned slice0;   // first LDS byte of the wave's slices

  __device__ __forceinline__ void init(int wave, int lane) {
    slice0 = static_cast<unsigned>(wave * PER_WAVE * 1024);
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int byte = (wave * PER_WAVE + j) * 1024 + lane * 16;
      const int row = byte / ROWB;
      const int lch = ((byte % ROWB) / 16) ^ chunk_swz<D>(row);
      voff[j] = static_cast<unsigned>(row * ROWB + lch * 16 - j * 1024);
    }
  }

  __device__ __forceinline__ static u32x4 rsrc(const unsigned char* base, int bytes) {
    const unsigned long long a = reinterpret_cast<unsigned long long>(base);
    u32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(a));
    r[1] = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(a >> 32) & 0xffffu);   // stride 0
    r[2] = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(bytes));
    r[3] = kRsrcWord3;
    return r;
  }

  // The wave's buffer_load_dwordx4 ... lds instructions for one tile, written
  // as inline asm so that the compiler does not count them as pending writes
  // to the tile being read: the loop orders every tile's reads after its own
  // copy with an explicit vmcnt wait and a barrier, and the copy into the
  // other stage stays in flight meanwhile.  M0 is restored afterwards.
  __device__ __forceinline__ void issue_one(const unsigned char* g, int key0, int N, TBS_LDS unsigned char* dst) const {
    const u32x4 r = rsrc(g + static_cast<long long>(key0) * ROWB, (N - key0) * ROWB);
    const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(unsigned long)dst) + slice0;
    unsigned saved;
    if (PER_WAVE == 1) {
      asm volatile(
          "s_mov_b32 %0, m0\n\t"
          "s_mov_b32 m0, %1\n\t"
          "s_nop 0\n\t"
          "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
          "s_mov_b32 m0, %0"
          : "=&s"(saved)
          : "s"(m0), "v"(voff[0]), "s"(r)
          : "memory");
    } else if (PER_WAVE == 2) {
      asm volatile(
          "s_mov_b32 %0, m0\n\t"
          "s_mov_b32 m0, %1\n\t"
          "s_nop 0\n\t"
          "buffer_load_dwordx4 %2, %4, 0 offen lds\n\t"
          "buffer_load_dwordx4 %3, %4, 0 offen offset:1024 lds\n\t"
          "s_mov_b32 m0, %0"
          : "=&s"(saved)
          : "s"(m0), "v"(voff[0]), "v"(voff[PER_WAVE > 1 ? 1 : 0]), "s"(r)
          : "memory");
    } else {
      asm volatile(
          "s_mov_b32 %0, m0\n\t"
          "s_mov_b32 m0, %1\n\t"
          "s_nop 0\n\t"
          "buffer_load_dwordx4 %2, %6, 0 offen lds\n\t"
          "buffer_load_dwordx4 %3, %6, 0 offen offset:1024 lds\n\t"
          "buffer_load_dwordx4 %4, %6, 0 offen offset:2048 lds\n\t"
          "buffer_load_dwordx4 %5, %6, 0 offen offset:3072 lds\n\t"
          "s_mov_b32 m0, %0"
          : "=&s"(saved)
          : "s"(m0), "v"(voff[0]), "v"(voff[PER_WAVE > 1 ? 1 : 0]), "v"(voff[PER_WAVE > 2 ? 2 : 0]),
            "v"(voff[PER_WAVE > 3 ? 3 : 0]), "s"(r)
          : "memory");
    }
  }
};

// Copies one float (the scale of a K tile) from `src` into LDS with a
// buffer_load_dword ... lds issued by one wave: every lane fetches the same
// word, so dwords dst[0..63] all receive it.  Like the tile copies it is
// written as inline asm and waited for with the explicit vmcnt wait and
// barrier of the copy protocol.
__device__ __forceinline__ void copy_scale(const float* src, TBS_LDS float* dst) {
  const unsigned long long a = reinterpret_cast<unsigned long long>(src);
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(a));
  r[1] = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(a >> 32) & 0xffffu);
  r[2] = 4u;
  r[3] = kRsrcWord3;
  const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(unsigned long)dst);
  const unsigned zero = 0u;
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0), "v"(zero), "s"(r)
      : "memory");
}

// A work item is a group of G consecutive query blocks of one (b, h).  The
// workgroup loads every 64-key K/V tile in the union of the group's key
// blocks once; each wave (32 query rows of one member block) computes only
// the tiles its own block selected.  Adjacent query blocks select largely the
// same key blocks, so grouping cuts tile traffic without wasting much MFMA.
constexpr int kMaxListBlocks = 2048;   // nb limit of the in-LDS union list
constexpr int kMaxListWords = kMaxListBlocks / 32;

template <int BQ, int G, int MODE>
struct GroupInfo {
  int bh, i0, gsz;   // head, first query block, member blocks present (1..G)
  int g;             // work item
  int tb, te;        // key tiles [tb, te) of this part (te: an upper bound when not split)
  int part, nparts;  // part of the item and the item's number of parts

  __device__ __forceinline__ void decode(const FwdParams& p, int qpos) {
    tb = 0;
    te = 0x7fffffff;
    part = 0;
    nparts = 1;
    if (MODE == kCausal && p.split_tiles > 0) {
      // Split dense causal: the queue runs item rows gi = ng-1 .. 0 (the last
      // query blocks have the most keys); row gi holds, for every head, the
      // ceil(tiles(gi) / split_tiles) equal parts of its item, consecutively.
      int rem = qpos;
      int gi = p.ng - 1;
      int ntg = 1, npg = 1;
      for (;; --gi) {
        ntg = (min(p.N, (gi + 1) * G * BQ) + kKeyTile - 1) / kKeyTile;
        npg = (ntg + p.split_tiles - 1) / p.split_tiles;
        if (rem < p.BH * npg || gi == 0) break;
        rem -= p.BH * npg;
      }
      bh = rem / npg;
      part = rem - bh * npg;
      nparts = npg;
      // equal parts: lengths differ by at most one tile
      tb = part * ntg / npg;
      te = (part + 1) * ntg / npg;
      g = bh * p.ng + gi;
    } else if (fwd_listed(MODE) && p.entries) {
      // Split sparse items: the entry names the item, the part and its range
      // of the item's union tiles.
      const int4 en = p.entries[qpos];
      g = min(max(en.x, 0), p.U - 1);
      part = en.y;
      nparts = max(en.z, 1);
      tb = en.w & 0xffff;
      te = static_cast<int>(static_cast<unsigned>(en.w) >> 16);
      bh = g / p.ng;
    } else if (MODE == kCausal) {
      // Longest first: the last query blocks of every head have the most keys.
      const int gi = p.ng - 1 - qpos / p.BH;
      bh = qpos % p.BH;
      g = bh * p.ng + gi;
    } else {
      g = qpos;
      if (fwd_listed(MODE) && p.work_list) g = min(max(p.work_list[qpos], 0), p.U - 1);
      bh = g / p.ng;
    }
    i0 = (g - bh * p.ng) * G;
    gsz = min(G, p.nb - i0);
  }
};

// ------------------------------------------------------- bf16, two groups ---
//
// Workgroup of 8 waves covering 256 query rows: G = 256 / block consecutive
// query blocks of one (b, h), each 32-row slice owned by one wave.  Waves
// w and w + 4 share a SIMD, so the workgroup splits into two groups (waves
// 0-3 and 4-7) with one wave of each group on every SIMD.  A wave's work on
// tile t is an MFMA part M(t) = S(t) = K(t) Q^T, then O^T += V^T P^T for
// tile t - 1, and a VALU part V(t) = the online-softmax update of tile t.
// The workgroup advances in steps of one part each; group 1 runs one
// step behind group 0, so on every SIMD one wave issues MFMAs while the other
// computes exponentials and the matrix core and the VALU work side by side:
//
//   step       2t            2t+1          2t+2
//   group 0    M(t)          V(t)          M(t+1)
//   group 1    V(t-1)        M(t)          V(t)
//
// K(t) is read in steps 2t and 2t+1 and V(t) in steps 2t+2 and 2t+3; both
// have two LDS stages.  The copies of K(t+1) and V(t) are issued in steps 2t
// and 2t+1 and land by the end of step 2t+1.  Only the end of every odd step
// is a barrier, so the two groups need not change parts at the same moment.
constexpr int kWaves = 8;

template <int D, int BQ, int BK, int MODE, bool F8>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2))) void flash_fwd_bf16_pp(
    FwdParams p) {
  constexpr int G = 256 / BQ;           // query blocks per work item
  constexpr int NWB = BQ / 32;          // waves per member block
  constexpr int NT = kWaves * 64;
  constexpr int ROWB = D * 2;           // bytes of a V row (and of a bf16 K or Q row)
  constexpr int TILEB = kKeyTile * ROWB;
  constexpr int ROWK = F8 ? D : ROWB;   // bytes of a K row
  constexpr int TILEK = kKeyTile * ROWK;
  constexpr int SPB = BK / kKeyTile;    // key tiles per key block (BK keys)
  constexpr int NS = F8 ? D / 64 : D / 16;   // k-steps of S^T
  constexpr int NO = D / 32;            // 32-dim tiles of O^T
  static_assert(!F8 || D == 128, "the fp8 path takes head_dim 128");
  // LDS: K stage 0, K stage 1, V stage 0, V stage 1.
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * TILEK + 2 * TILEB];
  __shared__ unsigned s_bm[fwd_listed(MODE) ? G * kMaxListWords : 1];
  // Union list: key block index in the low 16 bits, member-block bits above.
  __shared__ unsigned s_lt[fwd_listed(MODE) ? kMaxListBlocks : 1];
  __shared__ int s_unit;
  __shared__ int s_nlist;
  __shared__ int s_last;
  __shared__ float s_ksc[F8 ? 2 : 1][64];   // fp8 path: scale of the K tile in each stage

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int h = lane >> 5;
  const int col = lane & 31;
  const int grp = wave >> 2;
  const int member = wave / NWB;
  const float sl2 = p.scale_log2;
  TBS_LDS unsigned char* lds = (TBS_LDS unsigned char*)smem;

  if (p.prof && tid == 0) p.prof[2 * blockIdx.x] = wall_clock64();

  const unsigned char* qg_all = static_cast<const unsigned char*>(p.q);
  const unsigned char* kg_all = static_cast<const unsigned char*>(p.k);
  const unsigned char* vg_all = static_cast<const unsigned char*>(p.v);
  TileLoader<D, kWaves> loader;        // V tiles, and K tiles of the bf16 path
  loader.init(wave, lane);
  TileLoader<F8 ? D / 2 : D, kWaves> loader8;   // K tiles of the fp8 path (D-byte rows)
  if (F8) loader8.init(wave, lane);
  const int krow0 = swap_bits23(col);   // K operand row: bits 2 and 3 swapped

  // Lane byte offsets of the MFMA operands inside a K or V tile.  K (A
  // operand of S^T): row krow0 (+32 for the second half), 16-byte chunk
  // 2s + h of k-step s.  V^T (A operand of O^T, read transposed): for
  // 32-dim tile mo and half-read hf, row 8h + 4hf + (lane&15)/4 and dims
  // 32mo + 16((lane>>4)&1) + 4(lane&3) .. +3; key step kk adds 16 rows.  The
  // chunk swizzle depends on the low four row bits only, which neither the
  // half (+32 rows) nor the key step (+16 rows) changes, so both are
  // immediate offsets.
  //
  // fp8 path: K (A operand of the 32x32x64 product) holds one byte per
  // element; for k-step s lane (h, col) supplies the 32 bytes of dims
  // 64s + 32h .. +31 (chunks 4s + 2h and 4s + 2h + 1 of its row), and Q^T
  // (B operand) the same dims of its query.  A and B share the assignment of
  // dims to (lane half, byte), so the product sums every dim once.
  unsigned koff[F8 ? 2 * NS : NS];
  if (F8) {
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int e = 0; e < 2; ++e)
        koff[2 * s + e] = krow0 * ROWK + (((4 * s + 2 * h + e) ^ chunk_swz<D / 2>(krow0)) * 16);
  } else {
#pragma unroll
    for (int s = 0; s < NS; ++s) koff[s] = krow0 * ROWB + (((2 * s + h) ^ chunk_swz<D>(krow0)) * 16);
  }
  unsigned voff[NO][2];
#pragma unroll
  for (int mo = 0; mo < NO; ++mo)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int ii = lane & 15;
      const int row = 8 * h + 4 * hf + (ii >> 2);
      const int dim = 32 * mo + 16 * ((lane >> 4) & 1) + 4 * (ii & 3);
      voff[mo][hf] = row * ROWB + ((dim >> 3) ^ chunk_swz<D>(row)) * 16 + (dim & 7) * 2;
    }

  // Queue length: the work items, or (split sparse items) the entries the
  // planning kernels wrote, of which this workgroup runs its own range.
  const bool own_range = fwd_listed(MODE) && p.starts != nullptr;
  const int n_queue = own_range ? *p.n_entries : p.U;
  int next = own_range ? p.starts[blockIdx.x] : 0;
  const int last = own_range ? min(p.starts[blockIdx.x + 1], n_queue) : 0;
  for (;;) {
    int qpos;
    if (own_range) {
      // every wave is done with the previous item's LDS before it is reused
      __syncthreads();
      qpos = next++;
      if (qpos >= last) break;
    } else {
      if (tid == 0) s_unit = static_cast<int>(atomicAdd(p.ctrl, 1u));
      __syncthreads();
      qpos = s_unit;
      __syncthreads();
      if (qpos >= n_queue) break;
    }

    GroupInfo<BQ, G, MODE> gi;
    gi.decode(p, qpos);
    const long long head_off = static_cast<long long>(gi.bh) * p.N * ROWB;
    const unsigned char* kg = kg_all + static_cast<long long>(gi.bh) * p.N * ROWK;
    const unsigned char* vg = vg_all + head_off;
    const bool active = member < gi.gsz;
    const int qblk = gi.i0 + member;
    const int q0w = qblk * BQ + (wave % NWB) * 32;
    const int qrow = q0w + col;

    // Tile list of the work item: the union of its blocks' key blocks, with
    // a bit per member block saying whether that block selected it.
    int nt;
    if (fwd_listed(MODE)) {
      const int nwords = (p.nbk + 31) / 32;
      for (int x = tid; x < G * kMaxListWords; x += NT) s_bm[x] = 0u;
      __syncthreads();
      for (int m = 0; m < gi.gsz; ++m) {
        const long long u = static_cast<long long>(gi.bh) * p.nb + gi.i0 + m;
        const int cnt = min(max(p.row_cnt[u], 0), p.nbk);
        const int32_t* lst = p.row_idx + u * p.nbk;
        for (int x = tid; x < cnt; x += NT) {
          const int j = min(max(lst[x], 0), p.nbk - 1);
          atomicOr(&s_bm[m * kMaxListWords + (j >> 5)], 1u << (j & 31));
        }
      }
      __syncthreads();
      if (wave == 0) {
        unsigned wm[G];
        unsigned un = 0u;
#pragma unroll
        for (int m = 0; m < G; ++m) {
          wm[m] = lane < nwords ? s_bm[m * kMaxListWords + lane] : 0u;
          un |= wm[m];
        }
        const int c = __popc(un);
        int incl = c;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int y = __shfl_up(incl, off, 64);
          if (lane >= off) incl += y;
        }
        int pos = incl - c;
        while (un) {
          const int bit = __ffs(un) - 1;
          un &= un - 1;
          unsigned msk = 0u;
#pragma unroll
          for (int m = 0; m < G; ++m) msk |= ((wm[m] >> bit) & 1u) << m;
          s_lt[pos] = static_cast<unsigned>(lane * 32 + bit) | (msk << 16);
          ++pos;
        }
        if (lane == 63) s_nlist = incl;
      }
      __syncthreads();
      const int nl = s_nlist;
      nt = nl * SPB;
      if (SPB > 1 && nl > 0 && static_cast<int>(s_lt[nl - 1] & 0xffffu) == p.nbk - 1) {
        const int tail = p.N - (p.nbk - 1) * BK;
        nt = (nl - 1) * SPB + (tail + kKeyTile - 1) / kKeyTile;
      }
      nt = max(min(nt, gi.te) - gi.tb, 0);   // a part runs union tiles [tb, te)
    } else if (MODE == kDense) {
      nt = (p.N + kKeyTile - 1) / kKeyTile;
    } else {
      nt = min((min(p.N, (gi.i0 + gi.gsz) * BQ) + kKeyTile - 1) / kKeyTile, gi.te) - gi.tb;
    }
    const int tb = gi.tb;   // first key tile of this part (0 unless split)
    // Per-tile facts from the tile's union-list word w (listed modes): its
    // first key and whether this wave's block selected it.  The loop keeps
    // the words of tiles t-1 .. t+3 in scalar registers and reads the next
    // ones from LDS one iteration ahead, so no lookup waits on LDS.
    auto wkey0 = [&](unsigned w, int t) __attribute__((always_inline)) -> int {
      if (fwd_listed(MODE)) return static_cast<int>(w & 0xffffu) * BK + ((tb + t) % SPB) * kKeyTile;
      return (tb + t) * kKeyTile;
    };
    // Under a causal mask a wave skips tiles whose keys all follow its 32
    // query rows (the second tile of a 128-row diagonal block, for the first
    // half of its rows).
    auto wmine = [&](unsigned w, int t) __attribute__((always_inline)) -> bool {
      if (!active) return false;
      if (MODE == kSparseCausal) return ((w >> (16 + member)) & 1u) && wkey0(w, t) < q0w + 32;
      if (MODE == kSparse) return (w >> (16 + member)) & 1u;
      if (MODE == kCausal) return (tb + t) * kKeyTile < q0w + 32;
      return true;
    };
    auto wread = [&](int t) __attribute__((always_inline)) -> unsigned {
      if (fwd_listed(MODE)) return s_lt[min(max(tb + t, 0) / SPB, kMaxListBlocks - 1)];
      return 0u;
    };
    auto wuni = [&](unsigned v) __attribute__((always_inline)) -> unsigned {
      return fwd_listed(MODE) ? __builtin_amdgcn_readfirstlane(v) : 0u;
    };

    // Q^T as B operand: lane (h, col) holds Q[qrow][16s + 8h .. +7] (bf16)
    // or the codes of Q[qrow][64s + 32h .. +31] (fp8), with the row's scale.
    using QFrag = typename std::conditional<F8, i32x8, bf16x8>::type;
    QFrag qf[NS];
    float q_sc = 1.f;
    {
      const long long qtok = static_cast<long long>(gi.bh) * p.N + min(qrow, p.N - 1);
      if constexpr (F8) {
        const unsigned char* qr = qg_all + qtok * D;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const u32x4 lo = *reinterpret_cast<const u32x4*>(qr + 64 * s + 32 * h);
          const u32x4 hi = *reinterpret_cast<const u32x4*>(qr + 64 * s + 32 * h + 16);
          qf[s] = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
        q_sc = p.q_scale[qtok];
      } else {
        const unsigned char* qr = qg_all + qtok * ROWB;
#pragma unroll
        for (int s = 0; s < NS; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qr + (16 * s + 8 * h) * 2);
      }
    }
    // fp8 path: scale of K tile t.  Wave 0 copies it into the tile's LDS
    // stage slot together with the tile (same wait and barrier); M(t) reads
    // it and V(t) uses it.
    float k_sc = 1.f;
    const float* ksc_head = F8 ? p.k_scale + static_cast<long long>(gi.bh) * p.nkt : nullptr;

    f32x16 acc_o[NO];
#pragma unroll
    for (int mo = 0; mo < NO; ++mo)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc_o[mo][e] = 0.f;
    // Running maximum (raw logits), its scaled value (0 while no finite
    // logit has been seen) and the threshold past which it is moved.
    float m_run = -INFINITY;
    float m_b = 0.f;
    float m_thr = -INFINITY;
    float l_run = 0.f;
    const float grow_span = 8.f / sl2;   // weights stay <= 2^8 below it
    f32x16 sacc[2];                      // S^T of the current tile (two 32-key halves)
    bf16x8 pb[2][2];                     // P^T of the previous tile, per half and key step

    // M(t): S(t) from K stage KS, then O^T += V^T P^T of tile t - 1 from V
    // stage VS.  All 32 A-operand fragments (16 of K, 16 of V^T) stream
    // through one ring of TBS_KPF registers, read that many MFMAs ahead.
    auto mpart = [&](auto ks, auto vs, int t, unsigned w_t, unsigned w_tm1) __attribute__((always_inline)) {
      constexpr int KS = decltype(ks)::value;
      constexpr int VS = decltype(vs)::value;
      const bool s_on = t < nt && wmine(w_t, t);
      const bool pv_on = t >= 1 && t - 1 < nt && wmine(w_tm1, t - 1);
      const TBS_LDS unsigned char* lk = lds + KS * TILEK;
      const TBS_LDS unsigned char* lv = lds + 2 * TILEK + VS * TILEB;
      constexpr int NF = 2 * NS;          // fragments of each product
      constexpr int KP = TBS_KPF < NF ? TBS_KPF : NF;
      if constexpr (F8) {
        if (s_on) {
          k_sc = s_ksc[KS][0];
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int e = 0; e < 16; ++e) sacc[mt][e] = 0.f;
          // All NF fragments (two 16-byte reads each) are read up front.
          i32x8 kr[NF];
#pragma unroll
          for (int f = 0; f < NF; ++f) {
            const TBS_LDS unsigned char* row = lk + (f / NS) * 32 * ROWK;
            const u32x4 lo = *(const TBS_LDS u32x4*)(row + koff[2 * (f % NS)]);
            const u32x4 hi = *(const TBS_LDS u32x4*)(row + koff[2 * (f % NS) + 1]);
            kr[f] = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          }
#pragma unroll
          for (int f = 0; f < NF; ++f)
            sacc[f / NS] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kr[f], qf[f % NS], sacc[f / NS], 0, 0, 0, 0,
                                                                           0, 0);
        }
      } else if (s_on) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int e = 0; e < 16; ++e) sacc[mt][e] = 0.f;
        auto kread = [&](int f) __attribute__((always_inline)) -> bf16x8 {
          return *(const TBS_LDS bf16x8*)(lk + (f / NS) * 32 * ROWB + koff[f % NS]);
        };
        bf16x8 kr[KP];
#pragma unroll
        for (int f = 0; f < KP; ++f) kr[f] = kread(f);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const bf16x8 a = kr[f % KP];
          if (f + KP < NF) kr[f % KP] = kread(f + KP);
          sacc[f / NS] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[f % NS], sacc[f / NS], 0, 0, 0);
        }
#if TBS_KPF_PIN
        __builtin_amdgcn_sched_group_barrier(0x100, KP, 0);
#pragma unroll
        for (int f = 0; f < NF - KP; ++f) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, KP, 0);
#endif
      }
      if (pv_on) {
        // Fragment f = kk * NO + mo: key step kk (keys 16kk .. 16kk+15), dims
        // 32mo .. 32mo+31; lane (h, col) supplies P for keys 16kk + 8h + 0..7.
        constexpr int NV = 4 * NO;
        constexpr int VP = TBS_KPF < NV ? TBS_KPF : NV;
        auto vread = [&](int f) __attribute__((always_inline)) -> bf16x8 {
          const int kk = f / NO, mo = f % NO;
          const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((TBS_LDS bf16x4*)(lv + 16 * kk * ROWB + voff[mo][0]));
          const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((TBS_LDS bf16x4*)(lv + 16 * kk * ROWB + voff[mo][1]));
          return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        };
        bf16x8 vr[VP];
#pragma unroll
        for (int f = 0; f < VP; ++f) vr[f] = vread(f);
#pragma unroll
        for (int f = 0; f < NV; ++f) {
          const bf16x8 a = vr[f % VP];
          if (f + VP < NV) vr[f % VP] = vread(f + VP);
          const int kk = f / NO, mo = f % NO;
          acc_o[mo] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kk >> 1][kk & 1], acc_o[mo], 0, 0, 0);
        }
#if TBS_KPF_PIN
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * VP, 1);
#pragma unroll
        for (int f = 0; f < NV - VP; ++f) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, VP, 1);
#endif
      }
    };

    // V(t): online-softmax update with the logits of tile t; leaves P^T(t) in
    // pb.  The whole tile (both halves) shares one reference maximum: its
    // P V product is accumulated only in M(t+1), after the rescale below has
    // been applied to everything accumulated so far.
    auto vpart = [&](int t, unsigned w_t) __attribute__((always_inline)) {
      if (!(t < nt && wmine(w_t, t))) return;
      const int key0 = wkey0(w_t, t);
      const bool need_mask = (key0 + kKeyTile > p.N) || (fwd_causal(MODE) && key0 + kKeyTile - 1 > q0w);
      if (need_mask) {
        // Mask keys past the sequence end (ragged tail) and, if causal, keys
        // after the query.  Lane value e of half mt is key 32mt + 16(e>>3) + 8h + (e&7).
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = key0 + 32 * mt + 16 * (e >> 3) + 8 * h + (e & 7);
            const bool bad = key >= p.N || (fwd_causal(MODE) && key > qrow);
            if (bad) sacc[mt][e] = -INFINITY;
          }
      }
      float m4[4];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        m4[2 * mt] = max3f(max3f(sacc[mt][0], sacc[mt][1], sacc[mt][2]), max3f(sacc[mt][3], sacc[mt][4], sacc[mt][5]),
                           max3f(sacc[mt][6], sacc[mt][7], sacc[mt][8]));
        m4[2 * mt + 1] = max3f(max3f(sacc[mt][9], sacc[mt][10], sacc[mt][11]),
                               max3f(sacc[mt][12], sacc[mt][13], sacc[mt][14]), sacc[mt][15]);
      }
      float mx = max3f(m4[0], m4[1], max3f(m4[2], m4[3], m4[3]));
      const float mo32 = xor32(mx);
      mx = max3f(mx, mo32, mo32);
      // fp8 path: accumulators hold dot products of codes; f = q_sc * k_sc
      // converts them to dot products of the dequantised rows (f > 0, so the
      // maximum carries over).  The floors keep 0 * -inf out of masked keys
      // when a scale is 0, in which case the codes and accumulators are 0.
      float sl2t = sl2;
      if constexpr (F8) {
        constexpr float kMinNormal = 1.17549435e-38f;
        mx *= fmaxf(q_sc * k_sc, kMinNormal);
        sl2t = fmaxf(sl2 * fmaxf(q_sc * k_sc, kMinNormal), kMinNormal);
      }
      // The reference maximum of a row moves only when the tile maximum
      // exceeds it by more than 2^8 in weight (any reference gives the exact
      // result; the bound keeps every weight <= 2^8).  Lanes l and l^32 hold
      // the same row and take the same decision.
      const bool grow = mx > m_thr;
      if (__any(grow)) {
        const float alpha = grow ? fast_exp2((m_run - mx) * sl2) : 1.f;   // 0 on the first move
#pragma unroll
        for (int mo = 0; mo < NO; ++mo)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc_o[mo][e] *= alpha;
        l_run *= alpha;
        if (grow) {
          m_run = mx;
          m_b = mx * sl2;
          m_thr = mx + grow_span;
        }
      }
      // Weights in fp32 (their row sum) and rounded to bf16 (the P V operand).
      float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float pv = fast_exp2(fmaf(sacc[mt][8 * t2 + e], sl2t, -m_b));
            ls[e & 3] += pv;
            pb[mt][t2][e] = static_cast<__bf16>(pv);
          }
      l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
    };

    auto step_barrier = []() __attribute__((always_inline)) {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };

    // The copies of tile t's interval: K(t+1) into K stage (t+1)&1 and V(t)
    // into V stage t&1 (P = t&1); every wave issues its share.
    auto issue_k = [&](auto stage, int key0) __attribute__((always_inline)) {
      constexpr int ST = decltype(stage)::value;
      if constexpr (F8) {
        loader8.issue_one(kg, key0, p.N, lds + ST * TILEK);
        if (wave == 0) copy_scale(ksc_head + key0 / kKeyTile, (TBS_LDS float*)&s_ksc[ST][0]);
      } else {
        loader.issue_one(kg, key0, p.N, lds + ST * TILEK);
      }
    };
    auto issue = [&](auto pp, int t, unsigned w_tp1, unsigned w_t) __attribute__((always_inline)) {
      constexpr int P = decltype(pp)::value;
      if (t + 1 < nt) issue_k(Stage<P ^ 1>{}, wkey0(w_tp1, t + 1));
      if (t < nt) loader.issue_one(vg, wkey0(w_t, t), p.N, lds + 2 * TILEK + P * TILEB);
    };

    // Both groups run the same sequence M(0) V(0) M(1) V(1) ... M(nt), group
    // 1 one part behind group 0.  There is one barrier per tile, where each
    // group has waited for its copies: group 0 after V(t), group 1 after
    // M(t).  Between two barriers group 0 runs M(t) V(t) and group 1 V(t-1)
    // M(t), and every wave issues its share of the copies of K(t+1) and V(t)
    // just before its softmax part (group 1 right after the barrier, group 0
    // after M(t)), so a wave about to issue MFMAs never waits behind a burst
    // of copies.  Those copies land before the barrier that ends the
    // interval, ahead of their first reads (K(t+1) in M(t+1), V(t) in
    // M(t+1)), and the stages they fill were last read in M(t-1) (K(t-1),
    // V(t-2)), before the barrier that opened it.  The loop is unrolled
    // twice so the LDS stages of K(t) and V(t-1) are compile-time constants.
    auto end_m = [&]() __attribute__((always_inline)) {
      if (grp == 1) {
        wait_vmem();
        step_barrier();
      }
    };
    auto end_v = [&]() __attribute__((always_inline)) {
      if (grp == 0) {
        wait_vmem();
        step_barrier();
      }
    };
    if (nt > 0) {
      // Union-list words of tiles t-1 .. t+3 (uniform).
      unsigned w_m1 = 0u, w_0 = wuni(wread(0)), w_1 = wuni(wread(1)), w_2 = wuni(wread(2)), w_3 = wuni(wread(3));
      issue_k(Stage<0>{}, wkey0(w_0, 0));
      wait_vmem();
      step_barrier();
      if (grp == 1) issue(Stage<0>{}, 0, w_1, w_0);
      for (int t = 0;; t += 2) {
        const unsigned pf_a = wread(t + 4), pf_b = wread(t + 5);   // tiles t+4, t+5, for the next iteration
        mpart(Stage<0>{}, Stage<1>{}, t, w_0, w_m1);
        end_m();
        if (t == nt) break;
        if (grp == 0) issue(Stage<0>{}, t, w_1, w_0);
        if (grp == 1) issue(Stage<1>{}, t + 1, w_2, w_1);
        vpart(t, w_0);
        end_v();

        mpart(Stage<1>{}, Stage<0>{}, t + 1, w_1, w_0);
        end_m();
        if (t + 1 == nt) break;
        if (grp == 0) issue(Stage<1>{}, t + 1, w_2, w_1);
        if (grp == 1) issue(Stage<0>{}, t + 2, w_3, w_2);
        vpart(t + 1, w_1);
        end_v();
        w_m1 = w_1;
        w_0 = w_2;
        w_1 = w_3;
        w_2 = wuni(pf_a);
        w_3 = wuni(pf_b);
      }
      if (grp == 0) step_barrier();
    }

    // Epilogue: lane (h, col) holds O[qrow][32mo + 8j + 4h + r] in acc_o[mo][4j + r].
    const float l_tot = l_run + xor32(l_run);
    if ((MODE == kCausal || fwd_listed(MODE)) && gi.nparts > 1) {
      // A part of a split item: its O (unnormalised, relative to its own
      // reference maximum m_run), m_run and row sum go to the part's slot;
      // the item's last part to finish merges every part, in part order.
      // Parts run on any XCD, whose L2 caches are not coherent with each
      // other, so the slots are written through to memory and read past the
      // caches (buffer stores and loads with sc0 sc1), in the lanes' own
      // fragment order (1 KB contiguous per wave and instruction); every store
      // has completed (vmcnt 0, then the workgroup barrier) before the part
      // counter moves, so no fence has to write back a whole L2.
      constexpr int PW = NO * 4 * 256 + 2 * 64;    // floats per wave: O fragments, then m and l per lane
      constexpr int PS = kWaves * PW;              // floats per part
      constexpr int kThrough = 17;                 // sc0 | sc1
      auto frag = [&](long long e, int f) __attribute__((always_inline)) -> int {   // byte offset of fragment f
        return static_cast<int>(((e * PS + wave * PW + f * 256) + lane * 4) * 4);
      };
      auto lanef = [&](long long e, int w) __attribute__((always_inline)) -> int {  // m (w = 0) or l (w = 1)
        return static_cast<int>((e * PS + wave * PW + NO * 4 * 256 + w * 64 + lane) * 4);
      };
      const __amdgpu_buffer_rsrc_t rsrc_t = __builtin_amdgcn_make_buffer_rsrc(p.part_buf, 0, 0x7fffffff, kRsrcWord3);
#pragma unroll
      for (int mo = 0; mo < NO; ++mo)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u32x4 ov;
#pragma unroll
          for (int r = 0; r < 4; ++r) ov[r] = __float_as_uint(acc_o[mo][4 * j + r]);
          __builtin_amdgcn_raw_buffer_store_b128(ov, rsrc_t, frag(qpos, mo * 4 + j), 0, kThrough);
        }
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m_run), rsrc_t, lanef(qpos, 0), 0, kThrough);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(l_tot), rsrc_t, lanef(qpos, 1), 0, kThrough);
      wait_vmem();
      __syncthreads();
      if (tid == 0) s_last = atomicAdd(p.part_cnt + gi.g, 1u) == static_cast<unsigned>(gi.nparts - 1);
      __syncthreads();
      if (s_last) {
        const long long e0 = qpos - gi.part;
        float mm = -INFINITY;
        for (int q = 0; q < gi.nparts; ++q)
          mm = fmaxf(mm, __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc_t, lanef(e0 + q, 0), 0, kThrough)));
        float ll = 0.f;
#pragma unroll
        for (int mo = 0; mo < NO; ++mo)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc_o[mo][e] = 0.f;
        for (int q = 0; q < gi.nparts; ++q) {
          const float mq = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc_t, lanef(e0 + q, 0), 0, kThrough));
          const float lq = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc_t, lanef(e0 + q, 1), 0, kThrough));
          const float f = mq == -INFINITY ? 0.f : fast_exp2((mq - mm) * sl2);
          ll += f * lq;
#pragma unroll
          for (int mo = 0; mo < NO; ++mo)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const u32x4 ov = __builtin_amdgcn_raw_buffer_load_b128(rsrc_t, frag(e0 + q, mo * 4 + j), 0, kThrough);
#pragma unroll
              for (int r = 0; r < 4; ++r) acc_o[mo][4 * j + r] += f * __uint_as_float(ov[r]);
            }
        }
        const float inv = ll > 0.f ? 1.f / ll : 0.f;
        if (active && qrow < p.N) {
          unsigned short* orow = static_cast<unsigned short*>(p.o) +
                                 (static_cast<long long>(gi.bh) * p.N + qrow) * D;
#pragma unroll
          for (int mo = 0; mo < NO; ++mo)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              bf16x4 ov;
#pragma unroll
              for (int r = 0; r < 4; ++r) ov[r] = static_cast<__bf16>(acc_o[mo][4 * j + r] * inv);
              *reinterpret_cast<bf16x4*>(orow + 32 * mo + 8 * j + 4 * h) = ov;
            }
          if (h == 0 && p.lse)
            p.lse[static_cast<long long>(gi.bh) * p.N + qrow] = ll > 0.f ? mm * p.scale + logf(ll) : -INFINITY;
        }
      }
      continue;
    }
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (active && qrow < p.N) {
      unsigned short* orow = static_cast<unsigned short*>(p.o) +
                             (static_cast<long long>(gi.bh) * p.N + qrow) * D;
#pragma unroll
      for (int mo = 0; mo < NO; ++mo)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bf16x4 ov;
#pragma unroll
          for (int r = 0; r < 4; ++r) ov[r] = static_cast<__bf16>(acc_o[mo][4 * j + r] * inv);
          *reinterpret_cast<bf16x4*>(orow + 32 * mo + 8 * j + 4 * h) = ov;
        }
      if (h == 0 && p.lse)
        p.lse[static_cast<long long>(gi.bh) * p.N + qrow] =
            l_tot > 0.f ? m_run * p.scale + logf(l_tot) : -INFINITY;
    }
  }

  if (tid == 0) {
    if (p.prof) p.prof[2 * blockIdx.x + 1] = wall_clock64();
    // The last workgroup to finish leaves the queue counters at zero.
    if (atomicAdd(p.ctrl + 1, 1u) == gridDim.x - 1) {
      atomicExch(p.ctrl, 0u);
      atomicExch(p.ctrl + 1, 0u);
    }
  }
}

// ---------------------------------------------------------------- fp32 ---

template <int D, int BQ, int BK, int MODE>
__global__ __launch_bounds__(BQ * 2) void flash_fwd_f32(FwdParams p) {
  constexpr int NW = BQ / 32;
  constexpr int NT = NW * 64;
  constexpr int LD = D + 1;           // padded row stride (floats)
  constexpr int NQ = D / 2;           // k-steps of S^T (2 dims each)
  constexpr int NO = D / 32;
  __shared__ float ks[kKeyTile * LD];
  __shared__ float vs[kKeyTile * LD];
  __shared__ int s_unit;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int h = lane >> 5;
  const int col = lane & 31;
  const float sl2 = p.scale_log2;
  const float* qa = static_cast<const float*>(p.q);
  const float* ka = static_cast<const float*>(p.k);
  const float* va = static_cast<const float*>(p.v);

  if (p.prof && tid == 0) p.prof[2 * blockIdx.x] = wall_clock64();

  for (;;) {
    if (tid == 0) s_unit = static_cast<int>(atomicAdd(p.ctrl, 1u));
    __syncthreads();
    const int qpos = s_unit;
    __syncthreads();
    if (qpos >= p.U) break;

    UnitInfo<BQ, BK, MODE> ui;
    ui.decode(p, qpos);
    const long long head_off = static_cast<long long>(ui.bh) * p.N * D;
    const int q0w = ui.i * BQ + wave * 32;
    const int qrow = q0w + col;

    float qf[NQ];   // lane (h, col): Q[qrow][2s + h]
    {
      const float* qr = qa + head_off + static_cast<long long>(min(qrow, p.N - 1)) * D;
#pragma unroll
      for (int s = 0; s < NQ; ++s) qf[s] = qr[2 * s + h];
    }
    f32x16 acc_o[NO];
#pragma unroll
    for (int mo = 0; mo < NO; ++mo)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc_o[mo][e] = 0.f;
    float m_run = -INFINITY;
    float l_run = 0.f;

    for (int t = 0; t < ui.ntiles; ++t) {
      const int key0 = ui.key0(p, t);
      __syncthreads();
      // 16-byte global loads (rows are 16-byte aligned: d is a multiple of
      // 4 and the inputs 16-byte aligned), stored to the padded LDS rows
      // element by element.
      for (int x = tid; x < kKeyTile * D / 4; x += NT) {
        const int r = (4 * x) / D, c = (4 * x) % D;
        const long long key = min(key0 + r, p.N - 1);
        const float4 k4 = *reinterpret_cast<const float4*>(ka + head_off + key * D + c);
        const float4 v4 = *reinterpret_cast<const float4*>(va + head_off + key * D + c);
        float* kd = ks + r * LD + c;
        float* vd = vs + r * LD + c;
        kd[0] = k4.x;
        kd[1] = k4.y;
        kd[2] = k4.z;
        kd[3] = k4.w;
        vd[0] = v4.x;
        vd[1] = v4.y;
        vd[2] = v4.z;
        vd[3] = v4.w;
      }
      __syncthreads();

      f32x16 sacc[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[mt][e] = 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int s = 0; s < NQ; ++s)
          sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x2f32(ks[(32 * mt + col) * LD + 2 * s + h], qf[s],
                                                          sacc[mt], 0, 0, 0);
      // Lane value e of tile mt is key 32mt + 8(e>>2) + 4h + (e&3).
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = key0 + 32 * mt + 8 * (e >> 2) + 4 * h + (e & 3);
          if (key >= p.N || (fwd_causal(MODE) && key > qrow)) sacc[mt][e] = -INFINITY;
        }
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sacc[mt][e]);
      mx = fmaxf(mx, xor32(mx));
      const float m_new = fmaxf(m_run, mx);
      if (m_new != m_run) {
        const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2((m_run - m_new) * sl2);
#pragma unroll
        for (int mo = 0; mo < NO; ++mo)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc_o[mo][e] *= alpha;
        l_run *= alpha;
        m_run = m_new;
      }
      const float mb = (m_run == -INFINITY) ? 0.f : m_run * sl2;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float pv = fast_exp2(fmaf(sacc[mt][e], sl2, -mb));
          l_run += pv;
          sacc[mt][e] = pv;
        }
      // O^T += V^T P^T, two keys per step: step (mt, e) pairs slot h with key
      // 32mt + 8(e>>2) + 4h + (e&3), the key this lane's P value belongs to.
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int kl = 32 * mt + 8 * (e >> 2) + 4 * h + (e & 3);
#pragma unroll
          for (int mo = 0; mo < NO; ++mo)
            acc_o[mo] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[kl * LD + 32 * mo + col], sacc[mt][e],
                                                             acc_o[mo], 0, 0, 0);
        }
    }

    const float l_tot = l_run + xor32(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (qrow < p.N) {
      float* orow = static_cast<float*>(p.o) + head_off + static_cast<long long>(qrow) * D;
#pragma unroll
      for (int mo = 0; mo < NO; ++mo)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4 ov;
#pragma unroll
          for (int r = 0; r < 4; ++r) ov[r] = acc_o[mo][4 * j + r] * inv;
          *reinterpret_cast<f32x4*>(orow + 32 * mo + 8 * j + 4 * h) = ov;
        }
      if (h == 0 && p.lse)
        p.lse[static_cast<long long>(ui.bh) * p.N + qrow] =
            l_tot > 0.f ? m_run * p.scale + logf(l_tot) : -INFINITY;
    }
  }

  if (tid == 0) {
    if (p.prof) p.prof[2 * blockIdx.x + 1] = wall_clock64();
    if (atomicAdd(p.ctrl + 1, 1u) == gridDim.x - 1) {
      atomicExch(p.ctrl, 0u);
      atomicExch(p.ctrl + 1, 0u);
    }
  }
}

// ------------------------------------------------------------- dispatch ---

typedef void (*KernelFn)(FwdParams);

// Query blocks per work item: bf16 work items hold 256 query rows (four
// 64-row or two 128-row blocks, one 8-wave workgroup); fp32 inputs use
// single blocks.
constexpr int group_for(int dtype, int block) { return dtype == 0 ? 256 / block : 1; }

// Every variant is instantiated explicitly: referencing a kernel template
// only through a function-pointer table does not always emit its host stub.
#define TBS_INSTANTIATE(D, BQ, BKX, F8)                                                    \
  template __global__ void flash_fwd_bf16_pp<D, BQ, BQ, kSparse, F8>(FwdParams);           \
  template __global__ void flash_fwd_bf16_pp<D, BQ, BQ, kDense, F8>(FwdParams);            \
  template __global__ void flash_fwd_bf16_pp<D, BQ, BQ, kCausal, F8>(FwdParams);           \
  template __global__ void flash_fwd_bf16_pp<D, BQ, BQ, kSparseCausal, F8>(FwdParams);     \
  template __global__ void flash_fwd_bf16_pp<D, BQ, BKX, kSparse, F8>(FwdParams);          \
  template __global__ void flash_fwd_bf16_pp<D, BQ, BKX, kSparseCausal, F8>(FwdParams);
#define TBS_INSTANTIATE_F32(D, BQ, BKX)                                                \
  template __global__ void flash_fwd_f32<D, BQ, BQ, kSparse>(FwdParams);               \
  template __global__ void flash_fwd_f32<D, BQ, BQ, kDense>(FwdParams);                \
  template __global__ void flash_fwd_f32<D, BQ, BQ, kCausal>(FwdParams);               \
  template __global__ void flash_fwd_f32<D, BQ, BQ, kSparseCausal>(FwdParams);         \
  template __global__ void flash_fwd_f32<D, BQ, BKX, kSparse>(FwdParams);              \
  template __global__ void flash_fwd_f32<D, BQ, BKX, kSparseCausal>(FwdParams);
TBS_INSTANTIATE(128, 64, 128, false)
TBS_INSTANTIATE(128, 128, 64, false)
TBS_INSTANTIATE(64, 64, 128, false)
TBS_INSTANTIATE(64, 128, 64, false)
TBS_INSTANTIATE(128, 64, 128, true)
TBS_INSTANTIATE(128, 128, 64, true)
TBS_INSTANTIATE_F32(128, 64, 128)
TBS_INSTANTIATE_F32(128, 128, 64)
TBS_INSTANTIATE_F32(64, 64, 128)
TBS_INSTANTIATE_F32(64, 128, 64)
#undef TBS_INSTANTIATE
#undef TBS_INSTANTIATE_F32

// Key blocks enter only the listed modes; dense and causal take BK = BQ.
// Element kinds: 0 bf16, 1 fp32, 2 bf16 with fp8 Q and K (head_dim 128).
template <int D, int BQ, int BK>
KernelFn pick_mode(int kind, int mode) {
  static const KernelFn bf16_fns[4] = {
      flash_fwd_bf16_pp<D, BQ, BK, kSparse, false>, flash_fwd_bf16_pp<D, BQ, BQ, kDense, false>,
      flash_fwd_bf16_pp<D, BQ, BQ, kCausal, false>, flash_fwd_bf16_pp<D, BQ, BK, kSparseCausal, false>};
  static const KernelFn f32_fns[4] = {flash_fwd_f32<D, BQ, BK, kSparse>, flash_fwd_f32<D, BQ, BQ, kDense>,
                                      flash_fwd_f32<D, BQ, BQ, kCausal>, flash_fwd_f32<D, BQ, BK, kSparseCausal>};
  if (kind == 2) {
    if constexpr (D == 128) {
      static const KernelFn f8_fns[4] = {
          flash_fwd_bf16_pp<D, BQ, BK, kSparse, true>, flash_fwd_bf16_pp<D, BQ, BQ, kDense, true>,
          flash_fwd_bf16_pp<D, BQ, BQ, kCausal, true>, flash_fwd_bf16_pp<D, BQ, BK, kSparseCausal, true>};
      return f8_fns[mode];
    }
    return nullptr;
  }
  return kind == 0 ? bf16_fns[mode] : f32_fns[mode];
}

template <int D>
KernelFn pick_blocks(const Shape& s, int kind, int mode) {
  if (s.block == 128) return s.kb == 128 ? pick_mode<D, 128, 128>(kind, mode) : pick_mode<D, 128, 64>(kind, mode);
  return s.kb == 128 ? pick_mode<D, 64, 128>(kind, mode) : pick_mode<D, 64, 64>(kind, mode);
}

KernelFn pick_kernel(const Shape& s, int mode, bool fp8) {
  const int kind = fp8 ? 2 : s.dtype;
  return s.d == 128 ? pick_blocks<128>(s, kind, mode) : pick_blocks<64>(s, kind, mode);
}

}  // namespace

int group_size(const Shape& s) { return group_for(s.dtype, s.block); }

// Threads per workgroup: 8 waves for bf16 (two groups of four), one wave per
// 32 query rows for fp32.
int fwd_threads(const Shape& s) {
  if (s.dtype == 0) return kWaves * 64;
  return group_size(s) * s.block * 2;
}

long long work_items(const Shape& s) {
  const int G = group_size(s);
  return static_cast<long long>(s.B) * s.H * ((s.nb + G - 1) / G);
}

constexpr int kSplitMinTiles = 16;     // shortest part of a split item
constexpr int kSplitItemsPerCu = 4;    // split below this many items per compute unit
constexpr int kPlanThreads = 1024;     // split sparse problems hold at most this many items
constexpr int kPlanMaxWorkers = 1024;  // and run on at most this many workgroups

namespace {
__global__ __launch_bounds__(256) void zero_u32_kernel(uint32_t* __restrict__ x, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) x[i] = 0u;
}

// Inclusive prefix sum over the kPlanThreads threads of one workgroup (every
// thread calls it; s_w holds one int per wave).  Returns the thread's
// inclusive sum and sets *total to the workgroup's sum.
__device__ __forceinline__ long long plan_scan(long long x, long long* s_w, long long* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  long long incl = x;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const long long y = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += y;
  }
  __syncthreads();
  if (lane == kWave - 1) s_w[wv] = incl;
  __syncthreads();
  long long base = 0, all = 0;
  for (int w = 0; w < kPlanThreads / kWave; ++w) {
    if (w < wv) base += s_w[w];
    all += s_w[w];
  }
  *total = all;
  return base + incl;
}

// Work of a split sparse problem, cut into equal shares (one workgroup, one
// thread per item).  The items' union tiles are laid end to end in item
// order (so the parts, and the results, do not depend on a work list) and
// the sequence is cut into `workers`
// contiguous chunks of C = ceil(total / workers) tiles; worker w runs chunk
// w.  An item crossing a chunk boundary becomes several parts (consecutive
// entries, {item, part, parts, first tile | end tile << 16}); an item without
// tiles is one entry of the chunk its position falls in.  starts[w] is the
// first entry of worker w (starts[workers] = number of entries); the per-item
// part counters are zeroed.
__global__ __launch_bounds__(kPlanThreads) void split_plan_kernel(const int* __restrict__ item_tiles, int items,
                                                                  int workers, int4* __restrict__ entries,
                                                                  int* __restrict__ n_entries,
                                                                  int* __restrict__ starts,
                                                                  uint32_t* __restrict__ part_cnt) {
  __shared__ long long s_w[kPlanThreads / kWave];
  __shared__ int s_chunk[kPlanThreads + kPlanMaxWorkers];
  const int t = threadIdx.x;
  const bool live = t < items;
  const int g = t;
  const long long tiles = live ? item_tiles[g] : 0;
  long long total = 0;
  const long long s0 = plan_scan(tiles, s_w, &total) - tiles;    // first tile of the item in the sequence
  const long long e0 = s0 + tiles;
  const long long C = total > 0 ? (total + workers - 1) / workers : 1;
  const int cfirst = static_cast<int>(min(s0 / C, static_cast<long long>(workers - 1)));
  const int parts = !live ? 0 : tiles == 0 ? 1 : static_cast<int>((e0 - 1) / C - s0 / C + 1);
  long long n = 0;
  const int off0 = static_cast<int>(plan_scan(parts, s_w, &n) - parts);
  for (int q = 0; q < parts; ++q) {
    const long long lo = q == 0 ? s0 : (cfirst + q) * C;
    const long long hi = min(e0, (cfirst + q + 1) * C);
    const int tb = static_cast<int>(lo - s0);
    const int te = static_cast<int>(hi - s0);
    entries[off0 + q] = make_int4(g, q, parts, tb | (te << 16));
    s_chunk[off0 + q] = cfirst + q;
  }
  if (live) part_cnt[g] = 0u;
  __syncthreads();
  // Entries are in chunk order: worker c starts at the first entry whose
  // chunk is c or later.
  const int ne = static_cast<int>(n);
  for (int e = t; e <= ne; e += kPlanThreads) {
    const int lo = e == 0 ? 0 : s_chunk[e - 1] + 1;
    const int hi = e == ne ? workers : s_chunk[e];
    for (int c = lo; c <= hi; ++c) starts[c] = e;
  }
  if (t == 0) n_entries[0] = ne;
}
}  // namespace

// Key tiles of dense causal item row gi (256 query rows).
static long long causal_item_tiles(const Shape& s, int gi) {
  const int G = group_size(s);
  const long long rows = std::min<long long>(s.N, static_cast<long long>(gi + 1) * G * s.block);
  return (rows + kKeyTile - 1) / kKeyTile;
}

int causal_split_tiles(const Shape& s, int mode) {
  if (mode != kCausal || s.dtype != 0 || (s.flags & kFlagNoSplit)) return 0;
  const int cus = device_cu_count();
  if (work_items(s) >= static_cast<long long>(kSplitItemsPerCu) * cus) return 0;
  // Parts of half the mean work per compute unit (at least 16 tiles), so
  // that every compute unit takes about two: only the items longer than that
  // are split.
  const int G = group_size(s);
  const int ng = (s.nb + G - 1) / G;
  long long total = 0;
  for (int gi = 0; gi < ng; ++gi) total += causal_item_tiles(s, gi);
  total *= static_cast<long long>(s.B) * s.H;
  const long long mean = (total + cus - 1) / cus;
  const long long t = std::max<long long>(kSplitMinTiles, (mean + 1) / 2);
  if (causal_item_tiles(s, ng - 1) <= t) return 0;
  return static_cast<int>(t);
}

long long causal_split_entries(const Shape& s, int split_tiles) {
  const int G = group_size(s);
  const int ng = (s.nb + G - 1) / G;
  long long per_head = 0;
  for (int gi = 0; gi < ng; ++gi) per_head += (causal_item_tiles(s, gi) + split_tiles - 1) / split_tiles;
  return per_head * s.B * s.H;
}

bool sparse_split(const Shape& s, int mode) {
  if (!fwd_listed(mode) || s.dtype != 0 || (s.flags & kFlagNoSplit)) return false;
  // entries hold tile indices of an item in 16 bits
  if ((s.N + kKeyTile - 1) / kKeyTile >= (1 << 16)) return false;
  const long long items = work_items(s);
  return items < static_cast<long long>(kSplitItemsPerCu) * device_cu_count() && items <= kPlanThreads &&
         device_cu_count() <= kPlanMaxWorkers / 2;
}

namespace {
size_t align256(size_t n) { return (n + 255) / 256 * 256; }
size_t part_bytes(const Shape& s) {
  return static_cast<size_t>(kWaves) * ((s.d / 32) * 4 * 256 + 2 * 64) * sizeof(float);
}
// Split sparse problems run on at most 2 workgroups per compute unit; each
// chunk boundary cuts at most one item, so there are at most items + workers
// entries.
long long sparse_split_max_workers() { return 2LL * device_cu_count(); }
long long sparse_split_max_entries(const Shape& s) { return work_items(s) + sparse_split_max_workers(); }

// Workspace of a split sparse problem: part counters, entry count, item tile
// counts, workgroup starts, entries, then the parts' partial results.
struct SparseSplitLayout {
  size_t counters, n_entries, item_tiles, starts, entries, parts, total;
};
SparseSplitLayout sparse_split_layout(const Shape& s) {
  SparseSplitLayout l;
  const size_t items = static_cast<size_t>(work_items(s));
  const size_t maxe = static_cast<size_t>(sparse_split_max_entries(s));
  l.counters = 0;
  l.n_entries = align256(items * sizeof(uint32_t));
  l.item_tiles = l.n_entries + 256;
  l.starts = l.item_tiles + align256(items * sizeof(int));
  l.entries = l.starts + align256((static_cast<size_t>(sparse_split_max_workers()) + 1) * sizeof(int));
  l.parts = l.entries + align256(maxe * sizeof(int4));
  l.total = l.parts + maxe * part_bytes(s);
  return l;
}
}  // namespace

size_t causal_split_bytes(const Shape& s, int mode) {
  if (sparse_split(s, mode)) return sparse_split_layout(s).total;
  const int t = causal_split_tiles(s, mode);
  if (t == 0) return 0;
  const size_t counters = align256(static_cast<size_t>(work_items(s)) * sizeof(uint32_t));
  return counters + static_cast<size_t>(causal_split_entries(s, t)) * part_bytes(s);
}

int fwd_workers(const Shape& s, int mode, bool fp8) {
  KernelFn fn = pick_kernel(s, mode, fp8);
  if (!fn) return 0;
  const int threads = fwd_threads(s);
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(fn), threads, 0) !=
          hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  const long long want = static_cast<long long>(device_cu_count()) * per_cu;
  // split sparse problems: the entry count is known on the device only
  if (sparse_split(s, mode)) return static_cast<int>(std::min(want, sparse_split_max_workers()));
  const int split = causal_split_tiles(s, mode);
  const long long items = split ? causal_split_entries(s, split) : work_items(s);
  return static_cast<int>(want < items ? want : items);
}

hipError_t launch_fwd(const Shape& s, int mode, const FwdArgs& a, hipStream_t stream) {
  FwdParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.lse = a.lse;
  p.row_cnt = a.row_cnt;
  p.row_idx = a.row_idx;
  p.work_list = a.work_list;
  p.ctrl = a.ctrl;
  p.prof = reinterpret_cast<unsigned long long*>(a.prof);
  p.q_scale = a.q_scale;
  p.k_scale = a.k_scale;
  p.nkt = (s.N + kKeyTile - 1) / kKeyTile;
  p.BH = s.B * s.H;
  p.N = s.N;
  p.nb = s.nb;
  p.nbk = s.nbk;
  p.G = group_size(s);
  p.ng = (s.nb + p.G - 1) / p.G;
  p.U = static_cast<int>(work_items(s));
  p.scale = static_cast<float>(s.scale);
  p.scale_log2 = static_cast<float>(s.scale * 1.4426950408889634);
  p.split_tiles = causal_split_tiles(s, mode);
  p.part_cnt = nullptr;
  p.part_buf = nullptr;
  p.entries = nullptr;
  p.n_entries = nullptr;
  p.starts = nullptr;
  const int grid = fwd_workers(s, mode, a.fp8);
  if (sparse_split(s, mode)) {
    // Split sparse items: union tile counts per item, then the queue of parts.
    if (!a.split_ws) return hipErrorInvalidValue;
    const SparseSplitLayout l = sparse_split_layout(s);
    auto* ws = static_cast<unsigned char*>(a.split_ws);
    p.part_cnt = reinterpret_cast<uint32_t*>(ws + l.counters);
    int* n_entries = reinterpret_cast<int*>(ws + l.n_entries);
    int* item_tiles = reinterpret_cast<int*>(ws + l.item_tiles);
    int* starts = reinterpret_cast<int*>(ws + l.starts);
    int4* entries = reinterpret_cast<int4*>(ws + l.entries);
    p.part_buf = reinterpret_cast<float*>(ws + l.parts);
    p.entries = entries;
    p.n_entries = n_entries;
    p.starts = starts;
    if (grid < 1 || grid > sparse_split_max_workers()) return hipErrorInvalidValue;
    const int items = static_cast<int>(work_items(s));
    hipError_t e = launch_item_union(s, a.row_cnt, a.row_idx, item_tiles, nullptr, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(split_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, item_tiles, items, grid, entries,
                       n_entries, starts, p.part_cnt);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else if (p.split_tiles > 0) {
    if (!a.split_ws) return hipErrorInvalidValue;
    const long long items = work_items(s);
    p.U = static_cast<int>(causal_split_entries(s, p.split_tiles));
    p.part_cnt = static_cast<uint32_t*>(a.split_ws);
    p.part_buf = reinterpret_cast<float*>(static_cast<unsigned char*>(a.split_ws) +
                                          (static_cast<size_t>(items) * sizeof(uint32_t) + 255) / 256 * 256);
    // The part counters start at zero on every call (the workspace region
    // may hold another call's data).
    const int n = static_cast<int>(items);
    hipLaunchKernelGGL(zero_u32_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, p.part_cnt, n);
    // A failed fill would leave the counters that pick each item's merging
    // part undefined: report it before the attention kernel is enqueued.
    const hipError_t ze = hipGetLastError();
    if (ze != hipSuccess) return ze;
  }
  KernelFn fn = pick_kernel(s, mode, a.fp8);
  if (!fn || grid < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(fwd_threads(s)), 0, stream, p);
  return hipGetLastError();
}

}  // namespace tbs
