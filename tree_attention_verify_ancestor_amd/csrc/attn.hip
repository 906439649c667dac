// tree_verify_attn: tree-masked verification attention over a shared KV prefix.
//
// "Technical analysis of EAGLE-4", section "EAGLE-4 verification trees and the
// harness": a custom mask lets every draft token attend to the shared prefix, its
// ancestors and itself, hiding siblings and other branches, so all branches are
// scored in one target pass ("EAGLE" notes, "3. Verify").  That section and "Why
// speculative decoding" also say why the shape matters: small-batch decoding is
// bound by memory bandwidth, and verifying many draft tokens per pass reuses each
// byte read.  Here every (node, query-head) row of one KV head streams the same
// prefix K/V, so the prefix is read from HBM once per KV head and all rows of the
// group share it -- a dense contraction per byte, done on bf16 MFMA.
//
// bf16 path (gfx950):
//   attn_bf16      grid = (sequence, KV head, row block, key chunk), XCD-aware.  A
//     workgroup owns up to 256 query rows of one KV head (rows = node * G + head in the
//     group) and one chunk of prefix keys; chunk 0 also owns the tree keys.  Stages of
//     64 or 128 keys of K and V go from HBM straight into XOR-swizzled LDS by LDS DMA
//     (global_load_lds), up to four stages in flight.  A wave computes S^T = K Q^T on
//     v_mfma_f32_32x32x16_bf16 (a lane holds 16 keys of one query row), masks the tree
//     stage with the query node's 64-bit ancestor bitset, turns scores into weights
//     2^(s - m) against a fixed per-row reference m (the row maximum of its first
//     visible subtile; an exact two-pass recompute takes over if a weight could pass
//     2^48) and accumulates O^T += V^T P^T, reading V^T with ds_read_b64_tr_b16.
//     Shapes: up to 32 rows, 4 waves split each stage's keys; up to 64 rows, the same
//     with two row tiles per wave; up to 128 rows, 8 waves as 4 row groups x 2 key
//     halves; beyond, 8 waves of one 32-row tile each (or 64-row units of the second
//     shape when such 256-row units are few).  With 8 waves two share each SIMD, so
//     one wave's softmax (vector ALUs) runs beside the other's products.
//     Key-split waves merge their (m, l, O) through LDS.  The output per row and chunk
//     is the final bf16 row when one chunk covers the prefix, else an unnormalised
//     fp32 partial plus (m, l).
//   attn_combine   sixteen lanes per output row, four or eight rows per workgroup,
//     merge the chunk partials (eight chunks in flight at a time), write bf16 out and
//     the natural-log lse.
// fp32 path: attn_f32, one workgroup per output row on the vector ALUs (the
// fp32 workloads are small correctness cases).
#include <math.h>

#include <mutex>

#include <stdint.h>

#include <type_traits>

#include "tv_internal.h"

namespace tv {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttnArgs {
  const __bf16* q;
  const __bf16* k_tree;
  const __bf16* v_tree;
  const __bf16* k_prefix;
  const __bf16* v_prefix;
  const int64_t* offsets;
  const int32_t* n_nodes;
  const uint64_t* anc;
  __bf16* out;
  float* lse;
  int32_t* seq_status;
  float* part_o;      // [unit][chunk][row in unit][D]   unnormalised fp32 partial outputs
  float2* part_ml;    // [unit][chunk][row in unit]      (reference max in log2 units, sum)
  int B, Hq, Hkv, G, n_max, max_prefix;
  int rows_per_wg, chunk_keys, n_chunks, n_rb, total_wgs;
  int rank_pairs;     // ragged batches: (sequence, chunk) pairs ranked by work in-kernel
  float sl2;          // scale * log2(e)
};

struct AttnPlan {
  int waves, wq, wk, qt, rows_per_wg, n_rb, chunk_keys, n_chunks, units, total_wgs, grid;
  size_t part_o_bytes, part_ml_bytes, ws_bytes;
};

constexpr int kMaxChunks = 32;                       // key chunks per work unit (merge width)
constexpr int kMaxRankPairs = 256;                   // (sequence, chunk) pairs ranked in-kernel
constexpr int kRankMinBatch = 8;                     // sequences from which they are ranked
constexpr int kLdsBudget = 128 * 1024;               // the ring of prefix stages
constexpr int kLdsMax = 160 * 1024;                  // LDS of one CU

__host__ __device__ constexpr int stage_keys(int wk) { return 32 * (wk > 2 ? wk : 2); }
__host__ __device__ constexpr int stage_bytes(int D, int wk) { return 2 * stage_keys(wk) * 2 * D; }
__host__ __device__ constexpr int n_buffers(int D, int wk) {
  return kLdsBudget / stage_bytes(D, wk) < 4 ? kLdsBudget / stage_bytes(D, wk) : 4;
}

// Work split of one workgroup: WQ query groups x WK key splits, each wave owning QT
// tiles of 32 rows (rows = node * G + head within the group).  Small row counts use
// four waves that split the keys; from 128 rows on, eight waves of one tile each, two
// per SIMD, so that one wave's softmax runs on the vector ALUs while the other's
// products occupy the matrix core.  When 256-row units are few (one or two sequences
// with many rows), filling the chip would take so many key chunks that the fp32
// partials outweigh the K/V they summarise; those batches use 64-row units instead
// (the row blocks of one KV head re-read its keys from L2) and one workgroup per CU,
// which quarters the chunk count.
static AttnPlan make_plan(int B, int n_max, int Hq, int Hkv, int D, int max_prefix) {
  AttnPlan p{};
  const int G = Hq / Hkv;
  const int R = n_max * G;
  if (R <= 32) { p.wq = 1; p.wk = 4; p.qt = 1; }
  else if (R <= 64) { p.wq = 1; p.wk = 4; p.qt = 2; }
  else if (R <= 128) { p.wq = 4; p.wk = 2; p.qt = 1; }
  else { p.wq = 8; p.wk = 1; p.qt = 1; }
  const bool split_rows = R > 128 && (long)B * Hkv * ((R + 255) / 256) < 32;
  if (split_rows) { p.wq = 1; p.wk = 4; p.qt = 2; }
  p.waves = p.wq * p.wk;
  p.rows_per_wg = 32 * p.qt * p.wq;
  p.n_rb = (R + p.rows_per_wg - 1) / p.rows_per_wg;
  const int kt = stage_keys(p.wk);
  p.units = B * Hkv * p.n_rb;
  // about two workgroups per CU over 256 CUs (one for split rows); every chunk at
  // least two stages
  const long target = split_rows ? 256 : 512;
  long want = (target + p.units - 1) / p.units;
  if (want < 1) want = 1;
  long ck = (max_prefix + want - 1) / want;
  ck = (ck + kt - 1) / kt * kt;
  if (ck < 2 * kt) ck = 2 * kt;
  if (max_prefix > 0 && (max_prefix + ck - 1) / ck > kMaxChunks)
    ck = ((max_prefix + kMaxChunks - 1) / kMaxChunks + kt - 1) / kt * kt;
  p.chunk_keys = (int)ck;
  p.n_chunks = max_prefix > 0 ? (int)((max_prefix + ck - 1) / ck) : 1;
  p.total_wgs = p.units * p.n_chunks;
  p.grid = (p.total_wgs + 7) / 8 * 8 + (kPlanVariant ? 64 : 0);
  const size_t slots = (size_t)p.units * p.n_chunks * p.rows_per_wg;
  p.part_o_bytes = slots * D * 4;
  p.part_ml_bytes = slots * 8;
  p.ws_bytes = p.n_chunks > 1 ? p.part_o_bytes + p.part_ml_bytes : 0;
  return p;
}

template <int D>
__device__ __forceinline__ int swz(int row) {
  // XOR pattern over the 16-byte chunks of a row: conflict-free for 16 consecutive rows
  // reading one chunk column (K operand) and spread for the transpose reads of V.
  if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return ((row & 3) << 1) | ((row >> 2) & 1);
}

// s_waitcnt vmcnt(N) with the other counters unconstrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that does not drain outstanding LDS DMA (the caller waits for
// exactly the stages it needs with wait_vmcnt first); a compiler memory barrier too.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// One 16-byte global -> LDS DMA per lane: lane i's bytes land at lds_base + 16 * i.
// Issued as inline asm so that the compiler keeps no alias bookkeeping for it (it
// would otherwise drain every outstanding DMA before each LDS read).  The caller
// orders it: wait_vmcnt + lds_barrier before reading the data, and a barrier before
// reusing a buffer.  M0 carries the LDS base; nothing else in these kernels uses M0.
__device__ __forceinline__ void lds_dma16(const void* gsrc, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(gsrc), "s"(lds_base) : "m0");
}
// The same with a uniform 64-bit base in SGPRs and a 32-bit per-lane byte offset.
__device__ __forceinline__ void lds_dma16_s(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds_base) : "m0");
}

// Maximum of a value over the two lanes l and l ^ 32 (which hold the two key halves of
// one query row), in every lane.
__device__ __forceinline__ float max_halves(float v) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}
__device__ __forceinline__ float sum_halves(float v) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

template <int N>
using ic = std::integral_constant<int, N>;

enum StageMode { kFull = 0, kMasked = 1 };

// Key chunks per workgroup for a sequence with R rows per KV head.  The plan is sized by
// n_max: where a tree fills every row block of the eight-wave shape (256 rows a block),
// a workgroup takes two adjacent chunks as one pass, so that such a call runs as many
// workgroups as one with half the rows (about one per CU) instead of a second round;
// smaller trees leave the row blocks past their rows idle and keep one chunk each.  The
// attention kernel, its ranking of pairs and the merge all take the span from here.
__device__ __forceinline__ int chunk_span(const AttnArgs& a, int R) {
  return a.rows_per_wg == 256 && a.n_rb >= 2 && R > (a.n_rb - 1) * a.rows_per_wg ? 2 : 1;
}

template <int D, int WQ, int WK, int QT>
__global__ __launch_bounds__(64 * WQ * WK) void attn_bf16(AttnArgs a) {
  constexpr int W = WQ * WK;
  constexpr int NT = 64 * W;
  static_assert(W == 4 || W == 8, "four or eight waves per workgroup");
  constexpr int KT = stage_keys(WK);            // keys per stage
  constexpr int NS = KT / 32;                   // 32-key subtiles per stage
  constexpr int NSW = NS / WK;                  // subtiles per wave and stage
  constexpr int ROWB = 2 * D;                   // LDS bytes per K/V row (bf16, swizzled)
  constexpr int TILEB = KT * ROWB;              // K (or V) bytes per stage
  constexpr int STAGEB = 2 * TILEB;
  constexpr int NBUF = n_buffers(D, WK);
  constexpr int DMA = STAGEB / (NT * 16);             // 16-byte LDS DMAs per thread per stage
  constexpr int ROWS_PER_KB = 1024 / ROWB;
  constexpr int KBLKS = TILEB / 1024;
  constexpr int DS = D / 16;
  constexpr int DT = D / 32;
  static_assert(DMA * NT * 16 == STAGEB, "stage must split into 1 KB DMA blocks");
  static_assert(NBUF >= 2 && NBUF <= 4, "two to four stage buffers");
  static_assert(NBUF * DMA < 64, "the DMAs in flight fit the vmcnt counter");
  static_assert(NSW * WK == NS && NSW >= 1, "whole subtiles per wave");
  static_assert(QT == 1 || QT == 2, "one or two row tiles per wave");

  // LDS: the ring of NBUF prefix stages, then, with a ring of two, an area of its own
  // for the tree stage's K and V (at most 64 rows each), so that the tree stage does
  // not hold back a prefix stage.  All of it is reused at the end for the rows of all
  // waves (fp32, padded).
  constexpr int TREE_TILEB = TV_MAX_NODES * ROWB;
  constexpr int RING = NBUF * STAGEB;
  constexpr bool SEP_TREE = NBUF == 2 && RING + 2 * TREE_TILEB <= kLdsMax;
  constexpr int OSTR = D + 4;
  constexpr int OB_FLOATS = W * QT * 32 * OSTR;
  constexpr int OUT_BYTES = OB_FLOATS * 4 + W * QT * 32 * 8;
  constexpr int STAGE_AREA = RING + (SEP_TREE ? 2 * TREE_TILEB : 0);
  constexpr int SMEM = STAGE_AREA > OUT_BYTES ? STAGE_AREA : OUT_BYTES;
  static_assert(SMEM <= kLdsMax, "LDS of one workgroup");
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];

  // ---- work item.  The order puts KV heads fastest, then row blocks, then chunks:
  // workgroups running together read the same token range of every head, i.e. whole
  // contiguous prefix rows, and the row blocks of one (head, chunk) stay close in time.
  // The blockIdx -> item map is XCD-aware: consecutive items land on one XCD (and L2).
  // A ragged batch (prefix lengths or node counts that differ) instead takes its
  // (sequence, chunk) pairs in order of their work, keys times row tiles, largest
  // first: the longest items are dispatched first and the short ones fill in at the
  // end.  Every workgroup ranks the pairs itself (the stage ring is not in use yet and
  // holds the ranking) and takes the pair at its place; consecutive workgroups take
  // the KV heads and row blocks of one pair.
  const int x = blockIdx.x;
  int kvh, rb, chunk, b;
  bool by_work = false;
  if (a.rank_pairs) {
    int* s_work = (int*)smem;
    volatile int* s_pick = s_work + kMaxRankPairs;
    volatile int* s_ragged = s_pick + 1;
    const int per = a.Hkv * a.n_rb;
    const int P = a.B * a.n_chunks;
    if (threadIdx.x == 0) *s_ragged = 0;
    __syncthreads();
    const int n0 = a.n_nodes[0];
    const int64_t L0 = a.offsets[0] < 0 ? -1 : a.offsets[1] - a.offsets[0];
    for (int j = threadIdx.x; j < P; j += blockDim.x) {
      const int bj = j / a.n_chunks, cj = j % a.n_chunks;
      const int nj = a.n_nodes[bj];
      const int64_t Lj = a.offsets[bj] < 0 ? -1 : a.offsets[bj + 1] - a.offsets[bj];
      if (nj != n0 || Lj != L0) *s_ragged = 1;
      int w = 0;
      if (nj >= 1 && nj <= a.n_max && Lj >= 0 && Lj <= a.max_prefix) {
        const int sj = chunk_span(a, nj * a.G);
        const int64_t lo = (int64_t)cj * a.chunk_keys;
        const int keys = (int)max((int64_t)0, min((int64_t)sj * a.chunk_keys, Lj - lo)) + (cj == 0 ? nj : 0);
        w = cj % sj == 0 && (cj == 0 || lo < Lj) ? keys * ((nj * a.G + 31) / 32) : 0;
      }
      s_work[j] = w;
    }
    __syncthreads();
    by_work = kPlanVariant || *s_ragged != 0;
    if (by_work) {
      const int place = x / per;
      for (int j = threadIdx.x; j < P; j += blockDim.x) {
        const int wj = s_work[j];
        int r = 0;
        for (int i = 0; i < P; ++i)                  // branch-free: no exec-mask jumps
          r += (int)(s_work[i] > wj) | ((int)(s_work[i] == wj) & (int)(i < j));
        if (r == place) *s_pick = j;
      }
      __syncthreads();
      if (place >= P) return;                        // padding of the grid: no item
      const int pick = *s_pick;
      b = pick / a.n_chunks;
      chunk = pick % a.n_chunks;
      kvh = (x % per) % a.Hkv;
      rb = (x % per) / a.Hkv;
    }
    __syncthreads();                                 // every wave has read the ranking
  }
  if (!by_work) {
    const int logical = (x % 8) * (gridDim.x / 8) + x / 8;
    if (logical >= a.total_wgs) return;              // padding of the grid: no item
    int t = logical;
    kvh = t % a.Hkv; t /= a.Hkv;
    rb = t % a.n_rb; t /= a.n_rb;
    chunk = t % a.n_chunks;
    b = t / a.n_chunks;
  }
  // the item is uniform over the workgroup (the ranked pick comes through LDS): keep it,
  // and everything derived from it, in scalar registers so that branches on it are
  // plain jumps
  b = __builtin_amdgcn_readfirstlane(b);
  chunk = __builtin_amdgcn_readfirstlane(chunk);
  kvh = __builtin_amdgcn_readfirstlane(kvh);
  rb = __builtin_amdgcn_readfirstlane(rb);
  const int unit = (b * a.Hkv + kvh) * a.n_rb + rb;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wq = wave / WK;
  const int wk = wave % WK;
  const int g = lane >> 5;
  const int ql = lane & 31;

  const int n = a.n_nodes[b];
  const int64_t off = a.offsets[b];
  const int64_t Lw = a.offsets[b + 1] - off;
  const bool n_ok = n >= 1 && n <= a.n_max;
  const bool seq_ok = n_ok && off >= 0 && Lw >= 0 && Lw <= a.max_prefix;
  const int L = seq_ok ? (int)Lw : 0;
  const int G = a.G;
  const int R = n_ok ? n * G : 0;
  const int row0 = rb * a.rows_per_wg;
  const int span = chunk_span(a, R);
  const int c0 = chunk * a.chunk_keys;
  const int c1 = min(L, c0 + span * a.chunk_keys);
  const bool active = seq_ok && row0 < R && chunk % span == 0 && (chunk == 0 || c0 < L);

  if (active) {
    const int has_tree = chunk == 0 ? 1 : 0;
    const int n_full = c1 > c0 ? (c1 - c0) / KT : 0;           // prefix stages without a mask
    const int nst = (c1 > c0 ? (c1 - c0 + KT - 1) / KT : 0) + has_tree;

    // queries of this wave: Q^T operands and node ancestor bitsets of its QT tiles.  A
    // wave whose rows all lie beyond the tree's rows still queues its DMA share and
    // joins every barrier, but computes nothing.
    const int rw0 = row0 + wq * 32 * QT;
    const bool wave_live = rw0 < R;
    const bool live1 = rw0 + 32 < R;                 // the wave's second tile has rows
    int rho[QT], qnode[QT], qhead[QT];
    bf16x8 qop[QT][DS];
    uint64_t qanc[QT];
#pragma unroll
    for (int u = 0; u < QT; ++u) {
      rho[u] = rw0 + 32 * u + ql;
      const int rc = rho[u] < R ? rho[u] : R - 1;
      qnode[u] = rc / G;
      qhead[u] = kvh * G + rc % G;
      const __bf16* qp = a.q + (((size_t)b * a.n_max + qnode[u]) * a.Hq + qhead[u]) * D + 8 * g;
#pragma unroll
      for (int s = 0; s < DS; ++s) qop[u][s] = *(const bf16x8*)(qp + 16 * s);
      qanc[u] = a.anc[(size_t)b * a.n_max + qnode[u]];
    }

    f32x16 o[QT][DT];
    float m_run[QT], l_run[QT];
#pragma unroll
    for (int u = 0; u < QT; ++u) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[u][dt] = f32x16{};
      m_run[u] = -INFINITY;
      l_run[u] = 0.f;
    }

    const size_t kv_row = (size_t)a.Hkv * D;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;
    static_assert(KBLKS == (W / 2) * DMA, "half the waves cover one tile");
    // queue the DMA of stage st into its buffer.  Waves 0..W/2-1 fetch K rows, the
    // others V rows; each wave covers DMA consecutive 1 KB blocks (ROWS_PER_KB rows
    // each) and each lane one 16-byte chunk, placed at its XOR-swizzled position.
    const bool dma_v = wave >= W / 2;
    const int dma_blk0 = (wave % (W / 2)) * DMA;
    const __bf16* tree_base = (dma_v ? a.v_tree : a.k_tree) + ((size_t)b * a.n_max * a.Hkv + kvh) * D;
    const __bf16* pref_base = (dma_v ? a.v_prefix : a.k_prefix) + (size_t)off * kv_row + (size_t)kvh * D;
    const int dma_pos = lane % (ROWB / 16);
    const int dma_row = lane / (ROWB / 16);
    auto stage_kbase = [&](int st) { return (has_tree && st == 0) ? 0 : c0 + (st - has_tree) * KT; };
    // LDS byte offsets of stage st's K tile and of its V tile from the K tile: the tree
    // stage has its own area when it fits, the prefix stages cycle through the ring,
    // whose K tiles fill its first half and V tiles its second.  The first prefix stage
    // takes slot 0 (a tree stage in the ring the last slot), so that a loop over the
    // prefix stages knows each stage's slot at compile time when unrolled by NBUF.
    const int extra = SEP_TREE && has_tree ? 1 : 0;       // stages outside the ring
    const int rot = has_tree ? 1 : 0;
    auto k_tile = [&](int st) {
      return (SEP_TREE && has_tree && st == 0) ? RING : ((st - rot + NBUF) % NBUF) * TILEB;
    };
    auto v_tile = [&](int st) { return (SEP_TREE && has_tree && st == 0) ? TREE_TILEB : NBUF * TILEB; };
    // per-lane byte offset of this thread's first DMA within a full prefix stage (the
    // stage's first key row is added to the uniform base).  DMA i reads ROWS_PER_KB * i
    // rows further on (a uniform term) at a chunk whose index differs by XOR with i & 3
    // for D = 128 (the swizzle of the row) and not at all for D = 64.
    static_assert(DMA % 4 == 0 || D == 64, "the chunk XOR repeats every four DMAs");
    const uint32_t dma_off0 = (uint32_t)(((size_t)(dma_blk0 * ROWS_PER_KB + dma_row) * kv_row +
                                          (dma_pos ^ swz<D>(dma_blk0 * ROWS_PER_KB + dma_row)) * 8) * 2);
    auto issue = [&](int st) __attribute__((always_inline)) {
      const bool tree = has_tree && st == 0;
      const int kbase = stage_kbase(st);
      const int kend = tree ? n : c1;
      // uniform values, made explicitly scalar for the asm operands
      const uint32_t dst0 = __builtin_amdgcn_readfirstlane(
          lds0 + k_tile(st) + (dma_v ? v_tile(st) : 0) + dma_blk0 * 1024);
      if (!tree && kbase + KT <= kend) {
        const uintptr_t sbv = (uintptr_t)(pref_base + (size_t)kbase * kv_row);
        const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)sbv);
        const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(sbv >> 32));
#pragma unroll
        for (int i = 0; i < DMA; ++i) {
          const uint64_t sbi = (((uint64_t)hi << 32) | lo) + (uint64_t)i * ROWS_PER_KB * kv_row * 2;
          const uint32_t ilo = __builtin_amdgcn_readfirstlane((uint32_t)sbi);
          const uint32_t ihi = __builtin_amdgcn_readfirstlane((uint32_t)(sbi >> 32));
          lds_dma16_s((const void*)(((uint64_t)ihi << 32) | ilo),
                      D == 128 ? dma_off0 ^ ((i & 3) << 4) : dma_off0, dst0 + i * 1024);
        }
        return;
      }
      const __bf16* base = tree ? tree_base : pref_base;
      const size_t rstride = tree ? (size_t)a.Hkv * D : kv_row;
      const uintptr_t sbv = (uintptr_t)(base + (size_t)kbase * rstride);
      const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)sbv);
      const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(sbv >> 32));
      const void* sb = (const void*)(((uint64_t)hi << 32) | lo);
      // the tree stage only fetches the 32-row subtiles that hold nodes; the others are
      // never read (their subtiles are skipped).  Rows past the stage's last key repeat
      // that key (their weights are zero).
      const int rows_needed = tree ? (n + 31) / 32 * 32 : KT;
      const int last = kend - 1 - kbase;
#pragma unroll
      for (int i = 0; i < DMA; ++i) {
        if ((dma_blk0 + i) * ROWS_PER_KB >= rows_needed) continue;      // wave-uniform
        const int lrow = (dma_blk0 + i) * ROWS_PER_KB + dma_row;
        const int chk = dma_pos ^ swz<D>(lrow);
        lds_dma16_s(sb, (uint32_t)(min(lrow, last) * rstride * 2) + chk * 16, dst0 + i * 1024);
      }
    };
    // Start of stage st: its data has landed (this wave's DMAs by vmcnt, the others'
    // by the barrier), and every wave has finished its LDS reads of stage st-1; a
    // prefix stage's buffer is then refilled with stage st+NBUF-1.  The DMAs complete
    // in issue order, so stage st has landed once at most the DMAs of the stages issued
    // after it are outstanding: stages up to extra+NBUF-1 at the start, then one more
    // per refill.  (The tree stage may issue fewer DMAs; it is always the oldest.)
    auto begin_stage = [&](int st) __attribute__((always_inline)) {
      const int ahead = min(nst - 1, max(extra + NBUF - 1, st + NBUF - 2)) - st;
      if (ahead <= 0) wait_vmcnt<0>();
      else if (ahead == 1) wait_vmcnt<DMA>();
      else if (ahead == 2) wait_vmcnt<2 * DMA>();
      else if (ahead == 3) wait_vmcnt<3 * DMA>();
      else wait_vmcnt<NBUF * DMA>();                       // the tree stage, NBUF = 4
      __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): this wave's LDS reads are done
      lds_barrier();
      if (st - extra >= 1 && st + NBUF - 1 < nst) issue(st + NBUF - 1);
    };

    // lane-constant LDS byte offsets of the first K and V^T operand reads.  The others
    // differ from them by XOR in the chunk bits of the row (the swizzle only depends on
    // the low four row bits), and every subtile and buffer base is a multiple of the
    // row size, so one register per operand serves all reads:
    //   K operand s:       (base + koff0) ^ (s << 5)
    //   V^T operand dt:    A = (base + voff0) ^ (dt << 6) for rows 0-7 of the 16-key
    //                      step, (A ^ VHI) + 8 rows for rows 8-15
    const uint32_t koff0 = ql * ROWB + ((g ^ swz<D>(ql)) << 4);
    uint32_t voff0;
    {
      const int s16 = lane & 15;
      const int rlo = 4 * g + (s16 >> 2);
      const int chk = 2 * ((lane >> 4) & 1) + ((s16 & 3) >> 1);
      voff0 = rlo * ROWB + ((chk ^ swz<D>(rlo)) << 4) + ((s16 & 1) << 3);
    }
    constexpr uint32_t VHI = D == 128 ? 32 : 0;   // swz(row + 8) ^ swz(row), in bytes

    // ---- building blocks on one 32-key subtile.  sub is its index within the stage,
    // kb / vb the stage's K and V tiles in LDS.
    struct KOps { bf16x8 v[DS]; };
    struct VOps { bf16x8 v[2][DT]; };
    typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    auto lds_addr = [](const char* p) {
      return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
    };
    auto load_k = [&](const char* kb, int sub) {
      KOps k;
      const uint32_t a0 = lds_addr(kb) + sub * 32 * ROWB + koff0;
#pragma unroll
      for (int s = 0; s < DS; ++s) k.v[s] = *(lds_bf16x8*)(uintptr_t)(a0 ^ (s << 5));
      return k;
    };
    auto load_v = [&](const char* vb, int sub) {
      VOps v;
      const uint32_t a0 = lds_addr(vb) + sub * 32 * ROWB + voff0;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const uint32_t lo_a = (a0 ^ (dt << 6)) + ks * 16 * ROWB;
          const uint32_t hi_a = ((a0 ^ (dt << 6)) ^ VHI) + 8 * ROWB + ks * 16 * ROWB;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)lo_a);
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)hi_a);
          const s16x4 both[2] = {lo, hi};
          v.v[ks][dt] = *(const bf16x8*)both;
        }
      return v;
    };
    // the same operands straight from global memory (the slow path): key kbase + k of
    // the stage; keys at or past kend are clamped (their weights are zero)
    auto key_row = [&](bool tree, int key, bool is_v) {
      const __bf16* base = tree ? (is_v ? a.v_tree : a.k_tree) + ((size_t)b * a.n_max * a.Hkv + kvh) * D
                                : (is_v ? a.v_prefix : a.k_prefix) + (size_t)off * kv_row + (size_t)kvh * D;
      return base + (size_t)key * (tree ? (size_t)a.Hkv * D : kv_row);
    };
    auto load_k_global = [&](bool tree, int k0, int kend) {
      KOps k;
      const __bf16* row = key_row(tree, min(k0 + ql, kend - 1), false) + 8 * g;
#pragma unroll
      for (int s = 0; s < DS; ++s) k.v[s] = *(const bf16x8*)(row + 16 * s);
      return k;
    };
    auto load_v_global = [&](bool tree, int k0, int kend) {
      // A operand lane (d, g), element e: V[key 16 ks + 8 (e >> 2) + 4 g + (e & 3)][d],
      // the key order of the softmax weights in the B operand
      VOps v;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int key = min(k0 + 16 * ks + 8 * (e >> 2) + 4 * g + (e & 3), kend - 1);
            v.v[ks][dt][e] = key_row(tree, key, true)[32 * dt + ql];
          }
      return v;
    };
    // S^T = K Q^T for row tile U: a lane holds 16 keys of query row ql
    auto qk = [&](auto u_tag, const KOps& k) {
      constexpr int U = decltype(u_tag)::value;
      f32x16 s = f32x16{};
#pragma unroll
      for (int i = 0; i < DS; ++i) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k.v[i], qop[U][i], s, 0, 0, 0);
      return s;
    };
    // O^T += V^T P^T for row tile U, with P^T the softmax weights as the B operand
    auto pv = [&](auto u_tag, const VOps& v, const bf16x8 (&pb)[2]) {
      constexpr int U = decltype(u_tag)::value;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          o[U][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v.v[ks][dt], pb[ks], o[U][dt], 0, 0, 0);
    };
    // masking of a stage that is not full: keys >= kend and, through amask (the
    // query's ancestor bitset in the tree stage, all ones otherwise), keys off the
    // query's root path are -inf
    // A lane's keys are key0 + 8 (r >> 2) + (r & 3), all within 28 of key0 (and below 64
    // in the tree stage, where key0 < 64 too), so one 32-bit mask holds them all.
    auto apply_mask = [&](f32x16& s, int key0, int kend, uint64_t amask) {
      const int lim = kend - key0;
      const uint32_t below = lim >= 32 ? ~0u : (lim <= 0 ? 0u : (1u << lim) - 1u);
      const uint32_t vis = (uint32_t)(amask >> (key0 & 63)) & below;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        s[r] = (vis & (1u << (8 * (r >> 2) + (r & 3)))) ? s[r] : -INFINITY;
    };
    auto lane_max = [&](const f32x16& s) {
      float m = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) m = fmaxf(m, s[r]);
      return m * a.sl2;
    };
    // Fixed reference (fast path): the first subtile with a visible key sets m_run to
    // that subtile's row maximum (both key halves of a row agree through the lane
    // swap); after that m_run never moves and O is touched by MFMAs only.  Weights
    // 2^(s - m_run) stay exact in bf16/fp32 up to 2^48 and cannot overflow the
    // sums; a score beyond that sets `over`, and the wave recomputes this chunk on the
    // slow path.
    constexpr float kRefSpan = 48.f;
    auto reference = [&](auto u_tag, const f32x16& s) {
      constexpr int U = decltype(u_tag)::value;
      const float first = max_halves(lane_max(s));
      m_run[U] = m_run[U] == -INFINITY ? first : m_run[U];
    };
    // weights 2^(s*scale*log2e - m_run) as bf16 B operands; their sum (of the rounded
    // weights, the ones the products use) is added to l and returned
    auto weights = [&](auto u_tag, const f32x16& s, bf16x8 (&pb)[2]) {
      constexpr int U = decltype(u_tag)::value;
      const float msub = m_run[U] == -INFINITY ? 0.f : m_run[U];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pb[0][e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[e], a.sl2, -msub));
        pb[1][e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[8 + e], a.sl2, -msub));
      }
      typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
      const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        psum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[0][2 * e], pb[0][2 * e + 1]}, one2, psum, false);
        psum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pb[1][2 * e], pb[1][2 * e + 1]}, one2, psum, false);
      }
      l_run[U] += psum;
      return psum;
    };
    // the fast path's overflow guard: a lane's 16 weights sum past 2^48 (or to inf or
    // NaN) whenever some weight may have left the range the fixed reference carries
    auto too_big = [&](float psum) { return !(psum <= 0x1p48f); };

    // one subtile from LDS, every row tile in turn (tree and tail stages, and the
    // one-tile layout)
    bool over = false;
    bool ref_open = true;        // some row of the wave has no reference yet (wave-uniform)
    auto subtile_fast = [&](auto mode_tag, auto ntile_tag, const char* kb, const char* vb, int sub,
                            int kbase, int kend, bool tree) {
      constexpr int MODE = decltype(mode_tag)::value;
      constexpr int NT = decltype(ntile_tag)::value;
      // eight waves: subtiles strictly one after another (the other wave of the SIMD
      // provides the overlap), which keeps the live registers within 256
      if constexpr (W == 8) __builtin_amdgcn_sched_barrier(0);
      const KOps k = load_k(kb, sub);
      f32x16 s[NT];
      // with two waves per SIMD, a wave raises its priority for its products so that
      // they issue back to back while the other wave works on the vector ALUs
      if constexpr (W == 8) __builtin_amdgcn_s_setprio(1);
      s[0] = qk(ic<0>{}, k);
      if constexpr (NT > 1) s[1] = qk(ic<1>{}, k);
      if constexpr (W == 8) __builtin_amdgcn_s_setprio(0);
      // with two waves per SIMD the other wave hides the V^T read latency: read V^T
      // only after the products that consume K, so K and V^T never occupy registers
      // together
      if constexpr (W == 8) __builtin_amdgcn_sched_barrier(0);
      const VOps v = load_v(vb, sub);
      const int key0 = kbase + sub * 32 + 4 * g;
      bf16x8 pb[NT][2];
      if constexpr (MODE == kMasked) apply_mask(s[0], key0, kend, tree ? qanc[0] : ~0ull);
      if constexpr (NT > 1)
        if constexpr (MODE == kMasked) apply_mask(s[1], key0, kend, tree ? qanc[1] : ~0ull);
      if (ref_open) {
        reference(ic<0>{}, s[0]);
        bool open = m_run[0] == -INFINITY;
        if constexpr (NT > 1) {
          reference(ic<1>{}, s[1]);
          open |= m_run[1] == -INFINITY;
        }
        ref_open = __ballot(open) != 0;
      }
      over |= too_big(weights(ic<0>{}, s[0], pb[0]));
      if constexpr (NT > 1) over |= too_big(weights(ic<1>{}, s[1], pb[1]));
      if constexpr (W == 8) __builtin_amdgcn_s_setprio(1);
      pv(ic<0>{}, v, pb[0]);
      if constexpr (NT > 1) pv(ic<1>{}, v, pb[1]);
      if constexpr (W == 8) __builtin_amdgcn_s_setprio(0);
    };
    auto stage_fast = [&](int st) {
      const char* kb = smem + k_tile(st);
      const char* vb = kb + v_tile(st);
      const bool tree = has_tree && st == 0;
      const int kbase = stage_kbase(st);
      const int kend = tree ? n : c1;
      const bool full = !tree && kbase + KT <= kend;
#pragma unroll
      for (int j = 0; j < NSW; ++j) {
        const int sub = wk + j * WK;
        if (kbase + sub * 32 >= kend) continue;                 // wave-uniform
        // a second tile whose rows all lie past the tree's rows is skipped
        if (QT > 1 && live1) {
          if (full) subtile_fast(ic<kFull>{}, ic<QT>{}, kb, vb, sub, kbase, kend, tree);
          else subtile_fast(ic<kMasked>{}, ic<QT>{}, kb, vb, sub, kbase, kend, tree);
        } else {
          if (full) subtile_fast(ic<kFull>{}, ic<1>{}, kb, vb, sub, kbase, kend, tree);
          else subtile_fast(ic<kMasked>{}, ic<1>{}, kb, vb, sub, kbase, kend, tree);
        }
      }
    };

    // a full prefix stage: no mask, every subtile present, a fixed number of row tiles
    auto stage_full = [&](auto ntile_tag, int st) {
      const char* kb = smem + k_tile(st);
      const char* vb = kb + v_tile(st);
      const int kbase = stage_kbase(st);
#pragma unroll
      for (int j = 0; j < NSW; ++j)
        subtile_fast(ic<kFull>{}, ntile_tag, kb, vb, wk + j * WK, kbase, c1, false);
    };

    // ---- pipeline over the stages: the tree stage and up to NBUF prefix stages in
    // flight.  Q and the bitsets were loaded before the first stage's DMAs; one wait
    // for all of them (stage 0 is needed first in any case) also tells the compiler
    // that its loads are done -- it counts only its own loads and would otherwise wait
    // for every outstanding DMA before each use of Q inside the loop.  Then the other
    // stages are queued.
    if (nst > 0) issue(0);
    wait_vmcnt<0>();
#pragma unroll
    for (int p = 1; p < NBUF + 1; ++p)
      if (p < nst && p < NBUF + extra) issue(p);
    if constexpr (WQ == 8 && WK == 1 && QT == 1) {
      // ---- eight waves of one row tile: software-pipelined over 32-key subtiles.
      // While a wave's softmax of subtile s (with its row sums) runs on the vector ALUs,
      // the products of subtile s+1 (S^T = K Q^T) run on the matrix core; then O^T +=
      // V^T P^T of subtile s, and K of subtile s+2 is read from LDS while those products
      // run.  Both waves of a SIMD issue the same mixed stream, so the matrix core is fed
      // from two waves; a wave's LDS reads hold up its vector instructions, and together
      // they, not the products, set the pace.
      //
      // Stage x+1 is opened (its DMAs waited for, then one barrier) when stage x starts,
      // before any read of its K.  At that barrier every wave has finished its reads of
      // stage x-1, whose buffer is then refilled with stage x+3 (stages 0..NBUF-1 were
      // issued above; opening stage y issues stage y+2 from y = 2 on).
      auto nsub = [&](int st) {
        const int kb0 = stage_kbase(st);
        const int ke = (has_tree && st == 0) ? n : c1;
        return (min(kb0 + KT, ke) - kb0 + 31) >> 5;
      };
      auto open_stage = [&](int x) __attribute__((always_inline)) {
        const int ahead = min(max(NBUF - 1, x + 1), nst - 1) - x;   // stages issued after x
        if (ahead <= 0) wait_vmcnt<0>();
        else if (ahead == 1) wait_vmcnt<DMA>();
        else if (ahead == 2) wait_vmcnt<2 * DMA>();
        else wait_vmcnt<3 * DMA>();
        __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): this wave's LDS reads are done
        lds_barrier();
        if (x >= 2 && x + NBUF - 2 < nst) issue(x + NBUF - 2);
      };
      if (!wave_live) {
        for (int x = 0; x < nst; ++x) open_stage(x);
      } else {
        bf16x8 kb[3];                             // K slices of the next subtile: a ring of three
        VOps vr;                                  // V^T operands of the current subtile
        f32x16 sa, sb;                            // scores of the current / next subtile
        float msub = 0.f;                         // the row's fixed reference
        auto k_addr = [&](int st, int sub) {
          return lds_addr(smem + k_tile(st)) + sub * 32 * ROWB + koff0;
        };
        auto v_addr = [&](int st, int sub) {
          return lds_addr(smem + k_tile(st) + v_tile(st)) + sub * 32 * ROWB + voff0;
        };
        auto read_k_slice = [&](uint32_t ka0, int i) __attribute__((always_inline)) {
          return *(lds_bf16x8*)(uintptr_t)(ka0 ^ (i << 5));
        };
        // V^T operand (ks, dt) of the subtile at va0: rows 0-7 and 8-15 of its 16-key step
        auto read_v_op = [&](uint32_t va0, int ks, int dt) __attribute__((always_inline)) {
          const uint32_t lo_a = (va0 ^ (dt << 6)) + ks * 16 * ROWB;
          const uint32_t hi_a = ((va0 ^ (dt << 6)) ^ VHI) + 8 * ROWB + ks * 16 * ROWB;
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)lo_a);
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)hi_a);
          const s16x4 both[2] = {lo, hi};
          vr.v[ks][dt] = *(const bf16x8*)both;
        };
        // This lane's LDS addresses in ring slot 0, subtile 0: K operand slice i, and the
        // V^T operands dt (rows 0-7, rows 8-15 of a 16-key step).  Slot, subtile and step
        // add multiples of the row size, which leave the XORed chunk bits alone, so any
        // read in the ring is one of these plus a constant: with the slot known at compile
        // time the constant is the read's immediate offset (below 64 KB: slots of K in the
        // ring's first half, of V in its second) and the read needs no address arithmetic.
        uint32_t kof[DS], vof[DT][2];
        {
          const uint32_t ring = lds_addr(smem);
#pragma unroll
          for (int i = 0; i < DS; ++i) kof[i] = (ring + koff0) ^ (i << 5);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            vof[dt][0] = (ring + NBUF * TILEB + voff0) ^ (dt << 6);
            vof[dt][1] = (vof[dt][0] ^ VHI) + 8 * ROWB;
          }
        }
        // the reads of one subtile: at run-time addresses (RtAddr: its K and V^T bases)
        // or at a compile-time offset from slot 0 (ic<offset>)
        struct RtAddr {
          uint32_t k, v;
        };
        auto rt = [&](int st, int sub) { return RtAddr{k_addr(st, sub), v_addr(st, sub)}; };
        auto kread = [&](auto at, int i) __attribute__((always_inline)) {
          if constexpr (std::is_same_v<decltype(at), RtAddr>) return read_k_slice(at.k, i);
          else return *(lds_bf16x8*)(uintptr_t)(kof[i] + (uint32_t)decltype(at)::value);
        };
        auto vread = [&](auto at, int ks, int dt) __attribute__((always_inline)) {
          if constexpr (std::is_same_v<decltype(at), RtAddr>) {
            read_v_op(at.v, ks, dt);
          } else {
            constexpr uint32_t O = decltype(at)::value;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)(uintptr_t)(vof[dt][0] + O + ks * 16 * ROWB));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)(uintptr_t)(vof[dt][1] + O + ks * 16 * ROWB));
            const s16x4 both[2] = {lo, hi};
            vr.v[ks][dt] = *(const bf16x8*)both;
          }
        };
        // One subtile s, in two phases whose issue order is pinned by scheduling fences.
        // A wave's LDS reads hold up its vector instructions, so the softmax goes beside
        // products with as few reads as possible:
        //  1. the products of subtile s+1 (S^T = K Q^T), each with its share of the
        //     weights of s (fma, exp2, bf16 conversion, row sum by fdot2); the K slices of
        //     s+1 (st1, sub1) pass through a ring of three, each read two products ahead
        //     (the first two were read in the previous step);
        //  2. O^T += V^T P^T of s, each product followed by the reload of its V^T operand
        //     with subtile s+1's, and the last two by the first two K slices of s+2
        //     (st2, sub2).
        // Where s+1 or s+2 does not exist, LDS data of the ring is read and the result
        // dropped.  a1: the reads of s+1, a2: those of s+2.
        auto step = [&](auto masked_tag, f32x16& s_cur, f32x16& s_nxt, int st, int sub, auto a1,
                        auto a2) __attribute__((always_inline)) {
          constexpr bool MASKED = decltype(masked_tag)::value;
          constexpr int EPG = 16 / DS;             // weights per product of the next subtile
          typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
          const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
          if constexpr (MASKED) {
            const bool tree = has_tree && st == 0;
            apply_mask(s_cur, stage_kbase(st) + sub * 32 + 4 * g, tree ? n : c1,
                       tree ? qanc[0] : ~0ull);
          }
          f32x16 sn = f32x16{};
          float e[16];
          bf16x2 pk[8];
          float psum = 0.f;
          __builtin_amdgcn_sched_barrier(0);
          // Empty asm operands pin each slot's vector work between its fences: the
          // scores enter in their slot and the weights, packed pairs and row sum leave
          // it (pure arithmetic otherwise moves freely across the fences, and the
          // optimiser gathers all of it behind the last product).
#pragma unroll
          for (int i = 0; i < DS; ++i) {
            sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb[i % 3], qop[0][i], sn, 0, 0, 0);
            if (i + 2 < DS) kb[(i + 2) % 3] = kread(a1, i + 2);
#pragma unroll
            for (int j = i * EPG; j < (i + 1) * EPG; ++j) {
              float sv = s_cur[j];
              asm volatile("" : "+v"(sv));
              e[j] = __builtin_amdgcn_exp2f(fmaf(sv, a.sl2, -msub));
              asm volatile("" : "+v"(e[j]));
            }
            if (i > 0) {
#pragma unroll
              for (int j = (i - 1) * EPG; j < i * EPG; j += 2) {
                pk[j >> 1] = bf16x2{(__bf16)e[j], (__bf16)e[j + 1]};
                psum = __builtin_amdgcn_fdot2_f32_bf16(pk[j >> 1], one2, psum, false);
                uint32_t pku = __builtin_bit_cast(uint32_t, pk[j >> 1]);
                asm volatile("" : "+v"(pku), "+v"(psum));
                pk[j >> 1] = __builtin_bit_cast(bf16x2, pku);
              }
            }
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
          for (int j = (DS - 1) * EPG; j < 16; j += 2) {
            pk[j >> 1] = bf16x2{(__bf16)e[j], (__bf16)e[j + 1]};
            psum = __builtin_amdgcn_fdot2_f32_bf16(pk[j >> 1], one2, psum, false);
          }
          l_run[0] += psum;
          bf16x8 pb[2];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            pb[j >> 2][2 * (j & 3)] = pk[j][0];
            pb[j >> 2][2 * (j & 3) + 1] = pk[j][1];
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
              o[0][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr.v[ks][dt], pb[ks], o[0][dt], 0, 0, 0);
              vread(a1, ks, dt);
              const int q = ks * DT + dt;
              if (q >= 2 * DT - 2) kb[q - (2 * DT - 2)] = kread(a2, q - (2 * DT - 2));
              __builtin_amdgcn_sched_barrier(0);
            }
          s_nxt = sn;
        };
        constexpr ic<0> unmasked{};
        constexpr ic<1> masked{};

        // subtile 0: its scores set the reference (the root is visible to every row in
        // the tree stage; every key of a prefix stage is).  Stage 1 opens with stage 0.
        open_stage(0);
        if (nst > 1) open_stage(1);
        sa = qk(ic<0>{}, load_k(smem + k_tile(0), 0));
        if (has_tree || n_full == 0)
          apply_mask(sa, stage_kbase(0) + 4 * g, has_tree ? n : c1, has_tree ? qanc[0] : ~0ull);
        reference(ic<0>{}, sa);
        msub = m_run[0] == -INFINITY ? 0.f : m_run[0];
        {
          const uint32_t va0 = v_addr(0, 0);
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) read_v_op(va0, ks, dt);
        }
        // the first two K slices of subtile 1
        auto prefetch_k = [&](int st, int sub) __attribute__((always_inline)) {
          const uint32_t ka = k_addr(st, sub);
          kb[0] = read_k_slice(ka, 0);
          kb[1] = read_k_slice(ka, 1);
        };
        int x = 0;
        if (has_tree) {
          // the tree stage: one or two masked subtiles (the first one masked already)
          const bool more = nst > 1;
          const bool two1 = more && nsub(1) >= 2;          // stage 1 holds a second subtile
          if (nsub(0) == 2) {
            prefetch_k(0, 1);
            step(unmasked, sa, sb, 0, 0, rt(0, 1), rt(more ? 1 : 0, 0));
            step(masked, sb, sa, 0, 1, rt(more ? 1 : 0, more ? 0 : 1), rt(two1 ? 1 : 0, 1));
          } else {
            prefetch_k(more ? 1 : 0, 0);
            step(unmasked, sa, sb, 0, 0, rt(more ? 1 : 0, 0), rt(two1 ? 1 : 0, two1 ? 1 : 0));
            sa = sb;
          }
          x = 1;
        } else {
          prefetch_k(0, nsub(0) >= 2 ? 1 : 0);
        }
        // full prefix stages: two unmasked subtiles each.  The next stage opens first, so
        // that the steps can read its K and V^T while their products run; one code path
        // (where there is no next stage the reads repeat this stage's)
        const int full_end = has_tree + n_full;
        // unrolled over the ring: stage x in slot S, the next stage in slot S+1 (read
        // even where it does not exist; those results are dropped)
        auto ring_stage = [&](auto slot_tag, int xx) __attribute__((always_inline)) {
          constexpr int S = decltype(slot_tag)::value;
          constexpr int S1 = (S + 1) % NBUF;
          if (xx >= 1 && xx + 1 < nst) open_stage(xx + 1);
          step(unmasked, sa, sb, xx, 0, ic<S * TILEB + 32 * ROWB>{}, ic<S1 * TILEB>{});
          step(unmasked, sb, sa, xx, 1, ic<S1 * TILEB>{}, ic<S1 * TILEB + 32 * ROWB>{});
        };
        static_assert(NBUF == 4 && NSW == 2, "the unrolled loop takes four slots of two subtiles");
        for (; x + 3 < full_end; x += 4) {           // stage x is in slot 0 here
          ring_stage(ic<0>{}, x);
          ring_stage(ic<1>{}, x + 1);
          ring_stage(ic<2>{}, x + 2);
          ring_stage(ic<3>{}, x + 3);
        }
        for (; x < full_end; ++x) {
          const bool more = x + 1 < nst;
          const bool two = more && nsub(x + 1) >= 2;
          if (x >= 1 && more) open_stage(x + 1);
          step(unmasked, sa, sb, x, 0, rt(x, 1), rt(more ? x + 1 : x, 0));
          step(unmasked, sb, sa, x, 1, rt(more ? x + 1 : x, more ? 0 : 1), rt(two ? x + 1 : x, 1));
        }
        // a partial last prefix stage (masked; opened by the loop or above)
        if (x < nst) {
          if (nsub(x) >= 2) {
            step(masked, sa, sb, x, 0, rt(x, 1), rt(x, 0));
            step(masked, sb, sa, x, 1, rt(x, 1), rt(x, 1));
          } else {
            step(masked, sa, sb, x, 0, rt(x, 0), rt(x, 0));
          }
        }
        // weights past the fixed reference's range show in the row sum (all terms are
        // non-negative; inf and NaN included): the exact path below takes over
        over = !(l_run[0] <= 0x1p48f);
      }
    } else if (!wave_live) {
      for (int st = 0; st < nst; ++st) begin_stage(st);
    } else {
      // The tree stage and a partial last prefix stage take the masked path outside the
      // loop over the full prefix stages.  The loop then has a single code path, so its
      // O accumulators stay in place (where two paths join inside a loop the compiler
      // copies all of them on every iteration).
      int st = 0;
      if (has_tree) {
        begin_stage(0);
        stage_fast(0);
        st = 1;
      }
      const int full_end = has_tree + n_full;
      auto full_loop = [&](auto ntile_tag) {
        for (; st < full_end; ++st) {
          begin_stage(st);
          stage_full(ntile_tag, st);
        }
      };
      if (QT > 1 && live1) full_loop(ic<QT>{});
      else full_loop(ic<1>{});
      if (st < nst) {
        begin_stage(st);
        stage_fast(st);
      }
    }

    // ---- slow path: a score left the fixed reference's range.  This wave recomputes
    // its rows of the chunk from global memory in two passes (exact row maximum first,
    // then the weighted sum against it), without barriers.
    if (__ballot(over)) {
      auto for_subtiles = [&](auto&& body) {
        for (int st = 0; st < nst; ++st) {
          const bool tree = has_tree && st == 0;
          const int kbase = stage_kbase(st);
          const int kend = tree ? n : c1;
          for (int j = 0; j < NSW; ++j) {
            const int k0 = kbase + (wk + j * WK) * 32;
            if (k0 < kend) body(tree, k0, kend);
          }
        }
      };
      float mx[QT];
#pragma unroll
      for (int u = 0; u < QT; ++u) mx[u] = -INFINITY;
      for_subtiles([&](bool tree, int k0, int kend) {
        const KOps k = load_k_global(tree, k0, kend);
        f32x16 s = qk(ic<0>{}, k);
        apply_mask(s, k0 + 4 * g, kend, tree ? qanc[0] : ~0ull);
        mx[0] = fmaxf(mx[0], lane_max(s));
        if constexpr (QT > 1) {
          s = qk(ic<1>{}, k);
          apply_mask(s, k0 + 4 * g, kend, tree ? qanc[1] : ~0ull);
          mx[1] = fmaxf(mx[1], lane_max(s));
        }
      });
#pragma unroll
      for (int u = 0; u < QT; ++u) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[u][dt] = f32x16{};
        m_run[u] = max_halves(mx[u]);
        l_run[u] = 0.f;
      }
      for_subtiles([&](bool tree, int k0, int kend) {
        const KOps k = load_k_global(tree, k0, kend);
        const VOps v = load_v_global(tree, k0, kend);
        bf16x8 pb[2];
        f32x16 s = qk(ic<0>{}, k);
        apply_mask(s, k0 + 4 * g, kend, tree ? qanc[0] : ~0ull);
        weights(ic<0>{}, s, pb);
        pv(ic<0>{}, v, pb);
        if constexpr (QT > 1) {
          s = qk(ic<1>{}, k);
          apply_mask(s, k0 + 4 * g, kend, tree ? qanc[1] : ~0ull);
          weights(ic<1>{}, s, pb);
          pv(ic<1>{}, v, pb);
        }
      });
    }
    const int nc = L > 0 ? (L + span * a.chunk_keys - 1) / (span * a.chunk_keys) : 1;
    if constexpr (WK == 1 && QT == 1) {
      // ---- one 32-row tile per wave and no key split: each wave writes its rows
      // straight from its accumulators (the two lanes of a row store 32 contiguous
      // bytes per instruction), with no LDS staging and no barrier: the final rows when
      // the sequence's prefix fits in one chunk, else unnormalised partials for
      // attn_combine.  The same arithmetic as the staged path below.
      const float lt = sum_halves(l_run[0]);
      const int i = wave * 32 + ql;                    // row within the workgroup
      const int rho_i = row0 + i;
      if (wave_live && rho_i < R) {
        const float M = m_run[0];
        const float sc = __builtin_amdgcn_exp2f(M - (M == -INFINITY ? 0.f : M));   // 0 without keys
        const float lsum = lt * sc;
        if (nc == 1) {
          const int node = rho_i / G;
          const int head = kvh * G + rho_i % G;
          const size_t orow = ((size_t)b * a.n_max + node) * a.Hq + head;
          const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              __bf16 ob4[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) ob4[e] = (__bf16)(o[0][dt][4 * r4 + e] * sc * inv);
              *(s16x4*)(a.out + orow * D + 32 * dt + 8 * r4 + 4 * g) = *(const s16x4*)ob4;
            }
          if (a.lse && g == 0) a.lse[orow] = lsum > 0.f ? (M + log2f(lsum)) * kLn2 : 0.f;
        } else {
          const size_t slot = ((size_t)unit * a.n_chunks + chunk) * a.rows_per_wg + i;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4)
              *(f32x4*)(a.part_o + slot * D + 32 * dt + 8 * r4 + 4 * g) =
                  f32x4{o[0][dt][4 * r4], o[0][dt][4 * r4 + 1], o[0][dt][4 * r4 + 2], o[0][dt][4 * r4 + 3]} * sc;
          if (g == 0) a.part_ml[slot] = make_float2(M, lsum);
        }
      }
    } else {
    // ---- every wave parks its rows (unnormalised O, reference m, sum l) in LDS, then
    // the whole workgroup combines the key-split waves of each row and writes the
    // chunk's output with coalesced stores: the final rows when the sequence's prefix
    // fits in one chunk, else unnormalised partials for attn_combine.
    __syncthreads();                                   // the stage ring is free now
    float* ob = (float*)smem;
    float2* mlb = (float2*)(ob + OB_FLOATS);
    {
      float lt[QT];
#pragma unroll
      for (int u = 0; u < QT; ++u) lt[u] = sum_halves(l_run[u]);
      if (wave_live) {
#pragma unroll
        for (int u = 0; u < QT; ++u) {
          if (u == 1 && !live1) break;
          float* orow = ob + ((wave * QT + u) * 32 + ql) * OSTR;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4)
              *(f32x4*)(orow + 32 * dt + 8 * r4 + 4 * g) =
                  f32x4{o[u][dt][4 * r4], o[u][dt][4 * r4 + 1], o[u][dt][4 * r4 + 2], o[u][dt][4 * r4 + 3]};
          if (g == 0) mlb[(wave * QT + u) * 32 + ql] = make_float2(m_run[u], lt[u]);
        }
      }
    }
    __syncthreads();
    constexpr int D4 = D / 4;
    // only the rows that hold tree nodes (chunk 0 zero-fills the others); unrolled, so
    // that the LDS reads of several rows are in flight together
    constexpr int ITEMS = 32 * QT * WQ * D4 / NT;
    static_assert(ITEMS * NT == 32 * QT * WQ * D4, "whole items per thread");
    const int live_items = min(a.rows_per_wg, R - row0) * D4;
#pragma unroll
    for (int it = 0; it < ITEMS; ++it) {
      const int idx = tid + it * NT;
      if (idx >= live_items) break;
      const int i = idx / D4;                          // row within the workgroup
      const int d = (idx % D4) * 4;
      const int rho_i = row0 + i;
      const int qg = i / (32 * QT);
      const int slot_w = (i / 32) % QT * 32 + i % 32;  // (tile, row) within a wave
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < WK; ++w) M = fmaxf(M, mlb[(qg * WK + w) * QT * 32 + slot_w].x);
      const float ms = M == -INFINITY ? 0.f : M;
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      float lsum = 0.f;
#pragma unroll
      for (int w = 0; w < WK; ++w) {
        const float2 ml = mlb[(qg * WK + w) * QT * 32 + slot_w];
        const float sc = __builtin_amdgcn_exp2f(ml.x - ms);      // 0 for a wave without keys
        acc += *(const f32x4*)(ob + ((qg * WK + w) * QT * 32 + slot_w) * OSTR + d) * sc;
        lsum += ml.y * sc;
      }
      if (nc == 1) {
        const int node = rho_i / G;
        const int head = kvh * G + rho_i % G;
        const size_t orow = ((size_t)b * a.n_max + node) * a.Hq + head;
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        __bf16 ob4[4] = {(__bf16)(acc[0] * inv), (__bf16)(acc[1] * inv), (__bf16)(acc[2] * inv),
                         (__bf16)(acc[3] * inv)};
        *(s16x4*)(a.out + orow * D + d) = *(const s16x4*)ob4;
        if (a.lse && d == 0) a.lse[orow] = lsum > 0.f ? (M + log2f(lsum)) * kLn2 : 0.f;
      } else {
        const size_t slot = ((size_t)unit * a.n_chunks + chunk) * a.rows_per_wg + i;
        *(f32x4*)(a.part_o + slot * D + d) = acc;
        if (d == 0) a.part_ml[slot] = make_float2(M, lsum);
      }
    }
    }
  }

  // ---- chunk 0 of every unit zero-fills the unit's rows that hold no tree node (all
  // of them when the sequence is invalid) and reports the sequence's status
  if (chunk == 0) {
    if (tid == 0 && a.seq_status && kvh == 0 && rb == 0)
      a.seq_status[b] = !n_ok ? TV_SEQ_BAD_N : (seq_ok ? TV_SEQ_OK : TV_SEQ_BAD_PREFIX);
    constexpr int V4 = D / 4;
    const int rows_total = a.n_max * G;
    const int first_dead = seq_ok ? R : 0;
    for (int idx = tid; idx < a.rows_per_wg * V4; idx += NT) {
      const int rho = row0 + idx / V4;
      if (rho < first_dead || rho >= rows_total) continue;
      const size_t orow = ((size_t)b * a.n_max + rho / G) * a.Hq + kvh * G + rho % G;
      *(s16x4*)(a.out + orow * D + (idx % V4) * 4) = s16x4{0, 0, 0, 0};
      if (a.lse && idx % V4 == 0) a.lse[orow] = 0.f;
    }
  }
}

// Merge of the key-chunk partials for the rows whose sequence spans more than one
// chunk (the others were written by attn_bf16).  Sixteen lanes per output row, four
// rows per wave, CR rows per workgroup: a lane owns D/16 consecutive dims (16-byte
// loads and one 8- or 16-byte store).  The partials are loaded eight chunks at a time
// before any is used and merged online against a running maximum.  Few output rows
// (one sequence) take four rows per workgroup, so that the live rows spread over
// more CUs; many take eight.
constexpr int kCombineLanes = 16;                    // lanes per output row
constexpr int kCombineBatch = 8;                     // chunk partials in flight per lane
constexpr int kCombineFewRows = 4096;                // up to this many: four rows per workgroup

template <int D, int CR>
__global__ __launch_bounds__(kCombineLanes * CR) void attn_combine(AttnArgs a) {
  constexpr int DPL = D / kCombineLanes;             // dims per lane: 8 or 4
  constexpr int V4 = DPL / 4;                        // f32x4 loads per lane and chunk
  const int row = blockIdx.x * CR + threadIdx.x / kCombineLanes;
  if (row >= a.B * a.n_max * a.Hq) return;
  const int d0 = (threadIdx.x % kCombineLanes) * DPL;
  const int h = row % a.Hq;
  const int i = (row / a.Hq) % a.n_max;
  const int b = row / (a.Hq * a.n_max);
  const int n = a.n_nodes[b];
  const int64_t Lw = a.offsets[b + 1] - a.offsets[b];
  if (n < 1 || n > a.n_max || a.offsets[b] < 0 || Lw < 0 || Lw > a.max_prefix || i >= n) return;
  const int L = (int)Lw;
  const int span = chunk_span(a, n * a.G);
  const int nc = L > 0 ? (L + span * a.chunk_keys - 1) / (span * a.chunk_keys) : 1;
  if (nc <= 1) return;
  const int G = a.G;
  const int kvh = h / G;
  const int rho = i * G + h % G;                       // row index within the KV head
  const int rb = rho / a.rows_per_wg;
  const int unit = (b * a.Hkv + kvh) * a.n_rb + rb;
  const size_t slot0 = (size_t)unit * a.n_chunks * a.rows_per_wg + rho % a.rows_per_wg;
  float M = -INFINITY, wsum = 0.f;
  f32x4 acc[V4];
#pragma unroll
  for (int v = 0; v < V4; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < nc; c0 += kCombineBatch) {
    float2 ml[kCombineBatch];
    f32x4 po[kCombineBatch][V4];
#pragma unroll
    for (int j = 0; j < kCombineBatch; ++j) {
      if (c0 + j < nc) {
        const size_t slot = slot0 + (size_t)(c0 + j) * span * a.rows_per_wg;
        ml[j] = a.part_ml[slot];
#pragma unroll
        for (int v = 0; v < V4; ++v) po[j][v] = *(const f32x4*)(a.part_o + slot * D + d0 + 4 * v);
      } else {
        ml[j] = make_float2(-INFINITY, 0.f);
      }
    }
    float mn = M;
#pragma unroll
    for (int j = 0; j < kCombineBatch; ++j) mn = fmaxf(mn, ml[j].x);
    const float ms = mn == -INFINITY ? 0.f : mn;
    const float sa = __builtin_amdgcn_exp2f(M - ms);          // 0 while nothing was merged
    wsum *= sa;
#pragma unroll
    for (int v = 0; v < V4; ++v) acc[v] *= sa;
#pragma unroll
    for (int j = 0; j < kCombineBatch; ++j) {
      if (c0 + j < nc) {
        const float sb = __builtin_amdgcn_exp2f(ml[j].x - ms);  // 0 for a chunk without keys
        wsum += ml[j].y * sb;
#pragma unroll
        for (int v = 0; v < V4; ++v) acc[v] += po[j][v] * sb;
      }
    }
    M = mn;
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  __bf16 ob[DPL];
#pragma unroll
  for (int v = 0; v < V4; ++v)
#pragma unroll
    for (int e = 0; e < 4; ++e) ob[4 * v + e] = (__bf16)(acc[v][e] * inv);
  if constexpr (DPL == 8) *(bf16x8*)(a.out + (size_t)row * D + d0) = *(const bf16x8*)ob;
  else *(s16x4*)(a.out + (size_t)row * D + d0) = *(const s16x4*)ob;
  if (a.lse && d0 == 0) a.lse[row] = wsum > 0.f ? (M + log2f(wsum)) * kLn2 : 0.f;
}

// fp32 inputs: one workgroup of 128 threads per output row, vector ALUs only.
__global__ __launch_bounds__(128) void attn_f32(
    int B, int Hq, int Hkv, int D, int n_max, int max_prefix, float scale,
    const float* __restrict__ q, const float* __restrict__ k_tree, const float* __restrict__ v_tree,
    const float* __restrict__ k_prefix, const float* __restrict__ v_prefix,
    const int64_t* __restrict__ offsets, const int32_t* __restrict__ n_nodes,
    const uint64_t* __restrict__ anc, float* __restrict__ out, float* __restrict__ lse,
    int32_t* __restrict__ seq_status) {
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x;
  const int G = Hq / Hkv;
  const int kvh = h / G;
  const int n = n_nodes[b];
  const int64_t off = offsets[b];
  const int64_t Lw = offsets[b + 1] - off;
  int status = TV_SEQ_OK;
  if (n < 1 || n > n_max) status = TV_SEQ_BAD_N;
  else if (off < 0 || Lw < 0 || Lw > max_prefix) status = TV_SEQ_BAD_PREFIX;
  if (seq_status && i == 0 && h == 0 && tid == 0) seq_status[b] = status;
  const size_t orow = (((size_t)b * n_max + i) * Hq + h);
  if (status != TV_SEQ_OK || i >= n) {
    for (int d = tid; d < D; d += 128) out[orow * D + d] = 0.f;
    if (lse && tid == 0) lse[orow] = 0.f;
    return;
  }
  const int L = (int)Lw;
  const uint64_t mask = anc[(size_t)b * n_max + i];
  __shared__ float s_q[256];
  __shared__ float s_p[128];
  __shared__ float s_red[4];
  for (int d = tid; d < D; d += 128) s_q[d] = q[orow * D + d];
  __syncthreads();
  float m = -INFINITY, l = 0.f, acc0 = 0.f, acc1 = 0.f;
  const int total = L + n;
  for (int base = 0; base < total; base += 128) {
    const int key = base + tid;
    float s = -INFINITY;
    if (key < L) {
      const float* kr = k_prefix + ((size_t)(off + key) * Hkv + kvh) * D;
      float dot = 0.f;
      for (int d = 0; d < D; d += 4) {
        const float4 kv = *(const float4*)(kr + d);
        dot += s_q[d] * kv.x + s_q[d + 1] * kv.y + s_q[d + 2] * kv.z + s_q[d + 3] * kv.w;
      }
      s = dot * scale;
    } else if (key < total && ((mask >> (key - L)) & 1ull)) {
      const float* kr = k_tree + (((size_t)b * n_max + (key - L)) * Hkv + kvh) * D;
      float dot = 0.f;
      for (int d = 0; d < D; d += 4) {
        const float4 kv = *(const float4*)(kr + d);
        dot += s_q[d] * kv.x + s_q[d + 1] * kv.y + s_q[d + 2] * kv.z + s_q[d + 3] * kv.w;
      }
      s = dot * scale;
    }
    float mc = s;
    for (int o = 32; o > 0; o >>= 1) mc = fmaxf(mc, __shfl_xor(mc, o));
    if ((tid & 63) == 0) s_red[tid >> 6] = mc;
    __syncthreads();
    mc = fmaxf(s_red[0], s_red[1]);
    __syncthreads();
    const float mnew = fmaxf(m, mc);
    const float msub = mnew == -INFINITY ? 0.f : mnew;
    const float alpha = expf(m - msub);
    const float p = expf(s - msub);
    s_p[tid] = p;
    float ps = p;
    for (int o = 32; o > 0; o >>= 1) ps += __shfl_xor(ps, o);
    if ((tid & 63) == 0) s_red[2 + (tid >> 6)] = ps;
    __syncthreads();
    l = l * alpha + s_red[2] + s_red[3];
    acc0 *= alpha;
    acc1 *= alpha;
    const int cnt = min(128, total - base);
    for (int t2 = 0; t2 < cnt; ++t2) {
      const float pt = s_p[t2];
      if (pt == 0.f) continue;
      const int kk = base + t2;
      const float* vr = kk < L ? v_prefix + ((size_t)(off + kk) * Hkv + kvh) * D
                               : v_tree + (((size_t)b * n_max + (kk - L)) * Hkv + kvh) * D;
      if (tid < D) acc0 += pt * vr[tid];
      if (tid + 128 < D) acc1 += pt * vr[tid + 128];
    }
    m = mnew;
    __syncthreads();
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (tid < D) out[orow * D + tid] = acc0 * inv;
  if (tid + 128 < D) out[orow * D + tid + 128] = acc1 * inv;
  if (lse && tid == 0) lse[orow] = l > 0.f ? m + logf(l) : 0.f;
}

template <int D>
static void launch_bf16(const AttnPlan& p, const AttnArgs& a, hipStream_t stream) {
  const dim3 grid(p.grid), block(64 * p.waves);
  if (p.wk == 4 && p.qt == 1) hipLaunchKernelGGL((attn_bf16<D, 1, 4, 1>), grid, block, 0, stream, a);
  else if (p.wk == 4) hipLaunchKernelGGL((attn_bf16<D, 1, 4, 2>), grid, block, 0, stream, a);
  else if (p.wk == 2) hipLaunchKernelGGL((attn_bf16<D, 4, 2, 1>), grid, block, 0, stream, a);
  else hipLaunchKernelGGL((attn_bf16<D, 8, 1, 1>), grid, block, 0, stream, a);
  if (p.n_chunks > 1) {
    const int rows = a.B * a.n_max * a.Hq;
    if ((rows <= kCombineFewRows) != kPlanVariant)
      hipLaunchKernelGGL((attn_combine<D, 4>), dim3((rows + 3) / 4), dim3(kCombineLanes * 4), 0, stream, a);
    else
      hipLaunchKernelGGL((attn_combine<D, 8>), dim3((rows + 7) / 8), dim3(kCombineLanes * 8), 0, stream, a);
  }
}

static bool aligned16(const void* p) { return (((uintptr_t)p) & 15) == 0; }

}  // namespace tv

namespace tv {

// Scratch of tree_verify_attn_noalloc: the fp32 chunk partials in a fixed device array
// (one copy per GPU, held until the process ends) instead of a caller workspace.  Host
// code reaches it only through the device address hipGetSymbolAddress returns for the
// current device, kept per device; the array's name is not a device address on the host.
constexpr size_t kScratchBytes = size_t(128) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[kScratchBytes];

static void* scratch_of_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  static std::mutex mu;
  static void* ptr[kMaxDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    ptr[dev] = p;
  }
  return ptr[dev];
}

}  // namespace tv

TV_API size_t tree_verify_attn_workspace_size(tv_dtype dt, int B, int n_max, int Hq, int Hkv,
                                              int D, int max_prefix_len) {
  if (!tv::known_dtype(dt) || dt != TV_BF16) return 0;
  if (B < 1 || n_max < 1 || n_max > TV_MAX_NODES || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 ||
      max_prefix_len < 0 || (D != 64 && D != 128))
    return 0;
  return tv::make_plan(B, n_max, Hq, Hkv, D, max_prefix_len).ws_bytes;
}

TV_API tv_status tree_verify_attn_plan(tv_dtype dt, int B, int n_max, int Hq, int Hkv, int D,
                                       int max_prefix_len, int32_t* plan) {
  if (!tv::known_dtype(dt)) return TV_ERR_DTYPE;
  if (!plan) return TV_ERR_NULL;
  if (B < 1 || n_max < 1 || n_max > TV_MAX_NODES || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 ||
      max_prefix_len < 0 || D < 1)
    return TV_ERR_SHAPE;
  if (dt == TV_F32) return TV_ERR_DTYPE;
  if (D != 64 && D != 128) return TV_ERR_UNSUPPORTED;
  const tv::AttnPlan p = tv::make_plan(B, n_max, Hq, Hkv, D, max_prefix_len);
  const int32_t v[8] = {p.waves, p.wq, p.wk, p.qt, p.rows_per_wg, p.chunk_keys, p.n_chunks, p.grid};
  for (int i = 0; i < 8; ++i) plan[i] = v[i];
  return TV_OK;
}

TV_API tv_status tree_verify_attn(tv_dtype dt, int B, int Hq, int Hkv, int D, int n_max,
                                  int max_prefix_len, float scale, const void* q,
                                  const void* k_tree, const void* v_tree, const void* k_prefix,
                                  const void* v_prefix, const int64_t* prefix_offsets,
                                  const int32_t* n_nodes, const uint64_t* anc, void* out,
                                  float* lse, void* ws, size_t ws_bytes, int32_t* seq_status,
                                  hipStream_t stream) {
  if (!tv::known_dtype(dt)) return TV_ERR_DTYPE;
  if (B < 1 || n_max < 1 || n_max > TV_MAX_NODES || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 ||
      max_prefix_len < 0 || D < 1)
    return TV_ERR_SHAPE;
  if (dt == TV_BF16 && D != 64 && D != 128) return TV_ERR_UNSUPPORTED;
  if (dt == TV_F32 && (D % 4 != 0 || D > 256)) return TV_ERR_UNSUPPORTED;
  if (!q || !k_tree || !v_tree || !prefix_offsets || !n_nodes || !anc || !out) return TV_ERR_NULL;
  if (max_prefix_len > 0 && (!k_prefix || !v_prefix)) return TV_ERR_NULL;
  if (!tv::aligned16(q) || !tv::aligned16(k_tree) || !tv::aligned16(v_tree) ||
      !tv::aligned16(out) || (max_prefix_len > 0 && (!tv::aligned16(k_prefix) ||
                                                     !tv::aligned16(v_prefix))))
    return TV_ERR_UNSUPPORTED;
  if (!(scale > 0.f)) scale = 1.0f / sqrtf((float)D);
  if (dt == TV_F32) {
    hipLaunchKernelGGL(tv::attn_f32, dim3(n_max, Hq, B), dim3(128), 0, stream, B, Hq, Hkv, D,
                       n_max, max_prefix_len, scale, (const float*)q, (const float*)k_tree,
                       (const float*)v_tree, (const float*)k_prefix, (const float*)v_prefix,
                       prefix_offsets, n_nodes, anc, (float*)out, lse, seq_status);
    return tv::launch_status();
  }
  const tv::AttnPlan p = tv::make_plan(B, n_max, Hq, Hkv, D, max_prefix_len);
  if (p.ws_bytes > 0 && (!ws || ws_bytes < p.ws_bytes || !tv::aligned16(ws)))
    return TV_ERR_WORKSPACE;
  tv::AttnArgs a{};
  a.q = (const __bf16*)q;
  a.k_tree = (const __bf16*)k_tree;
  a.v_tree = (const __bf16*)v_tree;
  a.k_prefix = (const __bf16*)k_prefix;
  a.v_prefix = (const __bf16*)v_prefix;
  a.offsets = prefix_offsets;
  a.n_nodes = n_nodes;
  a.anc = anc;
  a.out = (__bf16*)out;
  a.lse = lse;
  a.seq_status = seq_status;
  a.part_o = (float*)ws;
  a.part_ml = (float2*)((char*)ws + p.part_o_bytes);
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.n_max = n_max;
  a.max_prefix = max_prefix_len;
  a.rows_per_wg = p.rows_per_wg;
  a.chunk_keys = p.chunk_keys;
  a.n_chunks = p.n_chunks;
  a.n_rb = p.n_rb;
  a.total_wgs = p.total_wgs;
  // ranking pays where many sequences of different lengths share the GPU
  a.rank_pairs = B >= (tv::kPlanVariant ? 2 : tv::kRankMinBatch) &&
                 (long)B * p.n_chunks <= tv::kMaxRankPairs;
  a.sl2 = scale * tv::kLog2e;
  if (D == 128) tv::launch_bf16<128>(p, a, stream);
  else tv::launch_bf16<64>(p, a, stream);
  return tv::launch_status();
}

TV_API tv_status tree_verify_attn_noalloc(tv_dtype dt, int B, int Hq, int Hkv, int D, int n_max,
                                          int max_prefix_len, float scale, const void* q,
                                          const void* k_tree, const void* v_tree,
                                          const void* k_prefix, const void* v_prefix,
                                          const int64_t* prefix_offsets, const int32_t* n_nodes,
                                          const uint64_t* anc, void* out, float* lse,
                                          int32_t* seq_status, hipStream_t stream) {
  const size_t need = tree_verify_attn_workspace_size(dt, B, n_max, Hq, Hkv, D, max_prefix_len);
  if (need > tv::kScratchBytes) return TV_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    ws = tv::scratch_of_current_device();
    if (!ws) return TV_ERR_HIP;
  }
  return tree_verify_attn(dt, B, Hq, Hkv, D, n_max, max_prefix_len, scale, q, k_tree, v_tree,
                          k_prefix, v_prefix, prefix_offsets, n_nodes, anc, out, lse, ws,
                          need > 0 ? tv::kScratchBytes : 0, seq_status, stream);
}
