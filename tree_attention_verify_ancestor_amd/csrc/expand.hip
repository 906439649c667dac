// tree_expand_rerank: EAGLE-2 dynamic draft-tree construction, one level per call.
//
// "EAGLE" notes: "Well-Calibrated Draft Model" (confidence = softmax of the draft
// logits), "Expansion of tree" (a node's value is the product of confidences on its
// root path; keep the top-k), "Reranking Nodes" (keep the m nodes of largest value
// over all generated nodes).  Values are ranked by their logarithm: score = sum of
// log-confidences, with the row log-sum-exp taken in float64 and rounded once to
// float32, then fl32(parent + fl32(logit - lse)).  Every score bit is thereby fixed,
// so the kept set is exactly reproducible.
//
// Two kernels per call (and a third, draft_continue_kernel, for the per-level stop):
//   expand_rows_kernel   grid (chunk, frontier row, sequence).  Each workgroup reads
//                        one chunk of one logit row once (coalesced loads held in
//                        registers) and records the chunk's maximum, its float64 sum of
//                        exp(l - chunk max), a non-finite flag and its top-k.
//   expand_select_kernel one workgroup per sequence.  One wave per frontier row merges
//                        the chunk records into the row's log-sum-exp and top-k and
//                        appends the k children to the pool; then this level's
//                        children are ranked into the next frontier, and on the last
//                        level the whole pool is ranked, the best m-1 kept and the tree
//                        written in (depth, creation) order with remapped parents.
// Workspace per sequence: a header {status, pool count, next step, frontier slots and
// scores}, the pool of {parent slot, token, score, depth} records in creation order,
// then one record per (frontier row, chunk).
#include <float.h>
#include <math.h>

#include <type_traits>

#include "exp64.h"
#include "tv_internal.h"

namespace tv {

constexpr int kTopKMax = 16;
constexpr int kPoolMax = 4096;
static_assert(kPoolMax <= 4096, "pool slots fit 12 bits (depth-order keys) and a short");
constexpr int kChunkThreads = 256;
constexpr int kChunkWaves = kChunkThreads / kWave;
constexpr int kMaxRowChunks = 64;        // chunks per logit row (one lane each when merging)
constexpr int kMaxChunkElems = 64 * kChunkThreads;
constexpr int kMaxVocab = kMaxRowChunks * kMaxChunkElems;
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
static_assert(kSelWaves >= kTopKMax, "one select wave per frontier row");
static_assert(kChunkWaves * kTopKMax <= kWave, "the chunk's wave lists fit one wave");

struct PoolEntry {
  int32_t parent_slot;  // pool slot of the parent, -1 for the root
  int32_t token;
  float score;
  int32_t depth;
};

struct SeqHeader {
  int32_t status;
  int32_t count;
  int32_t next_step;
  int32_t pad[13];
  int32_t frontier[kTopKMax];          // pool slots of the frontier, best first
  float frontier_score[kTopKMax];      // and their scores (read without a pool lookup)
};

// What one workgroup of expand_rows_kernel learns about its chunk of a logit row.
struct ChunkRec {
  double sum;                // sum over the chunk of exp(l - max), float64
  float max;                 // chunk maximum
  int32_t bad;               // a NaN or infinite logit was seen
  float val[kTopKMax];       // chunk top-k, best first; -inf / INT32_MAX past its end
  int32_t id[kTopKMax];
};

__host__ __device__ inline int64_t pool_capacity(int k, int max_steps) {
  return (int64_t)k + (int64_t)(max_steps - 1) * k * k;
}
__host__ __device__ inline size_t chunk_rec_offset(int k, int max_steps) {
  size_t s = sizeof(SeqHeader) + (size_t)pool_capacity(k, max_steps) * sizeof(PoolEntry);
  return (s + 255) & ~(size_t)255;
}
__host__ __device__ inline size_t seq_stride_bytes(int k, int max_steps) {
  size_t s = chunk_rec_offset(k, max_steps) + (size_t)k * kMaxRowChunks * sizeof(ChunkRec);
  return (s + 255) & ~(size_t)255;
}
// pool slots used before level `step` (1-based): k after level 1, k*k per level after
__host__ __device__ inline int pool_base(int k, int step) {
  return step == 1 ? 0 : k + (step - 2) * k * k;
}

// ---- wave-wide reductions (every lane active; every lane gets the result)

// Order-preserving map of a float to an unsigned key: a larger value has a larger key,
// -0 and +0 share one key, and every finite value or -inf maps above 0, which is kept
// to mean "no candidate".
__device__ __forceinline__ uint32_t fkey(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  // 0 is the identity of unsigned max, so the compiler folds this into v_max_u32_dpp
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));    // quad_perm [1,0,3,2]
  v = max(v, dpp_u32<0x4E>(v));    // quad_perm [2,3,0,1]
  v = max(v, dpp_u32<0x141>(v));   // row_half_mirror: max over 8 lanes
  v = max(v, dpp_u32<0x140>(v));   // row_mirror: max over the 16-lane row
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return max(max(r0, r1), max(r2, r3));
}
__device__ __forceinline__ float wave_max_f32(float v) {
  const uint32_t k = wave_max_u32(fkey(v));
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
__device__ __forceinline__ int wave_min_i32(int v) {
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// One selection round over the wave: the lane whose candidate ranks first by (value
// descending, id ascending), given each lane's fkey (0 = no candidate) and id.
// Returns -1 when no lane has a candidate.
__device__ __forceinline__ int wave_argbest(uint32_t key, int id) {
  const uint32_t m = wave_max_u32(key);
  if (m == 0u) return -1;
  const uint64_t ball = __ballot(key == m);
  if (__popcll(ball) == 1) return __ffsll((unsigned long long)ball) - 1;
  const int mid = wave_min_i32(key == m ? id : INT32_MAX);         // equal values: lower id
  return __ffsll((unsigned long long)__ballot(key == m && id == mid)) - 1;
}

// The best two of this lane's elements x[j] by (value desc, j asc) among those ranked
// after (after_v, after_j); j = EPT marks an empty place.  -inf elements (past the chunk)
// are never taken.
template <int EPT>
__device__ __forceinline__ void best_two(const float (&x)[EPT], float after_v, int after_j,
                                         float& v1, int& j1, float& v2, int& j2) {
  v1 = v2 = -INFINITY;
  j1 = j2 = EPT;
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const float v = x[j];
    // bitwise, not short-circuit: the compiler would branch around every element
    const bool after = (v < after_v) | ((v == after_v) & (j > after_j));
    const bool c1 = after & (v > v1);
    const bool c2 = after & (v > v2);
    v2 = c1 ? v1 : (c2 ? v : v2);
    j2 = c1 ? j1 : (c2 ? j : j2);
    v1 = c1 ? v : v1;
    j1 = c1 ? j : j1;
  }
}

// float64 sum over the wave by DPP within rows of 16 lanes, then the four row sums
// (every lane gets the same value)
__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double wave_sum_f64_dpp(double v) {
  v += dpp_f64<0xB1>(v);     // quad_perm [1,0,3,2]
  v += dpp_f64<0x4E>(v);     // quad_perm [2,3,0,1]
  v += dpp_f64<0x141>(v);    // row_half_mirror: the 8-lane sum
  v += dpp_f64<0x140>(v);    // row_mirror: the 16-lane sum
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

// A lower bound on the k-th largest of the wave's keys (NS per lane; 0 marks no key):
// the largest T whose low 32 - BITS bits are 0 with at least k keys at or above it,
// found bit by bit from the top (BITS = 32: the k-th largest key itself).  0 when
// fewer than k keys are nonzero.
template <int NS, int BITS>
__device__ __forceinline__ uint32_t wave_kth_key(const uint32_t (&key)[NS], int k) {
  uint32_t T = 0;
#pragma unroll
  for (int bit = 31; bit >= 32 - BITS; --bit) {
    const uint32_t c = T | (1u << bit);
    int n = 0;
#pragma unroll
    for (int q = 0; q < NS; ++q) n += __popcll(__ballot(key[q] >= c));
    if (n >= k) T = c;
  }
  return T;
}

// An entry's rank key: larger value first, then lower id (ids >= 0)
__device__ __forceinline__ uint64_t rank_key(float v, int id) {
  return ((uint64_t)fkey(v) << 32) | (uint32_t)~id;
}
// the float a key was made from (+0 for -0)
__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}
// How many of keys[0..n) (in LDS) are larger than key.  Every lane reads the same
// address at a time (a broadcast), eight reads in flight, and compares in its own
// registers: no cross-lane or scalar step in the loop.
__device__ __forceinline__ int lds_rank_desc(const uint64_t* keys, int n, uint64_t key) {
  int rk = 0;
#pragma unroll 8
  for (int o = 0; o < n; ++o) rk += (int)(keys[o] > key);
  return rk;
}
__device__ __forceinline__ float key_float(uint64_t key) { return key_value((uint32_t)(key >> 32)); }
__device__ __forceinline__ int key_id(uint64_t key) { return (int)~(uint32_t)key; }

constexpr int kCandW = 64;               // threshold candidates kept per wave

// One chunk of one logit row per workgroup.  Each lane holds EPT logits; the chunk's
// maximum, its float64 sum of exp(l - max) and its top-k (value descending, id
// ascending) are recorded for expand_select_kernel.
//   sum   each lane sums exp(l - its own maximum) with exp_nonpos, then rescales by
//         exp(lane max - chunk max).  A NaN or infinite logit makes its lane's sum NaN,
//         which flags the chunk.
//   top-k T = the largest, over the waves, of the k-th largest lane maximum of a wave:
//         at least k logits of the chunk are >= T, so its top-k is among them.  Those
//         few (ballot-compacted per wave into LDS) are ranked by one wave across lanes.
//         When a wave gathers more than kCandW (heavy ties), the exact per-wave
//         selection rounds below run instead.
// Five waves per SIMD fit (EPT <= 32): a level's ~1280 workgroups are then resident at once.
template <int EPT, bool VEC>
__global__ __launch_bounds__(kChunkThreads) __attribute__((amdgpu_waves_per_eu(EPT >= 64 ? 4 : 5)))
void expand_rows_kernel(
    char* __restrict__ ws, size_t stride, size_t rec_off, int k, int step, int rows, int vocab,
    int chunk, const float* __restrict__ logits) {
  const int c = blockIdx.x;
  const int r = blockIdx.y;
  const int b = blockIdx.z;
  char* seq = ws + (size_t)b * stride;
  const SeqHeader* hdr = (const SeqHeader*)seq;
  if (step > 1 && (hdr->status != TV_SEQ_OK || hdr->next_step != step)) return;
  ChunkRec* rec = (ChunkRec*)(seq + rec_off) + (size_t)r * kMaxRowChunks + c;

  __shared__ double s_tab[kChunkWaves][kExpTab];
  __shared__ float s_cv[kChunkWaves][kCandW];
  __shared__ int s_ci[kChunkWaves][kCandW];
  __shared__ uint64_t s_ck[kWave];
  __shared__ uint32_t s_thr[kChunkWaves];
  __shared__ int s_cnt[kChunkWaves];
  __shared__ float s_wv[kChunkWaves][kTopKMax];
  __shared__ int s_wi[kChunkWaves][kTopKMax];
  __shared__ float s_max[kChunkWaves];
  __shared__ int s_bad[kChunkWaves];
  __shared__ double s_sum[kChunkWaves];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  // each wave its own copy of the exp table, written from immediates (no memory read
  // ahead of the logit loads) and read by the same wave only: no barrier
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < kExpTab; ++i) s_tab[wave][i] = kExp2Frac64[i];
  }
  const float* row = logits + ((size_t)b * rows + r) * (size_t)vocab;
  const int e0 = c * chunk;
  const int e1 = min(vocab, e0 + chunk);
  // element j of this thread; ids increase with j
  auto id_of = [&](int j) {
    return VEC ? e0 + 4 * (tid + kChunkThreads * (j >> 2)) + (j & 3) : e0 + tid + kChunkThreads * j;
  };

  // every load is issued before any is used (addresses clamped into the chunk), so
  // they are all in flight together
  float x[EPT];
  if constexpr (VEC) {
#pragma unroll
    for (int q = 0; q < EPT / 4; ++q) {
      const int i0 = min(id_of(4 * q), e1 - 4);           // chunk and vocab are 4-aligned
      const float4 v = *(const float4*)(row + i0);
      x[4 * q] = v.x;
      x[4 * q + 1] = v.y;
      x[4 * q + 2] = v.z;
      x[4 * q + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < EPT; ++j) x[j] = row[min(id_of(j), e1 - 1)];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const double* tab = s_tab[wave];

  // a chunk of exactly EPT logits per thread needs no bounds tests (every chunk of a
  // row but its last)
  auto body = [&](auto tail_tag) {
    constexpr bool TAIL = decltype(tail_tag)::value;
    auto in = [&](int j) { return !TAIL || id_of(j) < e1; };
    // logits past the chunk become -FLT_MAX: finite, never a candidate, summed as 0
    if constexpr (TAIL) {
#pragma unroll
      for (int j = 0; j < EPT; ++j) x[j] = in(j) ? x[j] : -FLT_MAX;
    }
    const bool has = in(0);
    float ml = -FLT_MAX;
#pragma unroll
    for (int j = 0; j < EPT; ++j) ml = fmaxf(ml, x[j]);
    const uint32_t lk[1] = {has ? fkey(ml) : 0u};
    // 20 key bits keep sign, exponent and 11 mantissa bits: a bound within about 1e-3
    // relative of the exact one, for 12 fewer ballot steps; the exact ranking follows
    const uint32_t tw = wave_kth_key<1, 20>(lk, k);
    const float mw = wave_max_f32(ml);
    const double md = (double)ml;
    double sum = 0.0;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const double e = exp_nonpos((double)x[j] - md, tab);
      sum += in(j) ? e : 0.0;
    }
    // the sum is complete here: otherwise the compiler sinks the exps past the barrier
    // below, and every element's partial results stay live across it
    asm volatile("" : "+v"(sum));
    // a NaN or infinite logit makes its lane's sum NaN (and only that does)
    const bool wbad = __ballot(sum != sum) != 0ull;
    if (lane == 0) {
      s_thr[wave] = tw;
      s_max[wave] = mw;
      s_bad[wave] = wbad;
    }
    __syncthreads();
    uint32_t T = s_thr[0];
    float M = s_max[0];
    int anybad = s_bad[0];
#pragma unroll
    for (int w = 1; w < kChunkWaves; ++w) {
      T = max(T, s_thr[w]);
      M = fmaxf(M, s_max[w]);
      anybad |= s_bad[w];
    }
    if (anybad) {
      if (tid == 0) rec->bad = 1;
      return;
    }
    // the candidates: logits >= T (every logit of the chunk when T is 0)
    const float tf = T == 0u ? -INFINITY : key_value(T);
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const bool cj = in(j) && x[j] >= tf;
      const uint64_t bm = __ballot(cj);
      if (bm != 0ull) {
        if (cj) {
          const int pos = cnt + (int)__builtin_amdgcn_mbcnt_hi(
                                    (uint32_t)(bm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0u));
          if (pos < kCandW) {
            s_cv[wave][pos] = x[j];
            s_ci[wave][pos] = id_of(j);
          }
        }
        cnt += __popcll(bm);
      }
    }
    // this lane's sum rescaled to the chunk maximum (lanes without logits hold 0)
    sum *= exp_nonpos(md - (double)M, tab);
    sum = wave_sum_f64_dpp(sum);
    if (lane == 0) {
      s_cnt[wave] = cnt;
      s_sum[wave] = sum;
    }
    __syncthreads();
    int n[kChunkWaves];
    int total = 0;
    bool over = false;
#pragma unroll
    for (int w = 0; w < kChunkWaves; ++w) {
      n[w] = s_cnt[w];
      total += n[w];
      over |= n[w] > kCandW;
    }
    if (tid == 0) {
      double S = 0.0;
#pragma unroll
      for (int w = 0; w < kChunkWaves; ++w) S += s_sum[w];
      rec->sum = S;
      rec->max = M;
      rec->bad = 0;
    }
    if (!over && total <= kWave) {
      // one wave ranks them (value descending, then id ascending): candidate `lane` in
      // registers, the others read across lanes
      if (wave == 0) {
        int w0 = 0, i0 = lane;
#pragma unroll
        for (int w = 0; w < kChunkWaves - 1; ++w)
          if (w0 == w && i0 >= n[w]) {
            i0 -= n[w];
            w0 = w + 1;
          }
        const bool mine = lane < total;
        const float v = mine ? s_cv[w0][i0] : 0.f;
        const int id = mine ? s_ci[w0][i0] : 0;
        const uint64_t key = rank_key(v, id);
        s_ck[lane] = key;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int rk = lds_rank_desc(s_ck, total, key);
        if (mine && rk < k) {
          rec->val[rk] = v;
          rec->id[rk] = id;
        }
        if (lane >= total && lane < k) {                 // fewer logits than k
          rec->val[lane] = -INFINITY;
          rec->id[lane] = INT32_MAX;
        }
      }
      return;
    }
    if (!over) {
      // rank of candidate tid among all, by every thread
      if (tid < total) {
        int w0 = 0, i0 = tid;
#pragma unroll
        for (int w = 0; w < kChunkWaves - 1; ++w)
          if (w0 == w && i0 >= n[w]) {
            i0 -= n[w];
            w0 = w + 1;
          }
        const float v = s_cv[w0][i0];
        const int id = s_ci[w0][i0];
        int rk = 0;
        for (int w = 0; w < kChunkWaves; ++w)
          for (int i = 0; i < n[w]; ++i) {
            const float ov = s_cv[w][i];
            const int oi = s_ci[w][i];
            rk += (int)(ov > v) | ((int)(ov == v) & (int)(oi < id));
          }
        if (rk < k) {
          rec->val[rk] = v;
          rec->id[rk] = id;
        }
      }
      if (tid >= total && tid < k) {                     // fewer logits than k
        rec->val[tid] = -INFINITY;
        rec->id[tid] = INT32_MAX;
      }
      return;
    }

    // Heavy ties: exact selection.  Each wave takes its top-k in k rounds over the
    // lanes' heads (a lane keeps its best two; when it wins with its second already
    // promoted, it rescans for the two after the winner); wave 0 then merges the lists.
    if constexpr (TAIL) {
#pragma unroll
      for (int j = 0; j < EPT; ++j) x[j] = in(j) ? x[j] : -INFINITY;
    }
    float h1v, h2v;
    int h1j, h2j;
    best_two(x, INFINITY, -1, h1v, h1j, h2v, h2j);
    bool second_known = true;
    for (int t = 0; t < k; ++t) {
      const int win = wave_argbest(h1j < EPT ? fkey(h1v) : 0u, id_of(h1j));
      if (win < 0) {
        if (lane == 0) {
          s_wv[wave][t] = -INFINITY;
          s_wi[wave][t] = INT32_MAX;
        }
        continue;
      }
      if (lane == win) {
        s_wv[wave][t] = h1v;
        s_wi[wave][t] = id_of(h1j);
        if (second_known) {
          h1v = h2v;
          h1j = h2j;
          second_known = false;
        } else {
          float a1v, a2v;
          int a1j, a2j;
          best_two(x, h1v, h1j, a1v, a1j, a2v, a2j);
          h1v = a1v;
          h1j = a1j;
          h2v = a2v;
          h2j = a2j;
          second_known = true;
        }
      }
    }
    __syncthreads();
    if (wave == 0) {
      // lane l holds candidate l % k of wave l / k
      const int nc = kChunkWaves * k;
      float cv = lane < nc ? s_wv[lane / k][lane % k] : -INFINITY;
      int ci = lane < nc ? s_wi[lane / k][lane % k] : INT32_MAX;
      for (int t = 0; t < k; ++t) {
        const int win = wave_argbest(ci != INT32_MAX ? fkey(cv) : 0u, ci);
        if (win < 0) {
          if (lane == 0) {
            rec->val[t] = -INFINITY;
            rec->id[t] = INT32_MAX;
          }
          continue;
        }
        if (lane == win) {
          rec->val[t] = cv;
          rec->id[t] = ci;
          cv = -INFINITY;
          ci = INT32_MAX;
        }
      }
    }
  };
  if (e1 - e0 == EPT * kChunkThreads)
    body(std::integral_constant<bool, false>());
  else
    body(std::integral_constant<bool, true>());
}

// wave-scope ordering of one wave's LDS writes before its reads of them
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The k best entries, by (value descending, id ascending), of up to 64 lists held one
// per lane, each best first: lane l's list has len entries, value(j) and id(j) (ids
// distinct, >= 0); at most max_total entries in all.  When they may exceed kWave and at
// least k lists are non-empty, T = the k-th best list head bounds them: every entry at
// or above it is a candidate, and at least k are.  Otherwise every entry is.  The
// candidates' rank keys are compacted into buf (kWave + 1 entries of this wave's LDS)
// and ranked there; emit(rank, key) is called for ranks below k.  Returns false,
// emitting nothing, when there are more than kWave candidates (heavy ties): the caller
// then merges another way.  Every lane must call.
template <class Val, class Id, class Emit>
__device__ __forceinline__ bool wave_topk_of_lists(int len, Val value, Id id_at, int k,
                                                  int max_total, uint64_t* buf, Emit emit) {
  const int lane = lane_id();
  uint64_t T = 0;
  if (max_total > kWave && __popcll(__ballot(len > 0)) >= k) {
    const uint64_t hk = len > 0 ? rank_key(value(0), id_at(0)) : 0ull;
    buf[lane] = hk;
    wave_lds_sync();
    if (len > 0 && lds_rank_desc(buf, kWave, hk) == k - 1) buf[kWave] = hk;
    wave_lds_sync();
    T = buf[kWave];
    wave_lds_sync();
  }
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < kTopKMax; ++j) cnt += (int)(j < len && rank_key(value(j), id_at(j)) >= T);
  // this lane's candidates go to buf[first ..], first = the counts of the lanes below
  // (cnt <= kTopKMax < 32); the places past cnt store into the spare word buf[kWave]
  // (T was read from it above), so that the stores need no branches
  static_assert(kTopKMax < 32, "counts fit five bits");
  int n;
  const int first = wave_prefix_small<5>(cnt, n);
  if (n > kWave) return false;
#pragma unroll
  for (int j = 0; j < kTopKMax; ++j) buf[j < cnt ? first + j : kWave] = rank_key(value(j), id_at(j));
  wave_lds_sync();
  if (lane < n) {
    const uint64_t key = buf[lane];
    const int rk = lds_rank_desc(buf, n, key);
    if (rk < k) emit(rk, key);
  }
  return true;
}

__device__ __forceinline__ bool better(float sa, int ia, float sb, int ib) {
  return sa > sb || (sa == sb && ia < ib);
}
// better() as 0/1 without short-circuit branches, for unrolled counting loops
__device__ __forceinline__ int beats(float sa, int ia, float sb, int ib) {
  return (int)(sa > sb) | ((int)(sa == sb) & (int)(ia < ib));
}

__global__ __launch_bounds__(kSelThreads) void expand_select_kernel(
    char* __restrict__ ws, size_t stride, size_t rec_off, int k, int step, int rows, int nch,
    int final_m, const int32_t* __restrict__ m_per_seq, const float* __restrict__ budget_log,
    const int32_t* __restrict__ root_token, int n_max, int32_t* __restrict__ parent,
    int32_t* __restrict__ token,
    float* __restrict__ score, int32_t* __restrict__ n_nodes, int32_t* __restrict__ frontier_token,
    int32_t* __restrict__ seq_status) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  char* seq = ws + (size_t)b * stride;
  SeqHeader* hdr = (SeqHeader*)seq;
  PoolEntry* pool = (PoolEntry*)(seq + sizeof(SeqHeader));
  const ChunkRec* recs = (const ChunkRec*)(seq + rec_off);

  __shared__ float s_score[kTopKMax * kTopKMax];
  __shared__ uint32_t s_key[kPoolMax];
  __shared__ uint8_t s_dep[kPoolMax];
  __shared__ short s_pos[kPoolMax];
  __shared__ short s_par[kPoolMax];
  __shared__ int s_ptok[kPoolMax];
  __shared__ float s_psc[kPoolMax];
  __shared__ uint32_t s_hist[256];
  __shared__ int s_wtot[kSelWaves];
  __shared__ int s_sel_digit, s_sel_before;
  __shared__ int s_tok[kTopKMax * kTopKMax];
  __shared__ int s_front[kTopKMax];
  __shared__ int s_kept[TV_MAX_NODES];
  __shared__ int s_kdep[TV_MAX_NODES];
  __shared__ int s_byrank[TV_MAX_NODES];
  __shared__ uint32_t s_kkey[TV_MAX_NODES];
  __shared__ int s_nkept, s_cut;
  __shared__ int s_status;
  __shared__ int s_m;
  __shared__ int s_rowbad;
  __shared__ uint64_t s_mk[kSelWaves][kWave + 1];    // per-wave merge candidates
  __shared__ uint64_t s_ckey[kTopKMax * kTopKMax];    // this level's children, rank keys

  const int base = pool_base(k, step);
  const int added = rows * k;
  const int count = base + added;

  // ---- every independent global read first: the header and m (thread 0), and per
  // frontier row (wave rr, lane c = chunk c) the chunk records and the parent node
  if (tid == 0) {
    int st = TV_SEQ_OK;
    if (step > 1) {
      st = hdr->status;
      if (st == TV_SEQ_OK && (hdr->next_step != step || hdr->count != base)) st = TV_SEQ_BAD_STATE;
    }
    s_status = st;
    s_m = final_m > 0 ? (m_per_seq ? m_per_seq[b] : final_m) : 0;
    s_nkept = 0;
    s_rowbad = 0;
  }
  if (tid < kTopKMax) s_front[tid] = -1;
  const int rr = wave;
  const bool merger = rr < rows;
  const bool has = merger && lane < nch;
  const ChunkRec* rec = recs + (size_t)rr * kMaxRowChunks + lane;
  float hv[kTopKMax];
  int hi[kTopKMax];
  float cmax = -INFINITY;
  double csum = 0.0;
  int cbad = 0;
  int pslot = -1;
  float pscore = 0.f;
  int pdepth = 0;
  if (merger) {
    // records of a sequence that is not ok are stale but never used
#pragma unroll
    for (int j = 0; j < kTopKMax; ++j) {
      hv[j] = -INFINITY;
      hi[j] = INT32_MAX;
    }
    if (has) {
      cbad = rec->bad;
      cmax = rec->max;
      csum = rec->sum;
      // whole 16-byte pieces (a record is 144 bytes, its lists 16-byte aligned), then the
      // places past k are cleared
#pragma unroll
      for (int q = 0; q < kTopKMax / 4; ++q) {
        const float4 v4 = ((const float4*)rec->val)[q];
        const int4 i4 = ((const int4*)rec->id)[q];
        hv[4 * q] = v4.x;
        hv[4 * q + 1] = v4.y;
        hv[4 * q + 2] = v4.z;
        hv[4 * q + 3] = v4.w;
        hi[4 * q] = i4.x;
        hi[4 * q + 1] = i4.y;
        hi[4 * q + 2] = i4.z;
        hi[4 * q + 3] = i4.w;
      }
#pragma unroll
      for (int j = 0; j < kTopKMax; ++j) {
        hv[j] = j < k ? hv[j] : -INFINITY;
        hi[j] = j < k ? hi[j] : INT32_MAX;
      }
    }
    if (step > 1) {
      // the frontier holds the previous level's children: depth step - 1
      pslot = hdr->frontier[rr];
      pslot = pslot < 0 ? 0 : (pslot >= base ? base - 1 : pslot);
      pscore = hdr->frontier_score[rr];
      pdepth = step - 1;
    }
  }
  __syncthreads();

  // ---- wave rr merges the chunk records of frontier row rr: lse = M + log(sum over
  // chunks of sum_c * exp(max_c - M)) in float64, rounded once to float32; the row's
  // top-k by a k-way merge of the sorted chunk lists
  if (s_status == TV_SEQ_OK && merger) {
    if (__ballot(has && cbad != 0) != 0ull) {
      if (lane == 0) s_rowbad = 1;
    } else {
      const float M = wave_max_f32(cmax);
      const double S = wave_sum_f64_dpp(has ? csum * exp((double)cmax - (double)M) : 0.0);
      const float lse32 = (float)((double)M + log(S));
      // a chunk's list holds its valid entries first (-inf / INT32_MAX past them)
      int len = 0;
#pragma unroll
      for (int j = 0; j < kTopKMax; ++j) len += (int)(hi[j] != INT32_MAX);
      auto put_child = [&](int t, float v, int tok) {
        PoolEntry e;
        e.parent_slot = pslot;
        e.token = tok;
        e.score = __fadd_rn(pscore, __fsub_rn(v, lse32));
        e.depth = pdepth + 1;
        pool[base + rr * k + t] = e;
        s_score[rr * k + t] = e.score;
        s_tok[rr * k + t] = e.token;
        s_ckey[rr * k + t] = rank_key(e.score, rr * k + t);
      };
      const bool merged = wave_topk_of_lists(
          len, [&](int j) { return hv[j]; }, [&](int j) { return hi[j]; }, k, nch * k, s_mk[rr],
          [&](int t, uint64_t key) { put_child(t, key_float(key), key_id(key)); });
      // heavy ties: k rounds of the best head
      for (int t = 0; !merged && t < k; ++t) {
        // the chunks together hold at least k finite candidates (vocab >= k)
        const int win = wave_argbest(hi[0] != INT32_MAX ? fkey(hv[0]) : 0u, hi[0]);
        if (lane == win) {
          put_child(t, hv[0], hi[0]);
#pragma unroll
          for (int j = 0; j < kTopKMax - 1; ++j) {
            hv[j] = hv[j + 1];
            hi[j] = hi[j + 1];
          }
          hv[kTopKMax - 1] = -INFINITY;
          hi[kTopKMax - 1] = INT32_MAX;
        }
      }
    }
  }
  __syncthreads();
  // every thread derives the status from the same LDS words
  int st = s_status;
  if (st == TV_SEQ_OK && s_rowbad) st = TV_SEQ_NONFINITE;
  if (st == TV_SEQ_OK && final_m > 0 && (s_m < 1 || s_m > n_max)) st = TV_SEQ_BAD_N;

  if (st == TV_SEQ_OK) {
    // next frontier: the k best children of this level by (score desc, creation asc):
    // each child's rank among all of them, from their rank keys in LDS
    for (int c = tid; c < added; c += kSelThreads) {
      const int rk = lds_rank_desc(s_ckey, added, s_ckey[c]);
      if (rk < k) s_front[rk] = c;
    }
    __syncthreads();
    if (tid < k) {
      hdr->frontier[tid] = base + s_front[tid];
      hdr->frontier_score[tid] = s_score[s_front[tid]];
      if (frontier_token) frontier_token[(size_t)b * k + tid] = s_tok[s_front[tid]];
    }
  } else if (frontier_token && tid < k) {
    frontier_token[(size_t)b * k + tid] = -1;
  }

  if (final_m > 0) {
    __syncthreads();
    int keep = 0;
    if (st == TV_SEQ_OK) {
      keep = min(s_m - 1, count);
      // the pool as order-preserving keys of the scores (and the depths) in LDS
      for (int c = tid; c < count; c += kSelThreads) {
        const PoolEntry e = pool[c];
        s_key[c] = fkey(e.score);
        s_dep[c] = (uint8_t)e.depth;
        s_pos[c] = -1;
        s_par[c] = (short)e.parent_slot;
        s_ptok[c] = e.token;
        s_psc[c] = e.score;
      }
      __syncthreads();
      if (keep == count) {                               // everything is kept
        for (int c = tid; c < count; c += kSelThreads) s_kept[c] = c;
        if (tid == 0) s_nkept = count;
        __syncthreads();
      } else if (keep > 0) {
        // T = the keep-th largest key, by radix selection 8 bits at a time from the top;
        // `need` ends as the number of entries equal to T that are kept
        uint32_t T = 0, tmask = 0;
        int need = keep;
        for (int shift = 24; shift >= 0; shift -= 8) {
          if (tid < 256) s_hist[tid] = 0u;
          __syncthreads();
          for (int c = tid; c < count; c += kSelThreads) {
            const uint32_t u = s_key[c];
            if ((u & tmask) == T) atomicAdd(&s_hist[(u >> shift) & 255u], 1u);
          }
          __syncthreads();
          if (wave == 0) {
            // lane l holds the digits 255-4l .. 252-4l, scanned from the top
            uint32_t h[4], sum = 0;
  #pragma unroll
            for (int j = 0; j < 4; ++j) {
              h[j] = s_hist[255 - 4 * lane - j];
              sum += h[j];
            }
            uint32_t incl = sum;
            for (int o = 1; o < kWave; o <<= 1) {
              const uint32_t t = __shfl_up(incl, o);
              if (lane >= o) incl += t;
            }
            const uint32_t before = incl - sum;
            if (before < (uint32_t)need && (uint32_t)need <= incl) {
              uint32_t cum = before;
              int d = 255 - 4 * lane;
  #pragma unroll
              for (int j = 0; j < 4; ++j) {
                if (cum + h[j] >= (uint32_t)need) {
                  d = 255 - 4 * lane - j;
                  break;
                }
                cum += h[j];
              }
              s_sel_digit = d;
              s_sel_before = (int)cum;
            }
          }
          __syncthreads();
          T |= (uint32_t)s_sel_digit << shift;
          tmask |= 255u << shift;
          need -= s_sel_before;
          __syncthreads();
        }
        // kept: keys above T, and the `need` earliest-created entries equal to T (the rank
        // among those comes from an in-order scan of per-thread tie counts)
        const int seg = (count + kSelThreads - 1) / kSelThreads;
        const int cs = tid * seg;
        int ties = 0;
        for (int j = 0; j < seg; ++j)
          if (cs + j < count && s_key[cs + j] == T) ++ties;
        static_assert(kPoolMax <= 7 * kSelThreads, "per-thread tie counts fit three bits");
        int wties;
        int rank = wave_prefix_small<3>(ties, wties);
        if (lane == 0) s_wtot[wave] = wties;
        __syncthreads();
        for (int w = 0; w < wave; ++w) rank += s_wtot[w];
        for (int j = 0; j < seg; ++j) {
          const int c = cs + j;
          if (c >= count) break;
          const uint32_t u = s_key[c];
          const bool kept = u > T || (u == T && rank < need);
          if (u == T) ++rank;
          if (kept) s_kept[atomicAdd(&s_nkept, 1)] = c;
        }
        __syncthreads();
      }
      // verify budget: rank the kept entries best first (score, then creation); the
      // leading run of places j whose score exceeds budget_log[j] stays
      if (budget_log && keep > 0) {
        if (tid == 0) s_cut = keep;
        if (tid < keep) s_kkey[tid] = s_key[s_kept[tid]];
        __syncthreads();
        if (tid < keep) {
          const int me = s_kept[tid];
          const uint32_t km = s_kkey[tid];
          int r = 0;
#pragma unroll 8
          for (int o = 0; o < keep; ++o) {
            const int other = s_kept[o];
            const uint32_t ko = s_kkey[o];
            r += (int)(ko > km) | ((int)(ko == km) & (int)(other < me));
          }
          s_byrank[r] = me;
          if (!(s_psc[me] > budget_log[r + 1])) atomicMin(&s_cut, r);
        }
        __syncthreads();
        keep = s_cut;
        if (tid < keep) s_kept[tid] = s_byrank[tid];
        __syncthreads();
      }
      // depth above the creation index (< kPoolMax = 2^12): one key orders by both
      if (tid < keep) s_kdep[tid] = ((int)s_dep[s_kept[tid]] << 12) | s_kept[tid];
      __syncthreads();
      // output position: root first, then by (depth, creation)
      if (tid < keep) {
        const int me = s_kept[tid];
        const int kme = s_kdep[tid];
        int before = 0;
#pragma unroll 8
        for (int o = 0; o < keep; ++o) before += s_kdep[o] < kme;
        s_pos[me] = (short)(1 + before);
      }
      __syncthreads();
      if (tid < keep) {
        const int me = s_kept[tid];
        const int pos = s_pos[me];
        const int ps = s_par[me];
        const size_t o = (size_t)b * n_max + pos;
        parent[o] = ps < 0 ? 0 : s_pos[ps];
        token[o] = s_ptok[me];
        score[o] = s_psc[me];
      }
    }
    const int n = (st == TV_SEQ_OK) ? keep + 1 : 0;
    for (int i = tid; i < n_max; i += kSelThreads) {
      const size_t o = (size_t)b * n_max + i;
      if (i == 0 && n > 0) {
        parent[o] = -1;
        token[o] = root_token[b];
        score[o] = 0.f;
      } else if (i >= n) {
        parent[o] = -1;
        token[o] = -1;
        score[o] = 0.f;
      }
    }
    if (tid == 0) n_nodes[b] = n;
  }
  __syncthreads();
  if (tid == 0) {
    hdr->status = st;
    hdr->count = (st == TV_SEQ_OK) ? count : 0;
    hdr->next_step = step + 1;
    if (seq_status) seq_status[b] = st;
  }
}

// The harness's per-level stop, one workgroup per sequence, after a level's select
// kernel: the latest level's best child (the frontier's rank 0) is at place p of the
// pool ranked best first; drafting goes on when p <= m - 1 and every place 1..p
// passes the verify budget, i.e. when that child would be kept if drafting stopped
// now.  Deeper nodes rank after their parents, so a 0 here never changes the tree.
__global__ __launch_bounds__(kSelThreads) void draft_continue_kernel(
    const char* __restrict__ ws, size_t stride, int m, const int32_t* __restrict__ m_per_seq,
    const float* __restrict__ budget_log, int32_t* __restrict__ more) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const char* seq = ws + (size_t)b * stride;
  const SeqHeader* hdr = (const SeqHeader*)seq;
  const PoolEntry* pool = (const PoolEntry*)(seq + sizeof(SeqHeader));
  __shared__ float s_sc[kPoolMax];
  __shared__ int s_place, s_fail;

  const int st = hdr->status;
  const int count = hdr->count;
  const int cs = hdr->frontier[0];
  const int mb = m_per_seq ? m_per_seq[b] : m;
  if (st != TV_SEQ_OK || count < 1 || count > kPoolMax || cs < 0 || cs >= count || mb < 2 ||
      mb > TV_MAX_NODES) {
    if (tid == 0) more[b] = 0;
    return;
  }
  if (tid == 0) {
    s_place = 1;
    s_fail = 0;
  }
  for (int c = tid; c < count; c += kSelThreads) s_sc[c] = pool[c].score;
  __syncthreads();
  const float ss = s_sc[cs];
  int ahead = 0;
  for (int c = tid; c < count; c += kSelThreads) ahead += beats(s_sc[c], c, ss, cs);
  if (ahead) atomicAdd(&s_place, ahead);
  __syncthreads();
  const int place = s_place;
  if (place > mb - 1) {                                   // beyond the kept count
    if (tid == 0) more[b] = 0;
    return;
  }
  if (budget_log) {
    // places 1..place hold the child itself and the entries ranked before it; each
    // must pass the bar of its own place
    for (int c = tid; c < count; c += kSelThreads) {
      const float sc = s_sc[c];
      if (c != cs && !better(sc, c, ss, cs)) continue;
      int r = 0;
      for (int o = 0; o < count; ++o) r += beats(s_sc[o], o, sc, c);
      if (!(sc > budget_log[r + 1])) s_fail = 1;
    }
    __syncthreads();
  }
  if (tid == 0) more[b] = s_fail ? 0 : 1;
}

// Chunking of a logit row: about 1024 workgroups in all, each chunk 2048, 4096, 8192 or
// 16384 logits (8 to 64 per thread), at most kMaxRowChunks chunks per row.
struct RowPlan {
  int nch, chunk, ept;
};
static RowPlan row_plan(int B, int rows, int vocab) {
  const long units = (long)B * rows;
  const long target = kPlanVariant ? 256 : 1024;
  const long want = (target + units - 1) / units;
  const long lo = (vocab + 8191) / 8192;
  const long hi = (vocab + 1023) / 1024;
  long n = want < hi ? want : hi;
  if (n < lo) n = lo;
  if (n > kMaxRowChunks) n = kMaxRowChunks;
  if (n < 1) n = 1;
  const int ch = (int)((vocab + n - 1) / n);
  RowPlan p;
  p.ept = ch <= 8 * kChunkThreads ? 8 : ch <= 16 * kChunkThreads ? 16 : ch <= 32 * kChunkThreads ? 32 : 64;
  // whole chunks of EPT logits per thread: only a row's last chunk takes bounds tests
  p.chunk = p.ept * kChunkThreads;
  p.nch = (vocab + p.chunk - 1) / p.chunk;
  return p;
}

template <int EPT>
static void launch_rows(bool vec, dim3 grid, hipStream_t stream, char* ws, size_t stride,
                        size_t rec_off, int k, int step, int rows, int vocab, int chunk,
                        const float* logits) {
  if (vec)
    hipLaunchKernelGGL((expand_rows_kernel<EPT, true>), grid, dim3(kChunkThreads), 0, stream, ws,
                       stride, rec_off, k, step, rows, vocab, chunk, logits);
  else
    hipLaunchKernelGGL((expand_rows_kernel<EPT, false>), grid, dim3(kChunkThreads), 0, stream, ws,
                       stride, rec_off, k, step, rows, vocab, chunk, logits);
}

}  // namespace tv

TV_API size_t tree_expand_workspace_size(int B, int k, int max_steps) {
  if (B < 1 || k < 1 || k > tv::kTopKMax || max_steps < 1) return 0;
  if (tv::pool_capacity(k, max_steps) > tv::kPoolMax) return 0;
  return (size_t)B * tv::seq_stride_bytes(k, max_steps);
}

TV_API tv_status tree_expand_rerank(void* ws, size_t ws_bytes, int B, int k, int max_steps,
                                    int step, int vocab, const float* logits, int final_m,
                                    const int32_t* m_per_seq, const float* budget_log,
                                    const int32_t* root_token, int n_max,
                                    int32_t* parent, int32_t* token, float* score,
                                    int32_t* n_nodes, int32_t* frontier_token, int32_t* seq_status,
                                    hipStream_t stream) {
  if (!logits) return TV_ERR_NULL;
  if (B < 1 || k < 1 || k > tv::kTopKMax || max_steps < 1 || step < 1 || step > max_steps ||
      vocab < k || vocab > tv::kMaxVocab || n_max < 1 || n_max > TV_MAX_NODES || final_m < 0 || final_m > n_max)
    return TV_ERR_SHAPE;
  if (tv::pool_capacity(k, max_steps) > tv::kPoolMax) return TV_ERR_SHAPE;
  if (final_m > 0 && (!parent || !token || !score || !n_nodes || !root_token)) return TV_ERR_NULL;
  const size_t need = tree_expand_workspace_size(B, k, max_steps);
  if (!ws || ws_bytes < need) return TV_ERR_WORKSPACE;
  const size_t stride = tv::seq_stride_bytes(k, max_steps);
  const size_t rec_off = tv::chunk_rec_offset(k, max_steps);
  const int rows = step == 1 ? 1 : k;
  const tv::RowPlan rp = tv::row_plan(B, rows, vocab);
  const bool vec = vocab % 4 == 0 && ((uintptr_t)logits & 15) == 0;
  const dim3 grid(rp.nch, rows, B);
  if (rp.ept == 8)
    tv::launch_rows<8>(vec, grid, stream, (char*)ws, stride, rec_off, k, step, rows, vocab, rp.chunk, logits);
  else if (rp.ept == 16)
    tv::launch_rows<16>(vec, grid, stream, (char*)ws, stride, rec_off, k, step, rows, vocab, rp.chunk, logits);
  else if (rp.ept == 32)
    tv::launch_rows<32>(vec, grid, stream, (char*)ws, stride, rec_off, k, step, rows, vocab, rp.chunk, logits);
  else
    tv::launch_rows<64>(vec, grid, stream, (char*)ws, stride, rec_off, k, step, rows, vocab, rp.chunk, logits);
  tv_status s = tv::launch_status();
  if (s != TV_OK) return s;
  hipLaunchKernelGGL(tv::expand_select_kernel, dim3(B), dim3(tv::kSelThreads), 0, stream,
                     (char*)ws, stride, rec_off, k, step, rows, rp.nch, final_m, m_per_seq,
                     budget_log, root_token, n_max, parent, token, score, n_nodes, frontier_token,
                     seq_status);
  return tv::launch_status();
}

TV_API tv_status tree_draft_continue(const void* ws, size_t ws_bytes, int B, int k, int max_steps,
                                     int m, const int32_t* m_per_seq, const float* budget_log,
                                     int32_t* more, hipStream_t stream) {
  if (!more) return TV_ERR_NULL;
  if (B < 1 || k < 1 || k > tv::kTopKMax || max_steps < 1 || m < 0 || m > TV_MAX_NODES ||
      (!m_per_seq && m < 1))
    return TV_ERR_SHAPE;
  if (tv::pool_capacity(k, max_steps) > tv::kPoolMax) return TV_ERR_SHAPE;
  const size_t need = tree_expand_workspace_size(B, k, max_steps);
  if (!ws || ws_bytes < need) return TV_ERR_WORKSPACE;
  hipLaunchKernelGGL(tv::draft_continue_kernel, dim3(B), dim3(tv::kSelThreads), 0, stream,
                     (const char*)ws, tv::seq_stride_bytes(k, max_steps), m, m_per_seq, budget_log,
                     more);
  return tv::launch_status();
}

TV_API tv_status tree_budget_thresholds(const float* cost_us, int n_max, float threshold,
                                        float* budget_log) {
  if (!cost_us || !budget_log) return TV_ERR_NULL;
  if (n_max < 1 || n_max > TV_MAX_NODES) return TV_ERR_SHAPE;
  for (int j = 0; j < TV_MAX_NODES; ++j) budget_log[j] = -INFINITY;
  for (int j = 1; j < n_max; ++j) {
    // candidate j brings the tree from j to j + 1 nodes
    const double marginal = (double)cost_us[j] - (double)cost_us[j - 1];
    if (threshold > 0.f && marginal > 0.0)
      budget_log[j] = (float)log((double)threshold * marginal);
  }
  return TV_OK;
}
