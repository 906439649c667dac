// tree_accept_stochastic: rejection-sampling acceptance over a draft tree.
//
// "EAGLE" notes, "Well-Calibrated Draft Model": under random sampling a draft token x
// is accepted with rate min(1, P_target(x) / P_draft(x)).  "What is EAGLE-3 ...",
// section 4 steps 3-4: a rejected token gives way to the target's own token, sampled
// from a corrected distribution, and the longest passing prefix of the tree is kept.
// "Technical analysis of EAGLE-4", "verification trees and the harness": rejection
// sampling keeps the output distribution unchanged.
//
// For a tree (the reading this library takes): from the root, try the current node's
// children in index order; child c with token x passes when
//     u_accept[c] * S * q(x) < r(x)            (float64, left to right)
// with r the current target weights (the node's p_target row, S = sum r); a passing
// child becomes the current node; a failing one turns r into the residual
//     r <- max(r - fl32(S) * q, 0)             (float32, product then difference)
// When no child passes the bonus token is the first v whose running sum of r passes
// u_bonus * S.
//
// One workgroup of 1024 threads per sequence walks the tree.  Up to 36864 tokens the
// current weights r live in LDS; rows of p_target and q_draft stream from HBM with
// coalesced loads.  Past that (a 128256-token vocabulary) r is never stored: after k
// rejections at the current node, r[v] is the node's p_target[v] taken through the k
// residual steps with the k scalars fl32(S_j) kept in LDS -- the same float32
// operations in the same order, so the same bits -- and every pass streams the node's
// p_target and q_draft rows.  Sums are float64: per thread (strided elements for the
// totals; contiguous elements for the bonus's running sum), then over the workgroup
// in a fixed order.
#include <algorithm>

#include "tv_internal.h"

namespace tv {

constexpr int kStochThreads = 1024;
constexpr int kStochBatch = 8;                // vocabulary loads in flight per thread
constexpr int kStochMaxVocab = 36864;                    // r in LDS: 144 KB

__device__ __forceinline__ double block_sum_f64(double v, double* sred) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();                                        // sred free from its last use
  if ((threadIdx.x & 63) == 0) sred[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int i = 0; i < kStochThreads / 64; ++i) t += sred[i];   // same order in every thread
  return t;
}

__global__ __launch_bounds__(kStochThreads) void accept_stochastic_kernel(
    int n_max, int V, const int32_t* __restrict__ parent, const uint64_t* __restrict__ anc,
    const int32_t* __restrict__ n_nodes, const int32_t* __restrict__ token,
    const float* __restrict__ p_target, const float* __restrict__ q_draft,
    const float* __restrict__ u_accept, const float* __restrict__ u_bonus,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ best_node,
    int32_t* __restrict__ bonus_token, int32_t* __restrict__ path) {
  __shared__ float sr[kStochMaxVocab];
  __shared__ double sred[kStochThreads / 64];
  __shared__ double sscan[kStochThreads / 64];
  __shared__ int skids[TV_MAX_NODES];
  __shared__ int snkids;
  __shared__ int schain[TV_MAX_NODES];
  __shared__ int spick, slastpos;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const size_t row = (size_t)b * n_max;
  const int n = n_nodes[b];
  const bool valid = n >= 1 && n <= n_max && anc[row] == 1ull;
  if (!valid) {
    if (tid == 0) {
      accept_len[b] = -1;
      best_node[b] = -1;
      bonus_token[b] = -1;
    }
    if (path && tid < n_max) path[row + tid] = -1;
    return;
  }
  // A thread's elements v = tid + i * kStochThreads are loaded kStochBatch at a time
  // from clamped addresses before any is used (a load used at once waits a full
  // memory round trip per element), then taken in increasing v as before.
  // r <- node u's target row; returns its sum
  auto load_row = [&](int u) {
    const float* pr = p_target + (row + u) * V;
    double s = 0.0;
    for (int v0 = tid; v0 < V; v0 += kStochBatch * kStochThreads) {
      float x[kStochBatch];
#pragma unroll
      for (int i = 0; i < kStochBatch; ++i) x[i] = pr[min(v0 + i * kStochThreads, V - 1)];
#pragma unroll
      for (int i = 0; i < kStochBatch; ++i) {
        const int v = v0 + i * kStochThreads;
        if (v < V) {
          sr[v] = x[i];
          s += (double)x[i];
        }
      }
    }
    return block_sum_f64(s, sred);                          // its barrier publishes sr
  };
  int u = 0, depth = 0;
  double S = load_row(0);
  while (true) {
    // children of u in index order
    if (tid < 64) {
      const bool kid = tid >= 1 && tid < n && parent[row + tid] == u;
      const uint64_t m = __ballot(kid);
      if (kid) skids[__popcll(m & ((1ull << tid) - 1ull))] = tid;
      if (tid == 0) snkids = __popcll(m);
    }
    __syncthreads();
    const int nk = snkids;
    const float* q = q_draft + (row + u) * V;
    bool moved = false;
    for (int j = 0; j < nk; ++j) {
      const int c = skids[j];
      const int x = token[row + c];
      const bool in_v = x >= 0 && x < V;
      const float rx = in_v ? sr[x] : 0.f;
      const float qx = in_v ? q[x] : 0.f;
      const bool pass = qx == 0.f ? rx > 0.f
                                  : (double)u_accept[row + c] * S * (double)qx < (double)rx;
      if (pass) {
        if (tid == 0) schain[depth] = c;
        u = c;
        ++depth;
        moved = true;
        __syncthreads();                                    // every thread has read sr[x]
        S = load_row(u);
        break;
      }
      // residual against this candidate's draft distribution: the product and the
      // difference each rounded to float32 (never contracted into one fma)
      __syncthreads();                                      // every thread has read sr[x]
      const float S32 = (float)S;
      double s = 0.0;
      for (int v0 = tid; v0 < V; v0 += kStochBatch * kStochThreads) {
        float qv[kStochBatch];
#pragma unroll
        for (int i = 0; i < kStochBatch; ++i) qv[i] = q[min(v0 + i * kStochThreads, V - 1)];
#pragma unroll
        for (int i = 0; i < kStochBatch; ++i) {
#pragma clang fp contract(off)
          const int v = v0 + i * kStochThreads;
          if (v < V) {
            const float prod = S32 * qv[i];
            const float nr = fmaxf(sr[v] - prod, 0.f);
            sr[v] = nr;
            s += (double)nr;
          }
        }
      }
      S = block_sum_f64(s, sred);
    }
    if (!moved) break;
    __syncthreads();                                        // skids reused
  }

  // bonus: first v whose running sum of r passes u_bonus * S (thread t scans the
  // contiguous slice [t*C, t*C + C); the slice sums are combined in thread order)
  const int C = (V + kStochThreads - 1) / kStochThreads;
  const int lo = min(tid * C, V);
  const int hi = min(lo + C, V);
  double local = 0.0;
  int lastpos = -1;
  for (int v = lo; v < hi; ++v) {
    local += (double)sr[v];
    if (sr[v] > 0.f) lastpos = v;
  }
  double incl = local;
  const int lane = tid & 63, wave = tid >> 6;
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) sscan[wave] = incl;
  if (tid == 0) {
    spick = V;
    slastpos = -1;
  }
  __syncthreads();
  double before = 0.0;
  for (int w = 0; w < wave; ++w) before += sscan[w];
  double run = before + incl - local;                       // sum of r below lo
  const double target = (double)u_bonus[b] * S;
  if (lo < hi && run + local > target) {
    for (int v = lo; v < hi; ++v) {
      run += (double)sr[v];
      if (run > target) {
        atomicMin(&spick, v);
        break;
      }
    }
  }
  if (lastpos >= 0) atomicMax(&slastpos, lastpos);
  __syncthreads();
  if (tid == 0) {
    int pick = spick;
    if (pick >= V) pick = slastpos >= 0 ? slastpos : V - 1;
    accept_len[b] = depth;
    best_node[b] = u;
    bonus_token[b] = pick;
  }
  if (path && tid < n_max) path[row + tid] = tid < depth ? schain[tid] : -1;
}

// Vocabularies past the LDS: r replayed from the node's p_target row (see the header).
constexpr int kStochScan = 4;                 // contiguous tokens per thread in the bonus scan

__global__ __launch_bounds__(kStochThreads) void accept_stochastic_stream_kernel(
    int n_max, int V, const int32_t* __restrict__ parent, const uint64_t* __restrict__ anc,
    const int32_t* __restrict__ n_nodes, const int32_t* __restrict__ token,
    const float* __restrict__ p_target, const float* __restrict__ q_draft,
    const float* __restrict__ u_accept, const float* __restrict__ u_bonus,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ best_node,
    int32_t* __restrict__ bonus_token, int32_t* __restrict__ path) {
  __shared__ float sS32[TV_MAX_NODES];        // fl32(S) of each rejection at the current node
  __shared__ double sred[kStochThreads / 64];
  __shared__ double sscan[kStochThreads / 64];
  __shared__ int skids[TV_MAX_NODES];
  __shared__ int snkids;
  __shared__ int schain[TV_MAX_NODES];
  __shared__ int spick, slastpos;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const size_t row = (size_t)b * n_max;
  const int n = n_nodes[b];
  const bool valid = n >= 1 && n <= n_max && anc[row] == 1ull;
  if (!valid) {
    if (tid == 0) {
      accept_len[b] = -1;
      best_node[b] = -1;
      bonus_token[b] = -1;
    }
    if (path && tid < n_max) path[row + tid] = -1;
    return;
  }
  int u = 0, depth = 0, nrej = 0;
  const float* pr = p_target + row * V;                    // node u's rows
  const float* q = q_draft + row * V;
  // r[v] after the nrej residual steps at u: product then difference, each float32
  auto r_of = [&](float pv, float qv) {
    float r = pv;
    for (int j = 0; j < nrej; ++j) {
#pragma clang fp contract(off)
      const float prod = sS32[j] * qv;
      r = fmaxf(r - prod, 0.f);
    }
    return r;
  };
  // S = sum of r over the vocabulary (the strided order of the LDS kernel)
  auto row_sum = [&]() {
    double s = 0.0;
    for (int v0 = tid; v0 < V; v0 += kStochBatch * kStochThreads) {
      float pv[kStochBatch], qv[kStochBatch];
#pragma unroll
      for (int i = 0; i < kStochBatch; ++i) {
        const int v = min(v0 + i * kStochThreads, V - 1);
        pv[i] = pr[v];
        qv[i] = q[v];
      }
#pragma unroll
      for (int i = 0; i < kStochBatch; ++i)
        if (v0 + i * kStochThreads < V) s += (double)r_of(pv[i], qv[i]);
    }
    return block_sum_f64(s, sred);
  };
  double S = row_sum();
  while (true) {
    if (tid < 64) {
      const bool kid = tid >= 1 && tid < n && parent[row + tid] == u;
      const uint64_t m = __ballot(kid);
      if (kid) skids[__popcll(m & ((1ull << tid) - 1ull))] = tid;
      if (tid == 0) snkids = __popcll(m);
    }
    __syncthreads();
    const int nk = snkids;
    bool moved = false;
    for (int j = 0; j < nk; ++j) {
      const int c = skids[j];
      const int x = token[row + c];
      const bool in_v = x >= 0 && x < V;
      const float qx = in_v ? q[x] : 0.f;
      const float rx = in_v ? r_of(pr[x], qx) : 0.f;
      const bool pass = qx == 0.f ? rx > 0.f
                                  : (double)u_accept[row + c] * S * (double)qx < (double)rx;
      if (pass) {
        if (tid == 0) schain[depth] = c;
        u = c;
        ++depth;
        moved = true;
        nrej = 0;
        pr = p_target + (row + u) * V;
        q = q_draft + (row + u) * V;
        S = row_sum();
        break;
      }
      __syncthreads();                                      // sS32[nrej] is free
      if (tid == 0) sS32[nrej] = (float)S;
      __syncthreads();
      ++nrej;
      S = row_sum();
    }
    if (!moved) break;
    __syncthreads();                                        // skids reused
  }

  // bonus: the first v whose running sum of r passes u_bonus * S, over tiles of
  // kStochScan * 1024 tokens (thread t owns kStochScan consecutive tokens of a tile);
  // the scan stops at the first tile that holds it
  const double target = (double)u_bonus[b] * S;
  if (tid == 0) {
    spick = V;
    slastpos = -1;
  }
  __syncthreads();
  const int lane = tid & 63, wave = tid >> 6;
  double base = 0.0;
  int lastpos = -1;
  for (int t0 = 0; t0 < V; t0 += kStochScan * kStochThreads) {
    const int v0 = t0 + tid * kStochScan;
    float r[kStochScan];
    double local = 0.0;
#pragma unroll
    for (int i = 0; i < kStochScan; ++i) {
      const int v = min(v0 + i, V - 1);
      r[i] = v0 + i < V ? r_of(pr[v], q[v]) : 0.f;
      local += (double)r[i];
      if (r[i] > 0.f) lastpos = v0 + i;
    }
    double incl = local;
    for (int o = 1; o < 64; o <<= 1) {
      const double y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    if (lane == 63) sscan[wave] = incl;
    __syncthreads();
    double before = base;
    for (int w = 0; w < wave; ++w) before += sscan[w];
    double run = before + incl - local;                     // sum of r below v0
    if (run + local > target) {
#pragma unroll
      for (int i = 0; i < kStochScan; ++i) {
        run += (double)r[i];
        if (run > target && v0 + i < V) {
          atomicMin(&spick, v0 + i);
          break;
        }
      }
    }
    double tile = 0.0;
    for (int w = 0; w < kStochThreads / 64; ++w) tile += sscan[w];
    base += tile;
    __syncthreads();                                        // spick settled, sscan reused
    if (spick < V) break;
  }
  if (lastpos >= 0) atomicMax(&slastpos, lastpos);
  __syncthreads();
  if (tid == 0) {
    int pick = spick;
    if (pick >= V) pick = slastpos >= 0 ? slastpos : V - 1;
    accept_len[b] = depth;
    best_node[b] = u;
    bonus_token[b] = pick;
  }
  if (path && tid < n_max) path[row + tid] = tid < depth ? schain[tid] : -1;
}


// ----------------------------------------------------------------------------------
// Several workgroups per sequence.  The vocabulary is cut into P slices of Vs tokens;
// workgroup (b, k) keeps slice k of the current weights r and of the draft row q in
// LDS, so no row is read twice.  Every change of r (a new current node, a residual
// step) ends in an exchange: each slice publishes its float64 total and its last
// token with r > 0, and every workgroup of the sequence adds the P totals in slice
// order -- the same S everywhere, so all of them take the same decisions.  r[x] of a
// candidate token is replayed from the node's p_target[x] through the residual
// scalars (as in the streaming kernel), so no slice has to publish it.
//
// An exchange record is three 64-bit words, each a 32-bit payload beside a 32-bit
// flag (a 64-bit store is single-copy atomic): the total's two halves and the last
// positive token.  Records are stored and polled with device-scope atomics; a cleared
// workspace (flags 0) starts every call.  The P workgroups of a sequence must run at
// the same time: the host keeps B * P within the compute units, and a wait that outlasts
// kSplitSpinMax polls ends the sequence with -1 outputs instead of hanging.
constexpr int kSplitThreads = 256;
constexpr int kSplitWaves = kSplitThreads / 64;
constexpr int kSplitMaxSlices = 64;          // one polling lane per slice
constexpr int kSplitSliceMax = 16384;        // r and q of a slice in LDS: 128 KB
constexpr int kSplitMinSlice = 1024;         // smaller slices would not pay for an exchange
constexpr int kSplitSpinMax = 1 << 20;       // polls of one exchange before giving up
constexpr uint32_t kLLFlag = 1u;

struct SplitPlan {
  int P, Vs;
};

// P = 0: one workgroup per sequence instead
inline SplitPlan split_plan(int B, int V, int cus) {
  int P = min(kSplitMaxSlices, cus / B);
  P = min(P, (V + kSplitMinSlice - 1) / kSplitMinSlice);
  const int p_min = (V + kSplitSliceMax - 1) / kSplitSliceMax;
  if (P < 2 || P < p_min) return {0, 0};
  const int Vs = (V + P - 1) / P;
  return {(V + Vs - 1) / Vs, Vs};                 // every slice non-empty
}

inline int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1) {
    (void)hipGetLastError();
    return 0;
  }
  return cus;
}

inline size_t split_ws_bytes(int B, int n_max, int P) {
  return ((size_t)B * n_max * P * 3 * sizeof(uint64_t) + 255) / 256 * 256;
}

__device__ __forceinline__ void ll_put(uint64_t* p, uint32_t v) {
  __hip_atomic_store(p, ((uint64_t)kLLFlag << 32) | v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t ll_get(uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(256) void split_clear_kernel(uint64_t* __restrict__ x, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) x[i] = 0;
}

__global__ __launch_bounds__(kSplitThreads) void accept_stochastic_split_kernel(
    int n_max, int V, int P, int Vs, const int32_t* __restrict__ parent,
    const uint64_t* __restrict__ anc, const int32_t* __restrict__ n_nodes,
    const int32_t* __restrict__ token, const float* __restrict__ p_target,
    const float* __restrict__ q_draft, const float* __restrict__ u_accept,
    const float* __restrict__ u_bonus, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ best_node, int32_t* __restrict__ bonus_token,
    int32_t* __restrict__ path, uint64_t* __restrict__ xch) {
  __shared__ float sr[kSplitSliceMax];          // r on this slice
  __shared__ float sq[kSplitSliceMax];          // q_draft[u] on this slice
  __shared__ double s_tot[kSplitMaxSlices];     // the last exchange: slice totals
  __shared__ int s_last[kSplitMaxSlices];       //   and last tokens with r > 0
  __shared__ double s_wsum[kSplitWaves];
  __shared__ int s_wlast[kSplitWaves];
  __shared__ float sS32[TV_MAX_NODES];          // fl32(S) of each rejection at the current node
  __shared__ int skids[TV_MAX_NODES], sktok[TV_MAX_NODES];
  __shared__ float skp[TV_MAX_NODES], skq[TV_MAX_NODES], sku[TV_MAX_NODES];
  __shared__ int snkids;
  __shared__ int schain[TV_MAX_NODES];
  __shared__ int s_fail, s_pick;
  const int b = blockIdx.x / P;
  const int k = blockIdx.x - b * P;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const size_t row = (size_t)b * n_max;
  const int v_lo = k * Vs;
  const int nv = min(V, v_lo + Vs) - v_lo;
  const int n = n_nodes[b];
  auto write_invalid = [&]() {
    if (k == 0) {
      if (tid == 0) {
        accept_len[b] = -1;
        best_node[b] = -1;
        bonus_token[b] = -1;
      }
      if (path && tid < n_max) path[row + tid] = -1;
    }
  };
  if (!(n >= 1 && n <= n_max && anc[row] == 1ull)) {   // the same in every slice
    write_invalid();
    return;
  }
  if (tid == 0) s_fail = 0;

  // this slice's float64 total (per-thread strided order, then lanes by butterfly, then
  // waves in order) and last token with r > 0, in every thread
  auto block_total = [&](double s, int last, double& tot, int& lst) {
    for (int o = 32; o > 0; o >>= 1) {
      s += __shfl_xor(s, o);
      last = max(last, __shfl_xor(last, o));
    }
    __syncthreads();                                        // s_wsum free from its last use
    if (lane == 0) {
      s_wsum[wave] = s;
      s_wlast[wave] = last;
    }
    __syncthreads();
    tot = 0.0;
    lst = -1;
#pragma unroll
    for (int w = 0; w < kSplitWaves; ++w) {
      tot += s_wsum[w];
      lst = max(lst, s_wlast[w]);
    }
  };
  // publish (tot, lst) as exchange e of this sequence and return S, the P totals added in
  // slice order; s_tot / s_last then hold every slice's record
  int e = 0;
  auto exchange = [&](double tot, int lst) {
    if (e >= n_max) {                 // a walk tries each node once: at most n exchanges
      if (tid == 0) s_fail = 1;
      __syncthreads();
      return 0.0;
    }
    uint64_t* slot = xch + ((size_t)b * n_max + e) * P * 3;
    ++e;
    if (tid == 0) {
      const uint64_t bits = (uint64_t)__double_as_longlong(tot);
      ll_put(slot + 3 * k, (uint32_t)bits);
      ll_put(slot + 3 * k + 1, (uint32_t)(bits >> 32));
      ll_put(slot + 3 * k + 2, (uint32_t)lst);
    }
    if (wave == 0) {
      bool ok = lane >= P;
      uint64_t w0 = 0, w1 = 0, w2 = 0;
      for (int spins = 0;; ++spins) {
        if (!ok) {
          w0 = ll_get(slot + 3 * lane);
          w1 = ll_get(slot + 3 * lane + 1);
          w2 = ll_get(slot + 3 * lane + 2);
          ok = (uint32_t)(w0 >> 32) == kLLFlag && (uint32_t)(w1 >> 32) == kLLFlag &&
               (uint32_t)(w2 >> 32) == kLLFlag;
        }
        if (__ballot(!ok) == 0ull) break;
        if (spins >= kSplitSpinMax) {
          if (lane == 0) s_fail = 1;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (lane < P) {
        s_tot[lane] = __longlong_as_double((long long)((w1 << 32) | (w0 & 0xFFFFFFFFull)));
        s_last[lane] = (int)(uint32_t)w2;
      }
    }
    __syncthreads();
    double S = 0.0;
    for (int j = 0; j < P; ++j) S += s_tot[j];
    return S;
  };
  // node uu becomes current: its slice of p_target (r) and q_draft into LDS, its
  // children in index order with their tokens, u_accept and the two rows at their
  // tokens; returns S
  auto enter = [&](int uu) {
    const size_t nrow = (row + uu) * (size_t)V;
    if (wave == 0) {
      const bool kid = lane >= 1 && lane < n && parent[row + lane] == uu;
      const uint64_t m = __ballot(kid);
      if (kid) {
        const int j = __popcll(m & ((1ull << lane) - 1ull));
        const int x = token[row + lane];
        const bool in_v = x >= 0 && x < V;
        skids[j] = lane;
        sktok[j] = x;
        sku[j] = u_accept[row + lane];
        skp[j] = in_v ? p_target[nrow + x] : 0.f;
        skq[j] = in_v ? q_draft[nrow + x] : 0.f;
      }
      if (lane == 0) snkids = __popcll(m);
    }
    const float* pr = p_target + nrow + v_lo;
    const float* qr = q_draft + nrow + v_lo;
    double s = 0.0;
    int last = -1;
    for (int i0 = tid; i0 < nv; i0 += kStochBatch * kSplitThreads) {
      float pv[kStochBatch], qv[kStochBatch];
#pragma unroll
      for (int i = 0; i < kStochBatch; ++i) {
        const int v = min(i0 + i * kSplitThreads, nv - 1);
        pv[i] = pr[v];
        qv[i] = qr[v];
      }
#pragma unroll
      for (int i = 0; i < kStochBatch; ++i) {
        const int v = i0 + i * kSplitThreads;
        if (v < nv) {
          sr[v] = pv[i];
          sq[v] = qv[i];
          s += (double)pv[i];
          if (pv[i] > 0.f) last = v_lo + v;
        }
      }
    }
    double tot;
    int lst;
    block_total(s, last, tot, lst);
    return exchange(tot, lst);
  };

  int u = 0, depth = 0, nrej = 0;
  double S = enter(0);
  bool failed = s_fail != 0;
  while (!failed) {
    const int nk = snkids;
    bool moved = false;
    for (int j = 0; j < nk && !failed; ++j) {
      const int c = skids[j];
      const int x = sktok[j];
      const bool in_v = x >= 0 && x < V;
      const float qx = skq[j];
      float rx = skp[j];
      for (int i = 0; i < nrej; ++i) {
#pragma clang fp contract(off)
        const float prod = sS32[i] * qx;
        rx = fmaxf(rx - prod, 0.f);
      }
      if (!in_v) rx = 0.f;
      const bool pass = qx == 0.f ? rx > 0.f : (double)sku[j] * S * (double)qx < (double)rx;
      if (pass) {
        if (tid == 0) schain[depth] = c;
        u = c;
        ++depth;
        nrej = 0;
        moved = true;
        __syncthreads();                                    // the children's entries are read
        S = enter(u);
        failed = s_fail != 0;
        break;
      }
      // residual against q_draft[u]: the product and the difference each rounded to
      // float32 (never contracted into one fma)
      const float S32 = (float)S;
      if (tid == 0) sS32[nrej] = S32;
      ++nrej;
      double s = 0.0;
      int last = -1;
      for (int v = tid; v < nv; v += kSplitThreads) {
#pragma clang fp contract(off)
        const float prod = S32 * sq[v];
        const float nr = fmaxf(sr[v] - prod, 0.f);
        sr[v] = nr;
        s += (double)nr;
        if (nr > 0.f) last = v_lo + v;
      }
      double tot;
      int lst;
      block_total(s, last, tot, lst);
      S = exchange(tot, lst);
      failed = s_fail != 0;
    }
    if (!moved) break;
  }
  if (failed) {
    write_invalid();
    return;
  }

  // bonus: the first token whose running sum of r passes u_bonus * S, the running sum
  // taken over the slices in order (their exchanged totals), then within the slice
  // that crosses, token by token
  const double target = (double)u_bonus[b] * S;
  double run = 0.0;
  int kc = -1;
  for (int j = 0; j < P; ++j) {
    if (run + s_tot[j] > target) {
      kc = j;
      break;
    }
    run += s_tot[j];
  }
  if (k == 0) {
    if (tid == 0) {
      accept_len[b] = depth;
      best_node[b] = u;
      if (kc < 0) {                                         // rounding left none
        int lp = -1;
        for (int j = 0; j < P; ++j) lp = max(lp, s_last[j]);
        bonus_token[b] = lp >= 0 ? lp : V - 1;
      }
    }
    if (path && tid < n_max) path[row + tid] = tid < depth ? schain[tid] : -1;
  }
  if (k != kc) return;
  // thread t scans the contiguous tokens [t*C, t*C + C) of the slice; the threads'
  // sums are combined in thread order
  const int C = (nv + kSplitThreads - 1) / kSplitThreads;
  const int lo = min(tid * C, nv);
  const int hi = min(lo + C, nv);
  double local = 0.0;
  for (int v = lo; v < hi; ++v) local += (double)sr[v];
  double incl = local;
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  __syncthreads();                                          // s_wsum free
  if (lane == 63) s_wsum[wave] = incl;
  if (tid == 0) s_pick = INT32_MAX;
  __syncthreads();
  double before = run;
  for (int w = 0; w < wave; ++w) before += s_wsum[w];
  before += incl - local;                                   // sum of r below lo
  if (lo < hi && before + local > target) {
    for (int v = lo; v < hi; ++v) {
      before += (double)sr[v];
      if (before > target) {
        atomicMin(&s_pick, v_lo + v);
        break;
      }
    }
  }
  __syncthreads();
  if (tid == 0) bonus_token[b] = s_pick != INT32_MAX ? s_pick : s_last[k];
}

}  // namespace tv

TV_API size_t tree_accept_stochastic_workspace_size(int B, int n_max, int vocab) {
  if (B < 1 || n_max < 1 || n_max > TV_MAX_NODES || vocab < 1) return 0;
  const tv::SplitPlan sp = tv::split_plan(B, vocab, tv::device_cus());
  return sp.P ? tv::split_ws_bytes(B, n_max, sp.P) : 0;
}

TV_API tv_status tree_accept_stochastic(int B, int n_max, int vocab, const int32_t* parent,
                                        const uint64_t* anc, const int32_t* n_nodes,
                                        const int32_t* token, const float* p_target,
                                        const float* q_draft, const float* u_accept,
                                        const float* u_bonus, int32_t* accept_len,
                                        int32_t* best_node, int32_t* bonus_token, int32_t* path,
                                        void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!parent || !anc || !n_nodes || !token || !p_target || !q_draft || !u_accept || !u_bonus ||
      !accept_len || !best_node || !bonus_token)
    return TV_ERR_NULL;
  if (B < 1 || n_max < 1 || n_max > TV_MAX_NODES || vocab < 1) return TV_ERR_SHAPE;
  const tv::SplitPlan sp = ws ? tv::split_plan(B, vocab, tv::device_cus()) : tv::SplitPlan{0, 0};
  if (sp.P) {
    const size_t need = tv::split_ws_bytes(B, n_max, sp.P);
    if (ws_bytes < need || (((uintptr_t)ws) & 15) != 0) return TV_ERR_WORKSPACE;
    const size_t words = need / sizeof(uint64_t);
    const int cgrid = (int)std::min<size_t>((words + 255) / 256, 1024);
    hipLaunchKernelGGL(tv::split_clear_kernel, dim3(cgrid), dim3(256), 0, stream, (uint64_t*)ws,
                       words);
    hipLaunchKernelGGL(tv::accept_stochastic_split_kernel, dim3(B * sp.P), dim3(tv::kSplitThreads),
                       0, stream, n_max, vocab, sp.P, sp.Vs, parent, anc, n_nodes, token, p_target,
                       q_draft, u_accept, u_bonus, accept_len, best_node, bonus_token, path,
                       (uint64_t*)ws);
  } else if (vocab <= tv::kStochMaxVocab) {
    hipLaunchKernelGGL(tv::accept_stochastic_kernel, dim3(B), dim3(tv::kStochThreads), 0, stream,
                       n_max, vocab, parent, anc, n_nodes, token, p_target, q_draft, u_accept,
                       u_bonus, accept_len, best_node, bonus_token, path);
  } else {
    hipLaunchKernelGGL(tv::accept_stochastic_stream_kernel, dim3(B), dim3(tv::kStochThreads), 0,
                       stream, n_max, vocab, parent, anc, n_nodes, token, p_target, q_draft,
                       u_accept, u_bonus, accept_len, best_node, bonus_token, path);
  }
  return tv::launch_status();
}
