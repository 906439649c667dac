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

}  // namespace tv

TV_API tv_status tree_accept_stochastic(int B, int n_max, int vocab, const int32_t* parent,
                                        const uint64_t* anc, const int32_t* n_nodes,
                                        const int32_t* token, const float* p_target,
                                        const float* q_draft, const float* u_accept,
                                        const float* u_bonus, int32_t* accept_len,
                                        int32_t* best_node, int32_t* bonus_token, int32_t* path,
                                        hipStream_t stream) {
  if (!parent || !anc || !n_nodes || !token || !p_target || !q_draft || !u_accept || !u_bonus ||
      !accept_len || !best_node || !bonus_token)
    return TV_ERR_NULL;
  if (B < 1 || n_max < 1 || n_max > TV_MAX_NODES || vocab < 1) return TV_ERR_SHAPE;
  if (vocab <= tv::kStochMaxVocab)
    hipLaunchKernelGGL(tv::accept_stochastic_kernel, dim3(B), dim3(tv::kStochThreads), 0, stream,
                       n_max, vocab, parent, anc, n_nodes, token, p_target, q_draft, u_accept,
                       u_bonus, accept_len, best_node, bonus_token, path);
  else
    hipLaunchKernelGGL(tv::accept_stochastic_stream_kernel, dim3(B), dim3(tv::kStochThreads), 0,
                       stream, n_max, vocab, parent, anc, n_nodes, token, p_target, q_draft,
                       u_accept, u_bonus, accept_len, best_node, bonus_token, path);
  return tv::launch_status();
}
