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
// Two kernels per call:
//   expand_rows_kernel   one workgroup per (sequence, frontier row): streams the
//                        vocabulary once for max, finiteness and a per-thread top-k,
//                        once more (L2-resident) for the float64 sum of exponentials,
//                        and appends k children to the sequence's pool.
//   expand_select_kernel one workgroup per sequence: ranks this level's children
//                        into the next frontier; on the last level ranks the whole
//                        pool, keeps the best m-1 and writes the tree in (depth,
//                        creation) order with remapped parents.
// Workspace per sequence: a header {status, pool count, next step}, the frontier
// (pool slots by rank), one bad-row flag per frontier row, then the pool of
// {parent slot, token, score, depth} records in creation order.
#include <math.h>

#include "tv_internal.h"

namespace tv {

constexpr int kTopKMax = 16;
constexpr int kPoolMax = 4096;
constexpr int kRowThreads = 512;
constexpr int kSelThreads = 1024;

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
  int32_t frontier[kTopKMax];
  int32_t row_bad[kTopKMax];
};

__host__ __device__ inline int64_t pool_capacity(int k, int max_steps) {
  return (int64_t)k + (int64_t)(max_steps - 1) * k * k;
}
__host__ __device__ inline size_t seq_stride_bytes(int k, int max_steps) {
  size_t s = sizeof(SeqHeader) + (size_t)pool_capacity(k, max_steps) * sizeof(PoolEntry);
  return (s + 255) & ~(size_t)255;
}
// pool slots used before level `step` (1-based): k after level 1, k*k per level after
__host__ __device__ inline int pool_base(int k, int step) {
  return step == 1 ? 0 : k + (step - 2) * k * k;
}

__device__ __forceinline__ uint32_t ordered(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);  // -0 -> +0 so equal values compare equal
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// a (value, id) pair as one integer: larger value first, then lower id
__device__ __forceinline__ uint64_t rank_key(float v, int id) {
  return ((uint64_t)ordered(v) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)id);
}

// Insert (v, id) into a list sorted best first; ids arrive in increasing order.
__device__ __forceinline__ void topk_insert(float (&val)[kTopKMax], int (&idx)[kTopKMax], int k,
                                            float v, int id) {
  if (!(v > val[k - 1])) return;
  float cv = v;
  int ci = id;
#pragma unroll
  for (int j = 0; j < kTopKMax; ++j) {
    if (j < k) {
      const bool beats = cv > val[j] || (cv == val[j] && ci < idx[j]);
      if (beats) {
        const float tv = val[j];
        const int ti = idx[j];
        val[j] = cv;
        idx[j] = ci;
        cv = tv;
        ci = ti;
      }
    }
  }
}

// k rounds of a wave-wide maximum over each lane's list head; the winner pops its head.
// Result (valid in every lane): out_v/out_i[0..k) best first.
__device__ __forceinline__ void wave_merge_topk(float (&val)[kTopKMax], int (&idx)[kTopKMax], int k,
                                                float* out_v, int* out_i, bool write) {
  for (int t = 0; t < k; ++t) {
    const uint64_t mine = idx[0] == INT32_MAX ? 0ull : rank_key(val[0], idx[0]);
    const uint64_t best = wave_max_u64(mine);
    if (best != 0ull && mine == best) {
#pragma unroll
      for (int j = 0; j < kTopKMax - 1; ++j) {
        val[j] = val[j + 1];
        idx[j] = idx[j + 1];
      }
      val[kTopKMax - 1] = -INFINITY;
      idx[kTopKMax - 1] = INT32_MAX;
    }
    if (write && lane_id() == 0) {
      if (best == 0ull) {
        out_v[t] = -INFINITY;
        out_i[t] = INT32_MAX;
      } else {
        const uint32_t o = (uint32_t)(best >> 32);
        const uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
        out_v[t] = __uint_as_float(u);
        out_i[t] = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFu));
      }
    }
  }
}

__global__ __launch_bounds__(kRowThreads) void expand_rows_kernel(
    char* __restrict__ ws, size_t stride, int k, int step, int rows, int vocab,
    const float* __restrict__ logits) {
  const int r = blockIdx.x;
  const int b = blockIdx.y;
  SeqHeader* hdr = (SeqHeader*)(ws + (size_t)b * stride);
  PoolEntry* pool = (PoolEntry*)(ws + (size_t)b * stride + sizeof(SeqHeader));
  if (step > 1 && (hdr->status != TV_SEQ_OK || hdr->next_step != step)) return;

  __shared__ float s_wv[kRowThreads / kWave][kTopKMax];
  __shared__ int s_wi[kRowThreads / kWave][kTopKMax];
  __shared__ float s_max[kRowThreads / kWave];
  __shared__ double s_sum[kRowThreads / kWave];
  __shared__ int s_bad[kRowThreads / kWave];
  __shared__ float s_topv[kTopKMax];
  __shared__ int s_topi[kTopKMax];

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const float* row = logits + ((size_t)b * rows + r) * (size_t)vocab;

  float val[kTopKMax];
  int idx[kTopKMax];
#pragma unroll
  for (int j = 0; j < kTopKMax; ++j) {
    val[j] = -INFINITY;
    idx[j] = INT32_MAX;
  }
  float mx = -INFINITY;
  bool bad = false;

  const bool vec = (vocab % 4 == 0) && ((((uintptr_t)row) & 15) == 0);
  if (vec) {
    const float4* row4 = (const float4*)row;
    const int n4 = vocab / 4;
    for (int q = tid; q < n4; q += kRowThreads) {
      const float4 x = row4[q];
      const float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v = xs[e];
        bad |= !isfinite(v);
        mx = fmaxf(mx, v);
        topk_insert(val, idx, k, v, 4 * q + e);
      }
    }
  } else {
    for (int v = tid; v < vocab; v += kRowThreads) {
      const float x = row[v];
      bad |= !isfinite(x);
      mx = fmaxf(mx, x);
      topk_insert(val, idx, k, x, v);
    }
  }

  // block max and finiteness
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
  const bool wbad = __ballot(bad) != 0ull;
  if (lane_id() == 0) {
    s_max[wave] = mx;
    s_bad[wave] = wbad;
  }
  wave_merge_topk(val, idx, k, s_wv[wave], s_wi[wave], lane_id() == 0);
  __syncthreads();
  float M = s_max[0];
  int anybad = s_bad[0];
  for (int w = 1; w < kRowThreads / kWave; ++w) {
    M = fmaxf(M, s_max[w]);
    anybad |= s_bad[w];
  }
  if (anybad) {
    if (tid == 0) hdr->row_bad[r] = 1;
    return;
  }

  // second pass: float64 sum of exp(l - max); the row is still in L2
  double sum = 0.0;
  const double Md = (double)M;
  if (vec) {
    const float4* row4 = (const float4*)row;
    const int n4 = vocab / 4;
    for (int q = tid; q < n4; q += kRowThreads) {
      const float4 x = row4[q];
      sum += exp((double)x.x - Md) + exp((double)x.y - Md) + exp((double)x.z - Md) +
             exp((double)x.w - Md);
    }
  } else {
    for (int v = tid; v < vocab; v += kRowThreads) sum += exp((double)row[v] - Md);
  }
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
  if (lane_id() == 0) s_sum[wave] = sum;

  // merge the per-wave lists (wave 0; lane l takes candidates l and l+64)
  if (wave == 0) {
    const int nc = (kRowThreads / kWave) * k;
    float v2[kTopKMax];
    int i2[kTopKMax];
#pragma unroll
    for (int j = 0; j < kTopKMax; ++j) {
      v2[j] = -INFINITY;
      i2[j] = INT32_MAX;
    }
    for (int c = lane_id(); c < nc; c += kWave) {
      const float cv = s_wv[c / k][c % k];
      const int ci = s_wi[c / k][c % k];
      if (ci == INT32_MAX) continue;
      // small insertion by full comparison (candidate ids are not ordered here)
      float pv = cv;
      int pi = ci;
#pragma unroll
      for (int j = 0; j < kTopKMax; ++j) {
        if (j < k) {
          const bool beats = pv > v2[j] || (pv == v2[j] && pi < i2[j]);
          if (beats) {
            const float tv = v2[j];
            const int ti = i2[j];
            v2[j] = pv;
            i2[j] = pi;
            pv = tv;
            pi = ti;
          }
        }
      }
    }
    wave_merge_topk(v2, i2, k, s_topv, s_topi, lane_id() == 0);
  }
  __syncthreads();
  if (tid < k) {
    double S = 0.0;
    for (int w = 0; w < kRowThreads / kWave; ++w) S += s_sum[w];
    const float lse32 = (float)(Md + log(S));
    int pslot = -1;
    float pscore = 0.f;
    int pdepth = 0;
    if (step > 1) {
      pslot = hdr->frontier[r];
      pslot = pslot < 0 ? 0 : (pslot >= pool_base(k, step) ? pool_base(k, step) - 1 : pslot);
      pscore = pool[pslot].score;
      pdepth = pool[pslot].depth;
    }
    const float logp = __fsub_rn(s_topv[tid], lse32);
    PoolEntry e;
    e.parent_slot = pslot;
    e.token = s_topi[tid];
    e.score = __fadd_rn(pscore, logp);
    e.depth = pdepth + 1;
    pool[pool_base(k, step) + r * k + tid] = e;
    if (tid == 0) hdr->row_bad[r] = 0;
  }
}

__device__ __forceinline__ bool better(float sa, int ia, float sb, int ib) {
  return sa > sb || (sa == sb && ia < ib);
}

__global__ __launch_bounds__(kSelThreads) void expand_select_kernel(
    char* __restrict__ ws, size_t stride, int k, int step, int rows, int final_m,
    const int32_t* __restrict__ m_per_seq, const int32_t* __restrict__ root_token, int n_max,
    int32_t* __restrict__ parent, int32_t* __restrict__ token, float* __restrict__ score,
    int32_t* __restrict__ n_nodes, int32_t* __restrict__ frontier_token,
    int32_t* __restrict__ seq_status) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  SeqHeader* hdr = (SeqHeader*)(ws + (size_t)b * stride);
  PoolEntry* pool = (PoolEntry*)(ws + (size_t)b * stride + sizeof(SeqHeader));

  __shared__ float s_score[kPoolMax];
  __shared__ short s_pos[kPoolMax];
  __shared__ int s_front[kTopKMax];
  __shared__ int s_kept[TV_MAX_NODES];
  __shared__ int s_nkept;
  __shared__ int s_status;

  const int base = pool_base(k, step);
  const int added = rows * k;
  const int count = base + added;
  if (tid == 0) {
    int st = TV_SEQ_OK;
    if (step > 1) {
      st = hdr->status;
      if (st == TV_SEQ_OK && (hdr->next_step != step || hdr->count != base)) st = TV_SEQ_BAD_STATE;
    }
    if (st == TV_SEQ_OK) {
      for (int rr = 0; rr < rows; ++rr)
        if (hdr->row_bad[rr]) st = TV_SEQ_NONFINITE;
    }
    if (st == TV_SEQ_OK && final_m > 0) {
      const int m = m_per_seq ? m_per_seq[b] : final_m;
      if (m < 1 || m > n_max) st = TV_SEQ_BAD_N;
    }
    s_status = st;
    s_nkept = 0;
  }
  if (tid < kTopKMax) s_front[tid] = -1;
  __syncthreads();
  const int st = s_status;

  if (st == TV_SEQ_OK) {
    for (int c = tid; c < added; c += kSelThreads) s_score[c] = pool[base + c].score;
    __syncthreads();
    // next frontier: the k best children of this level by (score desc, creation asc)
    for (int c = tid; c < added; c += kSelThreads) {
      const float sc = s_score[c];
      int rank = 0;
      for (int o = 0; o < added; ++o) rank += better(s_score[o], o, sc, c);
      if (rank < k) s_front[rank] = base + c;
    }
    __syncthreads();
    if (tid < k) {
      hdr->frontier[tid] = s_front[tid];
      if (frontier_token) frontier_token[(size_t)b * k + tid] = pool[s_front[tid]].token;
    }
  } else if (frontier_token && tid < k) {
    frontier_token[(size_t)b * k + tid] = -1;
  }

  if (final_m > 0) {
    __syncthreads();
    int keep = 0;
    if (st == TV_SEQ_OK) {
      const int m = m_per_seq ? m_per_seq[b] : final_m;
      keep = min(m - 1, count);
      for (int c = tid; c < count; c += kSelThreads) {
        s_score[c] = pool[c].score;
        s_pos[c] = -1;
      }
      __syncthreads();
      for (int c = tid; c < count; c += kSelThreads) {
        const float sc = s_score[c];
        int rank = 0;
        for (int o = 0; o < count && rank < keep; ++o) rank += better(s_score[o], o, sc, c);
        if (rank < keep) s_kept[atomicAdd(&s_nkept, 1)] = c;
      }
      __syncthreads();
      // output position: root first, then by (depth, creation)
      if (tid < keep) {
        const int me = s_kept[tid];
        const int dme = pool[me].depth;
        int before = 0;
        for (int o = 0; o < keep; ++o) {
          const int other = s_kept[o];
          const int dot = pool[other].depth;
          before += (dot < dme) || (dot == dme && other < me);
        }
        s_pos[me] = (short)(1 + before);
      }
      __syncthreads();
      if (tid < keep) {
        const int me = s_kept[tid];
        const int pos = s_pos[me];
        const PoolEntry e = pool[me];
        const size_t o = (size_t)b * n_max + pos;
        parent[o] = e.parent_slot < 0 ? 0 : s_pos[e.parent_slot];
        token[o] = e.token;
        score[o] = e.score;
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

}  // namespace tv

TV_API size_t tree_expand_workspace_size(int B, int k, int max_steps) {
  if (B < 1 || k < 1 || k > tv::kTopKMax || max_steps < 1) return 0;
  if (tv::pool_capacity(k, max_steps) > tv::kPoolMax) return 0;
  return (size_t)B * tv::seq_stride_bytes(k, max_steps);
}

TV_API tv_status tree_expand_rerank(void* ws, size_t ws_bytes, int B, int k, int max_steps,
                                    int step, int vocab, const float* logits, int final_m,
                                    const int32_t* m_per_seq, const int32_t* root_token, int n_max,
                                    int32_t* parent, int32_t* token, float* score,
                                    int32_t* n_nodes, int32_t* frontier_token, int32_t* seq_status,
                                    hipStream_t stream) {
  if (!logits) return TV_ERR_NULL;
  if (B < 1 || k < 1 || k > tv::kTopKMax || max_steps < 1 || step < 1 || step > max_steps ||
      vocab < k || n_max < 1 || n_max > TV_MAX_NODES || final_m < 0 || final_m > n_max)
    return TV_ERR_SHAPE;
  if (tv::pool_capacity(k, max_steps) > tv::kPoolMax) return TV_ERR_SHAPE;
  if (final_m > 0 && (!parent || !token || !score || !n_nodes || !root_token)) return TV_ERR_NULL;
  const size_t need = tree_expand_workspace_size(B, k, max_steps);
  if (!ws || ws_bytes < need) return TV_ERR_WORKSPACE;
  const size_t stride = tv::seq_stride_bytes(k, max_steps);
  const int rows = step == 1 ? 1 : k;
  hipLaunchKernelGGL(tv::expand_rows_kernel, dim3(rows, B), dim3(tv::kRowThreads), 0, stream,
                     (char*)ws, stride, k, step, rows, vocab, logits);
  tv_status s = tv::launch_status();
  if (s != TV_OK) return s;
  hipLaunchKernelGGL(tv::expand_select_kernel, dim3(B), dim3(tv::kSelThreads), 0, stream,
                     (char*)ws, stride, k, step, rows, final_m, m_per_seq, root_token, n_max,
                     parent, token, score, n_nodes, frontier_token, seq_status);
  return tv::launch_status();
}
