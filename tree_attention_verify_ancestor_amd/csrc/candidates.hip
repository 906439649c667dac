// tree_candidate_logits: the low-rank candidate head of the draft model.
//
// "Technical analysis of EAGLE-4", section "EAGLE-4 architecture": a low-rank
// candidate head first scores the vocabulary in a smaller representation and then
// computes full logits only for the selected candidates, which cuts the cost of
// next-token prediction.  Here the smaller representation is a rank-r factorisation:
// z = A h, a low-rank score Bm[v] . z for every token v, and the exact logit W[v] . h
// for the C tokens of largest score (ties to the lower id).  The output row -- exact
// at the candidates, low-rank elsewhere -- is what tree_expand_rerank reads.
//
// Every dot product is summed in float64 from the exact bf16 (and, for the scores,
// float32) values and rounded once to float32, so the candidate set and every
// output bit are fixed up to the order of a float64 sum.
//
// Four kernels per call:
//   cand_z_kernel      one wave per (row, j): z[row][j], lanes split d, float64 sums
//   cand_score_kernel  four lanes per token (each a quarter of r), two tokens per
//                      thread, rows in groups of 8
//                      with z in LDS: the low-rank scores, written into the logits rows
//   cand_select_kernel one workgroup per row: a lower bound on the C-th best score from
//                      the threads' maxima, the few scores above it gathered in LDS and
//                      ranked there (ties to the lower id); with heavy ties, radix
//                      selection over the whole row on order-preserving keys
//   cand_exact_kernel  one wave per (row, candidate): its exact logit overwrites the
//                      score
// HBM traffic: Bm (V*r*2 B) once per group of 8 rows, the C rows of W per draft row
// (C*d*2 B), A once per row, and the logits rows written then read once.
#include "tv_internal.h"

namespace tv {

constexpr int kCandMaxC = 256;
constexpr int kCandMaxR = 512;
constexpr int kCandGroup = 8;                  // rows per score workgroup
constexpr int kCandSplit = 4;                  // lanes per token in the score kernel
constexpr int kScoreBatch = 8;                 // Bm loads in flight per score thread
constexpr int kCandSelThreads = 1024;
constexpr int kCandGather = 2048;              // keys above the lower bound ranked in LDS
constexpr int kCandCache = 32 * 1024;          // vocabularies whose keys stay in LDS

// Order-preserving map of a float to an unsigned key: a larger value has a larger key,
// -0 and +0 share one key.
__device__ __forceinline__ uint32_t cand_key(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ double wave_sum_d(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Sum over i of a[i] * b[i] for bf16 vectors of length d (d % 8 == 0) by one wave, in
// float64 (each product of two bf16 values is exact in float32); every lane returns it.
// A lane's 16-byte pieces are loaded kDotBatch at a time from clamped addresses
// before any is used, then summed in increasing i as one at a time would be.
constexpr int kDotBatch = 8;
__device__ __forceinline__ double wave_dot_bf16(const __bf16* a, const __bf16* b, int d, int lane) {
  double acc = 0.0;
  for (int i0 = lane * 8; i0 < d; i0 += kDotBatch * kWave * 8) {
    bf16x8 av[kDotBatch], bv[kDotBatch];
#pragma unroll
    for (int q = 0; q < kDotBatch; ++q) {
      const int i = min(i0 + q * kWave * 8, d - 8);
      av[q] = *(const bf16x8*)(a + i);
      bv[q] = *(const bf16x8*)(b + i);
    }
#pragma unroll
    for (int q = 0; q < kDotBatch; ++q) {
      if (i0 + q * kWave * 8 < d) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc += (double)((float)av[q][e] * (float)bv[q][e]);
      }
    }
  }
  return wave_sum_d(acc);
}

__global__ __launch_bounds__(256) void cand_z_kernel(int d, int r, const __bf16* __restrict__ h,
                                                    const __bf16* __restrict__ A, float* __restrict__ z) {
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int j = blockIdx.x * 4 + wave;
  const int row = blockIdx.y;
  if (j >= r) return;                                          // wave-uniform
  const double s = wave_dot_bf16(h + (size_t)row * d, A + (size_t)j * d, d, lane);
  if (lane == 0) z[(size_t)row * r + j] = (float)s;
}

// TPT tokens per thread (token u at v0 + u * 64): each z value is read from LDS and
// converted to float64 once for TPT products.  Every token's sum keeps the order of
// one token per thread: j increasing, then the four quarters combined.
template <int TPT>
__global__ __launch_bounds__(256) void cand_score_kernel(int rows, int r, int V,
                                                        const __bf16* __restrict__ Bm,
                                                        const float* __restrict__ z,
                                                        float* __restrict__ logits) {
  constexpr int kTok = 256 / kCandSplit;
  __shared__ float sz[kCandGroup * kCandMaxR];
  const int g0 = blockIdx.y * kCandGroup;
  const int gr = min(kCandGroup, rows - g0);
  for (int t = threadIdx.x; t < gr * r; t += blockDim.x) sz[t] = z[(size_t)g0 * r + t];
  __syncthreads();
  const int v0 = blockIdx.x * kTok * TPT + threadIdx.x / kCandSplit;
  const int part = threadIdx.x % kCandSplit;
  const int rq = r / kCandSplit;
  double acc[TPT][kCandGroup];
#pragma unroll
  for (int u = 0; u < TPT; ++u)
#pragma unroll
    for (int k = 0; k < kCandGroup; ++k) acc[u][k] = 0.0;
  const float* zp = sz + part * rq;
  for (int jb = 0; jb < rq; jb += 8 * kScoreBatch) {
    bf16x8 bv[TPT][kScoreBatch];
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const __bf16* bp = Bm + (size_t)min(v0 + u * kTok, V - 1) * r + part * rq;
#pragma unroll
      for (int q = 0; q < kScoreBatch; ++q) bv[u][q] = *(const bf16x8*)(bp + min(jb + 8 * q, rq - 8));
    }
#pragma unroll
    for (int q = 0; q < kScoreBatch; ++q) {
      const int j0 = jb + 8 * q;
      if (j0 < rq) {
#pragma unroll
        for (int k = 0; k < kCandGroup; ++k) {
          if (k < gr) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const double zv = (double)zp[k * r + j0 + e];
#pragma unroll
              for (int u = 0; u < TPT; ++u)
                acc[u][k] = fma((double)(float)bv[u][q][e], zv, acc[u][k]);
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < TPT; ++u)
#pragma unroll
    for (int k = 0; k < kCandGroup; ++k) {
      acc[u][k] += __shfl_xor(acc[u][k], 1);
      acc[u][k] += __shfl_xor(acc[u][k], 2);
    }
  if (part == 0) {
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int v = v0 + u * kTok;
      if (v < V) {
#pragma unroll
        for (int k = 0; k < kCandGroup; ++k)
          if (k < gr) logits[(size_t)(g0 + k) * V + v] = (float)acc[u][k];
      }
    }
  }
}

__global__ __launch_bounds__(kCandSelThreads) void cand_select_kernel(
    int V, int C, const float* __restrict__ logits, int32_t* __restrict__ cand) {
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const float* lrow = logits + (size_t)row * V;
  __shared__ uint32_t s_hist[256];
  __shared__ int s_digit, s_before, s_n, s_ties, s_cnt;
  __shared__ uint32_t s_tmax[kCandSelThreads];
  __shared__ uint32_t s_gk[kCandGather];
  __shared__ int s_gi[kCandGather];
  __shared__ int s_ids[kCandMaxC];
  __shared__ uint32_t s_keys[kCandMaxC];
  __shared__ int s_rank[kCandMaxC];
  __shared__ uint32_t s_row[kCandCache];

  // every pass over the row: 32 coalesced key loads per thread in flight, then the
  // body for each (id, key)
  constexpr int kBatch = 32;
  auto for_each_key = [&](auto&& body) {
    for (int base = 0; base < V; base += kBatch * kCandSelThreads) {
      // unconditional loads from clamped addresses, then the select: a load under a
      // condition is compiled into a branch that waits for it before the next one
      float x[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) x[j] = lrow[min(base + j * kCandSelThreads + tid, V - 1)];
      uint32_t u[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int v = base + j * kCandSelThreads + tid;
        u[j] = v < V ? cand_key(x[j]) : 0u;
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int v = base + j * kCandSelThreads + tid;
        if (v < V) body(v, u[j]);
      }
    }
  };
  // Radix selection, 8 bits at a time from the top, over the keys each_key visits:
  // T = the k-th largest key; `need` = how many entries equal to T complete the k.
  auto radix_select = [&](auto&& each_key, int k, uint32_t& T, int& need) {
    uint32_t tmask = 0;
    T = 0;
    need = k;
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (tid < 256) s_hist[tid] = 0u;
      __syncthreads();
      each_key([&](int, uint32_t u) {
        if ((u & tmask) == T) atomicAdd(&s_hist[(u >> shift) & 255u], 1u);
      });
      __syncthreads();
      if (wave == 0) {
        // lane l holds digits 255-4l .. 252-4l, scanned from the top
        uint32_t hv[4], sum = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          hv[q] = s_hist[255 - 4 * lane - q];
          sum += hv[q];
        }
        uint32_t incl = sum;
        for (int o = 1; o < kWave; o <<= 1) {
          const uint32_t t = __shfl_up(incl, o);
          if (lane >= o) incl += t;
        }
        const uint32_t before = incl - sum;
        if (before < (uint32_t)need && (uint32_t)need <= incl) {
          uint32_t cum = before;
          int dg = 255 - 4 * lane;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (cum + hv[q] >= (uint32_t)need) {
              dg = 255 - 4 * lane - q;
              break;
            }
            cum += hv[q];
          }
          s_digit = dg;
          s_before = (int)cum;
        }
      }
      __syncthreads();
      T |= (uint32_t)s_digit << shift;
      tmask |= 255u << shift;
      need -= s_before;
      __syncthreads();
    }
  };

  // the row's keys stay in LDS when they fit: one pass over global memory, the others
  // over LDS
  const bool cached = V <= kCandCache;
  auto each_key = [&](auto&& body) {
    if (cached) {
      for (int v = tid; v < V; v += kCandSelThreads) body(v, s_row[v]);
    } else {
      for_each_key(body);
    }
  };

  // A lower bound first: each thread's largest key, and T0 the C-th largest of those
  // (C threads hold a key >= T0, so the C best keys are all >= T0).  The keys >= T0
  // are usually few: they are gathered in LDS and ranked there.
  uint32_t tmax = 0;
  for_each_key([&](int v, uint32_t u) {
    tmax = max(tmax, u);
    if (cached) s_row[v] = u;
  });
  s_tmax[tid] = tmax;
  if (tid == 0) s_cnt = 0;
  __syncthreads();
  uint32_t T0;
  int need0;
  radix_select([&](auto&& body) { body(tid, s_tmax[tid]); }, C, T0, need0);
  int ge = 0;
  each_key([&](int, uint32_t u) { ge += u >= T0; });
  if (ge) atomicAdd(&s_cnt, ge);
  __syncthreads();
  const int n_ge = s_cnt;
  if (n_ge <= kCandGather) {
    if (tid == 0) s_n = 0;
    __syncthreads();
    each_key([&](int v, uint32_t u) {
      if (u >= T0) {
        const int slot = atomicAdd(&s_n, 1);
        s_gk[slot] = u;
        s_gi[slot] = v;
      }
    });
    __syncthreads();
    // rank by (larger key, lower id); the first C are the candidates
    for (int gi = tid; gi < n_ge; gi += kCandSelThreads) {
      const uint32_t km = s_gk[gi];
      const int im = s_gi[gi];
      int rk = 0;
      for (int o = 0; o < n_ge; ++o)                 // branch-free: no exec-mask jumps
        rk += (int)(s_gk[o] > km) | ((int)(s_gk[o] == km) & (int)(s_gi[o] < im));
      if (rk < C) s_rank[rk] = im;
    }
    __syncthreads();
    if (tid < C) cand[(size_t)row * C + tid] = s_rank[tid];
    return;
  }

  // Many keys >= T0 (heavy ties): the exact selection over the whole row.  Selected:
  // keys above T, and the `need` lowest ids with key T.  Usually every entry with key
  // T is taken, so no order among them is needed; otherwise one wave takes them in id
  // order.
  uint32_t T;
  int need;
  radix_select(for_each_key, C, T, need);
  if (tid == 0) {
    s_n = 0;
    s_ties = 0;
  }
  __syncthreads();
  int ties = 0;
  for_each_key([&](int, uint32_t u) { ties += u == T; });
  if (ties) atomicAdd(&s_ties, ties);
  __syncthreads();
  const bool take_all = s_ties == need;
  for_each_key([&](int v, uint32_t u) {
    if (u > T || (take_all && u == T)) {
      const int slot = atomicAdd(&s_n, 1);
      s_ids[slot] = v;
      s_keys[slot] = u;
    }
  });
  if (!take_all && wave == 0) {
    int taken = 0;
    for (int base = 0; base < V && taken < need; base += kWave) {
      const int v = base + lane;
      const bool t = v < V && cand_key(lrow[v]) == T;
      const uint64_t bal = __ballot(t);
      const int before = __popcll(bal & ((1ull << lane) - 1ull));
      if (t && taken + before < need) {
        const int slot = atomicAdd(&s_n, 1);
        s_ids[slot] = v;
        s_keys[slot] = T;
      }
      taken += __popcll(bal);
    }
  }
  __syncthreads();
  // rank the C selected best first: larger key, then lower id
  if (tid < C) {
    const uint32_t km = s_keys[tid];
    const int im = s_ids[tid];
    int rk = 0;
    for (int o = 0; o < C; ++o)
      rk += (int)(s_keys[o] > km) | ((int)(s_keys[o] == km) & (int)(s_ids[o] < im));
    s_rank[rk] = im;
  }
  __syncthreads();
  if (tid < C) cand[(size_t)row * C + tid] = s_rank[tid];
}

// The exact logit of each candidate, one wave per (row, candidate).
__global__ __launch_bounds__(256) void cand_exact_kernel(int d, int V, int C,
                                                        const __bf16* __restrict__ h,
                                                        const __bf16* __restrict__ W,
                                                        const int32_t* __restrict__ cand,
                                                        float* __restrict__ logits) {
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int c = blockIdx.x * 4 + wave;
  const int row = blockIdx.y;
  if (c >= C) return;                                          // wave-uniform
  const int v = cand[(size_t)row * C + c];
  const double s = wave_dot_bf16(W + (size_t)v * d, h + (size_t)row * d, d, lane);
  if (lane == 0) logits[(size_t)row * V + v] = (float)s;
}

}  // namespace tv

TV_API size_t tree_candidate_workspace_size(int rows, int r) {
  if (rows < 1 || r < 1 || r > tv::kCandMaxR) return 0;
  return ((size_t)rows * r * sizeof(float) + 255) / 256 * 256;
}

TV_API tv_status tree_candidate_logits(int rows, int d, int r, int vocab, int C, const void* h,
                                       const void* A, const void* Bm, const void* W,
                                       float* logits, int32_t* cand, void* ws, size_t ws_bytes,
                                       hipStream_t stream) {
  if (!h || !A || !Bm || !W || !logits || !cand) return TV_ERR_NULL;
  if (rows < 1 || d < 8 || d % 8 != 0 || r < 32 || r % 32 != 0 || r > tv::kCandMaxR ||
      C < 1 || C > tv::kCandMaxC || vocab < C)
    return TV_ERR_SHAPE;
  if ((((uintptr_t)h | (uintptr_t)A | (uintptr_t)Bm | (uintptr_t)W) & 15) != 0)
    return TV_ERR_UNSUPPORTED;
  const size_t need = tree_candidate_workspace_size(rows, r);
  if (!ws || ws_bytes < need) return TV_ERR_WORKSPACE;
  float* z = (float*)ws;
  hipLaunchKernelGGL(tv::cand_z_kernel, dim3((r + 3) / 4, rows), dim3(256), 0, stream, d, r,
                     (const __bf16*)h, (const __bf16*)A, z);
  constexpr int kTokensPerWg = 256 / tv::kCandSplit * 2;
  hipLaunchKernelGGL(tv::cand_score_kernel<2>,
                     dim3((vocab + kTokensPerWg - 1) / kTokensPerWg,
                          (rows + tv::kCandGroup - 1) / tv::kCandGroup),
                     dim3(256), 0, stream, rows, r, vocab, (const __bf16*)Bm, (const float*)z, logits);
  hipLaunchKernelGGL(tv::cand_select_kernel, dim3(rows), dim3(tv::kCandSelThreads), 0, stream,
                     vocab, C, (const float*)logits, cand);
  hipLaunchKernelGGL(tv::cand_exact_kernel, dim3((C + 3) / 4, rows), dim3(256), 0, stream, d, vocab,
                     C, (const __bf16*)h, (const __bf16*)W, (const int32_t*)cand, logits);
  return tv::launch_status();
}
