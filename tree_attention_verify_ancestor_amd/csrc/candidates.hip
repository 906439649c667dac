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
// Three kernels per call:
//   cand_z_kernel      one wave per (row, j): z[row][j], lanes split d, float64 sums
//   cand_score_kernel  one thread per token, rows in groups of 32 with z in LDS: the
//                      low-rank scores, written into the logits rows
//   cand_select_kernel one workgroup per row: the C best scores by radix selection on
//                      order-preserving keys (ties to the lower id), the candidates
//                      ranked best first, then one wave per candidate computes its
//                      exact logit and overwrites the score
// HBM traffic: Bm (V*r*2 B) once per group of 32 rows, the C rows of W per draft row
// (C*d*2 B), A once per row, and the logits rows written then read once.
#include "tv_internal.h"

namespace tv {

constexpr int kCandMaxC = 256;
constexpr int kCandMaxR = 512;
constexpr int kCandGroup = 32;                 // rows per score workgroup
constexpr int kCandSelThreads = 1024;
constexpr int kCandSelWaves = kCandSelThreads / kWave;

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
__device__ __forceinline__ double wave_dot_bf16(const __bf16* a, const __bf16* b, int d, int lane) {
  double acc = 0.0;
  for (int i = lane * 8; i < d; i += kWave * 8) {
    const bf16x8 av = *(const bf16x8*)(a + i);
    const bf16x8 bv = *(const bf16x8*)(b + i);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (double)((float)av[e] * (float)bv[e]);
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

__global__ __launch_bounds__(256) void cand_score_kernel(int rows, int r, int V,
                                                        const __bf16* __restrict__ Bm,
                                                        const float* __restrict__ z,
                                                        float* __restrict__ logits) {
  __shared__ float sz[kCandGroup * kCandMaxR];
  const int g0 = blockIdx.y * kCandGroup;
  const int gr = min(kCandGroup, rows - g0);
  for (int t = threadIdx.x; t < gr * r; t += blockDim.x) sz[t] = z[(size_t)g0 * r + t];
  __syncthreads();
  const int v = blockIdx.x * blockDim.x + threadIdx.x;
  if (v >= V) return;
  double acc[kCandGroup];
#pragma unroll
  for (int k = 0; k < kCandGroup; ++k) acc[k] = 0.0;
  const __bf16* bp = Bm + (size_t)v * r;
  for (int j0 = 0; j0 < r; j0 += 8) {
    const bf16x8 bv = *(const bf16x8*)(bp + j0);
#pragma unroll
    for (int k = 0; k < kCandGroup; ++k) {
      if (k < gr) {
#pragma unroll
        for (int e = 0; e < 8; ++e)                    // bf16 x float32: exact in float64
          acc[k] = fma((double)(float)bv[e], (double)sz[k * r + j0 + e], acc[k]);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kCandGroup; ++k)
    if (k < gr) logits[(size_t)(g0 + k) * V + v] = (float)acc[k];
}

__global__ __launch_bounds__(kCandSelThreads) void cand_select_kernel(
    int d, int V, int C, const __bf16* __restrict__ h, const __bf16* __restrict__ W,
    float* __restrict__ logits, int32_t* __restrict__ cand) {
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  float* lrow = logits + (size_t)row * V;
  __shared__ uint32_t s_hist[256];
  __shared__ int s_digit, s_before, s_n;
  __shared__ int s_wtot[kCandSelWaves];
  __shared__ int s_ids[kCandMaxC];
  __shared__ uint32_t s_keys[kCandMaxC];
  __shared__ int s_rank[kCandMaxC];

  // T = the C-th largest key, 8 bits at a time from the top; `need` ends as the number
  // of entries equal to T that are selected (the lowest ids among them)
  uint32_t T = 0, tmask = 0;
  int need = C;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) s_hist[tid] = 0u;
    __syncthreads();
    for (int v = tid; v < V; v += kCandSelThreads) {
      const uint32_t u = cand_key(lrow[v]);
      if ((u & tmask) == T) atomicAdd(&s_hist[(u >> shift) & 255u], 1u);
    }
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

  // selected: keys above T, and the `need` lowest ids with key T (each thread scans a
  // contiguous segment; a block scan of the per-thread tie counts orders the ties)
  if (tid == 0) s_n = 0;
  const int seg = (V + kCandSelThreads - 1) / kCandSelThreads;
  const int cs = tid * seg;
  int ties = 0;
  for (int q = 0; q < seg; ++q)
    if (cs + q < V && cand_key(lrow[cs + q]) == T) ++ties;
  int incl = ties;
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(incl, o);
    if (lane >= o) incl += t;
  }
  if (lane == kWave - 1) s_wtot[wave] = incl;
  __syncthreads();
  int trank = incl - ties;
  for (int w = 0; w < wave; ++w) trank += s_wtot[w];
  for (int q = 0; q < seg; ++q) {
    const int v = cs + q;
    if (v >= V) break;
    const uint32_t u = cand_key(lrow[v]);
    const bool take = u > T || (u == T && trank < need);
    if (u == T) ++trank;
    if (take) {
      const int slot = atomicAdd(&s_n, 1);
      s_ids[slot] = v;
      s_keys[slot] = u;
    }
  }
  __syncthreads();
  // rank the C selected best first: larger key, then lower id
  if (tid < C) {
    const uint32_t km = s_keys[tid];
    const int im = s_ids[tid];
    int rk = 0;
    for (int o = 0; o < C; ++o) rk += s_keys[o] > km || (s_keys[o] == km && s_ids[o] < im);
    s_rank[rk] = im;
  }
  __syncthreads();
  if (tid < C) cand[(size_t)row * C + tid] = s_rank[tid];
  // exact logits of the candidates (every read of the scores is done)
  for (int c = wave; c < C; c += kCandSelWaves) {
    const int v = s_rank[c];
    const double s = wave_dot_bf16(W + (size_t)v * d, h + (size_t)row * d, d, lane);
    if (lane == 0) lrow[v] = (float)s;
  }
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
  if (rows < 1 || d < 8 || d % 8 != 0 || r < 8 || r % 8 != 0 || r > tv::kCandMaxR ||
      C < 1 || C > tv::kCandMaxC || vocab < C)
    return TV_ERR_SHAPE;
  if ((((uintptr_t)h | (uintptr_t)A | (uintptr_t)Bm | (uintptr_t)W) & 15) != 0)
    return TV_ERR_UNSUPPORTED;
  const size_t need = tree_candidate_workspace_size(rows, r);
  if (!ws || ws_bytes < need) return TV_ERR_WORKSPACE;
  float* z = (float*)ws;
  hipLaunchKernelGGL(tv::cand_z_kernel, dim3((r + 3) / 4, rows), dim3(256), 0, stream, d, r,
                     (const __bf16*)h, (const __bf16*)A, z);
  hipLaunchKernelGGL(tv::cand_score_kernel,
                     dim3((vocab + 255) / 256, (rows + tv::kCandGroup - 1) / tv::kCandGroup),
                     dim3(256), 0, stream, rows, r, vocab, (const __bf16*)Bm, (const float*)z, logits);
  hipLaunchKernelGGL(tv::cand_select_kernel, dim3(rows), dim3(tv::kCandSelThreads), 0, stream, d,
                     vocab, C, (const __bf16*)h, (const __bf16*)W, logits, cand);
  return tv::launch_status();
}
