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
//   cand_z_kernel      one wave per (row, j): z[row][j], lanes split d, float64 sums;
//                      stored as float64 (the float32 value upcast) at [group][j][16],
//                      rows padded to whole groups of 16 with zeros
//   cand_score_kernel  64 tokens per workgroup: their Bm rows are read once, coalesced,
//                      into LDS; each of 4 waves takes a quarter of the group's rows, a
//                      lane one token, and sums over j in float64 with z read as scalars
//                      (the same for every lane): the low-rank scores, written into the
//                      logits rows.  At 10 rows this is about 10 flops per Bm byte, the
//                      float64 ridge of the vector ALUs, so exact sums cost about the
//                      HBM time.
//   cand_select_kernel one workgroup per row: the C-th largest of the score groups'
//                      maxima (one group per score wave, recorded by the score kernel)
//                      bounds the C-th best score from below; only the groups whose
//                      maximum reaches the bound are read, their scores at or above it
//                      gathered in LDS and ranked there (ties to the lower id); with
//                      heavy ties, radix selection over the whole row on
//                      order-preserving keys
//   cand_exact_kernel  one wave per (row, candidate): its exact logit overwrites the
//                      score
// HBM traffic: Bm (V*r*2 B) once per group of 16 rows, the C rows of W per draft row
// (C*d*2 B), A once per row, and the logits rows written then read once.
#include "tv_internal.h"

namespace tv {

constexpr int kCandMaxC = 256;
constexpr int kCandMaxR = 512;
constexpr int kCandGroup = 16;                 // rows per score pass (z padded to whole groups)
constexpr int kScoreWaves = 4;                 // waves per score workgroup
constexpr int kCandSelThreads = 1024;
constexpr int kCandGather = 2048;              // keys above the lower bound ranked in LDS
constexpr int kCandGroups = kCandSelThreads / 4;   // groups of four threads for the lower bound
constexpr int kMinTokW = 16;                   // the fewest tokens a score wave covers
constexpr int kGmaxPerThread = 8;              // score-group maxima per selection thread
constexpr int kCandQualMax = 512;              // score groups read by the bounded selection

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

// z[row][j] rounded once to float32, stored upcast at z64[(row/16 * r + j) * 16 + row%16];
// rows past the last one (up to the group's end) hold 0
__global__ __launch_bounds__(256) void cand_z_kernel(int rows, int d, int r, const __bf16* __restrict__ h,
                                                    const __bf16* __restrict__ A, double* __restrict__ z64) {
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int j = blockIdx.x * 4 + wave;
  const int row = blockIdx.y;
  if (j >= r) return;                                          // wave-uniform
  const double s = row < rows ? wave_dot_bf16(h + (size_t)row * d, A + (size_t)j * d, d, lane) : 0.0;
  if (lane == 0)
    z64[((size_t)(row / kCandGroup) * r + j) * kCandGroup + row % kCandGroup] = (double)(float)s;
}

// Eight lanes share a token row: lane (t, p), t = lane / 8, p = lane % 8, takes the
// 8-j chunks p, p + 8, p + 16, ... of the rows of its TPT tokens t0 + t + 8u (u < TPT),
// so the eight lanes' 16-byte loads of one chunk index cover a whole 128-byte line of a
// row.  ROWS (even) rows of the group, z zero past the last row; z comes from LDS, one
// 16-byte read giving two rows of one j, shared by the TPT tokens.  Each token's sum: a
// lane's j in increasing order, then the eight lanes combined by neighbours, pairs, then
// halves -- one fixed order.
// Besides the scores, each wave records, per row, the largest key (cand_key) of its
// 8 * TPT tokens (a score group) in gmax[row][group], group = the wave's index in the
// grid; tokens past the vocabulary count as key 0.
// WPE: waves per SIMD the register allocation must leave room for (8 rows fit three
// waves in 168 registers without spills; 10 rows would spill)
template <int ROWS, int TPT, int RMAX, int WPE>
__global__ __launch_bounds__(kScoreWaves * kWave) __attribute__((amdgpu_waves_per_eu(WPE))) void cand_score_kernel(
    int rows, int r, int V, const __bf16* __restrict__ Bm, const double* __restrict__ z64,
    float* __restrict__ logits, uint32_t* __restrict__ gmax, int ng) {
  static_assert(ROWS % 2 == 0 && ROWS <= kCandGroup, "rows in pairs, at most one group");
  constexpr int kQMax = (RMAX + 63) / 64;             // chunks per lane at most
  // lane part p's z: zs[p * kPart + (q * 8 + e) * ROWS + row] = z[row][(8q + p) * 8 + e];
  // each part padded by 16 bytes, so the eight parts of one read fall on distinct banks
  constexpr int kPart = kQMax * 8 * ROWS + 2;
  __shared__ __align__(16) double zs[8 * kPart];
  constexpr int kTokW = 8 * TPT;                      // tokens per wave
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int g = blockIdx.y;
  const int nch = r / 8;                              // 8-j chunks of a row
  const int nq = (nch + 7) / 8;                       // chunks per lane (the last may be partial)
  // the group's z: every load of a batch issued before any store
  const double* zg = z64 + (size_t)g * r * kCandGroup;
  constexpr int kThr = kScoreWaves * kWave;
  constexpr int kBatch = 16;
  const int nz = r * ROWS;
  for (int q0 = 0; q0 < nz; q0 += kBatch * kThr) {
    double zv[kBatch];
#pragma unroll
    for (int bt = 0; bt < kBatch; ++bt) {
      const int qq = min(q0 + bt * kThr + tid, nz - 1);
      zv[bt] = zg[(qq / ROWS) * kCandGroup + qq % ROWS];
    }
#pragma unroll
    for (int bt = 0; bt < kBatch; ++bt) {
      const int qq = q0 + bt * kThr + tid;
      if (qq < nz) {
        const int j = qq / ROWS, row = qq % ROWS, c = j / 8;
        zs[(c % 8) * kPart + ((c / 8) * 8 + j % 8) * ROWS + row] = zv[bt];
      }
    }
  }
  // chunks past the row (the last round when r is not a multiple of 64) read z as 0:
  // their Bm pieces are zeros, and 0 * z must not meet an unwritten (possibly NaN) word
  const int n_pad = (nq * 8 - nch) * 8 * ROWS;
  for (int qq = tid; qq < n_pad; qq += kThr) {
    const int c = nch + qq / (8 * ROWS), rest = qq % (8 * ROWS);
    zs[(c % 8) * kPart + (c / 8) * 8 * ROWS + rest] = 0.0;
  }
  __syncthreads();
  const int t = lane >> 3, p = lane & 7;
  const int tw0 = (blockIdx.x * kScoreWaves + wave) * kTokW;
  const __bf16* brow[TPT];
#pragma unroll
  for (int u = 0; u < TPT; ++u) brow[u] = Bm + (size_t)min(tw0 + t + 8 * u, V - 1) * r;
  const double* zp = zs + p * kPart;
  double acc[TPT][ROWS];
#pragma unroll
  for (int u = 0; u < TPT; ++u)
#pragma unroll
    for (int i = 0; i < ROWS; ++i) acc[u][i] = 0.0;
  // blocks of 4 chunks per lane: every 16-byte piece of the block, for each token, is
  // loaded before any is used (all of a lane's chunks when r <= 256); a chunk past the
  // row reads as zeros, which add nothing
  constexpr int kQB = 4;
  for (int qb = 0; qb < nq; qb += kQB) {
    uint4 piece[kQB][TPT];
#pragma unroll
    for (int q = 0; q < kQB; ++q) {
      const int c = (qb + q) * 8 + p;
#pragma unroll
      for (int u = 0; u < TPT; ++u) {
        piece[q][u] = *(const uint4*)(brow[u] + 8 * min(c, nch - 1));
        if (c >= nch) piece[q][u] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int q = 0; q < kQB; ++q) {
      if (qb + q >= nq) break;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double2* zj = (const double2*)(zp + ((qb + q) * 8 + e) * ROWS);
        double bd[TPT];
#pragma unroll
        for (int u = 0; u < TPT; ++u) {
          const uint32_t w32 = e < 2 ? piece[q][u].x : e < 4 ? piece[q][u].y : e < 6 ? piece[q][u].z : piece[q][u].w;
          bd[u] = (double)__uint_as_float((e & 1) ? (w32 & 0xFFFF0000u) : (w32 << 16));
        }
#pragma unroll
        for (int i2 = 0; i2 < ROWS / 2; ++i2) {
          const double2 zz = zj[i2];
#pragma unroll
          for (int u = 0; u < TPT; ++u) {
            acc[u][2 * i2] = fma(bd[u], zz.x, acc[u][2 * i2]);
            acc[u][2 * i2 + 1] = fma(bd[u], zz.y, acc[u][2 * i2 + 1]);
          }
        }
      }
    }
  }
  // the eight lanes of each token, by DPP within each group of eight: pairs (quad_perm
  // [1,0,3,2]), quads ([2,3,0,1]), then the two quads (half-row mirror); every lane of
  // a group ends with the same sum
#pragma unroll
  for (int u = 0; u < TPT; ++u)
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
      double a = acc[u][i];
      a += dpp_f64<0xB1>(a);
      a += dpp_f64<0x4E>(a);
      a += dpp_f64<0x141>(a);
      acc[u][i] = a;
    }
  // lane p of each group takes rows p and p + 8 of its tokens (selected from the sums
  // every lane of the group holds): it writes their scores, and keeps per row the largest
  // key (cand_key) over its tokens, tokens past the vocabulary counting as key 0
  const int grp = blockIdx.x * kScoreWaves + wave;
  const int row0 = g * kCandGroup + p;
  uint32_t m0 = 0u, m1 = 0u;
#pragma unroll
  for (int u = 0; u < TPT; ++u) {
    const int v = tw0 + t + 8 * u;
    double x0 = acc[u][0], x1 = acc[u][ROWS > 8 ? 8 : 0];
#pragma unroll
    for (int i = 1; i < (ROWS < 8 ? ROWS : 8); ++i) x0 = p == i ? acc[u][i] : x0;
#pragma unroll
    for (int i = 9; i < ROWS; ++i) x1 = p == i - 8 ? acc[u][i] : x1;
    const float f0 = (float)x0, f1 = (float)x1;
    if (p < ROWS && row0 < rows && v < V) logits[(size_t)row0 * V + v] = f0;
    if (p + 8 < ROWS && row0 + 8 < rows && v < V) logits[(size_t)(row0 + 8) * V + v] = f1;
    m0 = max(m0, v < V ? cand_key(f0) : 0u);
    m1 = max(m1, v < V ? cand_key(f1) : 0u);
  }
  // the same p across the wave's eight token groups: lanes p + 8t, t = 0..7 (row rotate
  // by eight, then lanes 16 and 32 apart); lane p (t = 0) writes the group maxima
  m0 = max(m0, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m0, 0x128, 0xF, 0xF, false));
  m1 = max(m1, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m1, 0x128, 0xF, 0xF, false));
  m0 = max(m0, (uint32_t)__shfl_xor((int)m0, 16));
  m1 = max(m1, (uint32_t)__shfl_xor((int)m1, 16));
  m0 = max(m0, (uint32_t)__shfl_xor((int)m0, 32));
  m1 = max(m1, (uint32_t)__shfl_xor((int)m1, 32));
  if (t == 0 && grp < ng) {
    if (p < ROWS && row0 < rows) gmax[(size_t)row0 * ng + grp] = m0;
    if (p + 8 < ROWS && row0 + 8 < rows) gmax[(size_t)(row0 + 8) * ng + grp] = m1;
  }
}

__global__ __launch_bounds__(kCandSelThreads) void cand_select_kernel(
    int V, int C, const float* __restrict__ logits, const uint32_t* __restrict__ gmax, int ng,
    int tokw, int32_t* __restrict__ cand) {
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const float* lrow = logits + (size_t)row * V;
  __shared__ uint32_t s_hist[256];
  __shared__ int s_digit, s_before, s_n, s_ties;
  __shared__ uint32_t s_gmax[kCandGroups];
  __shared__ uint64_t s_gk[kCandGather];
  __shared__ int s_ids[kCandMaxC];
  __shared__ uint32_t s_keys[kCandMaxC];
  __shared__ int s_rank[kCandMaxC];
  __shared__ int s_grp[kCandQualMax];
  __shared__ int s_nq;

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
  // With passes < 4, T is the k-th largest key's leading 8 * passes bits (the rest 0):
  // a lower bound with at least k keys at or above it.
  auto radix_select = [&](auto&& each_key, int k, uint32_t& T, int& need, int passes) {
    uint32_t tmask = 0;
    T = 0;
    need = k;
    for (int shift = 24; shift >= 32 - 8 * passes; shift -= 8) {
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

  // rank the gathered keys by (larger key, lower id); the first C are the candidates
  auto rank_gathered = [&](int n_ge) {
    for (int gi = tid; gi < n_ge; gi += kCandSelThreads) {
      const uint64_t km = s_gk[gi];
      int rk = 0;
#pragma unroll 8
      for (int o = 0; o < n_ge; ++o) rk += (int)(s_gk[o] > km);
      if (rk < C) s_rank[rk] = (int)~(uint32_t)km;
    }
    __syncthreads();
    if (tid < C) cand[(size_t)row * C + tid] = s_rank[tid];
  };

  // Bounded by the score groups' maxima (written by the score kernel): T0 = the leading
  // 16 bits of the C-th largest group maximum.  C distinct scores (the C largest group
  // maxima) are >= T0, so every one of the C best scores is too, and only a group whose
  // maximum is >= T0 can hold one: those groups are read, their keys >= T0 gathered in
  // LDS and ranked.  Usually about C groups of tokw tokens, instead of the whole row.
  // Too many such groups or keys (heavy ties) fall through to the exact selection below.
  // The bound needs at least C groups (fewer than C groups: the path further down).
  bool bounded = gmax != nullptr && ng >= C && ng <= kGmaxPerThread * kCandSelThreads;
  if (bounded) {
    uint32_t gm[kGmaxPerThread];
#pragma unroll
    for (int j = 0; j < kGmaxPerThread; ++j) {
      const int gi = j * kCandSelThreads + tid;
      gm[j] = gmax[(size_t)row * ng + min(gi, ng - 1)];
      gm[j] = gi < ng ? gm[j] : 0u;
    }
    if (tid == 0) {
      s_nq = 0;
      s_n = 0;
    }
    uint32_t T0;
    int need0;
    radix_select([&](auto&& body) {
#pragma unroll
      for (int j = 0; j < kGmaxPerThread; ++j)
        if (j * kCandSelThreads + tid < ng) body(0, gm[j]);
    }, C, T0, need0, 2);
    // the qualifying groups into s_grp: per-thread counts, a ballot scan, one atomic per wave
    int mine = 0;
#pragma unroll
    for (int j = 0; j < kGmaxPerThread; ++j) mine += (int)(gm[j] >= T0 && j * kCandSelThreads + tid < ng);
    int wtot;
    const int pre = wave_prefix_small<4>(mine, wtot);
    int wbase = 0;
    if (lane == 0 && wtot > 0) wbase = atomicAdd(&s_nq, wtot);
    int slot = __builtin_amdgcn_readfirstlane(wbase) + pre;
#pragma unroll
    for (int j = 0; j < kGmaxPerThread; ++j) {
      const int gi = j * kCandSelThreads + tid;
      if (gm[j] >= T0 && gi < ng) {
        if (slot < kCandQualMax) s_grp[slot] = gi;
        ++slot;
      }
    }
    __syncthreads();
    const int nq = s_nq;
    bounded = nq <= kCandQualMax;
    if (bounded) {
      // their tokens, kGB per thread in flight, keys >= T0 gathered by ballot scans
      constexpr int kGB = 4;
      const int ntok = nq * tokw;
      for (int base = 0; base < ntok; base += kGB * kCandSelThreads) {
        int vv[kGB];
        float xv[kGB];
#pragma unroll
        for (int i = 0; i < kGB; ++i) {
          const int q = base + i * kCandSelThreads + tid;
          const int qq = min(q, ntok - 1);
          vv[i] = s_grp[qq / tokw] * tokw + qq % tokw;
          xv[i] = lrow[min(vv[i], V - 1)];
          vv[i] = q < ntok && vv[i] < V ? vv[i] : -1;
        }
        int cnt = 0;
        uint32_t uk[kGB];
#pragma unroll
        for (int i = 0; i < kGB; ++i) {
          uk[i] = cand_key(xv[i]);
          cnt += (int)(vv[i] >= 0 && uk[i] >= T0);
        }
        int wt;
        const int pr = wave_prefix_small<3>(cnt, wt);
        int wb = 0;
        if (lane == 0 && wt > 0) wb = atomicAdd(&s_n, wt);
        int sl = __builtin_amdgcn_readfirstlane(wb) + pr;
#pragma unroll
        for (int i = 0; i < kGB; ++i) {
          if (vv[i] >= 0 && uk[i] >= T0) {
            if (sl < kCandGather) s_gk[sl] = ((uint64_t)uk[i] << 32) | (uint32_t)~vv[i];
            ++sl;
          }
        }
      }
      __syncthreads();
      // at least C keys reach T0 (the C largest group maxima do); the test keeps every
      // rank below C written should that ever fail
      const int n_ge = s_n;
      if (n_ge >= C && n_ge <= kCandGather) {
        rank_gathered(n_ge);
        return;
      }
    }
    // heavy ties: the exact selection below
  }

  // A lower bound first: the largest key of each group of four threads (their strided
  // tokens), and T0 the C-th largest of those 256 group maxima: C groups hold a key
  // >= T0, so the C best keys are all >= T0.  The keys >= T0 are usually few (C plus a
  // few dozen): they are gathered in LDS and ranked there.  A row of at most
  // kBatch * 1024 tokens is read once and its keys stay in registers.
  const bool one_pass = V <= kBatch * kCandSelThreads;
  uint32_t u1[kBatch];
  uint32_t tmax = 0;
  if (one_pass) {
    float x[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) x[j] = lrow[min(j * kCandSelThreads + tid, V - 1)];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      u1[j] = j * kCandSelThreads + tid < V ? cand_key(x[j]) : 0u;
      tmax = max(tmax, u1[j]);
    }
  } else {
    for_each_key([&](int, uint32_t u) { tmax = max(tmax, u); });
  }
  tmax = max(tmax, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)tmax, 0xB1, 0xF, 0xF, false));
  tmax = max(tmax, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)tmax, 0x4E, 0xF, 0xF, false));
  if ((tid & 3) == 0) s_gmax[tid >> 2] = tmax;
  if (tid == 0) s_n = 0;
  __syncthreads();
  // T0: the leading 16 bits of the C-th largest group maximum (C <= 256 groups), by two
  // radix passes; at least C group maxima, hence C keys, are >= T0
  uint32_t T0;
  int need0;
  radix_select([&](auto&& body) { if (tid < kCandGroups) body(tid, s_gmax[tid]); }, C, T0, need0, 2);
  // gather the keys >= T0: per-thread counts, a wave prefix sum, one atomic per wave
  int mine = 0;
  if (one_pass) {
#pragma unroll
    for (int j = 0; j < kBatch; ++j) mine += (int)(u1[j] >= T0 && j * kCandSelThreads + tid < V);
    static_assert(kBatch < 64, "per-thread counts fit six bits");
    int wtot;
    const int pre = wave_prefix_small<6>(mine, wtot);
    int wbase = 0;
    if (lane == 0) wbase = atomicAdd(&s_n, wtot);
    wbase = __builtin_amdgcn_readfirstlane(wbase);
    int slot = wbase + pre;
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int v = j * kCandSelThreads + tid;
      if (u1[j] >= T0 && v < V) {
        if (slot < kCandGather) s_gk[slot] = ((uint64_t)u1[j] << 32) | (uint32_t)~v;
        ++slot;
      }
    }
  } else {
    for_each_key([&](int v, uint32_t u) {
      if (u >= T0) {
        const int slot = atomicAdd(&s_n, 1);
        if (slot < kCandGather) s_gk[slot] = ((uint64_t)u << 32) | (uint32_t)~v;
      }
    });
  }
  __syncthreads();
  const int n_ge = s_n;
  if (n_ge <= kCandGather) {
    // rank by (larger key, lower id) from the packed keys; the first C are the candidates
    for (int gi = tid; gi < n_ge; gi += kCandSelThreads) {
      const uint64_t km = s_gk[gi];
      int rk = 0;
#pragma unroll 8
      for (int o = 0; o < n_ge; ++o) rk += (int)(s_gk[o] > km);
      if (rk < C) s_rank[rk] = (int)~(uint32_t)km;
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
  radix_select(for_each_key, C, T, need, 4);
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

// z64 (float64, rows padded to whole groups of 16), then the score-group maxima (one
// uint32 key per row and group of at least kMinTokW tokens)
static size_t cand_z_bytes(int rows, int r) {
  const size_t groups = ((size_t)rows + tv::kCandGroup - 1) / tv::kCandGroup;
  return (groups * tv::kCandGroup * r * sizeof(double) + 255) / 256 * 256;
}

TV_API size_t tree_candidate_workspace_size(int rows, int r, int vocab) {
  if (rows < 1 || r < 1 || r > tv::kCandMaxR || vocab < 1) return 0;
  const size_t ng = ((size_t)vocab + tv::kMinTokW - 1) / tv::kMinTokW;
  return cand_z_bytes(rows, r) + ((size_t)rows * ng * sizeof(uint32_t) + 255) / 256 * 256;
}

namespace tv {
// tokens per score wave (one score group) for a number of rows
static int score_tokens_per_wave(int rows) {
  const int rg = rows > kCandGroup ? kCandGroup : (rows + 1) & ~1;
  return rg <= 12 ? 32 : 16;
}
template <int ROWS, int RMAX>
static void launch_score_rows(int rows, int r, int vocab, const __bf16* Bm, const double* z64,
                              float* logits, uint32_t* gmax, int ng, hipStream_t stream) {
  constexpr int TPT = ROWS <= 12 ? 4 : 2;             // tokens per lane: acc stays <= 48 doubles
  const int per_wg = kScoreWaves * 8 * TPT;
  const dim3 grid((vocab + per_wg - 1) / per_wg, (rows + kCandGroup - 1) / kCandGroup);
  hipLaunchKernelGGL((cand_score_kernel<ROWS, TPT, RMAX, ROWS <= 8 ? 3 : 1>), grid, dim3(kScoreWaves * kWave), 0, stream,
                     rows, r, vocab, Bm, z64, logits, gmax, ng);
}
template <int RMAX>
static void launch_score(int rows, int r, int vocab, const __bf16* Bm, const double* z64,
                         float* logits, uint32_t* gmax, int ng, hipStream_t stream) {
  // the group's rows rounded up to even (whole groups of 16 past 16 rows)
  const int rg = rows > kCandGroup ? kCandGroup : (rows + 1) & ~1;
  switch (rg) {
    case 2: launch_score_rows<2, RMAX>(rows, r, vocab, Bm, z64, logits, gmax, ng, stream); break;
    case 4: launch_score_rows<4, RMAX>(rows, r, vocab, Bm, z64, logits, gmax, ng, stream); break;
    case 6: launch_score_rows<6, RMAX>(rows, r, vocab, Bm, z64, logits, gmax, ng, stream); break;
    case 8: launch_score_rows<8, RMAX>(rows, r, vocab, Bm, z64, logits, gmax, ng, stream); break;
    case 10: launch_score_rows<10, RMAX>(rows, r, vocab, Bm, z64, logits, gmax, ng, stream); break;
    case 12: launch_score_rows<12, RMAX>(rows, r, vocab, Bm, z64, logits, gmax, ng, stream); break;
    case 14: launch_score_rows<14, RMAX>(rows, r, vocab, Bm, z64, logits, gmax, ng, stream); break;
    default: launch_score_rows<16, RMAX>(rows, r, vocab, Bm, z64, logits, gmax, ng, stream); break;
  }
}
}  // namespace tv

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
  const size_t need = tree_candidate_workspace_size(rows, r, vocab);
  if (!ws || ws_bytes < need) return TV_ERR_WORKSPACE;
  double* z64 = (double*)ws;
  const int tokw = tv::score_tokens_per_wave(rows);
  const int ng = (vocab + tokw - 1) / tokw;
  uint32_t* gmax = (uint32_t*)((char*)ws + cand_z_bytes(rows, r));
  const int padded = (rows + tv::kCandGroup - 1) / tv::kCandGroup * tv::kCandGroup;
  hipLaunchKernelGGL(tv::cand_z_kernel, dim3((r + 3) / 4, padded), dim3(256), 0, stream, rows, d, r,
                     (const __bf16*)h, (const __bf16*)A, z64);
  if (r <= 256)
    tv::launch_score<256>(rows, r, vocab, (const __bf16*)Bm, z64, logits, gmax, ng, stream);
  else
    tv::launch_score<512>(rows, r, vocab, (const __bf16*)Bm, z64, logits, gmax, ng, stream);
  hipLaunchKernelGGL(tv::cand_select_kernel, dim3(rows), dim3(tv::kCandSelThreads), 0, stream,
                     vocab, C, (const float*)logits, (const uint32_t*)gmax, ng, tokw, cand);
  hipLaunchKernelGGL(tv::cand_exact_kernel, dim3((C + 3) / 4, rows), dim3(256), 0, stream, d, vocab,
                     C, (const __bf16*)h, (const __bf16*)W, (const int32_t*)cand, logits);
  return tv::launch_status();
}
