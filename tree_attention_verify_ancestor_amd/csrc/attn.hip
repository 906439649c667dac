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
//   attn_bf16_partial  grid = (sequence, KV head, key chunk, row block), XCD-aware.
//     A workgroup of 4 waves owns up to 32*QT*(4/WK) query rows (rows = node*G + head
//     in group) and one chunk of prefix keys; chunk 0 also owns the tree keys.  Each
//     stage stages 32*NS keys of K and V from HBM through registers into XOR-swizzled
//     LDS (double-buffered).  Each wave computes S^T = K Q^T with
//     v_mfma_f32_32x32x16_bf16, so a lane holds 16 keys of one query; the ancestor
//     bitset of that query's node sits in two registers and masks the tree stage
//     only.  Online softmax runs in the log2 domain (scale*log2e folded into one
//     multiply, exp2), and O^T += V^T P^T reuses the S^T accumulator as the B operand
//     directly; V^T comes from LDS through ds_read_b64_tr_b16.  With WK > 1 the four
//     waves split each stage's keys and merge their (m, l, O) through LDS.  The
//     result per row and chunk is an unnormalised fp32 partial plus (max, sum).
//   attn_combine       one wave per output row merges the chunk partials, writes
//     bf16 out and the natural-log lse, and zeroes padding rows.
// fp32 path: attn_f32, one workgroup per output row on the vector ALUs (the
// fp32 workloads are small correctness cases).
#include <math.h>

#include <type_traits>

#include "tv_internal.h"

namespace tv {

constexpr int kAttnThreads = 256;
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
  float* part_o;   // [B*n_max*Hq][n_chunks][D]
  float2* part_ml; // [B*n_max*Hq][n_chunks]
  int B, Hq, Hkv, G, n_max, max_prefix;
  int chunk_keys, n_chunks, n_rb, total_wgs;
  float sl2;       // scale * log2(e)
};

struct AttnPlan {
  int qt, wk, rows_per_wg, n_rb, chunk_keys, n_chunks, total_wgs, grid;
  size_t ws_bytes;
};

static AttnPlan make_plan(int B, int n_max, int Hq, int Hkv, int D, int max_prefix) {
  AttnPlan p{};
  const int G = Hq / Hkv;
  const int R = n_max * G;
  const int tiles = (R + 31) / 32;
  if (tiles <= 1) { p.qt = 1; p.wk = 4; }
  else if (tiles <= 2) { p.qt = 1; p.wk = 2; }
  else if (tiles <= 4) { p.qt = 1; p.wk = 1; }
  else { p.qt = 2; p.wk = 1; }
  const int wq = 4 / p.wk;
  p.rows_per_wg = 32 * p.qt * wq;
  p.n_rb = (R + p.rows_per_wg - 1) / p.rows_per_wg;
  const int kt = 32 * (p.wk > 2 ? p.wk : 2);
  const long units = (long)B * Hkv * p.n_rb;
  // aim at two resident workgroups per CU on 256 CUs, chunks of at least 4 stages
  const long target = 512;
  long want = (target + units - 1) / units;
  if (want < 1) want = 1;
  long ck = (max_prefix + want - 1) / want;
  ck = (ck + kt - 1) / kt * kt;
  if (ck < 4 * kt) ck = 4 * kt;
  p.chunk_keys = (int)ck;
  p.n_chunks = max_prefix > 0 ? (int)((max_prefix + ck - 1) / ck) : 1;
  p.total_wgs = (int)(units * p.n_chunks);
  p.grid = (p.total_wgs + 7) / 8 * 8;
  p.ws_bytes = (size_t)B * n_max * Hq * p.n_chunks * ((size_t)D * 4 + 8);
  return p;
}

template <int D>
__device__ __forceinline__ int swz(int row) {
  // XOR pattern over the 16-byte chunks of a row: conflict-free for 16 consecutive rows
  // reading one chunk column (K operand) and spread for the transpose reads of V.
  if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return ((row & 3) << 1) | ((row >> 2) & 1);
}

template <int D, int QT, int WK>
__global__ __launch_bounds__(kAttnThreads) void attn_bf16_partial(AttnArgs a) {
  constexpr int NS = WK > 2 ? WK : 2;       // 32-key subtiles per stage
  constexpr int KT = 32 * NS;               // keys per stage
  constexpr int WQ = 4 / WK;                // query groups per workgroup
  constexpr int CH = D / 8;                 // 16-byte chunks per K/V row
  constexpr int ROWB = D * 2;               // LDS bytes per row (bf16, swizzled, unpadded)
  constexpr int TILEB = KT * ROWB;          // LDS bytes of K (or V) per stage
  constexpr int LOADS = KT * CH / kAttnThreads;
  constexpr int DS = D / 16;                // k-steps of the S^T product
  constexpr int DT = D / 32;                // 32-wide dim tiles of O^T
  static_assert(LOADS * kAttnThreads == KT * CH, "stage must split evenly");

  __shared__ __attribute__((aligned(16))) char smem[4 * TILEB];   // [buf][K|V]

  // ---- which work unit (XCD-aware: consecutive logical units share an XCD)
  const int x = blockIdx.x;
  const int per_xcd = gridDim.x / 8;
  const int logical = (x % 8) * per_xcd + x / 8;
  if (logical >= a.total_wgs) return;
  int t = logical;
  const int rb = t % a.n_rb; t /= a.n_rb;
  const int chunk = t % a.n_chunks; t /= a.n_chunks;
  const int kvh = t % a.Hkv;
  const int b = t / a.Hkv;

  const int n = a.n_nodes[b];
  const int64_t off = a.offsets[b];
  const int64_t Lw = a.offsets[b + 1] - off;
  if (n < 1 || n > a.n_max || Lw < 0 || Lw > a.max_prefix) return;
  const int L = (int)Lw;
  const int G = a.G;
  const int R = n * G;
  const int row0 = rb * (32 * QT * WQ);
  if (row0 >= R) return;
  const int c0 = chunk * a.chunk_keys;
  if (chunk > 0 && c0 >= L) return;
  const int c1 = min(L, c0 + a.chunk_keys);
  const int n_pref_stages = c1 > c0 ? (c1 - c0 + KT - 1) / KT : 0;
  const int has_tree = chunk == 0 ? 1 : 0;
  const int nstages = n_pref_stages + has_tree;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wq = wave / WK;
  const int wk = wave % WK;
  const int g = lane >> 5;
  const int ql = lane & 31;

  // ---- queries of this wave: Q^T operands and ancestor bitsets in registers
  bf16x8 qop[QT][DS];
  uint64_t qanc[QT];
  int qnode[QT], qhead[QT], qrow[QT];
#pragma unroll
  for (int tq = 0; tq < QT; ++tq) {
    const int rho = row0 + (wq * QT + tq) * 32 + ql;
    qrow[tq] = rho;
    const int rc = rho < R ? rho : R - 1;
    qnode[tq] = rc / G;
    qhead[tq] = kvh * G + rc % G;
    const __bf16* qp = a.q + (((size_t)b * a.n_max + qnode[tq]) * a.Hq + qhead[tq]) * D + 8 * g;
#pragma unroll
    for (int s = 0; s < DS; ++s) qop[tq][s] = *(const bf16x8*)(qp + 16 * s);
    qanc[tq] = a.anc[(size_t)b * a.n_max + qnode[tq]];
  }

  f32x16 o[QT][DT];
  float m_run[QT], l_run[QT];
#pragma unroll
  for (int tq = 0; tq < QT; ++tq) {
    m_run[tq] = -INFINITY;
    l_run[tq] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[tq][dt] = f32x16{};
  }

  // ---- stage loader: global -> registers -> swizzled LDS
  const size_t kv_row_stride = (size_t)a.Hkv * D;
  u32x4 kreg[LOADS], vreg[LOADS];
  auto load_stage = [&](int st) {
    const bool tree = has_tree && st == 0;
    const int kbase = tree ? 0 : c0 + (st - has_tree) * KT;
    const int kend = tree ? n : c1;
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int c = tid + kAttnThreads * u;
      const int row = c / CH;
      const int ch = c % CH;
      int key = kbase + row;
      key = key < kend ? key : kend - 1;
      size_t elt;
      const __bf16 *kp, *vp;
      if (tree) {
        elt = (((size_t)b * a.n_max + key) * a.Hkv + kvh) * D + ch * 8;
        kp = a.k_tree;
        vp = a.v_tree;
      } else {
        elt = ((size_t)(off + key)) * kv_row_stride + (size_t)kvh * D + ch * 8;
        kp = a.k_prefix;
        vp = a.v_prefix;
      }
      kreg[u] = *(const u32x4*)(kp + elt);
      vreg[u] = *(const u32x4*)(vp + elt);
    }
  };
  auto store_stage = [&](int buf) {
    char* kb = smem + buf * 2 * TILEB;
    char* vb = kb + TILEB;
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int c = tid + kAttnThreads * u;
      const int row = c / CH;
      const int ch = c % CH;
      const int offb = row * ROWB + ((ch ^ swz<D>(row)) << 4);
      *(u32x4*)(kb + offb) = kreg[u];
      *(u32x4*)(vb + offb) = vreg[u];
    }
  };

  // ---- compute one stage held in LDS buffer `buf`.  TREE selects the masked tree
  // stage; the prefix stages only bound the tail.  The two are separate code paths
  // chosen before any MFMA is issued, so no branch sits between an MFMA chain and the
  // reads of its accumulators.
  auto compute_stage = [&](auto tree_tag, int buf, int kbase, int kend) {
    constexpr bool TREE = decltype(tree_tag)::value;
    const char* kb = smem + buf * 2 * TILEB;
    const char* vb = kb + TILEB;
#pragma unroll
    for (int sub = wk; sub < NS; sub += WK) {
      if (kbase + sub * 32 >= kend) break;            // wave-uniform: nothing left
      // S^T = K Q^T for this 32-key subtile
      f32x16 sacc[QT];
#pragma unroll
      for (int tq = 0; tq < QT; ++tq) sacc[tq] = f32x16{};
      const int krow = sub * 32 + ql;
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        const bf16x8 kop = *(const bf16x8*)(kb + krow * ROWB + (((2 * s + g) ^ swz<D>(krow)) << 4));
#pragma unroll
        for (int tq = 0; tq < QT; ++tq)
          sacc[tq] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[tq][s], sacc[tq], 0, 0, 0);
      }
      // online softmax (log2 domain) and P^T in bf16
      bf16x8 pb[QT][2];
      const int kb0 = kbase + sub * 32 + 4 * g;        // key of accumulator 0 in this lane
#pragma unroll
      for (int tq = 0; tq < QT; ++tq) {
        float xv[16];
        float mloc = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb0 + 8 * (r >> 2) + (r & 3);
          bool vis = key < kend;
          if constexpr (TREE) vis = vis & (((qanc[tq] >> (key & 63)) & 1ull) != 0ull);
          xv[r] = vis ? sacc[tq][r] * a.sl2 : -INFINITY;
          mloc = fmaxf(mloc, xv[r]);
        }
        mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
        const float mnew = fmaxf(m_run[tq], mloc);
        const float msub = mnew == -INFINITY ? 0.f : mnew;
        const float alpha = exp2f(m_run[tq] - msub);
        float psum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          xv[r] = exp2f(xv[r] - msub);
          psum += xv[r];
        }
        l_run[tq] = l_run[tq] * alpha + psum;
        m_run[tq] = mnew;
        if (__ballot(alpha != 1.f)) {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) o[tq][dt] *= alpha;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pb[tq][0][e] = (__bf16)xv[e];
          pb[tq][1][e] = (__bf16)xv[8 + e];
        }
      }
      // O^T += V^T P^T; V^T operand via LDS transpose reads
      const int grp = lane >> 4;
      const int s16 = lane & 15;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int rlo = sub * 32 + 16 * ks + 4 * g + (s16 >> 2);
          const int rhi = rlo + 8;
          const int chk = 4 * dt + 2 * (grp & 1) + ((s16 & 3) >> 1);
          const int half = (s16 & 1) << 3;
          typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
          const lds_s16x4* plo = (const lds_s16x4*)(__attribute__((address_space(3))) const char*)(
              vb + rlo * ROWB + ((chk ^ swz<D>(rlo)) << 4) + half);
          const lds_s16x4* phi = (const lds_s16x4*)(__attribute__((address_space(3))) const char*)(
              vb + rhi * ROWB + ((chk ^ swz<D>(rhi)) << 4) + half);
          const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)plo);
          const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)phi);
          const s16x4 both[2] = {lo, hi};
          const bf16x8 vop = *(const bf16x8*)both;
#pragma unroll
          for (int tq = 0; tq < QT; ++tq)
            o[tq][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[tq][ks], o[tq][dt], 0, 0, 0);
        }
      }
    }
  };

  // ---- software pipeline over the stages
  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int st = 0; st < nstages; ++st) {
    if (st + 1 < nstages) load_stage(st + 1);
    if (has_tree && st == 0)
      compute_stage(std::true_type{}, 0, 0, n);
    else
      compute_stage(std::false_type{}, st & 1, c0 + (st - has_tree) * KT, c1);
    if (st + 1 < nstages) store_stage((st + 1) & 1);
    __syncthreads();
  }

  // ---- merge the key-split waves of each query group through LDS
  if constexpr (WK > 1) {
    float* mb = (float*)smem;                       // reused after the final barrier
    constexpr int PER = QT * (DT * 16 + 2);         // floats per lane per wave
    if (wk > 0) {
      float* dst = mb + ((size_t)(wq * (WK - 1) + wk - 1) * PER) * 64;
#pragma unroll
      for (int tq = 0; tq < QT; ++tq) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) dst[((tq * DT + dt) * 16 + r) * 64 + lane] = o[tq][dt][r];
        dst[(QT * DT * 16 + 2 * tq) * 64 + lane] = m_run[tq];
        dst[(QT * DT * 16 + 2 * tq + 1) * 64 + lane] = l_run[tq];
      }
    }
    __syncthreads();
    if (wk == 0) {
      for (int w = 1; w < WK; ++w) {
        const float* src = mb + ((size_t)(wq * (WK - 1) + w - 1) * PER) * 64;
#pragma unroll
        for (int tq = 0; tq < QT; ++tq) {
          const float mo = src[(QT * DT * 16 + 2 * tq) * 64 + lane];
          const float lo = src[(QT * DT * 16 + 2 * tq + 1) * 64 + lane];
          const float mn = fmaxf(m_run[tq], mo);
          const float ms = mn == -INFINITY ? 0.f : mn;
          const float sa = exp2f(m_run[tq] - ms);
          const float sb = exp2f(mo - ms);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              o[tq][dt][r] = o[tq][dt][r] * sa + src[((tq * DT + dt) * 16 + r) * 64 + lane] * sb;
          l_run[tq] = l_run[tq] * sa + lo * sb;
          m_run[tq] = mn;
        }
      }
    }
  }

  // ---- write the unnormalised partials of this chunk
  if (wk == 0) {
#pragma unroll
    for (int tq = 0; tq < QT; ++tq) {
      const float ltot = l_run[tq] + __shfl_xor(l_run[tq], 32);
      if (qrow[tq] < R) {
        const size_t prow =
            (((size_t)b * a.n_max + qnode[tq]) * a.Hq + qhead[tq]) * a.n_chunks + chunk;
        float* po = a.part_o + prow * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int d = 32 * dt + 8 * r4 + 4 * g;
            *(f32x4*)(po + d) = f32x4{o[tq][dt][4 * r4], o[tq][dt][4 * r4 + 1],
                                      o[tq][dt][4 * r4 + 2], o[tq][dt][4 * r4 + 3]};
          }
        if (g == 0) a.part_ml[prow] = make_float2(m_run[tq], ltot);
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void attn_combine(AttnArgs a, __bf16* __restrict__ out,
                                                    float* __restrict__ lse,
                                                    int32_t* __restrict__ seq_status) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int total = a.B * a.n_max * a.Hq;
  if (row >= total) return;
  const int lane = threadIdx.x & 63;
  const int h = row % a.Hq;
  const int i = (row / a.Hq) % a.n_max;
  const int b = row / (a.Hq * a.n_max);
  const int n = a.n_nodes[b];
  const int64_t Lw = a.offsets[b + 1] - a.offsets[b];
  int status = TV_SEQ_OK;
  if (n < 1 || n > a.n_max) status = TV_SEQ_BAD_N;
  else if (Lw < 0 || Lw > a.max_prefix) status = TV_SEQ_BAD_PREFIX;
  if (seq_status && i == 0 && h == 0 && lane == 0) seq_status[b] = status;
  constexpr int PL = D / 64;   // dims per lane
  __bf16* orow = out + (size_t)row * D + lane * PL;
  if (status != TV_SEQ_OK || i >= n) {
#pragma unroll
    for (int e = 0; e < PL; ++e) orow[e] = (__bf16)0.f;
    if (lse && lane == 0) lse[row] = 0.f;
    return;
  }
  const int L = (int)Lw;
  const int nc = L > 0 ? (L + a.chunk_keys - 1) / a.chunk_keys : 1;
  const size_t prow = (size_t)row * a.n_chunks;
  float M = -INFINITY;
  for (int c = 0; c < nc; ++c) M = fmaxf(M, a.part_ml[prow + c].x);
  const float Ms = M == -INFINITY ? 0.f : M;
  float acc[PL];
#pragma unroll
  for (int e = 0; e < PL; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  for (int c = 0; c < nc; ++c) {
    const float2 ml = a.part_ml[prow + c];
    const float w = exp2f(ml.x - Ms);
    wsum += ml.y * w;
    const float* po = a.part_o + (prow + c) * D + lane * PL;
#pragma unroll
    for (int e = 0; e < PL; ++e) acc[e] += po[e] * w;
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
#pragma unroll
  for (int e = 0; e < PL; ++e) orow[e] = (__bf16)(acc[e] * inv);
  if (lse && lane == 0) lse[row] = wsum > 0.f ? (Ms + log2f(wsum)) * kLn2 : 0.f;
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
  else if (Lw < 0 || Lw > max_prefix) status = TV_SEQ_BAD_PREFIX;
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

template <int D, int QT, int WK>
static void launch_partial(const AttnPlan& p, const AttnArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((attn_bf16_partial<D, QT, WK>), dim3(p.grid), dim3(kAttnThreads), 0, stream, a);
}

template <int D>
static void launch_bf16(const AttnPlan& p, const AttnArgs& a, __bf16* out, float* lse,
                        int32_t* seq_status, hipStream_t stream) {
  if (p.qt == 1 && p.wk == 4) launch_partial<D, 1, 4>(p, a, stream);
  else if (p.qt == 1 && p.wk == 2) launch_partial<D, 1, 2>(p, a, stream);
  else if (p.qt == 1 && p.wk == 1) launch_partial<D, 1, 1>(p, a, stream);
  else launch_partial<D, 2, 1>(p, a, stream);
  const int rows = a.B * a.n_max * a.Hq;
  hipLaunchKernelGGL(attn_combine<D>, dim3((rows + 3) / 4), dim3(256), 0, stream, a, out, lse,
                     seq_status);
}

static bool aligned16(const void* p) { return (((uintptr_t)p) & 15) == 0; }

}  // namespace tv

TV_API size_t tree_verify_attn_workspace_size(tv_dtype dt, int B, int n_max, int Hq, int Hkv,
                                              int D, int max_prefix_len) {
  if (dt != TV_BF16) return 0;
  if (B < 1 || n_max < 1 || n_max > TV_MAX_NODES || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 ||
      max_prefix_len < 0 || (D != 64 && D != 128))
    return 0;
  return tv::make_plan(B, n_max, Hq, Hkv, D, max_prefix_len).ws_bytes;
}

TV_API tv_status tree_verify_attn(tv_dtype dt, int B, int Hq, int Hkv, int D, int n_max,
                                  int max_prefix_len, float scale, const void* q,
                                  const void* k_tree, const void* v_tree, const void* k_prefix,
                                  const void* v_prefix, const int64_t* prefix_offsets,
                                  const int32_t* n_nodes, const uint64_t* anc, void* out,
                                  float* lse, void* ws, size_t ws_bytes, int32_t* seq_status,
                                  hipStream_t stream) {
  if (dt != TV_F32 && dt != TV_BF16) return TV_ERR_DTYPE;
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
  if (!ws || ws_bytes < p.ws_bytes) return TV_ERR_WORKSPACE;
  if (!tv::aligned16(ws)) return TV_ERR_WORKSPACE;
  tv::AttnArgs a{};
  a.q = (const __bf16*)q;
  a.k_tree = (const __bf16*)k_tree;
  a.v_tree = (const __bf16*)v_tree;
  a.k_prefix = (const __bf16*)k_prefix;
  a.v_prefix = (const __bf16*)v_prefix;
  a.offsets = prefix_offsets;
  a.n_nodes = n_nodes;
  a.anc = anc;
  a.part_o = (float*)ws;
  a.part_ml = (float2*)((char*)ws + (size_t)B * n_max * Hq * p.n_chunks * D * 4);
  a.B = B;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.n_max = n_max;
  a.max_prefix = max_prefix_len;
  a.chunk_keys = p.chunk_keys;
  a.n_chunks = p.n_chunks;
  a.n_rb = p.n_rb;
  a.total_wgs = p.total_wgs;
  a.sl2 = scale * tv::kLog2e;
  if (D == 128) tv::launch_bf16<128>(p, a, (__bf16*)out, lse, seq_status, stream);
  else tv::launch_bf16<64>(p, a, (__bf16*)out, lse, seq_status, stream);
  return tv::launch_status();
}
