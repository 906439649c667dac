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
  float sl2;          // scale * log2(e)
};

struct AttnPlan {
  int wq, wk, rows_per_wg, n_rb, chunk_keys, n_chunks, units, total_wgs, grid;
  size_t part_o_bytes, part_ml_bytes, ws_bytes;
};

constexpr int kWaves = 8;
constexpr int kMaxChunks = 16;                       // key chunks per work unit (merge width)
constexpr int kAttnThreads = 64 * kWaves;
constexpr int kLdsBudget = 128 * 1024;

__host__ __device__ constexpr int stage_keys(int wk) { return 32 * (wk > 2 ? wk : 2); }
__host__ __device__ constexpr int stage_bytes(int D, int wk) { return 2 * stage_keys(wk) * 2 * D; }
__host__ __device__ constexpr int n_buffers(int D, int wk) {
  return kLdsBudget / stage_bytes(D, wk) < 4 ? kLdsBudget / stage_bytes(D, wk) : 4;
}

static AttnPlan make_plan(int B, int n_max, int Hq, int Hkv, int D, int max_prefix) {
  AttnPlan p{};
  const int G = Hq / Hkv;
  const int R = n_max * G;
  if (R <= 64) { p.wq = 2; p.wk = 4; }
  else if (R <= 128) { p.wq = 4; p.wk = 2; }
  else { p.wq = 8; p.wk = 1; }
  p.rows_per_wg = 32 * p.wq;
  p.n_rb = (R + p.rows_per_wg - 1) / p.rows_per_wg;
  const int kt = stage_keys(p.wk);
  p.units = B * Hkv * p.n_rb;
  // about two workgroups per CU over 256 CUs; every chunk at least two stages
  const long target = 512;
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
  p.grid = (p.total_wgs + 7) / 8 * 8;
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

enum StageMode { kFull = 0, kMasked = 1 };

template <int D, int WQ, int WK>
__global__ __launch_bounds__(kAttnThreads) void attn_bf16(AttnArgs a) {
  constexpr int W = WQ * WK;
  static_assert(W == kWaves, "eight waves per workgroup");
  constexpr int NS = stage_keys(WK) / 32;       // 32-key subtiles per stage
  constexpr int KT = stage_keys(WK);            // keys per stage
  constexpr int ROWB = 2 * D;                   // LDS bytes per K/V row (bf16, swizzled)
  constexpr int TILEB = KT * ROWB;              // K (or V) bytes per stage
  constexpr int STAGEB = 2 * TILEB;
  constexpr int NBUF = n_buffers(D, WK);
  constexpr int DMA = STAGEB / (kAttnThreads * 16);   // 16-byte LDS DMAs per thread per stage
  constexpr int ROWS_PER_KB = 1024 / ROWB;
  constexpr int KBLKS = TILEB / 1024;
  constexpr int DS = D / 16;
  constexpr int DT = D / 32;
  static_assert(DMA * kAttnThreads * 16 == STAGEB, "stage must split into 1 KB DMA blocks");
  static_assert(NBUF >= 2 && NBUF <= 4, "two to four stage buffers");

  __shared__ __attribute__((aligned(1024))) char smem[NBUF * STAGEB];

  // ---- work item.  The order puts KV heads fastest, then row blocks, then chunks:
  // workgroups running together read the same token range of every head, i.e. whole
  // contiguous prefix rows, and the row blocks of one (head, chunk) stay close in time.
  // The blockIdx -> item map is XCD-aware: consecutive items land on one XCD (and L2).
  const int x = blockIdx.x;
  const int logical = (x % 8) * (gridDim.x / 8) + x / 8;
  if (logical >= a.total_wgs) return;                // padding of the grid: no item
  int t = logical;
  const int kvh = t % a.Hkv; t /= a.Hkv;
  const int rb = t % a.n_rb; t /= a.n_rb;
  const int chunk = t % a.n_chunks;
  const int b = t / a.n_chunks;
  const int unit = (b * a.Hkv + kvh) * a.n_rb + rb;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wq = wave / WK;
  const int wk = wave % WK;
  const int g = lane >> 5;
  const int ql = lane & 31;

  const int n = a.n_nodes[b];
  const int64_t off = a.offsets[b];
  const int64_t Lw = a.offsets[b + 1] - off;
  const bool n_ok = n >= 1 && n <= a.n_max;
  const bool seq_ok = n_ok && Lw >= 0 && Lw <= a.max_prefix;
  const int L = seq_ok ? (int)Lw : 0;
  const int G = a.G;
  const int R = n_ok ? n * G : 0;
  const int row0 = rb * a.rows_per_wg;
  const int c0 = chunk * a.chunk_keys;
  const int c1 = min(L, c0 + a.chunk_keys);
  const bool active = seq_ok && row0 < R && (chunk == 0 || c0 < L);

  if (active) {
    const int has_tree = chunk == 0 ? 1 : 0;
    const int nst = (c1 > c0 ? (c1 - c0 + KT - 1) / KT : 0) + has_tree;

    // queries of this wave: Q^T operands and the node's ancestor bitset.  A wave whose
    // 32 rows all lie beyond the tree's rows still queues its DMA share and joins
    // every barrier, but computes nothing.
    const bool wave_live = row0 + wq * 32 < R;
    const int rho = row0 + wq * 32 + ql;
    const int rc = rho < R ? rho : R - 1;
    const int qnode = rc / G;
    const int qhead = kvh * G + rc % G;
    bf16x8 qop[DS];
    {
      const __bf16* qp = a.q + (((size_t)b * a.n_max + qnode) * a.Hq + qhead) * D + 8 * g;
#pragma unroll
      for (int s = 0; s < DS; ++s) qop[s] = *(const bf16x8*)(qp + 16 * s);
    }
    const uint64_t qanc = a.anc[(size_t)b * a.n_max + qnode];
    wait_vmcnt<0>();      // Q and the bitset are in registers before any DMA is queued

    f32x16 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    const size_t kv_row = (size_t)a.Hkv * D;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)smem;
    static_assert(KBLKS == (W / 2) * DMA, "half the waves cover one tile");
    // queue the DMA of stage st into buffer buf.  Waves 0..W/2-1 fetch K rows, the
    // others V rows; each wave covers DMA consecutive 1 KB blocks (ROWS_PER_KB rows
    // each) and each lane one 16-byte chunk, placed at its XOR-swizzled position.
    const bool dma_v = wave >= W / 2;
    const int dma_blk0 = (wave % (W / 2)) * DMA;
    const __bf16* tree_base = (dma_v ? a.v_tree : a.k_tree) + ((size_t)b * a.n_max * a.Hkv + kvh) * D;
    const __bf16* pref_base = (dma_v ? a.v_prefix : a.k_prefix) + (size_t)off * kv_row + (size_t)kvh * D;
    const int dma_pos = lane % (ROWB / 16);
    const int dma_row = lane / (ROWB / 16);
    auto issue = [&](int st, int buf) {
      const bool tree = has_tree && st == 0;
      const int kbase = tree ? 0 : c0 + (st - has_tree) * KT;
      const int kend = tree ? n : c1;
      const __bf16* base = tree ? tree_base : pref_base;
      const size_t rstride = tree ? (size_t)a.Hkv * D : kv_row;
      const uint32_t dst0 = lds0 + buf * STAGEB + (dma_v ? TILEB : 0) + dma_blk0 * 1024;
      // the tree stage only fetches the 32-row subtiles that hold nodes; the others are
      // never read (their subtiles are skipped), and fewer DMAs in flight only make the
      // later vmcnt waits finish sooner
      const int rows_needed = tree ? (n + 31) / 32 * 32 : KT;
#pragma unroll
      for (int i = 0; i < DMA; ++i) {
        if ((dma_blk0 + i) * ROWS_PER_KB >= rows_needed) continue;      // wave-uniform
        const int lrow = (dma_blk0 + i) * ROWS_PER_KB + dma_row;
        const int chk = dma_pos ^ swz<D>(lrow);
        const int key = min(kbase + lrow, kend - 1);
        lds_dma16(base + (size_t)key * rstride + chk * 8,
                  __builtin_amdgcn_readfirstlane(dst0 + i * 1024));
      }
    };

    // lane-constant LDS byte offsets (the swizzle only depends on the low four row bits,
    // so the subtile, k-step and buffer terms are uniform and added per use)
    int koff[DS];
#pragma unroll
    for (int s = 0; s < DS; ++s) koff[s] = ql * ROWB + (((2 * s + g) ^ swz<D>(ql)) << 4);
    uint32_t voff_lo[DT], voff_hi[DT];
    {
      const int s16 = lane & 15;
      const int rlo = 4 * g + (s16 >> 2);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int chk = 4 * dt + 2 * ((lane >> 4) & 1) + ((s16 & 3) >> 1);
        const int half = (s16 & 1) << 3;
        voff_lo[dt] = rlo * ROWB + ((chk ^ swz<D>(rlo)) << 4) + half;
        voff_hi[dt] = (rlo + 8) * ROWB + ((chk ^ swz<D>(rlo + 8)) << 4) + half;
      }
    }

    // NSUB (1 or 2) 32-key subtiles processed together: S^T = K Q^T for each (the two
    // MFMA chains interleave), one online-softmax update over all their scores, then
    // O^T += V^T P^T with the products of both subtiles interleaved per accumulator.
    // kMasked hides keys >= kend and, through amask (the query's ancestor bitset in the
    // tree stage, all ones otherwise), keys off the query's root path.
    auto subtiles = [&](auto mode_tag, auto nsub_tag, const char* kb, const char* vb, int sub0,
                        int kbase, int kend, uint64_t amask) {
      constexpr int MODE = decltype(mode_tag)::value;
      constexpr int NSUB = decltype(nsub_tag)::value;
      f32x16 sacc[NSUB];
#pragma unroll
      for (int u = 0; u < NSUB; ++u) sacc[u] = f32x16{};
#pragma unroll
      for (int s = 0; s < DS; ++s) {
#pragma unroll
        for (int u = 0; u < NSUB; ++u) {
          const bf16x8 kop = *(const bf16x8*)(kb + (sub0 + u * WK) * 32 * ROWB + koff[s]);
          sacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[s], sacc[u], 0, 0, 0);
        }
      }
      float mloc = -INFINITY;
#pragma unroll
      for (int u = 0; u < NSUB; ++u) {
        const int key0 = kbase + (sub0 + u * WK) * 32 + 4 * g;   // key of accumulator 0
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if constexpr (MODE == kMasked) {
            const int key = key0 + 8 * (r >> 2) + (r & 3);
            const bool vis = (key < kend) & (((amask >> (key & 63)) & 1ull) != 0ull);
            sacc[u][r] = vis ? sacc[u][r] : -INFINITY;
          }
          mloc = fmaxf(mloc, sacc[u][r]);
        }
      }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32)) * a.sl2;
      // Lazy rescaling: m_run is a reference, not necessarily the maximum.  It only
      // moves (and O, l are rescaled) when some lane's scores exceed it by more than
      // 2^8; otherwise the weights below are at most 256, exact in fp32 and bf16.
      if (__ballot(mloc > m_run + 8.f)) {
        const float mnew = fmaxf(m_run, mloc);
        const float alpha = __builtin_amdgcn_exp2f(m_run - mnew);   // 0 while m_run is -inf
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
        l_run *= alpha;
        m_run = mnew;
      }
      const float msub = m_run == -INFINITY ? 0.f : m_run;
      // v_exp_f32 directly; weights below 2^-126 of the reference may flush to zero
      float psum = 0.f;
      bf16x8 pb[NSUB][2];
#pragma unroll
      for (int u = 0; u < NSUB; ++u) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sacc[u][r] = __builtin_amdgcn_exp2f(fmaf(sacc[u][r], a.sl2, -msub));
          psum += sacc[u][r];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pb[u][0][e] = (__bf16)sacc[u][e];
          pb[u][1][e] = (__bf16)sacc[u][8 + e];
        }
      }
      l_run += psum;
      typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
      const uint32_t vb0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)vb;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
          for (int u = 0; u < NSUB; ++u) {
            const uint32_t vbs = vb0 + (sub0 + u * WK) * 32 * ROWB + ks * 16 * ROWB;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)(uintptr_t)(vbs + voff_lo[dt]));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)(uintptr_t)(vbs + voff_hi[dt]));
            const s16x4 both[2] = {lo, hi};
            const bf16x8 vop = *(const bf16x8*)both;
            o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pb[u][ks], o[dt], 0, 0, 0);
          }
        }
      }
    };

    auto compute = [&](int st) {
      const int buf = st % NBUF;
      const char* kb = smem + buf * STAGEB;
      const char* vb = kb + TILEB;
      const bool tree = has_tree && st == 0;
      const int kbase = tree ? 0 : c0 + (st - has_tree) * KT;
      const int kend = tree ? n : c1;
      const uint64_t amask = tree ? qanc : ~0ull;
      // The mode is fixed per stage and chosen before any MFMA is issued: a prefix
      // stage whose keys all lie below kend needs no mask at all.  A wave that owns two
      // subtiles of a full stage processes them as a pair.
      constexpr int PER_WAVE = NS / WK;
      static_assert(PER_WAVE == 1 || PER_WAVE == 2, "one or two subtiles per wave and stage");
      if (!tree && kbase + KT <= kend) {
        subtiles(std::integral_constant<int, kFull>{}, std::integral_constant<int, PER_WAVE>{},
                 kb, vb, wk, kbase, kend, amask);
      } else {
        auto one = [&](auto j_tag) {
          constexpr int J = decltype(j_tag)::value;
          const int sub = wk + J * WK;
          if (kbase + sub * 32 >= kend) return;            // wave-uniform
          subtiles(std::integral_constant<int, kMasked>{}, std::integral_constant<int, 1>{},
                   kb, vb, sub, kbase, kend, amask);
        };
        one(std::integral_constant<int, 0>{});
        if constexpr (PER_WAVE > 1) one(std::integral_constant<int, 1>{});
      }
    };

    // ---- pipeline: up to NBUF stages in flight; stage st+NBUF-1 is queued into the
    // buffer that stage st-1 released, right after the barrier that proves it free.
#pragma unroll
    for (int p = 0; p < NBUF; ++p)
      if (p < nst) issue(p, p);
    for (int st = 0; st < nst; ++st) {
      const int ahead = min(nst - 1 - st, st == 0 ? NBUF - 1 : NBUF - 2);
      if (ahead <= 0) wait_vmcnt<0>();
      else if (ahead == 1) wait_vmcnt<DMA>();
      else if (ahead == 2) wait_vmcnt<2 * DMA>();
      else wait_vmcnt<3 * DMA>();
      lds_barrier();
      if (st >= 1 && st + NBUF - 1 < nst) issue(st + NBUF - 1, (st - 1) % NBUF);
      if (wave_live) compute(st);
    }
    __syncthreads();

    // ---- merge the key-split waves of each query group through LDS
    if constexpr (WK > 1) {
      float* mb = (float*)smem;
      constexpr int PER = DT * 16 + 2;                 // floats per lane per wave
      if (wk > 0) {
        float* dst = mb + (size_t)(wq * (WK - 1) + wk - 1) * PER * 64;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) dst[(dt * 16 + r) * 64 + lane] = o[dt][r];
        dst[(DT * 16) * 64 + lane] = m_run;
        dst[(DT * 16 + 1) * 64 + lane] = l_run;
      }
      __syncthreads();
      if (wk == 0) {
        for (int w = 1; w < WK; ++w) {
          const float* src = mb + (size_t)(wq * (WK - 1) + w - 1) * PER * 64;
          const float mo = src[(DT * 16) * 64 + lane];
          const float lo = src[(DT * 16 + 1) * 64 + lane];
          const float mn = fmaxf(m_run, mo);
          const float ms = mn == -INFINITY ? 0.f : mn;
          const float sa = exp2f(m_run - ms);
          const float sb = exp2f(mo - ms);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[dt][r] = o[dt][r] * sa + src[(dt * 16 + r) * 64 + lane] * sb;
          l_run = l_run * sa + lo * sb;
          m_run = mn;
        }
      }
    }

    // ---- output of this chunk: the final row when the sequence's prefix fits in one
    // chunk, else an unnormalised partial for attn_combine
    if (wk == 0 && wave_live && rho < R) {
      const float ltot = l_run + __shfl_xor(l_run, 32);
      const int nc = L > 0 ? (L + a.chunk_keys - 1) / a.chunk_keys : 1;
      if (nc == 1) {
        const size_t orow = ((size_t)b * a.n_max + qnode) * a.Hq + qhead;
        const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
        __bf16* op = a.out + orow * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int d = 32 * dt + 8 * r4 + 4 * g;
            __bf16 ob[4] = {(__bf16)(o[dt][4 * r4] * inv), (__bf16)(o[dt][4 * r4 + 1] * inv),
                            (__bf16)(o[dt][4 * r4 + 2] * inv), (__bf16)(o[dt][4 * r4 + 3] * inv)};
            *(s16x4*)(op + d) = *(const s16x4*)ob;
          }
        if (a.lse && g == 0) a.lse[orow] = ltot > 0.f ? (m_run + log2f(ltot)) * kLn2 : 0.f;
      } else {
        const size_t slot = ((size_t)unit * a.n_chunks + chunk) * a.rows_per_wg + wq * 32 + ql;
        float* po = a.part_o + slot * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int d = 32 * dt + 8 * r4 + 4 * g;
            *(f32x4*)(po + d) = f32x4{o[dt][4 * r4], o[dt][4 * r4 + 1], o[dt][4 * r4 + 2],
                                      o[dt][4 * r4 + 3]};
          }
        if (g == 0) a.part_ml[slot] = make_float2(m_run, ltot);
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
    for (int idx = tid; idx < a.rows_per_wg * V4; idx += kAttnThreads) {
      const int rho = row0 + idx / V4;
      if (rho < first_dead || rho >= rows_total) continue;
      const size_t orow = ((size_t)b * a.n_max + rho / G) * a.Hq + kvh * G + rho % G;
      *(s16x4*)(a.out + orow * D + (idx % V4) * 4) = s16x4{0, 0, 0, 0};
      if (a.lse && idx % V4 == 0) a.lse[orow] = 0.f;
    }
  }
}

// Merge of the key-chunk partials: one wave per output row whose sequence spans more
// than one chunk (the others were written by attn_bf16).  All partials of the row are
// loaded first, then combined online.
template <int D>
__global__ __launch_bounds__(256) void attn_combine(AttnArgs a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.B * a.n_max * a.Hq) return;
  const int lane = threadIdx.x & 63;
  const int h = row % a.Hq;
  const int i = (row / a.Hq) % a.n_max;
  const int b = row / (a.Hq * a.n_max);
  const int n = a.n_nodes[b];
  const int64_t Lw = a.offsets[b + 1] - a.offsets[b];
  if (n < 1 || n > a.n_max || Lw < 0 || Lw > a.max_prefix || i >= n) return;
  const int L = (int)Lw;
  const int nc = L > 0 ? (L + a.chunk_keys - 1) / a.chunk_keys : 1;
  if (nc <= 1) return;
  const int G = a.G;
  const int kvh = h / G;
  const int rho = i * G + h % G;                       // row index within the KV head
  const int rb = rho / a.rows_per_wg;
  const int unit = (b * a.Hkv + kvh) * a.n_rb + rb;
  const size_t slot0 = (size_t)unit * a.n_chunks * a.rows_per_wg + rho % a.rows_per_wg;
  constexpr int PL = D / 64;                            // dims per lane
  float2 ml[kMaxChunks];
  float pv[kMaxChunks][PL];
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    if (c < nc) {
      const size_t slot = slot0 + (size_t)c * a.rows_per_wg;
      ml[c] = a.part_ml[slot];
#pragma unroll
      for (int e = 0; e < PL; ++e) pv[c][e] = a.part_o[slot * D + lane * PL + e];
    }
  }
  float M = -INFINITY, wsum = 0.f, acc[PL];
#pragma unroll
  for (int e = 0; e < PL; ++e) acc[e] = 0.f;
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    if (c < nc) {
      const float mn = fmaxf(M, ml[c].x);
      const float ms = mn == -INFINITY ? 0.f : mn;
      const float sa = __builtin_amdgcn_exp2f(M - ms);
      const float sb = __builtin_amdgcn_exp2f(ml[c].x - ms);
#pragma unroll
      for (int e = 0; e < PL; ++e) acc[e] = acc[e] * sa + pv[c][e] * sb;
      wsum = wsum * sa + ml[c].y * sb;
      M = mn;
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  __bf16* op = a.out + (size_t)row * D + lane * PL;
#pragma unroll
  for (int e = 0; e < PL; ++e) op[e] = (__bf16)(acc[e] * inv);
  if (a.lse && lane == 0) a.lse[row] = wsum > 0.f ? (M + log2f(wsum)) * kLn2 : 0.f;
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

template <int D>
static void launch_bf16(const AttnPlan& p, const AttnArgs& a, hipStream_t stream) {
  if (p.wk == 4) hipLaunchKernelGGL((attn_bf16<D, 2, 4>), dim3(p.grid), dim3(kAttnThreads), 0, stream, a);
  else if (p.wk == 2) hipLaunchKernelGGL((attn_bf16<D, 4, 2>), dim3(p.grid), dim3(kAttnThreads), 0, stream, a);
  else hipLaunchKernelGGL((attn_bf16<D, 8, 1>), dim3(p.grid), dim3(kAttnThreads), 0, stream, a);
  if (p.n_chunks > 1) {
    const int rows = a.B * a.n_max * a.Hq;
    hipLaunchKernelGGL(attn_combine<D>, dim3((rows + 3) / 4), dim3(256), 0, stream, a);
  }
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
  a.sl2 = scale * tv::kLog2e;
  if (D == 128) tv::launch_bf16<128>(p, a, stream);
  else tv::launch_bf16<64>(p, a, stream);
  return tv::launch_status();
}
