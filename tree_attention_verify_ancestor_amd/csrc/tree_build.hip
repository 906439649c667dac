// tree_build: depth, ancestor bitset and position of every draft-tree node.
//
// "EAGLE" notes, "1. EAGLE pipeline / Draft Model": the draft is a tree of depth m
// holding more than m tokens.  "Technical analysis of EAGLE-4", "verification trees":
// a node sees the prefix, its ancestors and itself.  The ancestor set of node i is
// the root path i -> parent[i] -> ... -> 0, kept as one 64-bit word per node.
//
// One wavefront per sequence, lane i <-> node i.  The bitsets are built by pointer
// jumping: start from {i} and parent[i]; each round ORs in the set of the current
// jump target and doubles the jump, so six rounds cover any depth below 64.
#include "tv_internal.h"

namespace tv {

__global__ __launch_bounds__(256) void tree_build_kernel(
    int B, int n_max, const int32_t* __restrict__ parent, const int32_t* __restrict__ n_nodes,
    const int32_t* __restrict__ prefix_len, uint64_t* __restrict__ anc, int32_t* __restrict__ depth,
    int32_t* __restrict__ pos, int32_t* __restrict__ seq_status) {
  const int b = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (b >= B) return;
  const int i = lane_id();
  const int n = n_nodes[b];
  const bool in_tree = i < n;
  int p = (i < n_max) ? parent[(size_t)b * n_max + i] : -1;

  int status = TV_SEQ_OK;
  if (n < 1 || n > n_max) {
    status = TV_SEQ_BAD_N;
  } else {
    int code = 0;
    if (in_tree) {
      if (i == 0) code = (p != -1) ? TV_SEQ_BAD_PARENT : 0;
      else if (p == -1) code = TV_SEQ_SECOND_ROOT;
      else if (p < -1 || p >= i) code = TV_SEQ_BAD_PARENT;
    }
    const uint64_t bad = __ballot(code != 0);
    if (bad) status = __shfl(code, __ffsll((unsigned long long)bad) - 1);
  }

  uint64_t a = 0;
  int d = -1, ps = -1;
  if (status == TV_SEQ_OK) {
    // pointer jumping over the parent links (valid links point to lower indices)
    uint64_t set = in_tree ? (1ull << i) : 0ull;
    int jump = in_tree ? p : -1;
#pragma unroll
    for (int r = 0; r < 6; ++r) {
      const uint64_t other = shfl_u64(set, jump < 0 ? 0 : jump);
      const int next = __shfl(jump, jump < 0 ? 0 : jump);
      if (jump >= 0) {
        set |= other;
        jump = next;
      }
    }
    if (in_tree) {
      a = set;
      d = __popcll(set) - 1;
      ps = (prefix_len ? prefix_len[b] : 0) + d;
    }
  }
  if (i < n_max) {
    const size_t o = (size_t)b * n_max + i;
    anc[o] = a;
    depth[o] = d;
    if (pos) pos[o] = ps;
  }
  if (seq_status && i == 0) seq_status[b] = status;
}

}  // namespace tv

TV_API tv_status tree_build(int B, int n_max, const int32_t* parent, const int32_t* n_nodes,
                            const int32_t* prefix_len, uint64_t* anc, int32_t* depth, int32_t* pos,
                            int32_t* seq_status, hipStream_t stream) {
  if (!parent || !n_nodes || !anc || !depth) return TV_ERR_NULL;
  if (B < 1 || n_max < 1 || n_max > TV_MAX_NODES) return TV_ERR_SHAPE;
  const int per_block = 4;
  const int grid = (B + per_block - 1) / per_block;
  hipLaunchKernelGGL(tv::tree_build_kernel, dim3(grid), dim3(per_block * tv::kWave), 0, stream, B,
                     n_max, parent, n_nodes, prefix_len, anc, depth, pos, seq_status);
  return tv::launch_status();
}
