// tree_accept: greedy acceptance of the longest matching root path.
//
// "EAGLE" notes, "Well-Calibrated Draft Model": under greedy decoding a draft token is
// accepted when it equals the target's most likely token.  "What is EAGLE-3 ...",
// section 4 step 4: the longest prefix of the tree whose tokens all pass is kept.
// "Technical analysis of EAGLE-4", "verification trees": generation then continues
// with the target's own token after the accepted path.
//
// One wavefront per sequence, lane i <-> node i: each lane tests its own token
// against the target's token after its parent, a ballot gathers the passing nodes,
// a node is reachable when its ancestor bitset lies inside that ballot, and a wave
// maximum over (depth, -index) picks the deepest reachable node.  All of a lane's
// inputs are loaded at once; values of other nodes come by lane shuffles.
#include "tv_internal.h"

namespace tv {

__global__ __launch_bounds__(256) void tree_accept_kernel(
    int B, int n_max, const int32_t* __restrict__ parent, const int32_t* __restrict__ depth,
    const uint64_t* __restrict__ anc, const int32_t* __restrict__ n_nodes,
    const int32_t* __restrict__ token, const int32_t* __restrict__ target_next,
    int32_t* __restrict__ accept_len, int32_t* __restrict__ best_node,
    int32_t* __restrict__ bonus_token, int32_t* __restrict__ path) {
  const int b = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (b >= B) return;
  const int i = lane_id();
  const size_t row = (size_t)b * n_max;
  // every load up front (one memory round trip); lanes past n_max read node 0
  const int il = i < n_max ? i : 0;
  const int n = n_nodes[b];
  const uint64_t a_in = anc[row + il];
  const int p_in = parent[row + il];
  const int tok = token[row + il];
  const int tgt = target_next[row + il];
  const int d_in = depth[row + il];
  bool valid = n >= 1 && n <= n_max;
  if (valid) valid = shfl_u64(a_in, 0) == 1ull;  // the root's set is exactly {0} in a built tree
  if (!valid) {
    if (i == 0) {
      accept_len[b] = -1;
      best_node[b] = -1;
      bonus_token[b] = -1;
    }
    if (path && i < n_max) path[row + i] = -1;
    return;
  }
  const bool in_tree = i < n;
  // the target's token after node p sits in lane p (p stays in bounds even for
  // malformed input)
  const int p = p_in < 0 ? 0 : (p_in >= n ? n - 1 : p_in);
  const int tgt_parent = __shfl(tgt, p);
  const bool hit = (i == 0) || (in_tree && tok == tgt_parent);
  const uint64_t a = in_tree ? a_in : 0ull;
  const uint64_t passing = __ballot(in_tree && hit) | 1ull;
  int key = -1;
  if (in_tree && (a & ~passing) == 0) {
    const int d = d_in < 0 ? 0 : (d_in > 63 ? 63 : d_in);
    key = (d << 8) | (63 - i);
  }
  key = wave_max_i32(key);
  const int best = 63 - (key & 0xFF);
  const int alen = key >> 8;
  const uint64_t best_set = shfl_u64(a, best) & ~1ull;   // chosen path without the root
  const int bonus = __shfl(tgt, best);
  if (i == 0) {
    accept_len[b] = alen;
    best_node[b] = best;
    bonus_token[b] = bonus;
  }
  if (path && i < n_max) {
    if ((best_set >> i) & 1ull) {
      const int slot = __popcll(best_set & ((1ull << i) - 1ull));
      path[row + slot] = i;
    }
    if (i >= __popcll(best_set)) path[row + i] = -1;
  }
}

}  // namespace tv

TV_API tv_status tree_accept(int B, int n_max, const int32_t* parent, const int32_t* depth,
                             const uint64_t* anc, const int32_t* n_nodes, const int32_t* token,
                             const int32_t* target_next, int32_t* accept_len, int32_t* best_node,
                             int32_t* bonus_token, int32_t* path, hipStream_t stream) {
  if (!parent || !depth || !anc || !n_nodes || !token || !target_next || !accept_len ||
      !best_node || !bonus_token)
    return TV_ERR_NULL;
  if (B < 1 || n_max < 1 || n_max > TV_MAX_NODES) return TV_ERR_SHAPE;
  const int per_block = 4;
  const int grid = (B + per_block - 1) / per_block;
  hipLaunchKernelGGL(tv::tree_accept_kernel, dim3(grid), dim3(per_block * tv::kWave), 0, stream, B,
                     n_max, parent, depth, anc, n_nodes, token, target_next, accept_len, best_node,
                     bonus_token, path);
  return tv::launch_status();
}
