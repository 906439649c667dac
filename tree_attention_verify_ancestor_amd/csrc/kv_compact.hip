// tree_kv_compact: the accepted continuation's K/V into the cache.
//
// "Technical analysis of EAGLE-4", section "EAGLE-4 verification trees and the
// harness": after verification the harness keeps the accepted continuation, frees
// the rejected KV-cache entries and starts the next round.  The continuation is the
// root (the target's last token, queried in this pass but not yet cached) and the
// accepted path, root to leaf; the rest of the tree is simply not copied.
//
// One workgroup per (destination row, sequence): row 0 takes the root, row j >= 1
// the path's j-th node.  It copies that node's K and V rows (all KV heads, contiguous
// in the per-node layout) with 16-byte loads and stores.
#include "tv_internal.h"

namespace tv {

__global__ __launch_bounds__(256) void kv_compact_kernel(
    int n_max, int row_chunks, const int4* __restrict__ k_tree, const int4* __restrict__ v_tree,
    const int32_t* __restrict__ path, const int32_t* __restrict__ accept_len,
    int4* __restrict__ k_dst, int4* __restrict__ v_dst, const int64_t* __restrict__ dst_row,
    int64_t dst_rows) {
  const int j = blockIdx.x;
  const int b = blockIdx.y;
  const int alen = accept_len[b];
  if (alen < 0 || j > alen) return;                       // rejected tree, or past the path
  const int node = j == 0 ? 0 : path[(size_t)b * n_max + j - 1];
  const int64_t r = dst_row[b] + j;
  if (node < 0 || node >= n_max || r < 0 || r >= dst_rows) return;
  const size_t src = ((size_t)b * n_max + node) * row_chunks;
  const size_t dst = (size_t)r * row_chunks;
  for (int c = threadIdx.x; c < row_chunks; c += blockDim.x) {
    const int4 kv = k_tree[src + c];
    const int4 vv = v_tree[src + c];
    k_dst[dst + c] = kv;
    v_dst[dst + c] = vv;
  }
}

}  // namespace tv

TV_API tv_status tree_kv_compact(tv_dtype dt, int B, int n_max, int Hkv, int D, const void* k_tree,
                                 const void* v_tree, const int32_t* path,
                                 const int32_t* accept_len, void* k_dst, void* v_dst,
                                 const int64_t* dst_row, int64_t dst_rows, hipStream_t stream) {
  if (!tv::known_dtype(dt)) return TV_ERR_DTYPE;
  if (B < 1 || n_max < 1 || n_max > TV_MAX_NODES || Hkv < 1 || D < 1 || dst_rows < 0)
    return TV_ERR_SHAPE;
  if (!k_tree || !v_tree || !path || !accept_len || !dst_row) return TV_ERR_NULL;
  if (dst_rows > 0 && (!k_dst || !v_dst)) return TV_ERR_NULL;
  const size_t row_bytes = (size_t)Hkv * D * (dt == TV_BF16 ? 2 : 4);
  if (row_bytes % 16 != 0 || ((uintptr_t)k_tree | (uintptr_t)v_tree | (uintptr_t)k_dst |
                              (uintptr_t)v_dst) % 16 != 0)
    return TV_ERR_UNSUPPORTED;
  if (dst_rows == 0) return TV_OK;
  hipLaunchKernelGGL(tv::kv_compact_kernel, dim3(n_max, B), dim3(64), 0, stream, n_max,
                     (int)(row_bytes / 16), (const int4*)k_tree, (const int4*)v_tree, path,
                     accept_len, (int4*)k_dst, (int4*)v_dst, dst_row, dst_rows);
  return tv::launch_status();
}
