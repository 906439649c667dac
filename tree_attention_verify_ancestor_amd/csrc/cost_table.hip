// tree_cost_lookup: the verification cost of one (batch, context) read off a table
// measured over a grid of batch sizes, context lengths and node counts.
//
// "Technical analysis of EAGLE-4", section "EAGLE-4 verification trees and the
// harness": a one-time calibration on the target GPU records verification latency
// against batch size, context length and the number of candidates; the harness reads
// the cost of verifying N candidates at the current batch and context from it.
//
// Host code only.  Between grid points the log of the latency is interpolated
// bilinearly in (log batch, log context) -- exact for latencies that follow a power
// law in batch and context, as streaming cost does -- and the latency linearly in the
// node count; outside the grid the nearest grid value is taken.  The result never
// falls with N (a tree with one more node costs at least as much), which the running
// maximum enforces.
#include <math.h>

#include "tv_internal.h"

namespace tv {

// the cell [i, i+1] of an ascending axis holding x (clamped) and the weight of i+1
static void cell(const int* axis, int n, double x, int* i0, double* w) {
  if (n == 1 || x <= axis[0]) {
    *i0 = 0;
    *w = 0.0;
    return;
  }
  if (x >= axis[n - 1]) {
    *i0 = n - 2;
    *w = 1.0;
    return;
  }
  int i = 0;
  while (x > axis[i + 1]) ++i;
  *i0 = i;
  *w = (log(x) - log((double)axis[i])) / (log((double)axis[i + 1]) - log((double)axis[i]));
}

static bool ascending_positive(const int* a, int n) {
  if (n < 1 || a[0] < 1) return false;
  for (int i = 1; i < n; ++i)
    if (a[i] <= a[i - 1]) return false;
  return true;
}

}  // namespace tv

TV_API tv_status tree_cost_lookup(const int32_t* batch, int n_batch, const int32_t* context,
                                  int n_context, const int32_t* nodes, int n_nodes_pts,
                                  const float* cost_us, int B, int L, int n_max,
                                  float* cost_out) {
  if (!batch || !context || !nodes || !cost_us || !cost_out) return TV_ERR_NULL;
  if (n_batch < 1 || n_context < 1 || n_nodes_pts < 1 || B < 1 || L < 0 || n_max < 1 ||
      n_max > TV_MAX_NODES)
    return TV_ERR_SHAPE;
  if (!tv::ascending_positive(batch, n_batch) || !tv::ascending_positive(context, n_context) ||
      !tv::ascending_positive(nodes, n_nodes_pts) || nodes[n_nodes_pts - 1] > TV_MAX_NODES)
    return TV_ERR_SHAPE;
  for (size_t i = 0; i < (size_t)n_batch * n_context * n_nodes_pts; ++i)
    if (!(cost_us[i] > 0.f) || isinf(cost_us[i])) return TV_ERR_SHAPE;    // latencies are positive
  int ib, il;
  double wb, wl;
  tv::cell(batch, n_batch, (double)B, &ib, &wb);
  tv::cell(context, n_context, (double)(L > 0 ? L : 1), &il, &wl);
  const int ib1 = n_batch > 1 ? ib + 1 : ib, il1 = n_context > 1 ? il + 1 : il;
  // the table's row over the node points at (B, L)
  auto lat = [&](int bi, int li, int ni) {
    return log((double)cost_us[((size_t)bi * n_context + li) * n_nodes_pts + ni]);
  };
  double row[TV_MAX_NODES];
  for (int k = 0; k < n_nodes_pts; ++k)
    row[k] = exp((1 - wb) * ((1 - wl) * lat(ib, il, k) + wl * lat(ib, il1, k)) +
                 wb * ((1 - wl) * lat(ib1, il, k) + wl * lat(ib1, il1, k)));
  double run = -INFINITY;
  for (int N = 1; N <= n_max; ++N) {
    double c;
    if (N <= nodes[0]) {
      c = row[0];
    } else if (N >= nodes[n_nodes_pts - 1]) {
      c = row[n_nodes_pts - 1];
    } else {
      int k = 0;
      while (N > nodes[k + 1]) ++k;
      const double t = (double)(N - nodes[k]) / (double)(nodes[k + 1] - nodes[k]);
      c = (1 - t) * row[k] + t * row[k + 1];
    }
    run = c > run ? c : run;
    cost_out[N - 1] = (float)run;
  }
  return TV_OK;
}
