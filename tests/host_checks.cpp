// Host-side checks of libtreeverify's C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer together with a host-only build of the library (no device
// code, nothing launched): every argument check, the launch-plan and workspace-size
// arithmetic over a sweep of sizes, the cost-table lookup and the budget bars.  Any
// out-of-bounds access, overflow or undefined operation in that host code aborts the
// run; a wrong status fails it.  Prints "host checks ok" on success.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "treeverify.h"

static int g_fail = 0;
#define CHECK(cond)                                                  \
  do {                                                               \
    if (!(cond)) {                                                   \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++g_fail;                                                      \
    }                                                                \
  } while (0)

int main() {
  char buf[4096] __attribute__((aligned(16)));
  void* P = buf;                                   // a non-null, aligned stand-in, never read
  CHECK(tv_abi_version() == 3);
  for (int s = 0; s <= 6; ++s) CHECK(tv_status_string((tv_status)s) != nullptr);

  // tree_build / tree_accept argument checks
  CHECK(tree_build(1, 64, nullptr, (int32_t*)P, nullptr, (uint64_t*)P, (int32_t*)P, nullptr, nullptr, nullptr) == TV_ERR_NULL);
  CHECK(tree_build(0, 64, (int32_t*)P, (int32_t*)P, nullptr, (uint64_t*)P, (int32_t*)P, nullptr, nullptr, nullptr) == TV_ERR_SHAPE);
  CHECK(tree_build(1, 65, (int32_t*)P, (int32_t*)P, nullptr, (uint64_t*)P, (int32_t*)P, nullptr, nullptr, nullptr) == TV_ERR_SHAPE);
  CHECK(tree_accept(0, 8, (int32_t*)P, (int32_t*)P, (uint64_t*)P, (int32_t*)P, (int32_t*)P, (int32_t*)P,
                    (int32_t*)P, (int32_t*)P, (int32_t*)P, nullptr, nullptr) == TV_ERR_SHAPE);

  // expansion: workspace sizing over a sweep, argument checks
  for (int B = 1; B <= 64; B *= 2)
    for (int k = 0; k <= 17; ++k)
      for (int S = 0; S <= 12; ++S) {
        const size_t ws = tree_expand_workspace_size(B, k, S);
        if (k < 1 || k > 16 || S < 1) CHECK(ws == 0);
      }
  const size_t ews = tree_expand_workspace_size(2, 4, 3);
  CHECK(ews > 0);
  CHECK(tree_expand_rerank(P, ews, 2, 17, 3, 1, 100, (float*)P, 0, nullptr, nullptr, nullptr, 64,
                           nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == TV_ERR_SHAPE);
  CHECK(tree_expand_rerank(P, ews - 1, 2, 4, 3, 1, 100, (float*)P, 0, nullptr, nullptr, nullptr, 64,
                           nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == TV_ERR_WORKSPACE);
  CHECK(tree_expand_rerank(P, ews, 2, 4, 3, 1, (1 << 20) + 1, (float*)P, 0, nullptr, nullptr, nullptr,
                           64, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == TV_ERR_SHAPE);
  CHECK(tree_draft_continue(P, ews, 2, 4, 3, 0, nullptr, nullptr, (int32_t*)P, nullptr) == TV_ERR_SHAPE);

  // attention: plan and workspace arithmetic over a sweep of sizes
  int32_t plan[8];
  const int Ds[] = {64, 128};
  const int Gs[] = {1, 2, 4, 8};
  const int Ls[] = {0, 1, 63, 64, 129, 1000, 4096, 32768, 1 << 20, 1 << 30};
  for (int B : {1, 2, 3, 8, 9, 33, 256, 1024})
    for (int n_max : {1, 16, 32, 33, 64})
      for (int G : Gs)
        for (int Hkv : {1, 2, 8})
          for (int D : Ds)
            for (int L : Ls) {
              const int Hq = G * Hkv;
              CHECK(tree_verify_attn_plan(TV_BF16, B, n_max, Hq, Hkv, D, L, plan) == TV_OK);
              CHECK(plan[0] == 4 || plan[0] == 8);
              CHECK(plan[1] * plan[2] == plan[0]);
              CHECK(plan[5] > 0 && plan[6] >= 1 && plan[6] <= 32 && plan[7] >= plan[6]);
              CHECK((long)plan[5] * plan[6] >= L);
              const size_t ws = tree_verify_attn_workspace_size(TV_BF16, B, n_max, Hq, Hkv, D, L);
              CHECK((plan[6] == 1) == (ws == 0));
              if (ws > 0)                        // rejected before anything is launched
                CHECK(tree_verify_attn(TV_BF16, B, Hq, Hkv, D, n_max, L, 0.f, P, P, P, P, P,
                                       (int64_t*)P, (int32_t*)P, (uint64_t*)P, P, nullptr,
                                       nullptr, ws - 1, nullptr, nullptr) == TV_ERR_WORKSPACE);
            }
  CHECK(tree_verify_attn_plan(TV_BF16, 1, 64, 32, 8, 96, 100, plan) == TV_ERR_UNSUPPORTED);
  CHECK(tree_verify_attn_plan(TV_BF16, 1, 64, 30, 8, 128, 100, plan) == TV_ERR_SHAPE);
  CHECK(tree_verify_attn_plan(TV_F32, 1, 64, 32, 8, 64, 100, plan) == TV_ERR_DTYPE);
  CHECK(tree_verify_attn(TV_BF16, 1, 6, 4, 128, 64, 10, 0.f, P, P, P, P, P, (int64_t*)P, (int32_t*)P,
                         (uint64_t*)P, P, nullptr, nullptr, 0, nullptr, nullptr) == TV_ERR_SHAPE);
  CHECK(tree_verify_attn(TV_BF16, 1, 8, 2, 128, 64, 10, 0.f, (char*)P + 2, P, P, P, P, (int64_t*)P,
                         (int32_t*)P, (uint64_t*)P, P, nullptr, nullptr, 0, nullptr, nullptr) ==
        TV_ERR_UNSUPPORTED);
  CHECK(tree_verify_attn_noalloc(TV_BF16, 511, 4, 1, 128, 64, 8192, 0.f, P, P, P, P, P, (int64_t*)P,
                                 (int32_t*)P, (uint64_t*)P, P, nullptr, nullptr, nullptr) ==
        TV_ERR_WORKSPACE);

  // stochastic acceptance, compaction, candidate head: argument checks
  CHECK(tree_accept_stochastic(1, 64, 0, (int32_t*)P, (uint64_t*)P, (int32_t*)P, (int32_t*)P, (float*)P,
                               (float*)P, (float*)P, (float*)P, (int32_t*)P, (int32_t*)P, (int32_t*)P,
                               nullptr, nullptr, 0, nullptr) == TV_ERR_SHAPE);
  CHECK(tree_accept_stochastic(1, 64, 100, (int32_t*)P, (uint64_t*)P, (int32_t*)P, (int32_t*)P, nullptr,
                               (float*)P, (float*)P, (float*)P, (int32_t*)P, (int32_t*)P, (int32_t*)P,
                               nullptr, nullptr, 0, nullptr) == TV_ERR_NULL);
  CHECK(tree_accept_stochastic_workspace_size(0, 64, 1000) == 0);
  CHECK(tree_accept_stochastic_workspace_size(2, 65, 1000) == 0);
  CHECK(tree_accept_stochastic_workspace_size(2, 64, 0) == 0);
  CHECK(tree_candidate_workspace_size(4, 513, 1000) == 0);
  CHECK(tree_candidate_workspace_size(4, 64, 0) == 0);
  const size_t cws = tree_candidate_workspace_size(4, 64, 1000);
  CHECK(cws > 0);
  for (int V : {1, 15, 16, 17, 32000, 128256, 1 << 24}) CHECK(tree_candidate_workspace_size(16, 512, V) > 0);
  CHECK(tree_candidate_logits(4, 12, 64, 1000, 8, P, P, P, P, (float*)P, (int32_t*)P, P, cws, nullptr) ==
        TV_ERR_SHAPE);

  // cost table lookup and budget bars
  const int32_t bs[] = {1, 4, 16}, ls[] = {1024, 4096, 32768}, ns[] = {1, 16, 64};
  std::vector<float> cost(27);
  for (int i = 0; i < 3; ++i)
    for (int j = 0; j < 3; ++j)
      for (int k = 0; k < 3; ++k) cost[(i * 3 + j) * 3 + k] = 10.f + bs[i] * ls[j] * 1e-3f + ns[k];
  float out[64], bars[64];
  for (int B : {1, 3, 4, 100})
    for (int L : {0, 1, 2000, 40000})
      for (int n_max : {1, 17, 64}) {
        CHECK(tree_cost_lookup(bs, 3, ls, 3, ns, 3, cost.data(), B, L, n_max, out) == TV_OK);
        for (int N = 1; N < n_max; ++N) CHECK(out[N] >= out[N - 1] && isfinite(out[N]));
        CHECK(tree_budget_thresholds(out, n_max, 1e-3f, bars) == TV_OK);
      }
  const int32_t bad_axis[] = {4, 1, 16};
  CHECK(tree_cost_lookup(bad_axis, 3, ls, 3, ns, 3, cost.data(), 2, 2000, 64, out) == TV_ERR_SHAPE);
  CHECK(tree_cost_lookup(bs, 3, ls, 3, ns, 3, cost.data(), 2, 2000, 65, out) == TV_ERR_SHAPE);
  CHECK(tree_budget_thresholds(out, 0, 1e-3f, bars) == TV_ERR_SHAPE);

  if (g_fail) {
    fprintf(stderr, "%d host checks failed\n", g_fail);
    return 1;
  }
  printf("host checks ok\n");
  return 0;
}
