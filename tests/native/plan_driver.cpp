// Test driver for the persistent-launch planner (host code only).
// stdin:  n_units n_wg n_xcd block overhead min_part has_weights tail, then
//         n_units step counts, then (has_weights) n_units weights
// stdout: "P n_slots max_load total_load n_items n_combine", then item_ptr,
//         then one "unit s0 s1 slot" line per item, one "unit slot0 nparts"
//         line per combine entry, then queue_ptr and the queue's items.
#include <cstdio>
#include <vector>

#include "plan.hpp"

int main() {
  int n, P, X, block, ovh, minp, hw;
  double tail;
  if (std::scanf("%d %d %d %d %d %d %d %lf", &n, &P, &X, &block, &ovh, &minp, &hw, &tail) != 8)
    return 2;
  std::vector<int32_t> steps(n);
  std::vector<float> weight(n, 1.0f);
  for (int i = 0; i < n; ++i)
    if (std::scanf("%d", &steps[i]) != 1) return 2;
  for (int i = 0; i < n && hw; ++i)
    if (std::scanf("%f", &weight[i]) != 1) return 2;
  svg::PlanResult r;
  svg::plan_persistent(steps.data(), hw ? weight.data() : nullptr, n, P, X, block, ovh, minp, tail,
                       r);
  std::printf("%d %d %lld %lld %zu %zu\n", P, r.n_slots, (long long)r.max_load,
              (long long)r.total_load, r.items.size(), r.combine.size());
  for (size_t i = 0; i < r.item_ptr.size(); ++i) std::printf("%d ", r.item_ptr[i]);
  std::printf("\n");
  for (const auto& it : r.items) std::printf("%d %d %d %d\n", it.unit, it.s0, it.s1, it.slot);
  for (const auto& c : r.combine) std::printf("%d %d %d\n", c.unit, c.slot0, c.nparts);
  for (size_t i = 0; i < r.queue_ptr.size(); ++i) std::printf("%d ", r.queue_ptr[i]);
  std::printf("\n");
  for (const auto& it : r.queue_items) std::printf("%d %d %d %d\n", it.unit, it.s0, it.s1, it.slot);
  return 0;
}
