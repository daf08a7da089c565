// Work plan of the persistent attention launch (host code, no HIP).
//
// The attention forward runs one workgroup per compute unit, each walking a
// fixed list of work items. A unit of work is one workgroup's share of a
// schedule row (a Q tile, or a 256-row slice of a wider one); its cost is the
// number of 64-key steps its schedule holds. The plan
//   * deals the unit sequence (head-major, Q tiles ascending) to the XCDs
//     in blocks of consecutive units, round by round, so that all XCDs work
//     on neighbouring Q tiles (which share KV tiles) at the same time, and
//     cuts the last units into one run per XCD so that the XCDs end level;
//   * gives each XCD's units, in order, to the workgroup that is free first
//     by the cost model (a greedy dispatch simulated ahead of time), so that
//     neighbouring units start at about the same time and share their KV
//     tiles in the XCD's L2;
//   * spreads each XCD's last units over its workgroups by cost, so that
//     every workgroup ends with the same cost: a unit cut between two or more
//     workgroups is a split unit, whose parts write partial results (the
//     unnormalised O, the running maximum and the row sum) that a combine
//     pass merges.
// Every step of every unit is executed exactly once: the parts of a unit are
// contiguous step ranges that start at 0, and the last part runs to the end
// of the row (kPlanToEnd), whatever its length.
#pragma once

#include <stdint.h>

#include <vector>

namespace svg {

constexpr int32_t kPlanToEnd = 0x7FFFFFFF;  // "to the last step of the row"

struct PlanItem {
  int32_t unit;  // row * nsub + sub
  int32_t s0;    // first step
  int32_t s1;    // one past the last step, or kPlanToEnd
  int32_t slot;  // partial-result slot, or -1: the item writes O itself
};

struct PlanCombine {
  int32_t unit;
  int32_t slot0;   // the unit's parts use slots slot0 .. slot0 + nparts - 1
  int32_t nparts;
  int32_t pad;
};

struct PlanResult {
  std::vector<int32_t> item_ptr;  // [n_wg + 1]: items of workgroup i
  std::vector<PlanItem> items;
  // The same items as one queue per XCD: queue_ptr[x] .. queue_ptr[x + 1]
  // index queue_items, ordered by the start time the plan gave them.
  std::vector<int32_t> queue_ptr;  // [n_xcd + 1]
  std::vector<PlanItem> queue_items;
  std::vector<PlanCombine> combine;
  int32_t n_slots = 0;
  int64_t max_load = 0;    // largest workgroup cost (weighted steps + per-item overhead)
  int64_t total_load = 0;  // sum over workgroups
};

// steps[u] < 0 marks a unit with no rows (a slice past the end of a ragged
// last Q tile); it gets no item. weight[u] (NULL: all 1) scales unit u's
// steps into cost: steps of one head kind can take longer than those of
// another, and the plan balances cost. Workgroup i runs on XCD i % n_xcd.
// block > 0: blocks of `block` consecutive units are dealt to the XCDs in
// rounds (all XCDs work on neighbouring Q tiles at one time, which the
// shared Infinity Cache rewards), the last units in one contiguous run per
// XCD; block == 0: one contiguous run per XCD. overhead: the cost of
// starting an item, in steps. min_part: a unit is not cut into parts of
// fewer steps than this where it can be avoided.
void plan_persistent(const int32_t* steps, const float* weight, int32_t n_units, int32_t n_wg,
                     int32_t n_xcd, int32_t block, int32_t overhead, int32_t min_part,
                     PlanResult& out);

// Upper bound of the partial-result slots a plan uses: the parts of split
// units, at most two per cut between workgroups.
inline int64_t plan_max_slots(int32_t n_wg) { return 2 * (int64_t)n_wg; }
// Upper bound of the items: every unit once, plus one more per part.
inline int64_t plan_max_items(int64_t n_units, int32_t n_wg) {
  return n_units + plan_max_slots(n_wg);
}

}  // namespace svg
