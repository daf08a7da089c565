// Work plan of the persistent attention launch (host code, no HIP).
//
// The attention forward runs one workgroup per compute unit, each walking a
// fixed list of work items. A unit of work is one workgroup's share of a
// schedule row (a Q tile, or a 256-row slice of a wider one); its cost is the
// number of 64-key steps its schedule holds. The plan
//   * keeps the last units of the sequence, a small share of the work, for a
//     shared tail (below), and
//   * deals the other units (head-major, Q tiles ascending) to the XCDs
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
//     pass merges;
//   * cuts the tail units into parts of falling size (each about the tail
//     work left over the workgroup count, and at least min_part steps) and
//     queues them for any workgroup whose own XCD's queue is empty. The XCDs
//     of one chip do not run equally fast (measured: 3-5% apart in steps
//     per second under the same load), so shares that end level by the cost
//     model do not end level on the device; the tail absorbs the difference,
//     and its last, short parts set how level the workgroups end.
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
  // Items by workgroup: the XCD queues' items as the plan simulated their
  // dispatch, and the tail's parts as a greedy dispatch would take them
  // (for the load statistics; the device takes tail parts as it goes).
  std::vector<int32_t> item_ptr;  // [n_wg + 1]: items of workgroup i
  std::vector<PlanItem> items;
  // The same items as queues: queue_ptr[x] .. queue_ptr[x + 1] index
  // queue_items; queue x < n_xcd holds XCD x's items ordered by the start
  // time the plan gave them, queue n_xcd the shared tail in the order it is
  // to be taken.
  std::vector<int32_t> queue_ptr;  // [n_xcd + 2]
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
// fewer steps than this where it can be avoided. tail: the share of the
// total cost kept for the shared tail (0: none); a tail is kept only when
// there are at least four units per workgroup, and its parts use at most
// kPlanTailSlotsPerWg * n_wg partial slots.
void plan_persistent(const int32_t* steps, const float* weight, int32_t n_units, int32_t n_wg,
                     int32_t n_xcd, int32_t block, int32_t overhead, int32_t min_part,
                     double tail, PlanResult& out);

constexpr int32_t kPlanTailSlotsPerWg = 3;
// Upper bound of the partial-result slots a plan uses: the parts of units
// split between the workgroups of an XCD (at most two per cut), and the
// parts of the tail.
inline int64_t plan_max_slots(int32_t n_wg) {
  return (2 + (int64_t)kPlanTailSlotsPerWg) * (int64_t)n_wg;
}
// Upper bound of the split units: each has at least two parts.
inline int64_t plan_max_combine(int32_t n_wg) { return plan_max_slots(n_wg) / 2; }
// Upper bound of the items: every unit once, plus one more per part.
inline int64_t plan_max_items(int64_t n_units, int32_t n_wg) {
  return n_units + plan_max_slots(n_wg);
}

}  // namespace svg
