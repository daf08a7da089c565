// Work plan of the persistent attention launch; see plan.hpp.
#include "plan.hpp"

#include <algorithm>
#include <cmath>
#include <functional>
#include <queue>
#include <utility>

namespace svg {

void plan_persistent(const int32_t* steps, const float* weight, int32_t n_units, int32_t n_wg,
                     int32_t n_xcd, int32_t block, int32_t overhead, int32_t min_part,
                     double tail, PlanResult& out) {
  out = PlanResult{};
  const int32_t P = std::max(1, n_wg);
  const int32_t X = std::max(1, std::min(n_xcd, P));
  std::vector<std::vector<PlanItem>> per_wg(P);
  std::vector<std::vector<double>> per_wg_start(P);  // simulated start of each item
  std::vector<double> load(P, 0.0);
  auto emit = [&](int32_t i, const PlanItem& it, double c) {
    per_wg[i].push_back(it);
    per_wg_start[i].push_back(load[i]);
    load[i] += c;
  };

  // Units that have rows, in order, and their costs.
  std::vector<int32_t> U;
  U.reserve(n_units);
  for (int32_t u = 0; u < n_units; ++u)
    if (steps[u] >= 0) U.push_back(u);
  const int64_t M = (int64_t)U.size();
  auto w = [&](int64_t j) { return weight ? (double)weight[U[j]] : 1.0; };
  auto work = [&](int64_t j) { return w(j) * (double)steps[U[j]]; };  // weighted steps
  auto cost = [&](int64_t j) { return work(j) + overhead; };
  std::vector<double> pre(M + 1, 0.0);  // cost prefix
  for (int64_t j = 0; j < M; ++j) pre[j + 1] = pre[j] + cost(j);
  const double total = pre[M];

  // The shared tail: the last units, whose cost is at most `tail` of the
  // total, kept when there are four units per workgroup. The XCDs share
  // units [0, Mx) as below.
  int64_t Mx = M;
  if (tail > 0.0 && M >= 4 * (int64_t)P) {
    const double want = tail * total;
    while (Mx > 0 && pre[M] - pre[Mx - 1] <= want) --Mx;
  }
  const double xtotal = pre[Mx];

  // Workgroups of XCD x: i = k * X + x for k < G[x].
  std::vector<int32_t> G(X);
  for (int32_t x = 0; x < X; ++x) G[x] = P / X + (x < P % X ? 1 : 0);

  // Each XCD's sequence of units (indices into U). With blocks: block
  // r * X + x of `block` consecutive units goes to XCD x in round r, so
  // that all XCDs work on neighbouring Q tiles at the same time; the units
  // after the last full round but one are cut into one contiguous run per
  // XCD, sized so that the XCDs' costs end proportional to G[x]. Without:
  // the whole sequence is cut that way.
  std::vector<std::vector<int64_t>> seq(X);
  {
    std::vector<double> have(X, 0.0);
    int64_t rest = 0;
    if (block > 0) {
      const int64_t nb = (Mx + block - 1) / block;
      const int64_t rounds = std::max<int64_t>(0, nb / X - 1);
      for (int64_t r = 0; r < rounds; ++r)
        for (int32_t x = 0; x < X; ++x)
          for (int64_t j = (r * X + x) * block; j < (r * X + x + 1) * block; ++j) {
            seq[x].push_back(j);
            have[x] += cost(j);
          }
      rest = rounds * X * block;
    }
    // the rest: contiguous runs, XCD x's run of cost (target - have), kept
    // at least empty and scaled to the rest's cost
    std::vector<double> need(X);
    double sneed = 0.0;
    for (int32_t x = 0; x < X; ++x) {
      need[x] = std::max(0.0, xtotal * (double)G[x] / (double)P - have[x]);
      sneed += need[x];
    }
    const double rcost = xtotal - pre[rest];
    double acc = pre[rest];
    int64_t j = rest;
    for (int32_t x = 0; x < X; ++x) {
      acc += sneed > 0.0 ? rcost * need[x] / sneed : rcost / X;
      // a unit goes to the run its cost midpoint falls in
      while (j < Mx && (x == X - 1 || pre[j] + 0.5 * cost(j) < acc)) seq[x].push_back(j++);
    }
  }

  int32_t next_slot = 0;
  for (int32_t x = 0; x < X; ++x) {
    const std::vector<int64_t>& sq = seq[x];
    const int64_t m = (int64_t)sq.size();
    const int32_t g = G[x];
    if (m <= 0 || g <= 0) continue;
    auto wg = [&](int32_t k) { return k * X + x; };
    // Whole units first, each to the workgroup that is free first (the
    // least loaded so far, the lowest index on a tie): the dispatch order a
    // greedy device would take, so that units neighbouring in the sequence
    // start at about the same time and share their KV tiles in the L2.
    // Between g and 2g - 1 units are left for the spread.
    const int64_t R = m >= 2 * (int64_t)g ? m / g - 1 : 0;
    std::vector<double> A(g, 0.0);
    std::vector<int32_t> kmap(g);  // workgroups of the spread, earliest free first
    {
      typedef std::pair<double, int32_t> Slot;
      std::priority_queue<Slot, std::vector<Slot>, std::greater<Slot>> freeq;
      for (int32_t k = 0; k < g; ++k) freeq.push(Slot(0.0, k));
      for (int64_t i = 0; i < R * g; ++i) {
        const int64_t jj = sq[i];
        const Slot f = freeq.top();
        freeq.pop();
        emit(wg(f.second), PlanItem{U[jj], 0, kPlanToEnd, -1}, cost(jj));
        A[f.second] += cost(jj);
        freeq.push(Slot(A[f.second], f.second));
      }
      for (int32_t k = 0; k < g; ++k) {
        kmap[k] = freeq.top().second;
        freeq.pop();
      }
    }
    // The rest, spread by weighted steps so that every workgroup ends level.
    double lwork = 0.0, xcost = 0.0;
    int64_t lsteps = 0;
    for (int64_t i = 0; i < m; ++i) {
      xcost += cost(sq[i]);
      if (i < R * g) continue;
      lwork += work(sq[i]);
      lsteps += steps[U[sq[i]]];
    }
    const double tau = xcost / (double)g;
    // Workgroups that take part in the spread: all of them after full
    // rounds; without rounds no more than keep parts at min_part steps.
    int32_t ge = g;
    if (R == 0)
      ge = (int32_t)std::max<int64_t>(1, std::min<int64_t>(g, lsteps / std::max(1, min_part)));
    std::vector<double> cap(ge, 0.0);
    double scap = 0.0;
    for (int32_t k = 0; k < ge; ++k) {
      cap[k] = std::max(0.0, tau - A[kmap[k]]);
      scap += cap[k];
    }
    if (!(scap > 0.0)) {
      for (int32_t k = 0; k < ge; ++k) cap[k] = 1.0;
      scap = ge;
    }
    // Cut points in the leftover work: workgroup k takes [pc[k], pc[k+1]).
    std::vector<double> pc(ge + 1, 0.0);
    {
      double acc = 0.0;
      for (int32_t k = 1; k < ge; ++k) {
        acc += cap[k - 1];
        pc[k] = std::min(lwork, std::max(pc[k - 1], lwork * acc / scap));
      }
      pc[ge] = lwork;
    }
    double u0 = 0.0;
    int32_t kk = 0;  // first workgroup whose range may hold u0
    for (int64_t i = R * g; i < m; ++i) {
      const int64_t j = sq[i];
      const int32_t unit = U[j];
      const int32_t n = steps[unit];
      const double wj = w(j), u1 = u0 + wj * n;
      while (kk + 1 < ge && pc[kk + 1] <= u0) ++kk;  // pc[kk] <= u0 < pc[kk+1], or the last
      // a cut point at work position c falls after step round((c - u0) / wj)
      auto step_at = [&](double c) {
        const double t = (c - u0) / wj;
        return (int32_t)std::min<double>(n, std::max(0.0, std::floor(t + 0.5)));
      };
      // parts: [cut(k), cut(k+1)) over the workgroups whose ranges meet it,
      // empty step ranges dropped
      std::vector<std::pair<int32_t, int32_t>> parts;  // (workgroup k, first step)
      int32_t prev = 0;
      for (int32_t k = kk; k < ge; ++k) {
        if (k > kk && pc[k] >= u1) break;
        const int32_t e = k + 1 < ge ? step_at(pc[k + 1]) : n;
        const int32_t s0 = k == kk ? 0 : prev;
        if (e > s0 || (n == 0 && parts.empty())) parts.emplace_back(k, s0);
        prev = std::max(prev, e);
        if (e >= n) break;
      }
      if (parts.size() <= 1) {
        const int32_t k = kmap[parts.empty() ? kk : parts[0].first];
        emit(wg(k), PlanItem{unit, 0, kPlanToEnd, -1}, wj * n + overhead);
      } else {
        const int32_t slot0 = next_slot;
        for (size_t i = 0; i < parts.size(); ++i) {
          const int32_t s0 = parts[i].second;
          const int32_t s1 = i + 1 < parts.size() ? parts[i + 1].second : kPlanToEnd;
          const int32_t e = i + 1 < parts.size() ? s1 : n;
          const int32_t k = kmap[parts[i].first];
          emit(wg(k), PlanItem{unit, s0, s1, next_slot++}, wj * (e - s0) + overhead);
        }
        out.combine.push_back(PlanCombine{unit, slot0, (int32_t)parts.size(), 0});
      }
      u0 = u1;
    }
  }

  // per XCD: its workgroups' items by simulated start (then workgroup and
  // position, for a fixed order)
  out.queue_ptr.assign(X + 2, 0);
  for (int32_t x = 0; x < X; ++x) {
    struct Q {
      double start;
      int32_t wg, pos;
    };
    std::vector<Q> q;
    for (int32_t i = x; i < P; i += X)
      for (int32_t k = 0; k < (int32_t)per_wg[i].size(); ++k) q.push_back(Q{per_wg_start[i][k], i, k});
    std::sort(q.begin(), q.end(), [](const Q& a, const Q& b) {
      return a.start != b.start ? a.start < b.start : (a.wg != b.wg ? a.wg < b.wg : a.pos < b.pos);
    });
    for (const Q& e : q) out.queue_items.push_back(per_wg[e.wg][e.pos]);
    out.queue_ptr[x + 1] = (int32_t)out.queue_items.size();
  }

  // The tail: each unit cut, in sequence order, into parts of about the
  // tail work left over the workgroups (at least mp steps; a rest shorter
  // than that joins the part before it), so that the parts shrink towards
  // the end; mp is min_part, raised where the parts would need more than the
  // tail's slots. The queue takes them longest first.
  {
    double tail_work = 0.0;
    int32_t longest = 0;
    for (int64_t j = Mx; j < M; ++j) {
      tail_work += work(j);
      longest = std::max(longest, steps[U[j]]);
    }
    const int64_t budget = (int64_t)kPlanTailSlotsPerWg * P;
    // parts of tail unit j, given the tail work r left before it
    auto cut = [&](int64_t j, double r, int32_t mp, std::vector<std::pair<int32_t, int32_t>>& parts) {
      const int32_t n = steps[U[j]];
      const double wj = w(j);
      parts.clear();
      for (int32_t s0 = 0; s0 < n;) {
        const double want = std::ceil(r / ((double)P * wj));
        int32_t len = (int32_t)std::min<double>(n - s0, std::max<double>(mp, want));
        if (n - s0 - len < mp) len = n - s0;
        parts.emplace_back(s0, s0 + len);
        s0 += len;
        r -= wj * len;
      }
    };
    std::vector<std::pair<int32_t, int32_t>> parts;  // [s0, e)
    auto slots_for = [&](int32_t mp) {
      int64_t n = 0;
      double r = tail_work;
      for (int64_t j = Mx; j < M; ++j) {
        cut(j, r, mp, parts);
        if (parts.size() > 1) n += (int64_t)parts.size();
        r -= work(j);
      }
      return n;
    };
    int32_t mp = std::max(1, min_part);
    while (mp <= longest && slots_for(mp) > budget) mp += std::max(1, mp / 8);
    std::vector<std::pair<PlanItem, double>> titems;  // item, cost
    double rem = tail_work;
    for (int64_t j = Mx; j < M; ++j) {
      const int32_t unit = U[j], n = steps[unit];
      const double wj = w(j);
      cut(j, rem, mp, parts);
      rem -= work(j);
      if (parts.size() <= 1) {
        titems.emplace_back(PlanItem{unit, 0, kPlanToEnd, -1}, wj * n + overhead);
      } else {
        out.combine.push_back(PlanCombine{unit, next_slot, (int32_t)parts.size(), 0});
        for (size_t i = 0; i < parts.size(); ++i) {
          const int32_t s1 = i + 1 < parts.size() ? parts[i].second : kPlanToEnd;
          titems.emplace_back(PlanItem{unit, parts[i].first, s1, next_slot++},
                              wj * (parts[i].second - parts[i].first) + overhead);
        }
      }
    }
    // longest first (stable), so that a rest joined to a part does not
    // come last
    std::stable_sort(titems.begin(), titems.end(),
                     [](const std::pair<PlanItem, double>& a, const std::pair<PlanItem, double>& b) {
                       return a.second > b.second;
                     });
    // queue X; for the statistics, each part goes to the workgroup that is
    // free first by the cost model
    typedef std::pair<double, int32_t> Slot;
    std::priority_queue<Slot, std::vector<Slot>, std::greater<Slot>> freeq;
    for (int32_t i = 0; i < P; ++i) freeq.push(Slot(load[i], i));
    for (const auto& ti : titems) {
      out.queue_items.push_back(ti.first);
      const Slot f = freeq.top();
      freeq.pop();
      emit(f.second, ti.first, ti.second);
      freeq.push(Slot(load[f.second], f.second));
    }
    out.queue_ptr[X + 1] = (int32_t)out.queue_items.size();
  }

  out.n_slots = next_slot;
  out.item_ptr.assign(P + 1, 0);
  for (int32_t i = 0; i < P; ++i) {
    out.item_ptr[i + 1] = out.item_ptr[i] + (int32_t)per_wg[i].size();
    out.items.insert(out.items.end(), per_wg[i].begin(), per_wg[i].end());
    out.max_load = std::max(out.max_load, (int64_t)std::llround(load[i]));
    out.total_load += (int64_t)std::llround(load[i]);
  }
}

}  // namespace svg
