// Quality-aware bitwidth planner (host code).
//
// "Technical summary: PagedWeight", Core components 2: an offline,
// Hessian-weighted sensitivity score per linear block; online routing
// statistics, with frequently routed (hot) experts protected by higher
// bitwidth floors and damage multipliers; a prompt-specific correction of the
// sensitivity; and, when memory pressure sets a target, a greedy choice of the
// reductions with the least damage per byte saved until the target is met.
//
// Damage of block b at bitwidth q:  D_b(q) = mu_b * (S_b(q) + R_b(q)).
// A reduction step lowers one block by one bit (saving its plane bytes at cost
// D_b(q-1) - D_b(q)); steps are taken in increasing cost per byte (equal: the
// lower block index) until the resident plane bytes fit the budget.  When they
// already fit, the mirror steps restore bits in decreasing gain per byte among
// the steps that still fit.  Each block's next step does not depend on the
// other blocks, so a heap of one candidate per block yields the same sequence
// as rescanning every block at every step.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <queue>
#include <vector>

#include "pw_internal.h"

namespace {

using pw::kMaxBits;
using pw::kMinBits;

struct Cand {
  double key;
  int32_t b;
};

// Reduction order: smaller key first, then lower block index.
struct ReduceLater {
  bool operator()(const Cand& x, const Cand& y) const { return x.key > y.key || (x.key == y.key && x.b > y.b); }
};
// Restoration order: larger key first, then lower block index.
struct RestoreLater {
  bool operator()(const Cand& x, const Cand& y) const { return x.key < y.key || (x.key == y.key && x.b > y.b); }
};

}  // namespace

extern "C" {

pw_status pw_plan_bitwidths(const pw_plan_problem* P, const int32_t* q_cur, int64_t budget_bytes, int32_t* q_out,
                            int64_t* plane_bytes_out, int32_t* fits) {
  if (!P || !q_cur || !q_out) return PW_ERR_INVALID_ARG;
  const int32_t B = P->num_blocks, E = P->num_experts;
  if (B <= 0 || E <= 0 || !P->expert_of || !P->plane_bytes || !P->sensitivity) return PW_ERR_INVALID_ARG;
  if (P->floor_cold < kMinBits || P->floor_cold > kMaxBits || P->floor_hot < kMinBits || P->floor_hot > kMaxBits)
    return PW_ERR_BITWIDTH;
  for (int32_t b = 0; b < B; ++b) {
    if (P->expert_of[b] < 0 || P->expert_of[b] >= E || P->plane_bytes[b] <= 0) return PW_ERR_INVALID_ARG;
    if (q_cur[b] < kMinBits || q_cur[b] > kMaxBits) return PW_ERR_BITWIDTH;
  }

  // hot experts: the ceil(hot_fraction * E) largest positive masses, lower id on ties
  std::vector<char> hot(E, 0);
  if (P->routing_mass) {
    const int32_t n = (int32_t)ceil(P->hot_fraction * (double)E);
    std::vector<int32_t> ranked;
    for (int32_t e = 0; e < E; ++e)
      if (P->routing_mass[e] > 0.f) ranked.push_back(e);
    std::stable_sort(ranked.begin(), ranked.end(),
                     [&](int32_t a, int32_t c) { return P->routing_mass[a] > P->routing_mass[c]; });
    for (int32_t i = 0; i < n && i < (int32_t)ranked.size(); ++i) hot[ranked[i]] = 1;
  }

  std::vector<double> mu(B);
  std::vector<int32_t> floor(B), q(B);
  int64_t used = 0;
  for (int32_t b = 0; b < B; ++b) {
    const bool h = hot[P->expert_of[b]] != 0;
    mu[b] = h ? (double)P->hot_multiplier : 1.0;
    floor[b] = h ? P->floor_hot : P->floor_cold;
    q[b] = std::max(q_cur[b], floor[b]);
    used += (int64_t)q[b] * P->plane_bytes[b];
  }
  auto damage = [&](int32_t b, int32_t bits) {
    const double s = (double)P->sensitivity[(size_t)b * 6 + (bits - kMinBits)];
    const double r = P->correction ? (double)P->correction[(size_t)b * 6 + (bits - kMinBits)] : 0.0;
    return mu[b] * (s + r);
  };

  if (used > budget_bytes) {
    std::priority_queue<Cand, std::vector<Cand>, ReduceLater> heap;
    auto push = [&](int32_t b) {
      if (q[b] - 1 >= floor[b])
        heap.push({(damage(b, q[b] - 1) - damage(b, q[b])) / (double)P->plane_bytes[b], b});
    };
    for (int32_t b = 0; b < B; ++b) push(b);
    while (used > budget_bytes && !heap.empty()) {
      const int32_t b = heap.top().b;
      heap.pop();
      q[b] -= 1;
      used -= P->plane_bytes[b];
      push(b);
    }
  } else {
    std::priority_queue<Cand, std::vector<Cand>, RestoreLater> heap;
    auto push = [&](int32_t b) {
      if (q[b] + 1 <= kMaxBits)
        heap.push({(damage(b, q[b]) - damage(b, q[b] + 1)) / (double)P->plane_bytes[b], b});
    };
    for (int32_t b = 0; b < B; ++b) push(b);
    while (!heap.empty()) {
      const int32_t b = heap.top().b;
      heap.pop();
      // the remaining budget only shrinks, so a step that does not fit now never will
      if (used + P->plane_bytes[b] > budget_bytes) continue;
      q[b] += 1;
      used += P->plane_bytes[b];
      push(b);
    }
  }
  for (int32_t b = 0; b < B; ++b) q_out[b] = q[b];
  if (plane_bytes_out) *plane_bytes_out = used;
  if (fits) *fits = used <= budget_bytes ? 1 : 0;
  return PW_OK;
}

}  // extern "C"
