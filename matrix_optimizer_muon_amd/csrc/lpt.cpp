// Host-side global LPT partition of Muon units over owner slots.
//
// DMuon "架构设计" (Architecture design) page, §3.1 "分区（全局 LPT）": a single
// greedy longest-processing-time pass over all units of the model, with two
// built-in constraints: units of one transformer layer go to distinct owner
// slots (so that per-layer broadcasts from different owners run concurrently),
// and same-layer units under a size threshold are merged into one unit with one
// owner.  The page quotes the LPT bound 4/3 − 1/(3R) and argues that only a
// global (not per-layer) pass can balance 7 matrices per layer over 8 slots.
//
// Runs once at set-up, off the step's hot path; a heap of slots keyed by
// (load, id) gives O(n log R) when the layer rule leaves the top slots eligible.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <map>
#include <numeric>
#include <set>
#include <string>
#include <tuple>
#include <unordered_map>
#include <utility>
#include <vector>

#include "../../include/dmuon_ns.h"

namespace dmuon {
int lpt_fail(int code, const char* msg);
void clear_error();
}

namespace {

struct Unit {
  int64_t first;                // input index of its first member
  std::vector<int64_t> members;
  int64_t cost;
  int32_t layer;
};

int64_t unit_cost(int64_t rows, int64_t cols, int64_t batch, int32_t kind) {
  if (kind == 0) return batch * rows * cols;
  const int64_t m = std::min(rows, cols), n = std::max(rows, cols);
  return batch * (4 * m * m * n + 2 * m * m * m);
}

}  // namespace

extern "C" int dmuon_lpt_assign(int64_t n, const int64_t* rows, const int64_t* cols, const int64_t* batch,
                                const int32_t* layer_id, int32_t n_slots, int64_t merge_below_elems,
                                int32_t cost_kind, int32_t* slot_of, int64_t* slot_load, int32_t owner_slot,
                                int64_t* owner_order, int64_t* n_owned, int64_t* group_offsets,
                                int32_t* n_groups) {
  using dmuon::lpt_fail;
  dmuon::clear_error();
  if (n < 0) return lpt_fail(DMUON_E_SHAPE, "n < 0");
  if (n_slots <= 0) return lpt_fail(DMUON_E_SHAPE, "n_slots must be positive");
  if (cost_kind != 0 && cost_kind != 1) return lpt_fail(DMUON_E_CFG, "cost_kind must be 0 or 1");
  if (merge_below_elems < 0) return lpt_fail(DMUON_E_CFG, "merge_below_elems must be >= 0");
  if (!slot_load) return lpt_fail(DMUON_E_NULL, "slot_load is NULL");
  if (n > 0 && (!rows || !cols || !batch || !layer_id || !slot_of))
    return lpt_fail(DMUON_E_NULL, "item arrays and slot_of must be set");
  const bool want_owner = owner_order || n_owned || group_offsets || n_groups;
  if (want_owner && !(owner_order && n_owned && group_offsets && n_groups))
    return lpt_fail(DMUON_E_NULL, "owner_order, n_owned, group_offsets and n_groups go together");
  if (want_owner && (owner_slot < 0 || owner_slot >= n_slots))
    return lpt_fail(DMUON_E_SHAPE, "owner_slot out of range");
  for (int64_t i = 0; i < n; ++i) {
    if (rows[i] < 0 || cols[i] < 0 || batch[i] < 1 || rows[i] > (1 << 20) || cols[i] > (1 << 20))
      return lpt_fail(DMUON_E_SHAPE, "item dims out of range (rows, cols in [0, 2^20], batch >= 1)");
  }

  // ---- units, with same-layer small items merged (constraint 2) ----
  std::vector<Unit> units;
  units.reserve((size_t)n);
  std::unordered_map<int32_t, size_t> merged_unit;  // layer → unit holding its small items
  for (int64_t i = 0; i < n; ++i) {
    const int64_t numel = batch[i] * rows[i] * cols[i];
    const int64_t c = unit_cost(rows[i], cols[i], batch[i], cost_kind);
    const int32_t lay = layer_id[i];
    if (merge_below_elems > 0 && lay >= 0 && numel < merge_below_elems) {
      auto it = merged_unit.find(lay);
      if (it != merged_unit.end()) {
        units[it->second].members.push_back(i);
        units[it->second].cost += c;
        continue;
      }
      merged_unit[lay] = units.size();
    }
    units.push_back(Unit{i, {i}, c, lay});
  }

  // ---- visit order: cost descending, ties in input order ----
  std::vector<size_t> order(units.size());
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](size_t x, size_t y) { return units[x].cost > units[y].cost; });

  // ---- greedy placement (constraint 1: distinct slots per layer) ----
  std::vector<int64_t> load((size_t)n_slots, 0);
  std::set<std::pair<int64_t, int32_t>> by_load;   // (load, slot)
  for (int32_t s = 0; s < n_slots; ++s) by_load.insert({0, s});
  std::unordered_map<int32_t, std::vector<char>> layer_slots;   // layer → slot flags
  std::vector<int64_t> assigned;
  assigned.reserve((size_t)n);
  for (size_t u : order) {
    const Unit& U = units[u];
    std::vector<char>* used = nullptr;
    if (U.layer >= 0) {
      auto& v = layer_slots[U.layer];
      if (v.empty()) v.assign((size_t)n_slots, 0);
      used = &v;
    }
    int32_t best = -1;
    for (const auto& ls : by_load) {          // least load first, then lowest id
      if (!used || !(*used)[(size_t)ls.second]) {
        best = ls.second;
        break;
      }
    }
    if (best < 0) best = by_load.begin()->second;   // every slot holds this layer
    by_load.erase({load[(size_t)best], best});
    load[(size_t)best] += U.cost;
    by_load.insert({load[(size_t)best], best});
    if (used) (*used)[(size_t)best] = 1;
    for (int64_t i : U.members) {
      slot_of[i] = best;
      assigned.push_back(i);
    }
  }
  for (int32_t s = 0; s < n_slots; ++s) slot_load[s] = load[(size_t)s];

  // ---- the owner's share, grouped by exact shape in order of first assignment ----
  if (want_owner) {
    std::vector<std::tuple<int64_t, int64_t, int64_t>> keys;
    std::map<std::tuple<int64_t, int64_t, int64_t>, std::vector<int64_t>> groups;
    for (int64_t i : assigned) {
      if (slot_of[i] != owner_slot) continue;
      const auto key = std::make_tuple(batch[i], rows[i], cols[i]);
      auto it = groups.find(key);
      if (it == groups.end()) {
        keys.push_back(key);
        groups[key] = {i};
      } else {
        it->second.push_back(i);
      }
    }
    int64_t pos = 0;
    int32_t g = 0;
    for (const auto& key : keys) {
      group_offsets[g++] = pos;
      for (int64_t i : groups[key]) owner_order[pos++] = i;
    }
    group_offsets[g] = pos;
    *n_owned = pos;
    *n_groups = g;
  }
  return DMUON_OK;
}
