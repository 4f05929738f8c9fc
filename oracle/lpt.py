"""Reference global LPT partition of Muon units over owner slots.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this module.  The product's C++
``dmuon_lpt_assign`` shares no code with it.

Follows the DMuon "架构设计" (Architecture design) page, §3.1 "分区（全局 LPT）"
(partition, global LPT):
* one greedy longest-processing-time pass over all Muon units at once;
* constraint 1: units of the same transformer layer go to different owner slots;
* constraint 2: same-layer units below a size threshold (default 5M elements)
  are merged into one unit with one owner;
* the LPT quality bound 4/3 − 1/(3R) and the per-layer counter-example
  (R = 8 slots, 7 matrices per layer leaves one slot idle every layer).

Readings where the page is silent:
* cost = element count (cost_kind 0) or the NS flop count batch·(4m²n + 2m³)
  (cost_kind 1);
* units are visited in a stable sort by cost, largest first, ties in input
  (registration) order; a merged unit sits at its first member's position;
* each unit goes to the least-loaded slot that holds no unit of its layer, ties
  to the lowest slot id; if every slot holds that layer, to the least-loaded
  slot overall; a negative layer id means "no layer constraint";
* the owner's share is listed in assignment order, grouped by exact shape
  (batch, rows, cols), groups in order of first appearance.
"""
from __future__ import annotations


def _cost(rows, cols, batch, cost_kind):
    if cost_kind == 0:
        return batch * rows * cols
    m, n = min(rows, cols), max(rows, cols)
    return batch * (4 * m * m * n + 2 * m * m * m)


def lpt_assign(rows, cols, batch, layer_id, n_slots, merge_below_elems=0,
               cost_kind=0, owner_slot=0):
    """Global LPT with the same-layer-distinct-slot rule and optional merge.

    Returns a dict with ``slot_of`` (per input item), ``slot_load`` (per slot),
    ``owner_order`` (item indices owned by ``owner_slot``, grouped by shape) and
    ``group_offsets`` (len n_groups + 1).
    """
    n = len(rows)
    if not (len(cols) == len(batch) == len(layer_id) == n):
        raise ValueError("item arrays differ in length")
    if n_slots <= 0:
        raise ValueError("n_slots must be positive")
    # --- build units (constraint 2: merge small same-layer items) ---
    units = []          # list of (first_index, members, cost, layer)
    merged_of_layer = {}
    for i in range(n):
        numel = batch[i] * rows[i] * cols[i]
        c = _cost(rows[i], cols[i], batch[i], cost_kind)
        lay = layer_id[i]
        if merge_below_elems > 0 and lay >= 0 and numel < merge_below_elems:
            if lay in merged_of_layer:
                u = merged_of_layer[lay]
                units[u][1].append(i)
                units[u][2] += c
                continue
            merged_of_layer[lay] = len(units)
        units.append([i, [i], c, lay])
    # --- stable sort by cost, largest first ---
    order = sorted(range(len(units)), key=lambda u: -units[u][2])
    load = [0] * n_slots
    layers_in_slot = [set() for _ in range(n_slots)]
    slot_of = [-1] * n
    assigned_seq = []   # item indices in the order they were assigned
    for u in order:
        first, members, c, lay = units[u]
        eligible = [s for s in range(n_slots)
                    if lay < 0 or lay not in layers_in_slot[s]]
        if not eligible:
            eligible = list(range(n_slots))
        best = min(eligible, key=lambda s: (load[s], s))
        load[best] += c
        if lay >= 0:
            layers_in_slot[best].add(lay)
        for i in members:
            slot_of[i] = best
            assigned_seq.append(i)
    # --- the owner's share, grouped by exact shape ---
    groups = {}
    group_keys = []
    for i in assigned_seq:
        if slot_of[i] != owner_slot:
            continue
        key = (batch[i], rows[i], cols[i])
        if key not in groups:
            groups[key] = []
            group_keys.append(key)
        groups[key].append(i)
    owner_order, offsets = [], [0]
    for key in group_keys:
        owner_order.extend(groups[key])
        offsets.append(len(owner_order))
    return {"slot_of": slot_of, "slot_load": load,
            "owner_order": owner_order, "group_offsets": offsets}


def per_layer_lpt(rows, cols, batch, layer_id, n_slots, cost_kind=0):
    """LPT run separately inside each layer, every layer starting from empty slots.

    This is the local scheme the architecture page §3.1 argues against ("why it
    must be global"): with 7 matrices per layer and 8 slots it never uses the
    last slot.  Returns the per-slot loads summed over layers.
    """
    total = [0] * n_slots
    layers = []
    for lay in layer_id:
        if lay not in layers:
            layers.append(lay)
    for lay in layers:
        idx = [i for i in range(len(rows)) if layer_id[i] == lay]
        res = lpt_assign([rows[i] for i in idx], [cols[i] for i in idx],
                         [batch[i] for i in idx], [0] * len(idx), n_slots,
                         cost_kind=cost_kind)
        for s in range(n_slots):
            total[s] += res["slot_load"][s]
    return total
