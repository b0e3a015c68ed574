"""Ragged head-group tables and their memory -- TEST INFRASTRUCTURE ONLY.

Plain Python written from the Tangram page (per-head budgets r_h; the heads of one
group share a slot-map table as long as the group's largest budget needs, each head
reading its own prefix): head h of a request of n tokens keeps ceil(r_h n) tokens, a
group's table has the largest of its heads' counts, and the memory counts whole
16-slot pages per head plus 4 bytes per table entry.  Page bytes per head follow the
cache layout: 16 tokens x 96 B (INT2), 160 B (INT4), 512 B (FP16).

Only the tests may import this module; the library shares nothing with it.
"""
import math

PAGE = 16
HEAD_PAGE_BYTES = {0: 16 * 96, 1: 16 * 160, 2: 16 * 512}   # INT2, INT4, FP16


def kept(budget, n):
    return math.ceil(float(budget) * n)


def group_cost(groups, budgets, n, cls):
    """Bytes of the given grouping (a list of lists of head ids) and its table lengths."""
    block = HEAD_PAGE_BYTES[cls]
    total, slots = 0, []
    for grp in groups:
        s = max(kept(budgets[h], n) for h in grp)
        slots.append(s)
        total += -(-s // PAGE) * len(grp) * block + 4 * s
    return total, slots


def head_group_plan(budgets, heads_per_group, n, cls):
    """(order, table_slots, [grouped, per-head, no-eviction] bytes) with heads grouped
    consecutively by decreasing budget (ties: lower id first)."""
    hkv = len(budgets)
    order = sorted(range(hkv), key=lambda h: (-float(budgets[h]), h))
    groups = [order[i:i + heads_per_group] for i in range(0, hkv, heads_per_group)]
    grouped, slots = group_cost(groups, budgets, n, cls)
    block = HEAD_PAGE_BYTES[cls]
    exact = sum(-(-kept(r, n) // PAGE) * block + 4 * kept(r, n) for r in budgets)
    dense = hkv * -(-n // PAGE) * (block + 4)
    return order, slots, [grouped, exact, dense]


def all_groupings(heads, size):
    """Every partition of heads into groups of the given size (small cases only)."""
    if not heads:
        yield []
        return
    first, rest = heads[0], heads[1:]
    from itertools import combinations
    for mates in combinations(rest, size - 1):
        left = [h for h in rest if h not in mates]
        for tail in all_groupings(left, size):
            yield [[first, *mates]] + tail
