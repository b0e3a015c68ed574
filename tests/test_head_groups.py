"""Ragged head-group tables and their memory (Tangram): the plain-Python plan in
oracle/plan.py pinned by brute force and a hand-worked example, then the library's
host function against it (CPU only)."""
import numpy as np
import pytest

from oracle import plan


def test_sorted_grouping_is_optimal_by_brute_force():
    """Over every partition of 6 heads into groups of 2 or 3 (and 8 into 2 or 4), the
    grouping by decreasing budget has the smallest grouped memory."""
    r = np.random.default_rng(3)
    for hkv, size in ((6, 2), (6, 3), (8, 2), (8, 4)):
        for _ in range(6):
            budgets = np.float32(r.uniform(0.05, 1.0, hkv))
            n = int(r.integers(100, 5000))
            best = min(plan.group_cost(gr, budgets, n, 1)[0] for gr in plan.all_groupings(list(range(hkv)), size))
            _, _, nbytes = plan.head_group_plan(budgets, size, n, 1)
            assert nbytes[0] == best


def test_hand_worked_example():
    """Budgets (1/8, 7/8, 1/2, 1/4) (exact in fp32), groups of 2, 96 tokens, INT4
    (2560 B per head-page): kept 12, 84, 48, 24 tokens; order 1, 2, 3, 0 -> groups
    {1, 2} (84 slots, 6 pages) and {3, 0} (24 slots, 2 pages):
    6*2*2560 + 4*84 + 2*2*2560 + 4*24 = 41392 B; per-head tables 1+6+3+2 = 12 pages:
    12*2560 + 4*168 = 31392 B; no eviction 4 heads * 6 pages * (2560 + 4) = 61536 B."""
    order, slots, nbytes = plan.head_group_plan(np.float32([0.125, 0.875, 0.5, 0.25]), 2, 96, 1)
    assert order == [1, 2, 3, 0] and slots == [84, 24]
    assert nbytes == [41392, 31392, 61536]


def test_library_matches_the_plan():
    from mixed_precision_quantized_amd import kvq
    r = np.random.default_rng(5)
    for hkv, size in ((8, 2), (8, 4), (8, 1), (8, 8), (16, 4), (4, 2)):
        for cls in (0, 1, 2):
            budgets = np.float32(r.uniform(0.01, 1.0, hkv))
            budgets[r.integers(0, hkv)] = budgets[0]                      # a tie
            n = int(r.integers(1, 200000))
            order, slots, nbytes = kvq.head_group_plan(budgets, size, n, cls)
            o2, s2, b2 = plan.head_group_plan(budgets, size, n, cls)
            assert list(order) == o2 and list(slots) == s2 and list(nbytes) == b2
    # the ragged workload's budgets 0.1 + 0.9 h / 7 in groups of 2
    r_h = np.float32([0.1 + 0.9 * h / 7 for h in range(8)])
    order, slots, _ = kvq.head_group_plan(r_h, 2, 4096, 1)
    assert list(order) == [7, 6, 5, 4, 3, 2, 1, 0]


def test_library_rejects_bad_arguments():
    from mixed_precision_quantized_amd import kvq
    with pytest.raises(kvq.KvqError):
        kvq.head_group_plan(np.float32([0.5, 0.5, 0.5]), 2, 100)        # 2 does not divide 3
    with pytest.raises(kvq.KvqError):
        kvq.head_group_plan(np.float32([0.5, 0.0]), 1, 100)             # budget 0
    with pytest.raises(kvq.KvqError):
        kvq.head_group_plan(np.float32([0.5, 1.5]), 1, 100)             # budget > 1
    with pytest.raises(kvq.KvqError):
        kvq.head_group_plan(np.float32([0.5, 0.5]), 1, 100, cls=7)
