"""Host checks of the synthetic workload recipes (seeded input generation only)."""
import numpy as np

import synth
from oracle import oracle


def _counts(entries):
    c = np.zeros((synth.N_TEMPORAL, synth.N_MODAL, synth.N_SEMANTIC), np.int64)
    for (t, m, s), n in entries.items():
        c[t, m, s] = n
    return c


def test_greedy_bits_walks_rho_order_and_stops_at_the_first_misfit():
    # rho = 0.96 D(2) / (2 N): A = 32/20, C = 16/160, B = 0.3/20, so the walk is A, C, B.
    A, B, C = (0, 0, 0), (3, 1, 6), (0, 0, 1)
    counts = _counts({A: 10, B: 10, C: 80})
    bits = synth.greedy_bits(counts, 2.6)       # 200 + 20 (A) fits 260, C would give 380
    assert bits[A] == 4 and bits[C] == 2 and bits[B] == 2   # B would fit but the walk stopped
    bits = synth.greedy_bits(counts, 3.9)       # A and C fit 390, B would give 400
    assert bits[A] == 4 and bits[C] == 4 and bits[B] == 2
    bits = synth.greedy_bits(counts, 4.0)
    assert (bits[counts > 0] == 4).all()
    assert (synth.greedy_bits(counts, 2.0)[counts > 0] == 2).all()


def test_agentic_recipe():
    w = synth.qwen3_vl_agentic(batch=2, lo=9000, hi=12000, chunk=4096)
    assert w.g == 8 and w.heads_per_page == 8 and w.n_tables == 2
    total = sum(len(c[1]) for c in w.calls)
    int4 = sum(int((c[1] == synth.INT4).sum()) for c in w.calls)
    assert 0.2 < int4 / total < 0.4                      # about 30 % INT4 at 2.6 bits
    for (t, flags, rows, _) in w.calls:
        assert len(flags) <= 4096
        classes = oracle.route(flags)[0]
        # every call leaves fewer than 32 INT2-flagged tokens to its INT4 residual
        assert int((flags == synth.INT2).sum()) - int((classes == synth.INT2).sum()) < 32
    # pools hold what placement needs
    lists = synth.place_all(w, lambda f: oracle.route(f)[0])
    assert len(lists.rows2) == 32 * len(lists.pages2)
    assert int(w.alloc.n_entries.max()) <= w.alloc.max_entries


def _oracle_rows(w, requests=None):
    import sys, os
    sys.path.insert(0, os.path.dirname(__file__))
    from harness import OracleRun
    out, lse = OracleRun(w).attend()
    return (out, lse) if requests is None else (out[requests], lse[requests])


def test_subset_reproduces_the_sampled_requests():
    """Full-size parity samples requests through subset(): the oracle on the subset must
    equal the oracle on the whole workload for those requests (page and slot maps)."""
    for make, req in ((lambda: synth.qwen3_8b(batch=3, n_tokens=1024), [0, 2]),
                      (lambda: synth.ragged_dead(batch=4, lo=512, hi=4096), [1, 3]),
                      (lambda: synth.hybrid_anchor(batch=2, n_tokens=2048), [1])):
        full_o, full_l = _oracle_rows(make(), req)
        sub_o, sub_l = _oracle_rows(synth.subset(make(), req))
        assert np.array_equal(full_o, sub_o) and np.array_equal(full_l, sub_l)


def test_ragged_lengths_match_the_workload():
    w = synth.ragged_dead(batch=6, lo=512, hi=4096)
    lens = synth.ragged_lengths(batch=6, lo=512, hi=4096)
    tl = w.head_tokens.reshape(6, -1).max(axis=1)
    assert np.array_equal(tl, np.ceil(lens * 1.0).astype(np.int64))
