"""Tri-axis tags and greedy widths (TriAxialKV key designs 1 and 2): the oracle pinned
by a hand-derived conversation (tests/golden/tag_examples.txt) and by hand-worked and
property checks of the greedy walk; the library's host code then matches the oracle
exactly on seeded synthetic conversations and distortion tables (CPU only)."""
import os

import numpy as np
import pytest

import synth
from oracle import tags as otags

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tag_examples.txt")


def _golden():
    markers, tokens, want = {}, [], []
    for line in open(GOLDEN):
        f = line.split()
        if not f or f[0].startswith("#"):
            continue
        if f[0] == "marker":
            markers[int(f[1])] = f[2]
        else:
            tokens.append(int(f[1]))
            want.append((f[2], f[3], f[4]))
    return markers, tokens, want


def test_oracle_tags_match_the_hand_derived_conversation():
    markers, tokens, want = _golden()
    got, turns = otags.tag_tokens(tokens, markers)
    assert turns == 4
    for i, (g, w) in enumerate(zip(got, want)):
        assert g == w, (i, tokens[i], g, w)
    plain, t0 = otags.tag_tokens([5, 6, 7], markers)     # no marker at all
    assert t0 == 0 and plain == [("current", "text", "inst")] * 3


def test_oracle_widths_hand_worked():
    """rho = [8/20, 4/80, 2/40, 1/60] = [0.4, 0.05, 0.05, 0.0167]: tag 0, then the tie
    1 before 2, then 3.  At B = 2.6 (260 token-bits of 100 tokens) tag 0 fits (220),
    tag 1 does not (300): the walk stops although tag 2 alone would fit (260)."""
    d2, d4, n = [8.0, 4.0, 2.0, 1.0], [0.0] * 4, [10, 40, 20, 30]
    assert otags.allocate_bits(d2, d4, n, 2.6) == ([4, 2, 2, 2], 2.2)
    assert otags.allocate_bits(d2, d4, n, 3.0) == ([4, 4, 2, 2], 3.0)
    assert otags.allocate_bits(d2, d4, n, 2.0) == ([2, 2, 2, 2], 2.0)
    assert otags.allocate_bits(d2, d4, n, 4.0) == ([4, 4, 4, 4], 4.0)
    assert otags.allocate_bits(d2, d4, [10, 0, 20, 30], 4.0)[0] == [4, 2, 4, 4]   # empty tags stay


def test_oracle_widths_properties():
    r = np.random.default_rng(9)
    for _ in range(50):
        n = r.integers(0, 500, 56)
        n[r.random(56) < 0.2] = 0
        d2 = r.random(56) * 10
        d4 = d2 * r.random(56) * 0.2
        budget = float(r.uniform(2.0, 4.0))
        bits, avg = otags.allocate_bits(d2, d4, n, budget)
        total = int(n.sum())
        assert sum(int(b) * int(c) for b, c in zip(bits, n)) <= budget * total + 1e-9
        live = [k for k in range(56) if n[k] > 0]
        order = sorted(live, key=lambda k: (-(d2[k] - d4[k]) / (2.0 * n[k]), k))
        up = [bits[k] == 4 for k in order]
        assert up == sorted(up, reverse=True)             # the upgraded tags lead the order
        m = sum(up)
        if m < len(order):                                # the next one would not fit
            assert (avg * total + 2 * n[order[m]]) > budget * total


def test_library_tags_match_the_oracle():
    from mixed_precision_quantized_amd import kvq
    ev = {name: i for i, name in enumerate(otags.EVENTS)}
    markers, tokens, want = _golden()
    tags, turns = kvq.tag_tokens(np.array(tokens, np.int32), {t: ev[e] for t, e in markers.items()})
    assert turns == 4
    assert [int(x) for x in tags] == [otags.tag_index(*w) for w in want]
    for seed in range(6):
        s = synth.agentic_token_stream(seed=seed, n_turns=int(3 + 7 * seed), tokens_per_turn=400)
        got, t_lib = kvq.tag_tokens(s.tokens, {t: ev[e] for t, e in s.markers.items()})
        ref, t_orc = otags.tag_tokens(s.tokens.tolist(), s.markers)
        assert t_lib == t_orc
        assert np.array_equal(got, np.array([otags.tag_index(*x) for x in ref], np.uint8))
    with pytest.raises(kvq.KvqError):
        kvq.tag_tokens(np.array([1], np.int32), {7: 99})


def test_library_widths_and_flags_match_the_oracle():
    from mixed_precision_quantized_amd import kvq
    r = np.random.default_rng(10)
    for _ in range(40):
        n = r.integers(0, 2000, 56)
        n[r.random(56) < 0.3] = 0
        d2 = r.random(56) * 10
        d4 = d2 * r.random(56) * 0.2
        budget = float(r.uniform(2.0, 4.0))
        bits, avg = kvq.allocate_bits(d2, d4, n, budget)
        ref, ravg = otags.allocate_bits(d2, d4, n, budget)
        assert bits.tolist() == ref and avg == pytest.approx(ravg, abs=1e-12)
        tags = r.integers(0, 56, 300).astype(np.uint8)
        flags = kvq.tag_flags(tags, bits)
        assert np.array_equal(flags, np.array([0 if ref[t] == 2 else 1 for t in tags], np.uint8))
    with pytest.raises(kvq.KvqError):
        kvq.allocate_bits([1.0], [0.0], [5], 4.5)


def test_count_tags_accumulates_a_histogram():
    from mixed_precision_quantized_amd import kvq
    r = np.random.default_rng(4)
    a, b = r.integers(0, 56, 1000).astype(np.uint8), r.integers(0, 56, 77).astype(np.uint8)
    c = kvq.count_tags(a)
    kvq.count_tags(b, c)
    assert np.array_equal(c, np.bincount(np.concatenate([a, b]), minlength=56))
    with pytest.raises(kvq.KvqError):
        kvq.count_tags(np.array([3, 56], np.uint8), c)
    assert np.array_equal(c, np.bincount(np.concatenate([a, b]), minlength=56))  # nothing added
