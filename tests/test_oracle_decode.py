"""Pins of the oracle's acceptance, rollback and decode loops.

* the worked example of Whisper-Flash Figure 1 (golden fixture);
* App. A.1 arithmetic: the cache keeps L+1+a positions after a round;
  accepting EOS finishes the request with no bonus; a budget of R tokens
  allows at most R-1 candidates;
* the lossless property of greedy verification (Whisper-Flash §3.1; the
  "Speculative Loop" paragraph of "Alignment Drift ..."): the speculative
  output equals plain greedy decoding for ANY drafts, checked against a
  brute-force decoder that recomputes every position from scratch;
* closed-form acceptance statistics for Bernoulli-copy drafts.
"""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import decode as od
from oracle import model as om
from synthetic import TINY, WORKLOADS, make_draft_table, make_encoder_out, make_prefixes, make_weights

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_figure1_worked_example():
    ex = json.load(open(os.path.join(GOLDEN, "fig1_worked_example.json")))
    drafts, g = ex["drafts"], ex["target_argmax_rows"]
    a, emitted, c, done = od.greedy_accept(drafts, g, eos=0, budget=100)
    assert a == ex["expected"]["accepted"]
    assert emitted == ex["expected"]["emitted"]
    assert c == ex["expected"]["next_anchor"]
    assert len(emitted) == ex["expected"]["advance"]
    assert not done
    assert od.rollback_length(40, a) == 43            # old anchor + 2 accepted


def test_eos_and_budget_rules():
    # accepted EOS: finished, no bonus
    a, em, c, done = od.greedy_accept([5, 9, 7], [5, 9, 3, 1], eos=9, budget=10)
    assert (a, em, c, done) == (2, [5, 9], None, True)
    # correction equals EOS: emitted, finished
    a, em, c, done = od.greedy_accept([5, 6], [5, 9, 1], eos=9, budget=10)
    assert (a, em, c, done) == (1, [5, 9], 9, True)
    # R = 1: no candidates, exactly one token, then done
    a, em, c, done = od.greedy_accept([], [4], eos=9, budget=1)
    assert (a, em, c, done) == (0, [4], 4, True)
    # all accepted exhausts the budget exactly (k = R-1)
    a, em, c, done = od.greedy_accept([1, 2, 3], [1, 2, 3, 4], eos=9, budget=4)
    assert (a, em, done) == (3, [1, 2, 3, 4], True)
    with pytest.raises(ValueError):
        od.greedy_accept([1, 2], [1, 2, 3], eos=9, budget=2)   # k > R-1


@settings(max_examples=300, deadline=None)
@given(st.data())
def test_accept_is_longest_agreeing_prefix(data):
    k = data.draw(st.integers(0, 8))
    V = data.draw(st.integers(2, 6))
    drafts = data.draw(st.lists(st.integers(0, V - 1), min_size=k, max_size=k))
    g = data.draw(st.lists(st.integers(0, V - 1), min_size=k + 1, max_size=k + 1))
    eos = data.draw(st.integers(0, V))          # V = an id that never occurs
    budget = data.draw(st.integers(k + 1, k + 3))
    a, em, c, done = od.greedy_accept(drafts, g, eos, budget)
    # a: drafts 1..a agree with the target, and (unless EOS stopped it) the
    # next one does not
    assert all(drafts[i] == g[i] for i in range(a))
    eos_stop = a > 0 and drafts[a - 1] == eos
    if eos_stop:
        assert eos not in drafts[:a - 1] and c is None and done and em == drafts[:a]
    else:
        assert eos not in drafts[:a]
        assert a == k or drafts[a] != g[a]
        assert em == drafts[:a] + [g[a]] and c == g[a]
        assert done == (g[a] == eos or a + 1 >= budget)
    assert len(em) <= budget


def test_acceptance_statistics_closed_form():
    """Drafts copy the target with probability p, else a uniform id (which
    matches by chance with probability 1/V): P(a >= j) = p'^j with
    p' = p + (1-p)/V, so E[a] = sum_{j=1..K} p'^j (2.1988 for p = 0.7,
    K = 8, large V)."""
    g = np.random.default_rng(11)
    V, K, p, n = 50, 8, 0.7, 20000
    pp = p + (1 - p) / V
    expect = sum(pp ** j for j in range(1, K + 1))
    acc = []
    for _ in range(n):
        tgt = g.integers(0, V, K + 1)
        keep = g.random(K) < p
        drafts = np.where(keep, tgt[:K], g.integers(0, V, K))
        a, *_ = od.greedy_accept(list(drafts), list(tgt), eos=V, budget=K + 1)
        acc.append(a)
    acc = np.asarray(acc)
    se = acc.std() / np.sqrt(n)
    assert abs(acc.mean() - expect) < 4 * se
    m = od.loop_metrics(list(acc), [K] * n, K)
    for j in range(1, K + 1):
        assert abs(m["s_k"][j - 1] - pp ** j) < 0.02
    assert abs(sum((0.7) ** j for j in range(1, 9)) - 2.1988) < 1e-4


@pytest.fixture(scope="module")
def tiny_setup():
    wl = WORKLOADS[0]
    wbits = make_weights(TINY, wl.cfg_id)
    m = om.Model(TINY, wbits)
    enc = make_encoder_out(TINY, wl.cfg_id, 0)
    prefix = make_prefixes(wl)[0]
    return wl, m, enc, prefix


def test_speculative_equals_greedy_equals_brute_force(tiny_setup):
    wl, m, enc, prefix = tiny_setup
    n_max, eos, K = wl.n_max, TINY.eos_id, wl.k_draft
    greedy = od.greedy_decode(m, enc, prefix, n_max, eos)
    brute = od.brute_force_decode(m, enc, prefix, n_max, eos)
    assert greedy == brute
    P = len(prefix)
    rngd = np.random.default_rng(12)
    families = {
        "all_correct": od.table_drafts(greedy, P, np.ones(TINY.n_ctx + 1, bool),
                                       np.zeros(TINY.n_ctx + 1, np.int32)),
        "all_wrong": lambda L, y, k: [int((greedy[L + i - P] + 1) % TINY.vocab)
                                      if 0 <= L + i - P < len(greedy) else 0
                                      for i in range(1, k + 1)],
        "uniform": lambda L, y, k: list(rngd.integers(0, TINY.vocab, k)),
        "p0.7_table": od.table_drafts(greedy, P, *make_draft_table(wl, 0)),
    }
    for name, fn in families.items():
        stats = od.LoopStats()
        spec = od.speculative_decode(m, enc, prefix, n_max, eos, K, fn, stats)
        assert spec == greedy, name
        if name == "all_correct":
            # every round but possibly the last accepts min(K, R-1)
            assert all(a == k for a, k in zip(stats.accepted, stats.proposed))
        if name == "all_wrong":
            assert all(a == 0 for a in stats.accepted)


def test_speculative_equals_greedy_with_eos_inside(tiny_setup):
    """Take a token that greedy decoding emits mid-way as the EOS id: both
    loops must stop at its first occurrence, whether it arrives as an
    accepted candidate or as the target's correction/bonus."""
    wl, m, enc, prefix = tiny_setup
    greedy_full = od.greedy_decode(m, enc, prefix, wl.n_max, TINY.eos_id)
    P = len(prefix)
    for j in (3, 7, 12):
        eos = greedy_full[j]
        first = greedy_full.index(eos)
        greedy = od.greedy_decode(m, enc, prefix, wl.n_max, eos)
        assert greedy == greedy_full[:first + 1]
        for keep_p in (1.0, 0.7, 0.0):
            wl_k = WORKLOADS[0]
            keep, repl = make_draft_table(wl_k, 1, p_keep=keep_p)
            fn = od.table_drafts(greedy_full, P, keep, repl)
            spec = od.speculative_decode(m, enc, prefix, wl.n_max, eos, wl.k_draft, fn)
            assert spec == greedy, (j, keep_p)


def test_budget_respected_for_every_n_max(tiny_setup):
    wl, m, enc, prefix = tiny_setup
    P = len(prefix)
    greedy32 = od.greedy_decode(m, enc, prefix, 32, TINY.eos_id)
    fn = od.table_drafts(greedy32, P, np.ones(TINY.n_ctx + 1, bool),
                         np.zeros(TINY.n_ctx + 1, np.int32))
    for n_max in (1, 2, 3, 5, 9, 10, 11):
        spec = od.speculative_decode(m, enc, prefix, n_max, TINY.eos_id, 4, fn)
        assert spec == greedy32[:n_max]
