"""Pins of the tree-verification oracle ("Alignment Drift ...", App. E.3).

* a tree with a single branch reproduces the linear pass (logits of one
  causal block over the same tokens) and the linear greedy round;
* tree acceptance equals the best linear round over all root-to-leaf paths
  (each path's drafts and target choices through the linear oracle, which
  the Whisper-Flash Figure 1 worked example pins), truncated to R - 1;
* the parent array is validated.
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import decode as od
from oracle import model as om
from oracle import tree as ot
from synthetic import TINY, WORKLOADS, make_encoder_out, make_prefixes, make_weights


@pytest.fixture(scope="module")
def tiny_model():
    wl = WORKLOADS[0]
    wbits = make_weights(TINY, wl.cfg_id, ln_random=True)
    m = om.Model(TINY, wbits)
    req = m.new_request(make_encoder_out(TINY, wl.cfg_id, 0))
    prefix = make_prefixes(wl)[0]
    m.rows(req, prefix, 0)
    return m, req, len(prefix)


def test_one_branch_tree_is_the_linear_pass(tiny_model):
    m, req, L = tiny_model
    toks = np.random.default_rng(3).integers(0, TINY.vocab - 1, 6)
    chain = [-1, 0, 1, 2, 3, 4]
    lt = ot.tree_rows(m, req, toks, chain, L)
    lin = m.rows(ot.copy_request(m, req), toks, L)
    np.testing.assert_allclose(lt, lin, rtol=0, atol=1e-9)


def test_tree_nodes_see_only_their_ancestors(tiny_model):
    """A node's logits are the last row of its own path run as a linear block;
    siblings and their subtrees do not change them."""
    m, req, L = tiny_model
    g = np.random.default_rng(4)
    parents = [-1, 0, 0, 1, 2, 1, 3]
    toks = g.integers(0, TINY.vocab - 1, len(parents))
    lt = ot.tree_rows(m, req, toks, parents, L)
    for i in range(len(parents)):
        p = ot.path_to(parents, i)
        lin = m.rows(ot.copy_request(m, req), toks[p], L)
        np.testing.assert_allclose(lt[i], lin[-1], rtol=0, atol=1e-9)
    # a node's logits do not depend on the rest of the tree
    sub = ot.tree_rows(m, req, toks[:4], parents[:4], L)
    np.testing.assert_allclose(sub, lt[:4], rtol=0, atol=1e-9)


def _random_tree(g, T):
    return [-1] + [int(g.integers(0, i)) for i in range(1, T)]


@settings(max_examples=300, deadline=None)
@given(st.integers(0, 10**9), st.integers(1, 12), st.integers(1, 14))
def test_tree_accept_is_best_linear_round_over_paths(seed, T, budget):
    g = np.random.default_rng(seed)
    V, eos = 4, 3
    parents = _random_tree(g, T)
    toks = g.integers(0, V, T)
    am = g.integers(0, V, T)
    a, path, emitted, c, done = ot.tree_accept(toks, parents, am, eos, budget)
    # brute force: every root-to-node path as a linear round (drafts along
    # the path, the target's choices at the path's nodes)
    best = None
    for leaf in range(T):
        p = ot.path_to(parents, leaf)
        k = min(len(p) - 1, budget - 1)
        p = p[:k + 1]
        al, em, cl, dl = od.greedy_accept([int(toks[j]) for j in p[1:]],
                                          [int(am[j]) for j in p], eos, budget)
        node = p[al]
        if best is None or al > best[0] or (al == best[0] and node < best[1]):
            best = (al, node, em, cl, dl)
    assert a == best[0] and path[-1] == best[1]
    assert emitted == best[2] and c == best[3] and done == best[4]
    assert len(path) == a + 1 and path[0] == 0


@given(st.integers(0, 10**9), st.integers(1, 10), st.integers(2, 12))
def test_one_branch_tree_accept_is_linear(seed, k, budget):
    g = np.random.default_rng(seed)
    k = min(k, budget - 1)
    toks = g.integers(0, 3, k + 1)
    am = g.integers(0, 3, k + 1)
    chain = [-1] + list(range(k))
    a, path, emitted, c, done = ot.tree_accept(toks, chain, am, 2, budget)
    al, em, cl, dl = od.greedy_accept([int(t) for t in toks[1:]], [int(x) for x in am], 2, budget)
    assert (a, emitted, c, done) == (al, em, cl, dl)
    assert path == list(range(a + 1))


def test_parent_array_is_validated():
    for bad in ([0, 0], [-1, 1], [-1, 0, 3], [-1, -1]):
        with pytest.raises(ValueError):
            ot.depths(bad)
    assert ot.depths([-1, 0, 0, 1, 3]) == [0, 1, 1, 2, 3]
