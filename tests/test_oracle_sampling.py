"""Pins of Philox4x64-10 and of the rejection-sampling rule.

* Philox against numpy's own ``numpy.random.Philox`` (an independent
  implementation of the same SC'11 generator; numpy advances the counter by
  one before its first block);
* the rule of Whisper-Flash §3.1 preserves the target distribution: the
  first emitted token follows p (chi-square), the first candidate is
  accepted with probability sum_v min(p_v, q_v) = 1 - TV(p, q), q = p always
  accepts, and disjoint supports always reject with the resample following p.
"""
import numpy as np
import pytest

from oracle import philox as ph
from oracle import sampling as osmp


@pytest.mark.parametrize("ctr,key", [((0, 0, 0, 0), (0, 0)),
                                     ((5, 6, 7, 8), (123, 456)),
                                     ((2**64 - 2, 2**63, 17, 3), (2**64 - 1, 99))])
def test_philox_matches_numpy(ctr, key):
    bg = np.random.Philox(counter=np.array(ctr, dtype=np.uint64),
                          key=np.array(key, dtype=np.uint64))
    raw = [int(x) for x in bg.random_raw(4)]
    nxt = ((ctr[0] + 1) % 2**64,) + tuple(ctr[1:])
    if ctr[0] == 2**64 - 1:
        pytest.skip("carry case not exercised")
    assert list(ph.philox4x64_10(nxt, key)) == raw


def test_philox_vectorised_equals_scalar():
    g = np.random.default_rng(0)
    c = g.integers(0, 2**63, size=(4, 64), dtype=np.uint64) * np.uint64(2) + np.uint64(1)
    k = g.integers(0, 2**63, size=(2, 64), dtype=np.uint64)
    out = ph.philox4x64_10_np(c[0], c[1], c[2], c[3], k[0], k[1])
    for j in range(64):
        ref = ph.philox4x64_10([int(c[i, j]) for i in range(4)], (int(k[0, j]), int(k[1, j])))
        assert tuple(int(o[j]) for o in out) == ref


def test_uniform_is_24bit_and_in_range():
    us = [ph.uniform(7, r, s, p, st) for r in range(3) for s in range(3)
          for p in range(3) for st in range(2)]
    assert all(0.0 <= u < 1.0 for u in us)
    assert all(float(np.float32(u)) == u for u in us)
    assert all((u * 2**24).is_integer() for u in us)


def _dists(V, g):
    p = g.random(V) ** 3
    q = g.random(V) ** 3
    return (p / p.sum()).astype(np.float32), (q / q.sum()).astype(np.float32)


def test_first_token_follows_target_distribution():
    g = np.random.default_rng(21)
    V, k, n = 5, 2, 60000
    p0, q0 = _dists(V, g)
    p1, q1 = _dists(V, g)
    p = np.stack([p0, p1, p1])
    q = np.stack([q0, q1])
    counts = np.zeros(V)
    acc1 = 0
    for _ in range(n):
        drafts = [int(g.choice(V, p=q0 / q0.sum())), int(g.choice(V, p=q1 / q1.sum()))]
        a, em, c, done = osmp.rejection_round(p, q, drafts, list(g.random(k)),
                                              list(g.random(k + 1)), eos=V, budget=10)
        counts[em[0]] += 1
        acc1 += a >= 1
    exp = n * p0 / p0.sum()
    chi2 = ((counts - exp) ** 2 / exp).sum()
    assert chi2 < 18.5            # chi-square, 4 dof, p ~ 0.001
    tv_accept = np.minimum(p0, q0).sum()
    assert abs(acc1 / n - tv_accept) < 4 * np.sqrt(tv_accept * (1 - tv_accept) / n)


def test_q_equal_p_always_accepts_and_bonus_follows_p():
    g = np.random.default_rng(22)
    V = 6
    p0, _ = _dists(V, g)
    p = np.stack([p0] * 4)
    counts = np.zeros(V)
    for _ in range(3000):
        drafts = [int(g.choice(V, p=p0 / p0.sum())) for _ in range(3)]
        a, em, c, done = osmp.rejection_round(p, p[:3], drafts, list(g.random(3)),
                                              list(g.random(4)), eos=V, budget=10)
        assert a == 3 and em[:3] == drafts
        counts[c] += 1
    exp = 3000 * p0 / p0.sum()
    assert ((counts - exp) ** 2 / exp).sum() < 20.5


def test_disjoint_supports_always_reject():
    V = 6
    p = np.array([[0.5, 0.5, 0, 0, 0, 0]] * 2, np.float32)
    q = np.array([[0, 0, 0, 0.25, 0.25, 0.5]], np.float32)
    g = np.random.default_rng(23)
    counts = np.zeros(V)
    for _ in range(2000):
        d = int(g.choice(V, p=q[0]))
        a, em, c, done = osmp.rejection_round(p, q, [d], [g.random()], [g.random(), g.random()],
                                              eos=V, budget=10)
        assert a == 0 and c in (0, 1)
        counts[c] += 1
    assert abs(counts[0] / 2000 - 0.5) < 0.05


def test_icdf_ascending_order():
    w = np.array([0.1, 0.0, 0.4, 0.5], np.float32)
    assert osmp.icdf(w, 0.0) == 0
    assert osmp.icdf(w, 0.0999) == 0
    assert osmp.icdf(w, 0.1001) == 2
    assert osmp.icdf(w, 0.9999) == 3


def test_sample_round_temperature_softmax():
    z = np.array([1.0, 2.0, 3.0], np.float32)
    p = osmp.probs(z, 0.5)
    e = np.exp((z - 3) / 0.5)
    np.testing.assert_allclose(p, e / e.sum(), rtol=1e-6)
    sup = np.array([False, False, True])
    p2 = osmp.probs(z, 0.5, sup)
    assert p2[2] == 0 and abs(p2.sum() - 1) < 1e-6
