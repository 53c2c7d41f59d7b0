"""Pins of the anchor readout oracle ("Alignment Drift ...", App. D.2).

* the per-head probabilities it averages are the ones the model's own
  cross-attention uses: weighted by the values they reproduce that layer's
  attention output (multi_head_attention), and each head's sum to 1;
* the peak follows a key built to match one query;
* ties go to the lowest frame.
"""
import math

import numpy as np

from oracle import model as om
from oracle import readout as orr
from synthetic import TINY, WORKLOADS, make_encoder_out, make_prefixes, make_weights


def test_probabilities_reproduce_the_attention_output():
    wl = WORKLOADS[0]
    m = om.Model(TINY, make_weights(TINY, wl.cfg_id, ln_random=True))
    req = m.new_request(make_encoder_out(TINY, wl.cfg_id, 0))
    prefix = make_prefixes(wl)[0]
    m.rows(req, prefix, 0)
    seen = {}

    def probe(l, qc, kc, vc):
        seen[l] = (qc.copy(), kc, vc)

    m.rows(req, [5, 6, 7], len(prefix), probe=probe)
    H = TINY.n_heads
    hd = TINY.d_model // H
    for l, (qc, kc, vc) in seen.items():
        n = qc.shape[0]
        qh = qc.reshape(n, H, hd).transpose(1, 0, 2)
        kh = kc.reshape(-1, H, hd).transpose(1, 0, 2)
        p = om.softmax(qh @ kh.transpose(0, 2, 1) / math.sqrt(hd), axis=-1)
        np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-12)
        o = (p @ vc.reshape(-1, H, hd).transpose(1, 0, 2)).transpose(1, 0, 2).reshape(n, -1)
        np.testing.assert_allclose(o, om.multi_head_attention(qc, kc, vc, H, None), rtol=0,
                                   atol=1e-12)
        np.testing.assert_allclose(orr.head_average(qc, kc, H), p.mean(0), rtol=0, atol=0)


def test_peak_follows_a_matching_key():
    g = np.random.default_rng(0)
    H, hd, F = 4, 16, 50
    q = g.normal(size=(3, H * hd))
    k = g.normal(size=(F, H * hd)) * 0.1
    for r, f in enumerate([7, 0, 49]):
        k[f] = 5.0 * q[r] / np.linalg.norm(q[r]) * math.sqrt(hd)
    assert list(orr.peak(orr.head_average(q, k, H))) == [7, 0, 49]


def test_ties_go_to_the_lowest_frame():
    assert list(orr.peak(np.array([[1.0, 3.0, 3.0], [2.0, 2.0, 2.0]]))) == [1, 0]
