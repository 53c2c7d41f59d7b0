"""Pins of the oracle's parallel drafter (Whisper-Flash §3.2, App. A.2).

The pages print no drafter values, so the drafter's parity is unpinned
beyond these checks:
* RoPE equals multiplying each (i, i + hd/2) pair, read as a complex
  number, by exp(i * pos * 10000^(-2i/hd));
* after RoPE a query-key product depends only on the position difference,
  so a history key cached in an earlier round stays valid in later ones;
* the architecture reading reproduces the page's 60.7M trainable parameters;
* the history built round by round from the accepted rows' taps equals the
  history built from one full recompute of the target;
* the drafter's one-softmax attention over [history; block] equals torch's
  scaled_dot_product_attention with no mask;
* structure: attention inside the block is bidirectional (a mask row
  changes when a later row is added), the block reads the audio memory
  (another request's audio changes every row, the same audio gives the same
  bits) and the history below the anchor (a perturbed accepted row changes
  every block row; rows at or past the anchor are never read).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import decode as od
from oracle import drafter as odr
from oracle import model as om
from synthetic import (LARGE_V3, TINY, WORKLOADS, global_tensor_shapes, layer_tensor_shapes,
                       make_drafter_weights, make_encoder_out, make_prefixes, make_weights)

TINY_TAPS = (1, 0, 1, 1, 0)


def test_rope_is_complex_rotation():
    g = np.random.default_rng(1)
    H, hd, n = 3, 16, 7
    x = g.standard_normal((n, H * hd))
    pos = np.array([0, 1, 5, 17, 100, 447, 3])
    out = odr.rope(x, pos, H)
    inv = 10000.0 ** (-(2.0 * np.arange(hd // 2)) / hd)
    for r in range(n):
        for h in range(H):
            seg = x[r, h * hd:(h + 1) * hd]
            z = (seg[:hd // 2] + 1j * seg[hd // 2:]) * np.exp(1j * pos[r] * inv)
            # the oracle's phases are fp32 (as the page fixes): allow their rounding
            tol = 4 * np.abs(seg).max() * (pos[r] + 1) * 2.0 ** -23
            np.testing.assert_allclose(out[r, h * hd:h * hd + hd // 2], z.real, atol=tol)
            np.testing.assert_allclose(out[r, h * hd + hd // 2:(h + 1) * hd], z.imag, atol=tol)


def test_rope_scores_depend_only_on_position_difference():
    g = np.random.default_rng(2)
    H, hd = 2, 64
    q = g.standard_normal((1, H * hd))
    k = g.standard_normal((1, H * hd))
    def score(pq, pk):
        a = odr.rope(q, np.array([pq]), H).reshape(H, hd)
        b = odr.rope(k, np.array([pk]), H).reshape(H, hd)
        return (a * b).sum(-1)
    np.testing.assert_allclose(score(10, 3), score(110, 103), atol=1e-3)
    np.testing.assert_allclose(score(200, 0), score(420, 220), atol=1e-3)
    assert np.abs(score(10, 3) - score(10, 4)).max() > 1e-3


def test_parameter_count_matches_the_page():
    s = LARGE_V3
    ls = layer_tensor_shapes(s)
    per_layer = sum(int(np.prod(v)) for v in ls.values())
    total = 2 * per_layer + s.d_model * 5 * s.d_model + s.d_model + 2 * s.d_model
    assert abs(total / 1e6 - 60.7) < 0.05, total


@pytest.fixture(scope="module")
def tiny_pair():
    wl = WORKLOADS[0]
    tw = make_weights(TINY, wl.cfg_id)
    dw = make_drafter_weights(TINY, wl.cfg_id)
    enc = make_encoder_out(TINY, wl.cfg_id, 0)
    m = om.Model(TINY, tw)
    dr = odr.Drafter(TINY, tw, dw, taps=TINY_TAPS)
    return m, dr, enc, make_prefixes(wl)[0]


def test_history_from_rounds_equals_full_recompute(tiny_pair):
    m, dr, enc, prefix = tiny_pair
    seq = np.concatenate([prefix, np.random.default_rng(3).integers(0, TINY.vocab, 20)])
    # round by round: prefill, then blocks of 5 of which 1 + a rows are kept
    req, dreq = m.new_request(enc), dr.new_request(enc)
    lg, taps = m.rows(req, seq[:4], 0, taps=set(TINY_TAPS))
    dr.append_history(dreq, taps, 0)
    L = 4
    for keep in (3, 1, 5, 2, 4):
        blk = seq[L:L + 5]
        lg, taps = m.rows(req, blk, L, taps=set(TINY_TAPS))
        dr.append_history(dreq, {t: v[:keep] for t, v in taps.items()}, L)
        L += keep
    full_req, full_dreq = m.new_request(enc), dr.new_request(enc)
    lg, taps = m.rows(full_req, seq[:L], 0, taps=set(TINY_TAPS))
    dr.append_history(full_dreq, taps, 0)
    np.testing.assert_allclose(dreq.h[:L], full_dreq.h[:L], atol=1e-12)
    a = dr.block(dreq, int(seq[L]), L, 4)
    b = dr.block(full_dreq, int(seq[L]), L, 4)
    np.testing.assert_allclose(a, b, atol=1e-12)


def test_one_softmax_over_history_and_block_matches_sdpa():
    g = np.random.default_rng(4)
    H, hd, nh, nb = 4, 16, 11, 5
    q = g.standard_normal((nb, H * hd))
    k = g.standard_normal((nh + nb, H * hd))
    v = g.standard_normal((nh + nb, H * hd))
    ours = odr._attend(q, k, v, H)
    t = lambda a, n: torch.from_numpy(a).view(n, H, hd).transpose(0, 1)
    ref = F.scaled_dot_product_attention(t(q, nb), t(k, nh + nb), t(v, nh + nb))
    np.testing.assert_allclose(ours, ref.transpose(0, 1).reshape(nb, H * hd).numpy(), atol=1e-12)


def test_draft_rows_predict_their_own_positions(tiny_pair):
    """Mask row i sits at position L+i and proposes the token for that
    position; with identical mask inputs, rows differ only through RoPE."""
    m, dr, enc, prefix = tiny_pair
    req, dreq = m.new_request(enc), dr.new_request(enc)
    lg, taps = m.rows(req, prefix, 0, taps=set(TINY_TAPS))
    dr.append_history(dreq, taps, 0)
    out = dr.block(dreq, 7, len(prefix), 8)
    assert out.shape == (9, TINY.vocab)
    assert np.abs(out[1] - out[2]).max() > 1e-6       # positions differ
    d = odr.draft_tokens(out, 8)
    assert len(d) == 8 and all(0 <= x < TINY.vocab for x in d)


def _primed(m, dr, enc, prefix):
    req, dreq = m.new_request(enc), dr.new_request(enc)
    lg, taps = m.rows(req, prefix, 0, taps=set(TINY_TAPS))
    dr.append_history(dreq, taps, 0)
    return dreq


def test_block_attention_is_bidirectional(tiny_pair):
    """Mask rows see the rows after them (WF eq. 2: one softmax over the
    history and the whole block): row 1 changes when a third row is added
    to the block. Under a causal mask inside the block it could not."""
    m, dr, enc, prefix = tiny_pair
    dreq = _primed(m, dr, enc, prefix)
    L = len(prefix)
    k1 = dr.block(dreq, 7, L, 1)
    k2 = dr.block(dreq, 7, L, 2)
    assert np.abs(k1[1] - k2[1]).max() > 1e-6
    assert np.abs(k1[0] - k2[0]).max() > 1e-6          # the anchor row sees the mask rows too


def test_block_reads_the_audio_through_cross_attention(tiny_pair):
    """Same history, same block, another request's audio memory: every row
    changes (the drafter cross-attends with its own acoustic K/V); the same
    audio gives the same rows exactly."""
    m, dr, enc, prefix = tiny_pair
    dreq = _primed(m, dr, enc, prefix)
    L = len(prefix)
    other = dr.new_request(make_encoder_out(TINY, WORKLOADS[0].cfg_id, 1))
    other.h[:L] = dreq.h[:L]
    a = dr.block(dreq, 7, L, 4)
    b = dr.block(other, 7, L, 4)
    same = dr.new_request(enc)
    same.h[:L] = dreq.h[:L]
    c = dr.block(same, 7, L, 4)
    assert (np.abs(a - b).max(axis=1) > 1e-6).all()
    np.testing.assert_array_equal(a, c)


def test_block_reads_the_history(tiny_pair):
    """Changing one accepted position's history row changes every block row
    (history keys and values enter each layer's softmax); history rows at
    or beyond L are never read."""
    m, dr, enc, prefix = tiny_pair
    dreq = _primed(m, dr, enc, prefix)
    L = len(prefix)
    a = dr.block(dreq, 7, L, 4)
    dreq.h[L:L + 8] = 123.0                             # past the history: ignored
    np.testing.assert_array_equal(a, dr.block(dreq, 7, L, 4))
    # (not a constant shift: the history goes through a layer norm)
    dreq.h[1] += 0.5 * np.random.default_rng(9).standard_normal(dreq.h.shape[1])
    b = dr.block(dreq, 7, L, 4)
    assert (np.abs(a - b).max(axis=1) > 1e-6).all()
