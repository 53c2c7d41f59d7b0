"""Pins of the oracle's decoder against independent definitions.

* sublayers against PyTorch's own CPU routines (layer_norm, exact GELU,
  scaled_dot_product_attention);
* the whole stack against ``torch.nn.TransformerDecoderLayer`` (pre-LN,
  GELU) — an independent implementation of the same block — run as a full
  recompute with a causal mask;
* the cache: block-with-cache = token-by-token = full recompute (the
  causal pass over anchor plus candidates of Whisper-Flash §3.1 must equal
  running those positions one at a time).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import model as om
from synthetic import TINY, WORKLOADS, bf16_bits_to_f32, make_encoder_out, make_weights

torch.set_default_dtype(torch.float64)


def _t(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


def test_layer_norm_matches_torch():
    g = np.random.default_rng(1)
    x = g.standard_normal((7, 64)) * 3 + 1
    gam = 1 + 0.1 * g.standard_normal(64)
    bet = 0.1 * g.standard_normal(64)
    ref = F.layer_norm(_t(x), (64,), _t(gam), _t(bet), eps=1e-5).numpy()
    np.testing.assert_allclose(om.layer_norm(x, gam, bet, 1e-5), ref, rtol=0, atol=1e-12)


def test_gelu_matches_torch_exact():
    x = np.linspace(-8, 8, 1001)
    ref = F.gelu(_t(x), approximate="none").numpy()
    np.testing.assert_allclose(om.gelu(x), ref, rtol=0, atol=1e-14)


@pytest.mark.parametrize("L,n", [(0, 5), (7, 1), (13, 9)])
def test_causal_attention_matches_sdpa(L, n):
    g = np.random.default_rng(2)
    H, hd = 4, 16
    d = H * hd
    q = g.standard_normal((n, d))
    k = g.standard_normal((L + n, d))
    v = g.standard_normal((L + n, d))
    pos = np.arange(L, L + n)
    allowed = np.arange(L + n)[None, :] <= pos[:, None]
    ours = om.multi_head_attention(q, k, v, H, allowed)
    qh = _t(q).view(n, H, hd).transpose(0, 1)
    kh = _t(k).view(L + n, H, hd).transpose(0, 1)
    vh = _t(v).view(L + n, H, hd).transpose(0, 1)
    ref = F.scaled_dot_product_attention(qh, kh, vh, attn_mask=torch.from_numpy(allowed))
    ref = ref.transpose(0, 1).reshape(n, d).numpy()
    np.testing.assert_allclose(ours, ref, rtol=0, atol=1e-12)


def test_cross_attention_matches_sdpa():
    g = np.random.default_rng(3)
    H, hd, F_ = 4, 16, 100
    d = H * hd
    q = g.standard_normal((9, d))
    k = g.standard_normal((F_, d))
    v = g.standard_normal((F_, d))
    ours = om.multi_head_attention(q, k, v, H, None)
    ref = F.scaled_dot_product_attention(
        _t(q).view(9, H, hd).transpose(0, 1), _t(k).view(F_, H, hd).transpose(0, 1),
        _t(v).view(F_, H, hd).transpose(0, 1)).transpose(0, 1).reshape(9, d).numpy()
    np.testing.assert_allclose(ours, ref, rtol=0, atol=1e-12)


def _torch_stack(shape, wbits):
    """The same decoder assembled from torch.nn.TransformerDecoderLayer."""
    W = {k: _t(bf16_bits_to_f32(v)) for k, v in wbits.items()}
    d = shape.d_model
    layers = []
    for l in range(shape.n_layers):
        w = lambda n: W[f"L{l}.{n}"]
        lay = torch.nn.TransformerDecoderLayer(
            d_model=d, nhead=shape.n_heads, dim_feedforward=shape.d_ffn, dropout=0.0,
            activation="gelu", layer_norm_eps=shape.ln_eps, batch_first=True,
            norm_first=True, dtype=torch.float64)
        with torch.no_grad():
            lay.self_attn.in_proj_weight.copy_(torch.cat([w("wq"), w("wk"), w("wv")]))
            lay.self_attn.in_proj_bias.copy_(torch.cat([w("bq"), torch.zeros(d), w("bv")]))
            lay.self_attn.out_proj.weight.copy_(w("wo"))
            lay.self_attn.out_proj.bias.copy_(w("bo"))
            lay.multihead_attn.in_proj_weight.copy_(torch.cat([w("wqc"), w("wkc"), w("wvc")]))
            lay.multihead_attn.in_proj_bias.copy_(torch.cat([w("bqc"), torch.zeros(d), w("bvc")]))
            lay.multihead_attn.out_proj.weight.copy_(w("woc"))
            lay.multihead_attn.out_proj.bias.copy_(w("boc"))
            lay.linear1.weight.copy_(w("w1"))
            lay.linear1.bias.copy_(w("b1"))
            lay.linear2.weight.copy_(w("w2"))
            lay.linear2.bias.copy_(w("b2"))
            for i in (1, 2, 3):
                getattr(lay, f"norm{i}").weight.copy_(w(f"ln{i}_g"))
                getattr(lay, f"norm{i}").bias.copy_(w(f"ln{i}_b"))
        lay.eval()
        layers.append(lay)

    def forward(tokens, enc):
        n = len(tokens)
        x = W["tok_emb"][torch.as_tensor(tokens)] + W["pos_emb"][:n]
        x = x[None]
        mem = _t(bf16_bits_to_f32(enc))[None]
        mask = torch.triu(torch.full((n, n), float("-inf")), diagonal=1)
        with torch.no_grad():
            for lay in layers:
                x = lay(x, mem, tgt_mask=mask)
            h = F.layer_norm(x[0], (d,), W["lnf_g"], W["lnf_b"], eps=shape.ln_eps)
            return (h @ W["tok_emb"].T).numpy()
    return forward


@pytest.fixture(scope="module")
def tiny():
    wl = WORKLOADS[0]
    wbits = make_weights(TINY, wl.cfg_id, ln_random=True)
    enc = make_encoder_out(TINY, wl.cfg_id, 0)
    return TINY, wbits, enc


def test_full_stack_matches_torch_decoder_layers(tiny):
    shape, wbits, enc = tiny
    ref_fwd = _torch_stack(shape, wbits)
    m = om.Model(shape, wbits)
    tokens = np.random.default_rng(4).integers(0, shape.vocab, 23)
    ours = m.rows(m.new_request(enc), tokens, 0)
    ref = ref_fwd(tokens, enc)
    # the scale of these logits is ~1; fp64 summation-order differences only
    np.testing.assert_allclose(ours, ref, rtol=0, atol=1e-10)


def test_block_incremental_and_full_recompute_agree(tiny):
    shape, wbits, enc = tiny
    m = om.Model(shape, wbits)
    toks = np.random.default_rng(5).integers(0, shape.vocab, 30)
    full = m.rows(m.new_request(enc), toks, 0)
    # token by token with the cache
    req = m.new_request(enc)
    inc = np.concatenate([m.rows(req, toks[i:i + 1], i) for i in range(30)])
    # prefix of 12, then blocks of 9 and 9
    req = m.new_request(enc)
    blk = np.concatenate([m.rows(req, toks[:12], 0), m.rows(req, toks[12:21], 12),
                          m.rows(req, toks[21:30], 21)])
    np.testing.assert_allclose(inc, full, rtol=0, atol=1e-12)
    np.testing.assert_allclose(blk, full, rtol=0, atol=1e-12)


def test_rejected_rows_are_dead_after_rollback(tiny):
    """Rows written past the kept length must not influence later rounds
    (Whisper-Flash App. A.5: the rows of rejected candidates keep their
    memory but are hidden from every later query)."""
    shape, wbits, enc = tiny
    m = om.Model(shape, wbits)
    g = np.random.default_rng(6)
    toks = g.integers(0, shape.vocab, 10)
    junk = g.integers(0, shape.vocab, 9)
    req = m.new_request(enc)
    m.rows(req, toks[:6], 0)
    m.rows(req, junk, 6)                       # a verify whose rows are all rejected
    after = m.rows(req, toks[6:10], 6)          # cache kept at length 6
    clean = m.rows(m.new_request(enc), toks, 0)[6:10]
    np.testing.assert_allclose(after, clean, rtol=0, atol=1e-12)


def test_logit_scale_matches_init_statistics():
    """With LN gain 1 / bias 0 the final hidden row has unit variance, so a
    tied-head logit is a sum of d products with N(0, 0.02^2) weights: its
    standard deviation is 0.02*sqrt(d), 0.16 at d = 64."""
    wl = WORKLOADS[0]
    wbits = make_weights(TINY, wl.cfg_id)
    m = om.Model(TINY, wbits)
    enc = make_encoder_out(TINY, wl.cfg_id, 0)
    toks = np.random.default_rng(7).integers(0, TINY.vocab, 40)
    lg = m.rows(m.new_request(enc), toks, 0)
    expect = 0.02 * math.sqrt(TINY.d_model)
    assert abs(lg.std() / expect - 1) < 0.1
