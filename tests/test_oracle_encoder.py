"""Pins of the oracle's audio encoder (oracle/encoder.py) to things other
than itself:

* the stem convolution equals torch's conv1d (a library routine) for
  stride 1 and 2, and an impulse at feature frame j reaches exactly the
  output frames t with |stride t - j| <= 1;
* the position table: frame 0 is [0 ... 0, 1 ... 1], sin^2 + cos^2 = 1 per
  frequency, the first frequency is 1 rad/frame and the last 1e-4 (which
  fixes the exponent's denominator h - 1);
* one block equals the same block written with torch's layer_norm,
  scaled_dot_product_attention (no mask) and exact gelu;
* blocks are permutation-equivariant over frames (a causal or windowed
  mask fails this), the stem halves the frame count, and the final norm
  gives rows of mean 0 and variance 1.
"""
import numpy as np
import pytest
import torch

from oracle import encoder as oe
from synthetic import ENC_SMALL, bf16_bits_to_f32, make_encoder_weights, make_mel


@pytest.mark.parametrize("stride", [1, 2])
def test_conv3_equals_torch_conv1d(stride):
    g = np.random.default_rng(1)
    x = g.standard_normal((5, 18))
    w = g.standard_normal((7, 5, 3))
    b = g.standard_normal(7)
    ref = torch.nn.functional.conv1d(torch.from_numpy(x)[None], torch.from_numpy(w),
                                     torch.from_numpy(b), stride=stride, padding=1)[0].numpy()
    got = oe.conv3(x, w, b, stride)
    assert got.shape == ref.shape
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_conv3_stride2_receptive_field():
    T = 16
    w = np.ones((1, 1, 3))
    for j in range(T):
        x = np.zeros((1, T))
        x[0, j] = 1.0
        out = oe.conv3(x, w, np.zeros(1), 2)[0]
        assert out.shape == (T // 2,)
        hit = {t for t in range(T // 2) if out[t] != 0}
        assert hit == {t for t in range(T // 2) if abs(2 * t - j) <= 1}, j


def test_sinusoids_closed_form():
    d, F = 64, 1500
    p = oe.sinusoids(F, d)
    h = d // 2
    assert np.array_equal(p[0], np.r_[np.zeros(h), np.ones(h)])
    np.testing.assert_allclose(p[:, :h] ** 2 + p[:, h:] ** 2, 1.0, atol=1e-12)
    t = np.arange(F)
    np.testing.assert_allclose(p[:, 0], np.sin(t), atol=1e-12)           # w_0 = 1
    np.testing.assert_allclose(p[:, h - 1], np.sin(t * 1e-4), atol=1e-12)  # w_{h-1} = 1e-4
    np.testing.assert_allclose(p[:, d - 1], np.cos(t * 1e-4), atol=1e-12)


def test_block_equals_torch_sublayers():
    s = ENC_SMALL
    wb = make_encoder_weights(s, 0, ln_random=True, n_layers=1)
    enc = oe.Encoder(s, wb, n_layers=1)
    x = np.random.default_rng(2).standard_normal((s.n_frames, s.d_model))
    got = enc.block(0, x)
    W = {k: torch.from_numpy(bf16_bits_to_f32(v).astype(np.float64)) for k, v in wb.items()}
    F_ = torch.nn.functional
    xt = torch.from_numpy(x)
    d, H = s.d_model, s.n_heads
    h = F_.layer_norm(xt, (d,), W["E0.ln1_g"], W["E0.ln1_b"], s.ln_eps)
    q = F_.linear(h, W["E0.wq"], W["E0.bq"]).view(-1, H, s.head_dim).transpose(0, 1)
    k = F_.linear(h, W["E0.wk"]).view(-1, H, s.head_dim).transpose(0, 1)
    v = F_.linear(h, W["E0.wv"], W["E0.bv"]).view(-1, H, s.head_dim).transpose(0, 1)
    o = F_.scaled_dot_product_attention(q, k, v, is_causal=False).transpose(0, 1).reshape(-1, d)
    xt = xt + F_.linear(o, W["E0.wo"], W["E0.bo"])
    h = F_.layer_norm(xt, (d,), W["E0.ln2_g"], W["E0.ln2_b"], s.ln_eps)
    xt = xt + F_.linear(F_.gelu(F_.linear(h, W["E0.w1"], W["E0.b1"])), W["E0.w2"], W["E0.b2"])
    np.testing.assert_allclose(got, xt.numpy(), rtol=1e-10, atol=1e-10)


def test_blocks_are_permutation_equivariant():
    s = ENC_SMALL
    enc = oe.Encoder(s, make_encoder_weights(s, 0))
    x = np.random.default_rng(3).standard_normal((s.n_frames, s.d_model))
    perm = np.random.default_rng(4).permutation(s.n_frames)
    y = enc.block(1, enc.block(0, x))
    yp = enc.block(1, enc.block(0, x[perm]))
    np.testing.assert_allclose(yp, y[perm], rtol=1e-10, atol=1e-10)


def test_forward_shape_and_final_norm():
    s = ENC_SMALL
    enc = oe.Encoder(s, make_encoder_weights(s, 0))
    mel = make_mel(s, 0, 0)
    assert mel.shape == (s.n_mels, 2 * s.n_frames)
    out = enc.forward(mel)
    assert out.shape == (s.n_frames, s.d_model)
    np.testing.assert_allclose(out.mean(axis=1), 0.0, atol=1e-10)
    np.testing.assert_allclose(out.var(axis=1), 1.0, rtol=1e-3)   # var / (var + eps)
    # the stem alone: GELU outputs plus a unit-amplitude table
    x = enc.stem(bf16_bits_to_f32(mel).astype(np.float64))
    assert x.shape == (s.n_frames, s.d_model)
    assert np.isfinite(x).all() and float(np.abs(x).max()) < 10
