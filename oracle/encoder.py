"""Audio encoder forward of the oracle (fp64) — test infrastructure (only
tests, smoke() and bench.py's CPU baseline may use it).

The Whisper-Flash page (§1, §2) describes the encoder only as the stage
that turns a fixed 30 s window of log-mel features into the acoustic
representation (1500 frames, the audio memory every decoder pass reads) in
one parallel pass, and App. A.3 (Table A2) times it as a fixed cost per
request. The SGLang-Omni "Whisper ASR" cookbook fixes the 30 s mel window
("Long Audio Chunking").

Readings where the pages leave the computation open (the architecture of
the Whisper paper the pages cite as [1]):

* stem: two width-3 convolutions over time with one frame of zero padding
  on each side, each followed by exact GELU; the second has stride 2, so
  2F feature frames give F frames (output frame t reads input frames
  2t-1, 2t, 2t+1);
* a fixed sinusoidal position table is added after the stem: for
  h = d/2 and w_j = 10000^(-j/(h-1)), channel j < h of frame t holds
  sin(t w_j) and channel h + j holds cos(t w_j);
* n pre-LN blocks: x += SelfAttn(LN1(x)) with every frame seeing every
  frame (no mask), scores scaled by 1/sqrt(head_dim), biases on q, v and
  the output projection, none on k; then x += W2 GELU(W1 LN2(x) + b1) + b2;
* a final layer norm gives the audio memory.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

from synthetic import EncoderShape, bf16_bits_to_f32

from .model import gelu, layer_norm, multi_head_attention


def sinusoids(n_frames: int, d: int) -> np.ndarray:
    """Position table [n_frames, d] (fp64)."""
    h = d // 2
    w = np.exp(-math.log(10000.0) / (h - 1) * np.arange(h, dtype=np.float64))
    ang = np.arange(n_frames, dtype=np.float64)[:, None] * w[None, :]
    return np.concatenate([np.sin(ang), np.cos(ang)], axis=1)


def conv3(x: np.ndarray, w: np.ndarray, b: np.ndarray, stride: int) -> np.ndarray:
    """Width-3 convolution over time, zero padding 1. x [C_in, T],
    w [C_out, C_in, 3] -> [C_out, T_out] with T_out = (T - 1) // stride + 1:
    out[:, t] = b + sum_k w[:, :, k] x[:, stride t + k - 1]."""
    c_in, T = x.shape
    xp = np.zeros((c_in, T + 2), dtype=x.dtype)
    xp[:, 1:T + 1] = x
    t_out = (T - 1) // stride + 1
    out = np.repeat(b[:, None], t_out, axis=1).astype(x.dtype)
    for k in range(3):
        # tap k reads input frame s t + k - 1, padded index s t + k
        out += (np.ascontiguousarray(w[:, :, k])
                @ np.ascontiguousarray(xp[:, k: k + stride * (t_out - 1) + 1: stride]))
    return out


class Encoder:
    """Encoder with bf16-rounded weights held in ``dtype`` (fp64 default)."""

    def __init__(self, shape: EncoderShape, weights_bits: Dict[str, np.ndarray],
                 dtype=np.float64, n_layers: Optional[int] = None):
        self.s = shape
        self.dtype = dtype
        self.n_layers = shape.n_layers if n_layers is None else n_layers
        self.W = {k: bf16_bits_to_f32(v).astype(dtype) for k, v in weights_bits.items()}

    def w(self, l: int, name: str) -> np.ndarray:
        return self.W[f"E{l}.{name}"]

    def stem(self, mel: np.ndarray) -> np.ndarray:
        """mel [n_mels, 2F] -> x [F, d]: both convolutions, GELU, positions."""
        h = gelu(conv3(mel, self.W["conv1_w"], self.W["conv1_b"], 1))
        h = gelu(conv3(h, self.W["conv2_w"], self.W["conv2_b"], 2))
        F = h.shape[1]
        return h.T + sinusoids(F, self.s.d_model).astype(self.dtype)

    def block(self, l: int, x: np.ndarray) -> np.ndarray:
        s = self.s
        h = layer_norm(x, self.w(l, "ln1_g"), self.w(l, "ln1_b"), s.ln_eps)
        q = h @ self.w(l, "wq").T + self.w(l, "bq")
        k = h @ self.w(l, "wk").T
        v = h @ self.w(l, "wv").T + self.w(l, "bv")
        o = multi_head_attention(q, k, v, s.n_heads, None)
        x = x + (o @ self.w(l, "wo").T + self.w(l, "bo"))
        h = layer_norm(x, self.w(l, "ln2_g"), self.w(l, "ln2_b"), s.ln_eps)
        return x + (gelu(h @ self.w(l, "w1").T + self.w(l, "b1")) @ self.w(l, "w2").T
                    + self.w(l, "b2"))

    def forward(self, mel_bits: np.ndarray) -> np.ndarray:
        """One request: bf16 bits [n_mels, 2F] -> audio memory [F, d]."""
        x = self.stem(bf16_bits_to_f32(mel_bits).astype(self.dtype))
        for l in range(self.n_layers):
            x = self.block(l, x)
        return layer_norm(x, self.W["lnp_g"], self.W["lnp_b"], self.s.ln_eps)
