"""Parallel drafter of Whisper-Flash — test infrastructure (parity unpinned
beyond self-consistency: the pages print no drafter values).

Whisper-Flash §3.2 (eq. 2) and App. A.2:

* the block is X_t = [Emb(y_t), m, ..., m]: the anchor's token embedding
  followed by the same trained vector m repeated K times, at text positions
  t .. t+K;
* the history memory holds, for every accepted position before the anchor,
  the target's residual streams leaving blocks 1, 8, 15, 22, 29 (counting
  from 0; before the final layer norm), concatenated (5 d) and
  projected to the drafter width d;
* in each drafter layer a block row's query scores the projected history
  rows and every row of the block (no causal mask within it) under a single
  softmax, with rotary embeddings (base 10,000, fp32 phases, explicit text
  positions); then cross-attention over the audio with the drafter's own
  key/value projections, then a feed-forward update;
* the drafter reuses the target's token embedding and output head; the
  i-th mask row gives the guess for position t + i.

Readings where the pages leave a step open: a drafter layer has the target block's
pre-LN structure (self-attention, cross-attention, GELU MLP, same biases);
history rows enter a layer's attention like block rows — k = RoPE(W_k
LN1(h), pos), v = W_v LN1(h) + b_v — and are not updated across layers;
the history projection has no bias; RoPE pairs dimension i with i + hd/2
(rotate-half) at angle pos * 10000^(-2i/hd); the drafter has its own final
layer norm before the shared head. The parameter count this gives
(2 layers x 26.2M + 8.2M) matches the 60.7M the page states.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional

import numpy as np

from synthetic import ModelShape, bf16_bits_to_f32

from .model import gelu, layer_norm, softmax

TAP_LAYERS = (1, 8, 15, 22, 29)
ROPE_BASE = 10000.0


def rope_angles(positions: np.ndarray, hd: int) -> np.ndarray:
    """Angles [n, hd/2] computed in fp32, as the page fixes (fp32 phases)."""
    i = np.arange(hd // 2, dtype=np.float32)
    inv = np.float32(ROPE_BASE) ** (-(np.float32(2.0) * i) / np.float32(hd))
    return positions.astype(np.float32)[:, None] * inv[None, :]


def rope(x: np.ndarray, positions: np.ndarray, n_heads: int) -> np.ndarray:
    """Rotate each head's pairs (i, i + hd/2) by pos * inv_freq_i.
    x [n, d]; the rotation itself is applied in the array's dtype."""
    n, d = x.shape
    hd = d // n_heads
    ang = rope_angles(positions, hd).astype(np.float64)
    cos = np.cos(ang).astype(x.dtype)[:, None, :]
    sin = np.sin(ang).astype(x.dtype)[:, None, :]
    xh = x.reshape(n, n_heads, hd)
    a, b = xh[..., : hd // 2], xh[..., hd // 2:]
    out = np.concatenate([a * cos - b * sin, a * sin + b * cos], axis=-1)
    return out.reshape(n, d)


class DraftRequest:
    def __init__(self, shape: ModelShape, xkv: List[tuple], dtype):
        self.xkv = xkv                                     # drafter's own cross K/V
        self.h = np.zeros((shape.n_ctx, shape.d_model), dtype)   # projected history


class Drafter:
    def __init__(self, shape: ModelShape, target_weights: Dict[str, np.ndarray],
                 drafter_bits: Dict[str, np.ndarray], n_layers: int = 2, dtype=np.float64,
                 taps=TAP_LAYERS):
        self.s = shape
        self.dtype = dtype
        self.n_layers = n_layers
        self.taps = tuple(taps)
        self.E = bf16_bits_to_f32(target_weights["tok_emb"]).astype(dtype)
        self.W = {k: bf16_bits_to_f32(v).astype(dtype) for k, v in drafter_bits.items()}

    def w(self, l: int, name: str) -> np.ndarray:
        return self.W[f"D{l}.{name}"]

    def encode_kv(self, enc_bits: np.ndarray) -> List[tuple]:
        enc = bf16_bits_to_f32(enc_bits).astype(self.dtype)
        return [(enc @ self.w(l, "wkc").T, enc @ self.w(l, "wvc").T + self.w(l, "bvc"))
                for l in range(self.n_layers)]

    def new_request(self, enc_bits: np.ndarray) -> DraftRequest:
        return DraftRequest(self.s, self.encode_kv(enc_bits), self.dtype)

    def append_history(self, req: DraftRequest, taps: Dict[int, np.ndarray], L: int):
        """Project the target's tapped residual streams of rows at positions
        L .. L+n-1 and store them as history."""
        feat = np.concatenate([taps[t] for t in self.taps], axis=-1)     # [n, 5d]
        req.h[L:L + feat.shape[0]] = feat @ self.W["w_hist"].T

    def _layer_kv(self, l: int, h: np.ndarray, pos: np.ndarray):
        a = layer_norm(h, self.w(l, "ln1_g"), self.w(l, "ln1_b"), self.s.ln_eps)
        k = rope(a @ self.w(l, "wk").T, pos, self.s.n_heads)
        v = a @ self.w(l, "wv").T + self.w(l, "bv")
        return k, v

    def block(self, req: DraftRequest, anchor: int, L: int, K: int,
              hist_kv: Optional[List[tuple]] = None) -> np.ndarray:
        """Drafter logits [K+1, V] for the block at positions L .. L+K; rows
        1..K give the drafts. ``hist_kv``: precomputed per-layer history K/V
        (else recomputed from the projected history)."""
        s = self.s
        H, hd = s.n_heads, s.head_dim
        pos = np.arange(L, L + K + 1)
        x = np.concatenate([self.E[anchor][None, :],
                            np.repeat(self.W["mask"][None, :], K, axis=0)])
        for l in range(self.n_layers):
            if hist_kv is not None:
                kh, vh = hist_kv[l]
            else:
                kh, vh = self._layer_kv(l, req.h[:L], np.arange(L))
            a = layer_norm(x, self.w(l, "ln1_g"), self.w(l, "ln1_b"), s.ln_eps)
            q = rope(a @ self.w(l, "wq").T + self.w(l, "bq"), pos, H)
            k = rope(a @ self.w(l, "wk").T, pos, H)
            v = a @ self.w(l, "wv").T + self.w(l, "bv")
            keys = np.concatenate([kh, k])
            vals = np.concatenate([vh, v])
            o = _attend(q, keys, vals, H)
            x = x + (o @ self.w(l, "wo").T + self.w(l, "bo"))
            a = layer_norm(x, self.w(l, "ln2_g"), self.w(l, "ln2_b"), s.ln_eps)
            qc = a @ self.w(l, "wqc").T + self.w(l, "bqc")
            kc, vc = req.xkv[l]
            o = _attend(qc, kc, vc, H)
            x = x + (o @ self.w(l, "woc").T + self.w(l, "boc"))
            a = layer_norm(x, self.w(l, "ln3_g"), self.w(l, "ln3_b"), s.ln_eps)
            x = x + (gelu(a @ self.w(l, "w1").T + self.w(l, "b1")) @ self.w(l, "w2").T
                     + self.w(l, "b2"))
        hfin = layer_norm(x, self.W["lnd_g"], self.W["lnd_b"], s.ln_eps)
        return hfin @ self.E.T

    def history_kv(self, req: DraftRequest, L: int) -> List[tuple]:
        return [self._layer_kv(l, req.h[:L], np.arange(L)) for l in range(self.n_layers)]


def _attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_heads: int) -> np.ndarray:
    """Unmasked multi-head attention (every query sees every key)."""
    n, d = q.shape
    m = k.shape[0]
    hd = d // n_heads
    qh = q.reshape(n, n_heads, hd).transpose(1, 0, 2)
    kh = k.reshape(m, n_heads, hd).transpose(1, 0, 2)
    vh = v.reshape(m, n_heads, hd).transpose(1, 0, 2)
    p = softmax(qh @ kh.transpose(0, 2, 1) / math.sqrt(hd), axis=-1)
    return (p @ vh).transpose(1, 0, 2).reshape(n, d)


def draft_tokens(logits: np.ndarray, K: int) -> List[int]:
    """Drafts d_1..d_K: the argmax of block rows 1..K (lowest id on ties)."""
    from .decode import argmax_lowest
    return [argmax_lowest(logits[i]) for i in range(1, K + 1)]
