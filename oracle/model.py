"""Decoder forward pass of the oracle (fp64 by default) — test infrastructure.

What is computed (Whisper decoder, pre-LN; shapes from the Whisper large-v3
model the Whisper-Flash page evaluates, §4):

    x_i   = E[tok_i] + P[L + i]                       learned positions
    per layer:
      x  += SelfAttn(LN1(x))  causal: row i sees keys 0 .. L+i
      x  += CrossAttn(LN2(x), K_c, V_c)  all audio frames, no mask
      x  += W2 GELU(W1 LN3(x) + b1) + b2
    logits = LN_f(x) E^T                              head tied to E

The causal pass over "the anchor plus the candidates" is the verification
step of Whisper-Flash §3.1; row i of a block starting at cache length L sits
at position L+i and predicts position L+i+1 (App. A.1). Cross-attention K/V
are a per-request constant written once (SGLang-Omni cookbook, "Breakable
Prefill CUDA Graph"); ``encode_kv`` computes them.

Readings where the pages are silent: learned
absolute positions of length 448; LN eps 1e-5 with gain/bias; biases on
q, v, o, cross q/v/o, fc1, fc2 but none on k (a key bias shifts all scores
of a row equally, so it cannot change the output); scores scaled by
1/sqrt(head_dim); exact erf GELU; tied LM head without bias.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional

import numpy as np
from scipy.special import erf

from synthetic import ModelShape, bf16_bits_to_f32


def layer_norm(x: np.ndarray, g: np.ndarray, b: np.ndarray, eps: float) -> np.ndarray:
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * g + b


def gelu(x: np.ndarray) -> np.ndarray:
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def softmax(s: np.ndarray, axis: int = -1) -> np.ndarray:
    m = s.max(axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=axis, keepdims=True)


def multi_head_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                         n_heads: int, allowed: Optional[np.ndarray]) -> np.ndarray:
    """q [n, d], k/v [m, d]; ``allowed`` [n, m] bool or None (all keys)."""
    n, d = q.shape
    m = k.shape[0]
    hd = d // n_heads
    qh = q.reshape(n, n_heads, hd).transpose(1, 0, 2)
    kh = k.reshape(m, n_heads, hd).transpose(1, 0, 2)
    vh = v.reshape(m, n_heads, hd).transpose(1, 0, 2)
    s = qh @ kh.transpose(0, 2, 1) / math.sqrt(hd)          # [H, n, m]
    if allowed is not None:
        s = np.where(allowed[None, :, :], s, -np.inf)
    p = softmax(s, axis=-1)
    o = p @ vh                                               # [H, n, hd]
    return o.transpose(1, 0, 2).reshape(n, d)


class Request:
    """Per-request state: the write-once cross K/V and the self-attention
    cache (preallocated to the 448-token context; only the first ``L``
    positions are live, later entries are dead until overwritten)."""

    def __init__(self, shape: ModelShape, xkv: List[tuple], dtype):
        self.xkv = xkv
        self.K = [np.zeros((shape.n_ctx, shape.d_model), dtype) for _ in range(shape.n_layers)]
        self.V = [np.zeros((shape.n_ctx, shape.d_model), dtype) for _ in range(shape.n_layers)]


class Model:
    """Decoder with bf16-rounded weights held in ``dtype`` (fp64 default)."""

    def __init__(self, shape: ModelShape, weights_bits: Dict[str, np.ndarray],
                 dtype=np.float64, n_layers: Optional[int] = None):
        self.s = shape
        self.dtype = dtype
        self.n_layers = shape.n_layers if n_layers is None else n_layers
        self.W = {k: bf16_bits_to_f32(v).astype(dtype) for k, v in weights_bits.items()}

    def w(self, l: int, name: str) -> np.ndarray:
        return self.W[f"L{l}.{name}"]

    # -- write-once cross-attention K/V ------------------------------------
    def encode_kv(self, enc_bits: np.ndarray) -> List[tuple]:
        enc = bf16_bits_to_f32(enc_bits).astype(self.dtype)
        out = []
        for l in range(self.n_layers):
            kc = enc @ self.w(l, "wkc").T
            vc = enc @ self.w(l, "wvc").T + self.w(l, "bvc")
            out.append((kc, vc))
        return out

    def new_request(self, enc_bits: np.ndarray) -> Request:
        return Request(self._shape_nl(), self.encode_kv(enc_bits), self.dtype)

    def _shape_nl(self):
        import dataclasses
        return dataclasses.replace(self.s, n_layers=self.n_layers)

    # -- one causal pass over a block of rows ------------------------------
    def rows(self, req: Request, tokens, L: int, taps: Optional[list] = None,
             return_hidden: bool = False, probe=None) -> np.ndarray:
        """Run ``tokens`` at positions L..L+n-1 through every layer, writing
        their self-attention K/V into the cache at those positions. Returns
        logits [n, V]. ``taps``: list of layer indices whose post-block
        residual stream is returned too (as ``(logits, {layer: x})``).
        ``probe(l, qc, kc, vc)``, if given, sees every layer's cross-attention
        queries and the request's cross K/V."""
        s = self.s
        tokens = np.asarray(tokens, dtype=np.int64)
        n = len(tokens)
        if L + n > s.n_ctx:
            raise ValueError("block runs past the decoder context")
        pos = np.arange(L, L + n)
        x = self.W["tok_emb"][tokens] + self.W["pos_emb"][pos]
        allowed = np.arange(L + n)[None, :] <= pos[:, None]      # [n, L+n]
        tapped = {}
        for l in range(self.n_layers):
            h = layer_norm(x, self.w(l, "ln1_g"), self.w(l, "ln1_b"), s.ln_eps)
            q = h @ self.w(l, "wq").T + self.w(l, "bq")
            k = h @ self.w(l, "wk").T
            v = h @ self.w(l, "wv").T + self.w(l, "bv")
            req.K[l][L:L + n] = k
            req.V[l][L:L + n] = v
            o = multi_head_attention(q, req.K[l][:L + n], req.V[l][:L + n], s.n_heads, allowed)
            x = x + (o @ self.w(l, "wo").T + self.w(l, "bo"))

            h = layer_norm(x, self.w(l, "ln2_g"), self.w(l, "ln2_b"), s.ln_eps)
            qc = h @ self.w(l, "wqc").T + self.w(l, "bqc")
            kc, vc = req.xkv[l]
            if probe is not None:
                probe(l, qc, kc, vc)
            o = multi_head_attention(qc, kc, vc, s.n_heads, None)
            x = x + (o @ self.w(l, "woc").T + self.w(l, "boc"))

            h = layer_norm(x, self.w(l, "ln3_g"), self.w(l, "ln3_b"), s.ln_eps)
            x = x + (gelu(h @ self.w(l, "w1").T + self.w(l, "b1")) @ self.w(l, "w2").T
                     + self.w(l, "b2"))
            if taps is not None and l in taps:
                tapped[l] = x.copy()
        hidden = layer_norm(x, self.W["lnf_g"], self.W["lnf_b"], s.ln_eps)
        logits = hidden @ self.W["tok_emb"].T
        if taps is not None:
            return logits, tapped
        if return_hidden:
            return logits, x
        return logits
