"""Verification-attention anchor readout — test infrastructure (the oracle:
only tests, smoke() and bench.py's CPU baseline may use it).

"Alignment Drift in Single-Model Speculative Decoding for ASR",
Verification-Attention Correction and App. D.2: at one decoder layer the
target's cross-attention over the audio frames, averaged over the heads,
has its maximum near the frame being transcribed; at inference that layer's
scores are computed again from the keys already cached, and the frame of
the maximum is the readout.

Readings where the pages leave a step open: the readout is given for every verify row
(the caller takes the row it needs, e.g. the last kept one); probabilities
are the layer's softmax over the audio frames with the 1/sqrt(head_dim)
scale, averaged over heads with equal weight; the peak is the lowest frame
among equal maxima.
"""
from __future__ import annotations

import math
from typing import Tuple

import numpy as np

from . import model as om


def head_average(qc: np.ndarray, kc: np.ndarray, n_heads: int) -> np.ndarray:
    """qc [n, d] cross-attention queries, kc [F, d] the layer's cross keys.
    Returns [n, F]: the per-head softmax over frames, averaged over heads."""
    n, d = qc.shape
    hd = d // n_heads
    qh = qc.reshape(n, n_heads, hd).transpose(1, 0, 2)
    kh = kc.reshape(-1, n_heads, hd).transpose(1, 0, 2)
    s = qh @ kh.transpose(0, 2, 1) / math.sqrt(hd)              # [H, n, F]
    p = om.softmax(s, axis=-1)
    return p.mean(axis=0)


def peak(pbar: np.ndarray) -> np.ndarray:
    """Per row, the frame of the largest value (lowest frame on ties)."""
    m = pbar.max(axis=-1, keepdims=True)
    return np.argmax(pbar == m, axis=-1)


def anchor_frames(model: "om.Model", req: "om.Request", tokens, L: int,
                  layer: int) -> Tuple[np.ndarray, np.ndarray]:
    """Run the block at positions L.. (on a copy of the request) and return
    (peak frame per row, head-averaged probabilities [n, F]) at ``layer``."""
    from .tree import copy_request
    got = {}

    def probe(l, qc, kc, vc):
        if l == layer:
            got["p"] = head_average(qc, kc, model.s.n_heads)

    model.rows(copy_request(model, req), tokens, L, probe=probe)
    return peak(got["p"]), got["p"]
