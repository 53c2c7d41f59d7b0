"""Temperature rejection sampling — test infrastructure.

Whisper-Flash §3.1: with target distribution p_i and draft distribution q_i
(same temperature and token suppression), candidate i is accepted with
probability min(1, p_i(y_i)/q_i(y_i)); at the first rejection the verifier
samples from the normalised residual (p_i - q_i)_+; when every candidate is
accepted it samples a bonus from the next row's p. App. A.4: the softmax and
the acceptance test run in single precision; the end-of-transcript token and
the budget work the same way as in greedy acceptance.

Readings where the pages leave a step open: the acceptance test is u*q(y) < p(y) with
u uniform on [0, 1), equivalent to u < p/q for q(y) > 0 (which holds since
y ~ q); a draw from weights w uses the inverse CDF in ascending token order,
c = min{v : sum_{w<=v} w > u * sum(w)}; if the residual sums to zero, which
exact arithmetic rules out after a rejection, the draw falls back to p.
"""
from __future__ import annotations

from typing import List, Optional, Tuple

import numpy as np

from .philox import STREAM_ACCEPT, STREAM_RESAMPLE, uniform

F32 = np.float32


def probs(logits_row: np.ndarray, temperature: float,
          suppress: Optional[np.ndarray] = None) -> np.ndarray:
    """softmax(z / T) in fp32 with suppressed ids set to probability 0."""
    z = np.asarray(logits_row, dtype=F32) / F32(temperature)
    if suppress is not None:
        z = np.where(suppress, F32(-np.inf), z)
    m = z.max()
    e = np.exp(z - m, dtype=F32)
    return (e / e.sum(dtype=F32)).astype(F32)


def icdf(weights: np.ndarray, u: float) -> int:
    w = np.asarray(weights, dtype=F32)
    c = np.cumsum(w, dtype=F32)
    thr = F32(u) * c[-1]
    return int(np.flatnonzero(c > thr)[0])


def rejection_round(p: np.ndarray, q: np.ndarray, drafts: List[int],
                    u_acc: List[float], u_res: List[float], eos: int,
                    budget: int) -> Tuple[int, List[int], Optional[int], bool]:
    """p: [k+1, V] target probabilities of rows 0..k; q: [k, V] draft
    probabilities of candidates 1..k; u_acc[i], u_res[i]: uniforms for
    candidate/row i. Returns (a, emitted, next anchor or None, done)."""
    k = len(drafts)
    if budget < 1 or k > budget - 1:
        raise ValueError("at most R-1 candidates may be proposed")
    emitted: List[int] = []
    for i in range(k):
        y = int(drafts[i])
        if F32(u_acc[i]) * F32(q[i][y]) < F32(p[i][y]):
            emitted.append(y)
            if y == eos:
                return i + 1, emitted, None, True
            continue
        r = np.maximum(p[i].astype(F32) - q[i].astype(F32), F32(0))
        w = r if r.sum(dtype=F32) > 0 else p[i]
        c = icdf(w, u_res[i])
        emitted.append(c)
        return i, emitted, c, c == eos or len(emitted) >= budget
    c = icdf(p[k], u_res[k])
    emitted.append(c)
    return k, emitted, c, c == eos or len(emitted) >= budget


def sample_round(logits_rows: np.ndarray, q: np.ndarray, drafts: List[int],
                 temperature: float, seed: int, request: int, step: int,
                 eos: int, budget: int, suppress: Optional[np.ndarray] = None):
    """One sampling round with Philox uniforms keyed by
    (seed, request, step, position, stream)."""
    k = len(drafts)
    p = np.stack([probs(logits_rows[i], temperature, suppress) for i in range(k + 1)])
    u_acc = [uniform(seed, request, step, i, STREAM_ACCEPT) for i in range(k)]
    u_res = [uniform(seed, request, step, i, STREAM_RESAMPLE) for i in range(k + 1)]
    return rejection_round(p, q, drafts, u_acc, u_res, eos, budget)
