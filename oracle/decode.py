"""Greedy acceptance, rollback and the decode loops — test infrastructure.

Whisper-Flash §3.1 and App. A.1 define one round:

* the anchor y (already emitted; the target cache holds the L positions
  before it, not y itself) and k candidates d_1..d_k form one block of rows
  run through the decoder with a causal mask; row i gives the target's
  choice g_i for position L+i+1 (eq. 1: argmax);
* a is the length of the longest prefix with d_i = g_{i-1} for every i in it;
* c = g_a, the target's choice after that prefix, is emitted as well (a
  correction when a < k, a bonus when a = k) and anchors the next round;
* once an accepted candidate is EOS the request is finished, with no bonus;
* rollback keeps L+1+a cache positions (old anchor plus accepted candidates);
* a request with R tokens of output budget left gets no more than R-1
  candidates.

Readings where the pages leave a step open: argmax ties go to the lowest token id; the
first anchor, emitted by prefill, counts toward the output budget; a request
is done when it has emitted ``n_max`` tokens or emitted EOS.
"""
from __future__ import annotations

from typing import Callable, List, Optional, Tuple

import numpy as np


def argmax_lowest(row: np.ndarray) -> int:
    """Index of the largest value; ties go to the lowest index."""
    if np.isnan(row).any():
        raise FloatingPointError("NaN logit")
    m = row.max()
    return int(np.flatnonzero(row == m)[0])


def greedy_accept(drafts: List[int], g: List[int], eos: int, budget: int
                  ) -> Tuple[int, List[int], Optional[int], bool]:
    """One greedy verification round.

    drafts: d_1..d_k; g: g_0..g_k (target argmax of rows 0..k); budget: R,
    the output tokens still allowed (k must be <= R-1).
    Returns (a, emitted tokens, next anchor or None, done).
    """
    k = len(drafts)
    if budget < 1 or k > budget - 1:
        raise ValueError("at most R-1 candidates may be proposed")
    if len(g) < k + 1:
        raise ValueError("need the target's choice for every row")
    emitted: List[int] = []
    a = 0
    while a < k and drafts[a] == g[a]:
        emitted.append(int(drafts[a]))
        a += 1
        if drafts[a - 1] == eos:          # accepted EOS: finished, no bonus
            return a, emitted, None, True
    c = int(g[a])
    emitted.append(c)
    done = c == eos or len(emitted) >= budget
    return a, emitted, c, done


def rollback_length(L: int, a: int) -> int:
    """Cache length kept after a round with a accepted candidates."""
    return L + 1 + a


DraftFn = Callable[[int, int, int], List[int]]   # (L, anchor, k) -> k drafts


class LoopStats:
    def __init__(self):
        self.rounds = 0
        self.accepted = []          # a per round
        self.proposed = []          # k per round

    @property
    def tau(self) -> float:
        """Tokens emitted per target call."""
        return (sum(self.accepted) + self.rounds) / max(self.rounds, 1)


def prefill(model, req, prefix) -> Tuple[int, int]:
    """Run the prompt; the argmax of its last row is the first anchor and
    the first emitted token. Returns (anchor, L)."""
    logits = model.rows(req, prefix, 0)
    return argmax_lowest(logits[-1]), len(prefix)


def greedy_decode(model, enc_bits, prefix, n_max: int, eos: int) -> List[int]:
    """Plain cached greedy decoding, one target call per token (eq. 1)."""
    req = model.new_request(enc_bits)
    y, L = prefill(model, req, prefix)
    out = [y]
    while y != eos and len(out) < n_max:
        logits = model.rows(req, [y], L)
        L += 1
        y = argmax_lowest(logits[0])
        out.append(y)
    return out


def brute_force_decode(model, enc_bits, prefix, n_max: int, eos: int) -> List[int]:
    """Greedy decoding with no cache: every step recomputes all positions
    from scratch on a fresh cache (eq. 1 taken literally)."""
    xkv = model.encode_kv(enc_bits)
    from .model import Request
    seq = list(int(t) for t in prefix)
    out: List[int] = []
    while True:
        req = Request(model._shape_nl(), xkv, model.dtype)
        logits = model.rows(req, seq, 0)
        y = argmax_lowest(logits[-1])
        out.append(y)
        seq.append(y)
        if y == eos or len(out) >= n_max:
            return out


def speculative_decode(model, enc_bits, prefix, n_max: int, eos: int, K: int,
                       draft_fn: DraftFn, stats: Optional[LoopStats] = None
                       ) -> List[int]:
    """Propose / verify / advance loop (Whisper-Flash §3.1, App. A.1)."""
    req = model.new_request(enc_bits)
    y, L = prefill(model, req, prefix)
    out = [y]
    done = y == eos or len(out) >= n_max
    while not done:
        R = n_max - len(out)
        k = min(K, R - 1)
        drafts = [int(d) for d in draft_fn(L, y, k)]
        logits = model.rows(req, [y] + drafts, L)
        g = [argmax_lowest(r) for r in logits]
        a, emitted, c, done = greedy_accept(drafts, g, eos, R)
        out.extend(emitted)
        L = rollback_length(L, a)
        if stats is not None:
            stats.rounds += 1
            stats.accepted.append(a)
            stats.proposed.append(k)
        y = c
    return out


def table_drafts(greedy_seq: List[int], prefix_len: int, keep: np.ndarray,
                 repl: np.ndarray) -> DraftFn:
    """Drafts that copy the greedy continuation where ``keep`` is set and
    take ``repl`` elsewhere, keyed by absolute position. ``greedy_seq`` is
    the greedy output (its j-th token sits at position prefix_len + j)."""
    def fn(L: int, anchor: int, k: int) -> List[int]:
        ds = []
        for i in range(1, k + 1):
            pos = L + i
            j = pos - prefix_len
            gtok = greedy_seq[j] if 0 <= j < len(greedy_seq) else int(repl[pos])
            ds.append(gtok if keep[pos] else int(repl[pos]))
        return ds
    return fn


def loop_metrics(accepted: List[int], proposed: List[int], K: int) -> dict:
    """s_k (survival), a_1, a_k^c, L (mean accepted), tau, alpha, as defined
    in "Alignment Drift ...", §"Speculative Loop", and Whisper-Flash §4."""
    acc = np.asarray(accepted)
    prop = np.asarray(proposed)
    s = [1.0]
    for k in range(1, K + 1):
        elig = prop >= k
        s.append(float((acc[elig] >= k).mean()) if elig.any() else float("nan"))
    ac = [s[k] / s[k - 1] if s[k - 1] > 0 else float("nan") for k in range(1, K + 1)]
    return {
        "rounds": int(len(acc)),
        "s_k": s[1:],
        "a1": s[1],
        "a_c": ac,
        "mean_accepted": float(acc.mean()) if len(acc) else 0.0,
        "tau": float((acc + 1).mean()) if len(acc) else 0.0,
        "alpha": float(acc.sum() / max(prop.sum(), 1)),
    }
