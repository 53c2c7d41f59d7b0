"""Tree verification — test infrastructure (the oracle: only tests, smoke()
and bench.py's CPU baseline may use it).

"Alignment Drift in Single-Model Speculative Decoding for ASR", App. E.3
(the tree-decoder implementation check): the draft is a fixed tree of
candidate tokens, one target forward scores all its nodes with each node
attending only to its ancestors, and a tree that is a single chain must give
exactly the tokens of the linear block.

Readings where the pages leave a step open:

* node 0 is the anchor (the root) and ``parents[i] < i`` for every other
  node, so a node's ancestors come before it;
* node i sits at position L + depth(i) and sees the L cached positions plus
  its ancestors and itself. That is the causal pass over its root-to-node
  path, so its logits are those of the path run alone — the definition this
  module computes, one path at a time;
* greedy acceptance: a node is accepted when its parent is (the root always
  is), the parent is not an accepted EOS, and its token equals the target's
  choice at the parent. The kept path ends at the deepest accepted node no
  deeper than R - 1 (R output tokens left), the lowest node index among
  equally deep ones. Then, as in the linear round, accepting EOS finishes
  the request with no bonus; otherwise the target's choice there is emitted
  and becomes the next anchor;
* rollback keeps the anchor and the path at positions L .. L + a.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np

from . import model as om


def check_parents(parents: Sequence[int]) -> None:
    if len(parents) == 0 or parents[0] != -1:
        raise ValueError("node 0 is the root: parents[0] must be -1")
    for i in range(1, len(parents)):
        if not 0 <= parents[i] < i:
            raise ValueError(f"parents[{i}] = {parents[i]} must be in [0, {i})")


def depths(parents: Sequence[int]) -> List[int]:
    check_parents(parents)
    d = [0] * len(parents)
    for i in range(1, len(parents)):
        d[i] = d[parents[i]] + 1
    return d


def path_to(parents: Sequence[int], i: int) -> List[int]:
    """Nodes from the root down to node i."""
    out = [i]
    while parents[out[-1]] >= 0:
        out.append(parents[out[-1]])
    return out[::-1]


def copy_request(model: "om.Model", req: "om.Request") -> "om.Request":
    tmp = om.Request(model._shape_nl(), req.xkv, model.dtype)
    for l in range(model.n_layers):
        tmp.K[l][:] = req.K[l]
        tmp.V[l][:] = req.V[l]
    return tmp


def tree_rows(model: "om.Model", req: "om.Request", tokens: Sequence[int],
              parents: Sequence[int], L: int) -> np.ndarray:
    """Logits [T, V] of every node: node i's root-to-node path run as a
    causal block at positions L .. L + depth(i) over the request's first L
    cached positions (req itself is left unchanged)."""
    check_parents(parents)
    out = []
    for i in range(len(parents)):
        p = path_to(parents, i)
        tmp = copy_request(model, req)
        out.append(model.rows(tmp, [tokens[j] for j in p], L)[-1])
    return np.stack(out)


def tree_accept(tokens: Sequence[int], parents: Sequence[int], g: Sequence[int], eos: int,
                budget: int) -> Tuple[int, List[int], List[int], Optional[int], bool]:
    """One greedy round on a tree. tokens[0] is the anchor, g[i] the target's
    choice at node i, budget R the output tokens still allowed.
    Returns (a, path nodes [root, ..., node at depth a], emitted tokens,
    next anchor or None, done)."""
    if budget < 1:
        raise ValueError("no output token left")
    d = depths(parents)
    T = len(parents)
    acc = [False] * T
    acc[0] = True
    for i in range(1, T):
        p = parents[i]
        acc[i] = (acc[p] and not (p > 0 and tokens[p] == eos) and tokens[i] == g[p])
    best = 0
    for i in range(1, T):
        if acc[i] and d[i] <= budget - 1 and d[i] > d[best]:
            best = i
    path = path_to(parents, best)
    a = len(path) - 1
    emitted = [int(tokens[j]) for j in path[1:]]
    if a > 0 and tokens[best] == eos:
        return a, path, emitted, None, True
    c = int(g[best])
    emitted.append(c)
    return a, path, emitted, c, c == eos or len(emitted) >= budget
