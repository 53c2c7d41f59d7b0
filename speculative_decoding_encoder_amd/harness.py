"""Host-side round loop around the engine: prefill, then propose / verify /
accept / rollback rounds (Whisper-Flash section 3.1, appendix A.1).

Drafts come from a caller-supplied function; ``table_drafter`` builds the
synthetic ones (copy a given greedy continuation with probability p, else a
replacement id, keyed by absolute position). The loop reads the accept
outputs back each round, which is what a test needs; the benchmark times the
device calls on their own.
"""
from __future__ import annotations

from typing import Callable, List, Optional, Sequence

import numpy as np


def prefill(eng, slots: Sequence[int], prefixes: Sequence[np.ndarray], logits: bool = False):
    """Run each prompt as one block, keep all of it (rollback a = P-1) and
    return the first anchors (argmax of each prompt's last row)."""
    torch = eng.torch
    n = len(slots)
    T = max(len(p) for p in prefixes)
    toks = np.zeros((n, T), np.int32)
    for b, p in enumerate(prefixes):
        toks[b, :len(p)] = p
    lens = np.array([len(p) for p in prefixes], np.int32)
    d_slots = eng.i32(slots)
    d_tok = eng.i32(toks)
    d_ntok = eng.i32(lens)
    d_am = torch.empty((n, T), dtype=torch.int32, device=eng.dev)
    d_lg = None
    if logits:
        d_lg = torch.empty((n, T, eng.shape.vocab), dtype=torch.float32, device=eng.dev)
    eng.wf_verify_block(d_slots, d_tok, d_ntok, d_am, d_lg)
    eng.wf_rollback(d_slots, eng.i32(lens - 1))
    am = d_am.cpu().numpy()
    anchors = np.array([am[b, lens[b] - 1] for b in range(n)], np.int32)
    return (anchors, d_lg) if logits else anchors


DraftFn = Callable[[int, int, int, int], List[int]]   # (request, L, anchor, k) -> drafts


def table_drafter(greedy: Sequence[Sequence[int]], prefix_lens: Sequence[int],
                  tables: Sequence[tuple]) -> DraftFn:
    """Draft i of a round whose anchor sits at position L is, at position
    L+i, the greedy token when keep[L+i] else repl[L+i]."""
    def fn(b: int, L: int, anchor: int, k: int) -> List[int]:
        keep, repl = tables[b]
        out = []
        for i in range(1, k + 1):
            pos = L + i
            j = pos - prefix_lens[b]
            g = greedy[b][j] if 0 <= j < len(greedy[b]) else int(repl[pos])
            out.append(int(g) if keep[pos] else int(repl[pos]))
        return out
    return fn


class LoopResult:
    def __init__(self, n):
        self.tokens = [[] for _ in range(n)]
        self.accepted = [[] for _ in range(n)]
        self.proposed = [[] for _ in range(n)]
        self.rounds = 0


def run_loop(eng, slots: Sequence[int], prefixes: Sequence[np.ndarray], n_max: int, K: int,
             draft_fn: Optional[DraftFn], eos: int,
             steer: Optional[Callable] = None) -> LoopResult:
    """Greedy speculative decoding of ``len(slots)`` requests with block
    length K+1 (K = 0 is plain greedy decoding, one row per call).

    ``steer(b, L, tokens_row, k, argmax_row, a, next)`` may return (a, c) to
    override the round's outcome (oracle-steered comparisons)."""
    torch = eng.torch
    n = len(slots)
    res = LoopResult(n)
    anchors = prefill(eng, slots, prefixes)
    L = [len(p) for p in prefixes]
    y = [int(a) for a in anchors]
    for b in range(n):
        res.tokens[b].append(y[b])
    done = [y[b] == eos or n_max <= 1 for b in range(n)]
    T = K + 1
    d_slots = eng.i32(slots)
    d_am = torch.empty((n, T), dtype=torch.int32, device=eng.dev)
    outs = [torch.empty(n, dtype=torch.int32, device=eng.dev) for _ in range(4)]
    while not all(done):
        toks = np.zeros((n, T), np.int32)
        ntok = np.zeros(n, np.int32)
        budget = np.ones(n, np.int32)
        for b in range(n):
            if done[b]:
                continue
            R = n_max - len(res.tokens[b])
            k = min(K, R - 1, eng.shape.n_ctx - L[b] - 1)
            drafts = draft_fn(b, L[b], y[b], k) if k > 0 else []
            toks[b, 0] = y[b]
            toks[b, 1:1 + k] = drafts
            ntok[b] = 1 + k
            budget[b] = R
        d_tok = eng.i32(toks)
        d_ntok = eng.i32(ntok)
        eng.wf_verify_block(d_slots, d_tok, d_ntok, d_am)
        eng.wf_accept(d_tok, d_ntok, eng.i32(budget), d_am, *outs)
        n_acc, nxt, n_emit, dn = (o.cpu().numpy() for o in outs)
        if steer is not None:
            am = d_am.cpu().numpy()
            for b in range(n):
                if ntok[b] == 0:
                    continue
                r = steer(b, L[b], toks[b], ntok[b] - 1, am[b], int(n_acc[b]), int(nxt[b]))
                if r is not None:
                    a, c = r
                    n_acc[b] = a
                    nxt[b] = c
                    emitted = list(toks[b, 1:1 + a]) + ([c] if c >= 0 else [])
                    n_emit[b] = len(emitted)
                    dn[b] = int(c < 0 or c == eos or
                                len(res.tokens[b]) + len(emitted) >= n_max)
            eng.wf_rollback(d_slots, eng.i32(n_acc))
        else:
            eng.wf_rollback(d_slots, outs[0])
        res.rounds += 1
        for b in range(n):
            if ntok[b] == 0:
                continue
            a = int(n_acc[b])
            if a < 0:
                raise RuntimeError(f"request {b}: accept failed")
            emitted = [int(t) for t in toks[b, 1:1 + a]]
            if nxt[b] >= 0:
                emitted.append(int(nxt[b]))
            res.tokens[b].extend(emitted)
            res.accepted[b].append(a)
            res.proposed[b].append(int(ntok[b] - 1))
            L[b] += 1 + a
            y[b] = int(nxt[b])
            done[b] = bool(dn[b])
    return res


def run_drafter_loop(eng, slots: Sequence[int], prefixes: Sequence[np.ndarray], n_max: int,
                     K: int, eos: int) -> LoopResult:
    """Speculative decoding with the engine's own parallel drafter: every
    round is wf_draft (anchor + K drafts on the device) -> wf_verify_block
    with k = min(K, R-1) candidates -> wf_accept -> wf_rollback."""
    torch = eng.torch
    n = len(slots)
    res = LoopResult(n)
    anchors = prefill(eng, slots, prefixes)
    y = [int(a) for a in anchors]
    for b in range(n):
        res.tokens[b].append(y[b])
    done = [y[b] == eos or n_max <= 1 for b in range(n)]
    T = K + 1
    L = [len(p) for p in prefixes]
    d_slots = eng.i32(slots)
    d_block = torch.empty((n, T), dtype=torch.int32, device=eng.dev)
    d_am = torch.empty((n, T), dtype=torch.int32, device=eng.dev)
    outs = [torch.empty(n, dtype=torch.int32, device=eng.dev) for _ in range(4)]
    while not all(done):
        ntok = np.zeros(n, np.int32)
        budget = np.ones(n, np.int32)
        for b in range(n):
            if done[b]:
                continue
            R = n_max - len(res.tokens[b])
            ntok[b] = 1 + min(K, R - 1, eng.shape.n_ctx - L[b] - 1)
            budget[b] = R
        anchor = np.array([max(v, 0) for v in y], np.int32)
        eng.wf_draft(d_slots, eng.i32(anchor), K, d_block)
        d_ntok = eng.i32(ntok)
        eng.wf_verify_block(d_slots, d_block, d_ntok, d_am)
        eng.wf_accept(d_block, d_ntok, eng.i32(budget), d_am, *outs)
        eng.wf_rollback(d_slots, outs[0])
        blk = d_block.cpu().numpy()
        n_acc, nxt, n_emit, dn = (o.cpu().numpy() for o in outs)
        res.rounds += 1
        for b in range(n):
            if ntok[b] == 0:
                continue
            a = int(n_acc[b])
            if a < 0:
                raise RuntimeError(f"request {b}: accept failed")
            emitted = [int(t) for t in blk[b, 1:1 + a]]
            if nxt[b] >= 0:
                emitted.append(int(nxt[b]))
            res.tokens[b].extend(emitted)
            res.accepted[b].append(a)
            res.proposed[b].append(int(ntok[b] - 1))
            L[b] += 1 + a
            y[b] = int(nxt[b])
            done[b] = bool(dn[b])
    return res


class DeviceLoop:
    """A speculative round loop whose state lives on the device, so that a
    round (build the block, wf_verify_block, wf_accept, wf_rollback, update
    the state) needs no host synchronisation and can be captured once and
    replayed as a HIP graph.

    Drafts: ``draft_table`` int32 [n][n_ctx + K + 2] gives the candidate at
    each absolute position (the synthetic table drafter: the greedy token
    there with probability p, else a replacement id), or ``drafter=True``
    takes the engine's own parallel drafter (wf_draft). Requests that are
    done get n_tok = 0 and are skipped by the engine. The round's bookkeeping
    (n_tok, budgets, the table block, the state update) runs in the
    library's wf_loop_prepare / wf_loop_finish kernels."""

    def __init__(self, eng, slots: Sequence[int], anchors: np.ndarray, lens: np.ndarray,
                 n_max: int, K: int, eos: int, draft_table: Optional[np.ndarray] = None,
                 drafter: bool = False, logits: bool = False):
        torch = eng.torch
        self.eng, self.torch, self.K, self.n_max, self.eos = eng, torch, K, n_max, eos
        n = len(slots)
        self.n = n
        dev = eng.dev
        i32 = dict(dtype=torch.int32, device=dev)
        self.d_slots = eng.i32(slots)
        self.anchor = torch.as_tensor(np.asarray(anchors, np.int32), device=dev)
        self.L = torch.as_tensor(np.asarray(lens, np.int32), device=dev)
        anchors = np.asarray(anchors)
        self.emitted = torch.ones(n, **i32)
        self.done = torch.as_tensor(((anchors == eos) | (n_max <= 1)).astype(np.int32), device=dev)
        self.acc_sum = torch.zeros(n, **i32)
        self.prop_sum = torch.zeros(n, **i32)
        self.rounds_active = torch.zeros(n, **i32)
        self.step = torch.zeros(n, **i32)
        self.tok_sum = torch.zeros(n, **i32)       # tokens emitted by the rounds
        self.hist = torch.zeros(K + 1, dtype=torch.int64, device=dev)   # accepted-length counts
        T = K + 1
        self.block = torch.zeros((n, T), **i32)
        self.ntok = torch.zeros(n, **i32)
        self.budget = torch.ones(n, **i32)
        self.am = torch.empty((n, T), **i32)
        self.outs = [torch.empty(n, **i32) for _ in range(4)]
        self.logits = (torch.empty((n, T, eng.shape.vocab), dtype=torch.float32, device=dev)
                       if logits else None)
        self.drafter = drafter
        self.table = None
        if draft_table is not None:
            self.table = torch.as_tensor(np.ascontiguousarray(draft_table, np.int32), device=dev)
        self.state = eng.loop_state(self.anchor, self.L, self.emitted, self.done, self.acc_sum,
                                    self.prop_sum, self.rounds_active, self.step, self.tok_sum,
                                    self.hist)

    def prepare(self):
        """This round's block, n_tok and budgets from the state."""
        self.eng.wf_loop_prepare(self.state, self.n, self.K, self.n_max,
                                 None if self.drafter else self.table, self.block, self.ntok,
                                 self.budget)
        if self.drafter:
            self.eng.wf_draft(self.d_slots, self.anchor, self.K, self.block)

    def verify(self):
        self.eng.wf_verify_block(self.d_slots, self.block, self.ntok, self.am, self.logits)

    def accept(self, **kw):
        self.eng.wf_accept(self.block, self.ntok, self.budget, self.am, *self.outs, **kw)

    def finish(self):
        """Rollback and the state update of the round."""
        n_acc, nxt, n_emit, dn = self.outs
        self.eng.wf_rollback(self.d_slots, n_acc)
        self.eng.wf_loop_finish(self.state, self.n, self.K, self.ntok, n_acc, nxt, n_emit, dn)

    def restart(self, anchors: np.ndarray, lens: np.ndarray):
        """Start every request again from a fresh prefill (anchors, lengths),
        in place, so that a captured round stays valid; the totals carry on."""
        torch = self.torch
        anchors = np.asarray(anchors, np.int32)
        self.anchor.copy_(torch.as_tensor(anchors, device=self.eng.dev))
        self.L.copy_(torch.as_tensor(np.asarray(lens, np.int32), device=self.eng.dev))
        self.emitted.fill_(1)
        self.done.copy_(torch.as_tensor(((anchors == self.eos) | (self.n_max <= 1)).astype(np.int32),
                                        device=self.eng.dev))

    def round(self, **accept_kw):
        self.prepare()
        self.verify()
        self.accept(**accept_kw)
        self.finish()

    def counters(self) -> dict:
        """Host copy of the totals: tokens emitted so far per request
        (including its first anchor), tokens the rounds emitted, accepted and proposed candidates, active request-rounds,
        the accepted-length histogram, and whether every request is done."""
        return {"emitted": self.emitted.cpu().numpy().copy(),
                "tokens": int(self.tok_sum.sum().item()),
                "accepted": int(self.acc_sum.sum().item()),
                "proposed": int(self.prop_sum.sum().item()),
                "request_rounds": int(self.rounds_active.sum().item()),
                "hist": self.hist.cpu().numpy().copy(),
                "all_done": bool((self.done > 0).all().item())}


def draft_table(greedy: Sequence[int], prefix_len: int, keep: np.ndarray, repl: np.ndarray,
                size: int) -> np.ndarray:
    """Per absolute position t < size: the table drafter's candidate there
    (greedy[t - prefix_len] when keep[t], else repl[t]; past the known greedy
    continuation, repl[t])."""
    out = np.zeros(size, np.int32)
    for t in range(size):
        j = t - prefix_len
        g = greedy[j] if 0 <= j < len(greedy) else int(repl[min(t, len(repl) - 1)])
        out[t] = int(g) if keep[min(t, len(keep) - 1)] else int(repl[min(t, len(repl) - 1)])
    return out
