"""wf_accept and wf_accept_tree at the method's edges, bit for bit against the
oracle's rules (Whisper-Flash section 3.1 and appendix A.1; AD appendix E.3).

Integer logic on random arrays, so every outcome is exact:

* greedy: random argmax rows and drafts built to agree for a chosen prefix
  length; an EOS accepted at a random position (no bonus after it), EOS as
  the target's correction and as the bonus, a rejected EOS draft, budgets
  R = 0..K+1 (so k > R - 1 is proposed too: the kernel refuses it with
  n_acc = -1 and done) and inactive requests. Against
  ``oracle.decode.greedy_accept``.
* sampling at T = 0.7, against ``oracle.sampling.rejection_round`` with the
  same Philox uniforms: q = p (every candidate accepted, EOS drafts accepted
  and ending the request, an EOS bonus, the budget ending it) and disjoint
  supports (the suppression mask zeroes p where q lives: the first candidate
  is always rejected and the correction comes from p, EOS included).
  Decisions within fp32 rounding of their boundary are not compared. Both
  on a 64-id vocabulary (the one-kernel draw) and on a 1000-id one, ragged
  against the 64-id tiles, whose engine holds the split draw's scratch (row
  statistics, segment sums, then the draw).
* trees: random parent arrays with accepted chains, an accepted EOS node,
  EOS as the next token, budgets 1..depth+1. Against ``oracle.tree.tree_accept``.
"""
import dataclasses

import numpy as np
import pytest

from gpu_common import log
from oracle import decode as od
from oracle import philox as ph
from oracle import sampling as osmp
from oracle import tree as ot
from synthetic import TINY, make_weights

pytestmark = pytest.mark.gpu
TEMP = 0.7
V = 64
EOS = V - 1


@pytest.fixture(scope="module")
def eng(request):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from speculative_decoding_encoder_amd.binding import Engine
    shape = dataclasses.replace(TINY, n_layers=1, d_ffn=64, vocab=V, n_frames=32, eos_id=EOS)
    e = Engine(shape, make_weights(shape, 91), max_batch=1024, max_rows=64)
    yield e
    e.close()


# A vocabulary that is no multiple of the LM head's 64-id tiles, on an engine
# whose per-tile maxima buffer (ceil(V / 64) x max_rows floats) can hold the
# split draw's scratch for 512 requests of K + 1 = 9 rows (2nT + 3n + 128n
# floats): sampling then takes the row-statistics / segment-sum / draw
# kernels, where the narrow engine above takes the one-kernel fallback.
V_WIDE = 1000
WIDE_ROWS = -(-(2 * 512 * 9 + 3 * 512 + 128 * 512) // -(-V_WIDE // 64))


@pytest.fixture(scope="module")
def eng_wide(request):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from speculative_decoding_encoder_amd.binding import Engine
    shape = dataclasses.replace(TINY, n_layers=1, d_ffn=64, vocab=V_WIDE, n_frames=32,
                                eos_id=V_WIDE - 1)
    e = Engine(shape, make_weights(shape, 92), max_batch=1024, max_rows=WIDE_ROWS)
    yield e
    e.close()


def _outs(eng, n):
    torch = eng.torch
    return [torch.empty(n, dtype=torch.int32, device=eng.dev) for _ in range(4)]


def _host(outs):
    return [o.cpu().numpy() for o in outs]      # .cpu() waits for the stream


def _other(g, avoid):
    """A non-EOS id different from ``avoid``."""
    while True:
        v = int(g.integers(0, EOS))
        if v != avoid:
            return v


def greedy_case(n=1024, K=8, seed=2024):
    """Argmax rows and blocks whose drafts agree with the target for a
    chosen prefix length, with the EOS and budget edges planted."""
    T = K + 1
    g = np.random.default_rng(seed)
    am = g.integers(0, EOS, (n, T)).astype(np.int32)
    tok = g.integers(0, EOS, (n, T)).astype(np.int32)
    n_tok = g.integers(1, T + 1, n).astype(np.int32)
    n_tok[g.random(n) < 0.06] = 0                      # inactive requests
    budget = g.integers(0, T + 2, n).astype(np.int32)  # 0 .. K+2
    budget[g.random(n) < 0.3] = 200
    kinds = g.integers(0, 6, n)
    for b in range(n):
        k = max(int(n_tok[b]) - 1, 0)
        m = int(g.integers(0, k + 1))                  # agreeing prefix length
        for i in range(m):
            tok[b, i + 1] = am[b, i]
        if m < k:
            tok[b, m + 1] = _other(g, am[b, m])
        kind = kinds[b]
        if kind == 1 and m > 0:                        # an accepted EOS inside the prefix
            j = int(g.integers(1, m + 1))
            tok[b, j] = am[b, j - 1] = EOS
        elif kind == 2:                                # EOS as the correction / bonus
            am[b, m] = EOS
        elif kind == 3 and m < k:                      # a rejected EOS draft
            tok[b, m + 1] = EOS
            am[b, m] = _other(g, EOS)
        elif kind == 4:                                # all accepted, EOS bonus
            tok[b, 1:k + 1] = am[b, :k]
            am[b, k] = EOS
        elif kind == 5 and n_tok[b] > 0:               # all accepted, the budget ends it
            tok[b, 1:k + 1] = am[b, :k]
            budget[b] = n_tok[b]
    return tok, am, n_tok, budget


def greedy_expected(tok, am, n_tok, budget):
    """Per request (n_acc, next, n_emit, done) by the oracle's rule, the
    kernel's refusal (-1, -1, 0, 1) for k > R - 1 or R < 1, and counts of
    the edges met."""
    out = []
    seen = {"eos_accepted": 0, "eos_next": 0, "refused": 0, "budget_end": 0, "inactive": 0}
    for b in range(tok.shape[0]):
        nt, R = int(n_tok[b]), int(budget[b])
        if nt == 0:
            exp = (0, -1, 0, 0)
            seen["inactive"] += 1
        elif R < 1 or nt - 1 > R - 1:
            exp = (-1, -1, 0, 1)
            seen["refused"] += 1
        else:
            a, em, c, dn = od.greedy_accept(list(tok[b, 1:nt]), list(am[b, :nt]), EOS, R)
            exp = (a, -1 if c is None else c, len(em), int(dn))
            seen["eos_accepted"] += c is None
            seen["eos_next"] += c == EOS
            seen["budget_end"] += (c is not None and c != EOS and dn)
        out.append(exp)
    return out, seen


def test_greedy_accept_random_arrays_bit_exact(eng):
    tok, am, n_tok, budget = greedy_case()
    n = tok.shape[0]
    outs = _outs(eng, n)
    eng.wf_accept(eng.i32(tok), eng.i32(n_tok), eng.i32(budget), eng.i32(am), *outs)
    n_acc, nxt, n_emit, done = _host(outs)
    exp, seen = greedy_expected(tok, am, n_tok, budget)
    for b in range(n):
        got = (int(n_acc[b]), int(nxt[b]), int(n_emit[b]), int(done[b]))
        assert got == exp[b], (b, got, exp[b], tok[b], am[b], int(n_tok[b]), int(budget[b]))
    log(f"greedy accept edges: {seen}")
    assert all(v >= 20 for v in seen.values()), seen


def _sampling_case(eng, logits, q, tok, n_tok, budget, suppress, seed, step):
    torch = eng.torch
    n = tok.shape[0]
    outs = _outs(eng, n)
    d_lg = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).to(eng.dev)
    d_q = torch.from_numpy(np.ascontiguousarray(q, np.float32)).to(eng.dev)
    d_sup = None if suppress is None else torch.from_numpy(suppress.astype(np.uint8)).to(eng.dev)
    am = torch.zeros(tok.shape, dtype=torch.int32, device=eng.dev)
    eng.wf_accept(eng.i32(tok), eng.i32(n_tok), eng.i32(budget), am, *outs, logits=d_lg, q=d_q,
                  temperature=TEMP, seed=seed, request_id=eng.i32(np.arange(n)),
                  step=eng.i32(np.full(n, step)), suppress=d_sup)
    return _host(outs)


def _oracle_round(logits, q, drafts, suppress, seed, req, step, R, eos=EOS):
    """The oracle's outcome and the smallest relative distance of any
    decision it took from its fp32 boundary."""
    k = len(drafts)
    p = np.stack([osmp.probs(logits[i], TEMP, suppress) for i in range(k + 1)])
    u_acc = [ph.uniform(seed, req, step, i, ph.STREAM_ACCEPT) for i in range(k)]
    u_res = [ph.uniform(seed, req, step, i, ph.STREAM_RESAMPLE) for i in range(k + 1)]
    a, em, c, dn = osmp.rejection_round(p, q[:k], drafts, u_acc, u_res, eos, R)
    worst = np.inf
    for i in range(min(a + 1, k)):
        y = drafts[i]
        lhs = np.float64(np.float32(u_acc[i]) * np.float32(q[i][y]))
        worst = min(worst, abs(lhs - p[i][y]) / max(float(p[i][y]), 1e-30))
    if c is not None:
        w = np.maximum(p[a] - q[a], 0) if a < k else p[a]
        if w.sum() <= 0:
            w = p[a]
        cum = np.cumsum(w.astype(np.float64))
        worst = min(worst, float(np.min(np.abs(cum - u_res[a] * cum[-1])) / cum[-1]))
    return (a, -1 if c is None else c, len(em), int(dn)), worst


def sampling_case(case, n=512, K=8, V=V):
    """Logits, draft distributions, blocks, n_tok, budgets and the
    suppression mask of one edge case of rejection sampling over a
    vocabulary of V ids, EOS the last."""
    T = K + 1
    EOS = V - 1
    g = np.random.default_rng(77 if case == "q_equals_p" else 78)
    logits = (g.standard_normal((n, T, V)) * 2.0).astype(np.float32)
    suppress = None
    allowed = np.ones(V, bool)
    if case == "disjoint_supports":
        suppress = np.zeros(V, bool)
        suppress[24:EOS] = True                        # p lives on 0..23 and EOS
        allowed = ~suppress
    budget = g.integers(0, T + 2, n).astype(np.int32)
    budget[g.random(n) < 0.3] = 200
    n_tok = np.array([min(K, max(int(r) - 1, 0)) + 1 for r in budget], np.int32)
    over = g.random(n) < 0.05                          # k > R - 1 proposed
    n_tok[over] = T
    tok = np.zeros((n, T), np.int32)
    q = np.zeros((n, K, V), np.float32)
    kinds = g.integers(0, 4, n)
    for b in range(n):
        k = int(n_tok[b]) - 1
        if kinds[b] == 1:                              # EOS bonus / correction row
            logits[b, k if case == "q_equals_p" else 0, EOS] = 40.0
        for i in range(K):
            if case == "q_equals_p":
                q[b, i] = osmp.probs(logits[b, i], TEMP)
            else:
                z = g.standard_normal(V) * 1.5
                z[allowed] = -np.inf
                e = np.exp(z - z[~allowed].max())
                q[b, i] = (e / e.sum()).astype(np.float32)
            qi = q[b, i].astype(np.float64)
            tok[b, i + 1] = g.choice(V, p=qi / qi.sum())
        if case == "q_equals_p" and kinds[b] == 2 and k > 0:   # an EOS draft
            tok[b, int(g.integers(1, k + 1))] = EOS
    return logits, q, tok, n_tok, budget, suppress


SEED, STEP = 31337, 5


def sampling_expected(logits, q, tok, n_tok, budget, suppress):
    """Per request: None when the kernel must refuse the block, else the
    oracle's (n_acc, next, n_emit, done) and its smallest decision margin."""
    eos = logits.shape[-1] - 1
    out = []
    for b in range(tok.shape[0]):
        nt, R = int(n_tok[b]), int(budget[b])
        if R < 1 or nt - 1 > R - 1:
            out.append(None)
        else:
            out.append(_oracle_round(logits[b], q[b], [int(t) for t in tok[b, 1:nt]], suppress,
                                     SEED, b, STEP, R, eos))
    return out


def sampling_edges_met(expected, EOS=EOS):
    seen = {"eos_accepted": 0, "eos_next": 0, "refused": 0, "budget_end": 0}
    for e in expected:
        if e is None:
            seen["refused"] += 1
            continue
        exp, worst = e
        if worst > 1e-5:
            seen["eos_accepted"] += exp[1] == -1
            seen["eos_next"] += exp[1] == EOS
            seen["budget_end"] += exp[1] not in (-1, EOS) and exp[3] == 1
    return seen


@pytest.mark.parametrize("vocab", [V, V_WIDE])
@pytest.mark.parametrize("case", ["q_equals_p", "disjoint_supports"])
def test_sampling_accept_edges_against_oracle(request, case, vocab):
    eng = request.getfixturevalue("eng" if vocab == V else "eng_wide")
    EOS = vocab - 1
    logits, q, tok, n_tok, budget, suppress = sampling_case(case, V=vocab)
    n = tok.shape[0]
    n_acc, nxt, n_emit, done = _sampling_case(eng, logits, q, tok, n_tok, budget, suppress,
                                              SEED, STEP)
    expected = sampling_expected(logits, q, tok, n_tok, budget, suppress)
    pinned = agree = 0
    for b in range(n):
        got = (int(n_acc[b]), int(nxt[b]), int(n_emit[b]), int(done[b]))
        if expected[b] is None:
            assert got == (-1, -1, 0, 1), (b, got)
            continue
        exp, worst = expected[b]
        agree += got == exp
        if worst > 1e-5:
            pinned += 1
            assert got == exp, (b, got, exp, worst)
        if case == "disjoint_supports":
            assert got[0] == 0 and (got[1] < 24 or got[1] == EOS), (b, got)
    seen = sampling_edges_met(expected, EOS)
    log(f"sampling edges {case} V={vocab}: {agree} identical, {pinned} pinned, {seen}")
    checked = n - seen["refused"]
    assert pinned >= 0.9 * checked and agree >= checked - 3
    assert seen["eos_next"] >= 10 and seen["budget_end"] >= 10 and seen["refused"] >= 10
    if case == "q_equals_p":
        assert seen["eos_accepted"] >= 10


def _random_tree(g, n_nodes, am_row, tok_row):
    """Parents with a few long chains; 70% of the nodes copy the target's
    choice at their parent (so chains are accepted)."""
    par = np.full(n_nodes, -1, np.int32)
    for i in range(1, n_nodes):
        par[i] = i - 1 if g.random() < 0.5 else int(g.integers(0, i))
    for i in range(1, n_nodes):
        tok_row[i] = am_row[par[i]] if g.random() < 0.7 else _other(g, am_row[par[i]])
    return par


def tree_case(n=512, T=16):
    g = np.random.default_rng(99)
    am = g.integers(0, EOS, (n, T)).astype(np.int32)
    tok = g.integers(0, EOS, (n, T)).astype(np.int32)
    n_tok = g.integers(1, T + 1, n).astype(np.int32)
    par = np.full((n, T), -1, np.int32)
    budget = np.zeros(n, np.int32)
    for b in range(n):
        nt = int(n_tok[b])
        par[b, :nt] = _random_tree(g, nt, am[b], tok[b])
        d = ot.depths(list(par[b, :nt]))
        kind = b % 4
        if kind == 1 and nt > 1:                       # an accepted node carries EOS
            i = int(g.integers(1, nt))
            tok[b, i] = am[b, par[b, i]] = EOS
        elif kind == 2:                                # EOS as the next token
            am[b, :nt][g.random(nt) < 0.5] = EOS
        budget[b] = int(g.integers(1, max(d) + 3))
    budget[g.random(n) < 0.05] = 0
    return tok, am, n_tok, par, budget


def tree_expected(tok, am, n_tok, par, budget):
    """Per request: None when the kernel must refuse (R < 1), else the
    oracle's ((n_acc, next, n_emit, done), path); and the edges met."""
    out = []
    seen = {"eos_accepted": 0, "eos_next": 0, "refused": 0, "deep": 0}
    for b in range(tok.shape[0]):
        nt, R = int(n_tok[b]), int(budget[b])
        if R < 1:
            out.append(None)
            seen["refused"] += 1
            continue
        a, p, em, c, dn = ot.tree_accept(list(tok[b, :nt]), list(par[b, :nt]), list(am[b, :nt]),
                                         EOS, R)
        out.append(((a, -1 if c is None else c, len(em), int(dn)), p))
        seen["eos_accepted"] += c is None
        seen["eos_next"] += c == EOS
        seen["deep"] += a >= 3
    return out, seen


def test_tree_accept_eos_paths_bit_exact(eng):
    tok, am, n_tok, par, budget = tree_case()
    n, T = tok.shape
    torch = eng.torch
    outs = _outs(eng, n)
    path = torch.empty((n, T), dtype=torch.int32, device=eng.dev)
    eng.wf_accept_tree(eng.i32(tok), eng.i32(par), eng.i32(n_tok), eng.i32(budget), eng.i32(am),
                       path, *outs)
    n_acc, nxt, n_emit, done = _host(outs)
    path = path.cpu().numpy()
    expected, seen = tree_expected(tok, am, n_tok, par, budget)
    for b in range(n):
        got = (int(n_acc[b]), int(nxt[b]), int(n_emit[b]), int(done[b]))
        if expected[b] is None:
            assert got == (-1, -1, 0, 1) and (path[b] == -1).all(), (b, got)
            continue
        exp, p = expected[b]
        assert got == exp, (b, got, exp)
        a = exp[0]
        assert list(path[b, :a + 1]) == p and (path[b, a + 1:] == -1).all(), (b, path[b], p)
    log(f"tree accept edges: {seen}")
    assert all(v >= 10 for v in seen.values()), seen
