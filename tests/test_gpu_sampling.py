"""GPU temperature rejection sampling (wf_accept with T > 0) against the oracle.

* kernel-level parity: seeded logits, draft distributions q and drafts drawn
  from q go to both the GPU and ``oracle.sampling.sample_round``; the
  accepted length and the next token must agree wherever no fp32 decision
  sits within rounding distance of its boundary (both sides compute the
  softmax and the acceptance test in fp32, Whisper-Flash App. A.4);
* distribution preservation on the GPU itself (Whisper-Flash §3.1): over many
  Philox-keyed trials the first emitted token follows p (chi-square) and the
  first candidate is accepted with probability sum_v min(p_v, q_v);
* end-to-end rounds on the tiny model: GPU verify + sampling against the
  oracle's own fp64 logits, compared where every decision holds for any
  logits within the measured error (accept tests by |log(u q / p)|, the
  final draw by bounds on the CDF); at least a third of the rounds count.
"""
import dataclasses

import numpy as np
import pytest

from gpu_common import log
from oracle import philox as ph
from oracle import sampling as osmp
from synthetic import TINY, WORKLOADS, make_encoder_out, make_prefixes, make_weights

pytestmark = pytest.mark.gpu
TEMP = 0.7


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _small_engine(vocab, max_batch, max_rows=64):
    from speculative_decoding_encoder_amd.binding import Engine
    shape = dataclasses.replace(TINY, n_layers=1, d_ffn=64, vocab=vocab, n_frames=32,
                                eos_id=vocab - 1)
    return Engine(shape, make_weights(shape, 90), max_batch=max_batch, max_rows=max_rows), shape


def _softmax(x):
    x = x - x.max(-1, keepdims=True)
    e = np.exp(x)
    return e / e.sum(-1, keepdims=True)


def _gpu_accept(eng, tokens, logits, q, seed, req_ids, steps, budget):
    torch = eng.torch
    n, T = tokens.shape
    outs = [torch.empty(n, dtype=torch.int32, device=eng.dev) for _ in range(4)]
    d_lg = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).to(eng.dev)
    d_q = torch.from_numpy(np.ascontiguousarray(q, np.float32)).to(eng.dev)
    am = torch.zeros((n, T), dtype=torch.int32, device=eng.dev)
    eng.wf_accept(eng.i32(tokens), eng.i32(np.full(n, T)), eng.i32(budget), am, *outs,
                  logits=d_lg, q=d_q, temperature=TEMP, seed=seed,
                  request_id=eng.i32(req_ids), step=eng.i32(steps))
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in outs]


def _margins(lrow, qrows, drafts, u_acc, u_res, a_ref):
    """Smallest relative distance of any decision the oracle took from its
    fp32 boundary (accept tests up to a, and the final draw)."""
    k = len(drafts)
    p = [osmp.probs(lrow[i], TEMP) for i in range(k + 1)]
    worst = np.inf
    for i in range(min(a_ref + 1, k)):
        y = drafts[i]
        lhs = np.float64(np.float32(u_acc[i]) * np.float32(qrows[i][y]))
        worst = min(worst, abs(lhs - p[i][y]) / max(p[i][y], 1e-30))
    i = a_ref
    w = np.maximum(p[i] - qrows[i], 0) if i < k else p[i]
    if w.sum() <= 0:
        w = p[i]
    c = np.cumsum(w.astype(np.float64))
    thr = u_res[i] * c[-1]
    worst = min(worst, np.min(np.abs(c - thr)) / c[-1])
    return worst


def test_sampling_kernel_parity_full_vocab(torch_cuda):
    V, n, K = 51866, 32, 8
    T = K + 1
    eng, shape = _small_engine(V, n)
    g = np.random.default_rng(41)
    logits = (g.standard_normal((n, T, V)) * 2.0).astype(np.float32)
    q = np.empty((n, K, V), np.float32)
    drafts = np.zeros((n, K), np.int64)
    for b in range(n):
        for i in range(K):
            p = osmp.probs(logits[b, i], TEMP).astype(np.float64)
            qi = 0.7 * p + 0.3 * _softmax(g.standard_normal(V))
            q[b, i] = qi.astype(np.float32)
            drafts[b, i] = g.choice(V, p=qi / qi.sum())
    tokens = np.zeros((n, T), np.int32)
    tokens[:, 1:] = drafts
    seed, step = 1234567, 3
    req_ids = np.arange(n) + 100
    n_acc, nxt, n_emit, done = _gpu_accept(eng, tokens, logits, q, seed, req_ids,
                                           np.full(n, step), np.full(n, 200))
    agree = pinned = 0
    for b in range(n):
        u_acc = [ph.uniform(seed, int(req_ids[b]), step, i, ph.STREAM_ACCEPT) for i in range(K)]
        u_res = [ph.uniform(seed, int(req_ids[b]), step, i, ph.STREAM_RESAMPLE) for i in range(K + 1)]
        pk = np.stack([osmp.probs(logits[b, i], TEMP) for i in range(T)])
        a, em, c, dn = osmp.rejection_round(pk, q[b], list(drafts[b]), u_acc, u_res,
                                            eos=shape.eos_id, budget=200)
        same = (int(n_acc[b]), int(nxt[b])) == (a, c)
        agree += same
        if _margins(logits[b], q[b], list(drafts[b]), u_acc, u_res, a) > 1e-5:
            pinned += 1
            assert same, (b, int(n_acc[b]), int(nxt[b]), a, c)
    log(f"sampling parity: {agree}/{n} identical, {pinned} pinned by margin")
    assert agree >= n - 2
    eng.close()


def test_sampling_preserves_target_distribution_on_gpu(torch_cuda):
    V, n, K = 8, 256, 2
    T = K + 1
    eng, shape = _small_engine(V, n)
    g = np.random.default_rng(42)
    row_logits = (g.standard_normal((T, V)) * 1.5).astype(np.float32)
    p = np.stack([osmp.probs(row_logits[i], TEMP) for i in range(T)]).astype(np.float64)
    q = np.stack([_softmax(g.standard_normal(V) * 1.5) for _ in range(K)]).astype(np.float32)
    logits = np.broadcast_to(row_logits, (n, T, V)).copy()
    qb = np.broadcast_to(q, (n, K, V)).copy()
    counts = np.zeros(V)
    acc1 = 0
    trials = 0
    for step in range(40):
        drafts = np.stack([[g.choice(V, p=q[i].astype(np.float64) / q[i].sum()) for i in range(K)]
                           for _ in range(n)])
        tokens = np.zeros((n, T), np.int32)
        tokens[:, 1:] = drafts
        n_acc, nxt, n_emit, done = _gpu_accept(eng, tokens, logits, qb, 99, np.arange(n),
                                               np.full(n, step), np.full(n, 100))
        first = np.where(n_acc >= 1, drafts[:, 0], nxt)
        for t in first:
            counts[t] += 1
        acc1 += int((n_acc >= 1).sum())
        trials += n
    exp = trials * p[0]
    mask = exp > 5
    chi2 = (((counts - exp) ** 2 / exp)[mask]).sum()
    assert chi2 < 24.3, chi2          # chi-square, 7 dof, p ~ 0.001
    pacc = np.minimum(p[0], q[0]).sum()
    assert abs(acc1 / trials - pacc) < 4 * np.sqrt(pacc * (1 - pacc) / trials)
    log(f"sampling distribution: chi2 {chi2:.2f} over {trials} trials, accept rate "
        f"{acc1 / trials:.4f} vs {pacc:.4f}")
    eng.close()


def _draw_pinned(z, qrow, u, c, delta):
    """Whether a draw with uniform u lands on id c for every logit vector
    within delta of z entry by entry: bounds on the (residual) CDF at c - 1
    and at c. With logits within delta, each probability lies within a
    factor exp(2 delta / T) of p; the CDF through id j, A / (A + B) with A
    the mass up to j and B the rest, is smallest with A low and B high."""
    z = np.asarray(z, np.float64) / TEMP
    e = np.exp(z - z.max())
    p = e / e.sum()
    f = np.exp(2 * delta / TEMP)
    if qrow is None:
        wlo, whi = p / f, p * f
    else:
        wlo, whi = np.maximum(p / f - qrow, 0), np.maximum(p * f - qrow, 0)
        if wlo.sum() <= 0:
            return False           # the residual may vanish: no bound
    def bounds(j):
        le_lo, le_hi = wlo[:j + 1].sum(), whi[:j + 1].sum()
        gt_lo, gt_hi = wlo[j + 1:].sum(), whi[j + 1:].sum()
        return le_lo / (le_lo + gt_hi), le_hi / (le_hi + gt_lo)
    ok = u < bounds(c)[0]
    if c > 0:
        ok = ok and u > bounds(c - 1)[1]
    return bool(ok)


def test_sampling_round_tiny_model_against_oracle(torch_cuda):
    """Rounds of GPU verify + GPU rejection sampling against the oracle's
    fp64 logits and rule. A round is compared when every decision the
    oracle took holds for any logits within the measured GPU error delta:
    the accept tests by |log(u q / p)| > 2 delta / T, the final draw by the
    CDF bounds of _draw_pinned. At least a third of the rounds must be
    compared."""
    from oracle import model as om
    from speculative_decoding_encoder_amd.binding import Engine
    wl = WORKLOADS[0]
    wbits = make_weights(TINY, wl.cfg_id)
    enc = make_encoder_out(TINY, wl.cfg_id, 0)
    prefix = make_prefixes(wl)[0]
    P = len(prefix)
    m = om.Model(TINY, wbits)
    eng = Engine(TINY, wbits, max_batch=1, max_rows=64)
    torch = eng.torch
    eng.wf_encode_kv(eng.i32([0]), eng.bf16(enc[None]))
    K = 4
    T = K + 1
    rounds = 24
    g = np.random.default_rng(43)
    checked = 0
    deltas = []
    for rnd in range(rounds):
        eng.wf_reset(eng.i32([0]))
        req = m.new_request(enc)
        m.rows(req, prefix, 0)
        am = torch.empty((1, P), dtype=torch.int32, device=eng.dev)
        eng.wf_verify_block(eng.i32([0]), eng.i32(prefix[None]), eng.i32([P]), am)
        eng.wf_rollback(eng.i32([0]), eng.i32([P - 1]))
        anchor = int(g.integers(0, TINY.vocab))
        qz = np.stack([_softmax(g.standard_normal(TINY.vocab) * 2) for _ in range(K)])
        drafts = [int(g.choice(TINY.vocab, p=qz[i])) for i in range(K)]
        block = np.array([anchor] + drafts, np.int32)
        lg = torch.empty((1, T, TINY.vocab), dtype=torch.float32, device=eng.dev)
        amb = torch.empty((1, T), dtype=torch.int32, device=eng.dev)
        eng.wf_verify_block(eng.i32([0]), eng.i32(block[None]), eng.i32([T]), amb, lg)
        outs = [torch.empty(1, dtype=torch.int32, device=eng.dev) for _ in range(4)]
        d_q = torch.from_numpy(qz.astype(np.float32)[None]).to(eng.dev)
        eng.wf_accept(eng.i32(block[None]), eng.i32([T]), eng.i32([50]), amb, *outs, logits=lg,
                      q=d_q, temperature=TEMP, seed=7, request_id=eng.i32([0]),
                      step=eng.i32([rnd]))
        a_gpu, c_gpu = int(outs[0].item()), int(outs[1].item())
        ref64 = m.rows(req, block, P)
        ref = ref64.astype(np.float32)
        # the GPU's logit error, plus slack for its own fp32 softmax rounding
        delta = float(np.abs(lg.cpu().numpy()[0] - ref64).max()) + 1e-6
        deltas.append(delta)
        u_acc = [ph.uniform(7, 0, rnd, i, ph.STREAM_ACCEPT) for i in range(K)]
        u_res = [ph.uniform(7, 0, rnd, i, ph.STREAM_RESAMPLE) for i in range(K + 1)]
        pk = np.stack([osmp.probs(ref[i], TEMP) for i in range(T)])
        a, em, c, dn = osmp.rejection_round(pk, qz.astype(np.float32), drafts, u_acc, u_res,
                                            eos=TINY.eos_id, budget=50)
        pinned = True
        for i in range(min(a + 1, K)):
            y = drafts[i]
            r = np.log(max(u_acc[i] * qz[i][y], 1e-30) / max(pk[i][y], 1e-30))
            if abs(r) <= 2 * delta / TEMP:
                pinned = False
        if c is not None and not _draw_pinned(ref64[a], qz[a] if a < K else None, u_res[a], c,
                                              delta):
            pinned = False
        if pinned:
            checked += 1
            assert (a_gpu, c_gpu) == (a, c), (rnd, a_gpu, c_gpu, a, c, delta)
    log(f"tiny sampling rounds: {checked}/{rounds} pinned and identical, max logit error "
        f"{max(deltas):.2e}")
    assert checked >= rounds // 3, (checked, max(deltas))
    eng.close()
