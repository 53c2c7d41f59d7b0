"""wf_loop_prepare and wf_loop_finish, the device bookkeeping of the running
speculative loop (Whisper-Flash section 3.1: a round emits the accepted
candidates and the next token, which anchors the next round; appendix A.1:
the output budget and EOS), bit for bit against the rules as the header
states them, written out here in numpy on random states.

Edges covered: requests already done, budgets used up or nearly (R <= 1),
blocks that would pass the context end (room <= 0), table reads past the
table's end (clamped), inactive requests in finish (n_tok = 0), rejected
EOS ends (next token -1), accepted lengths 0..K and the histogram's
atomics from hundreds of requests.
"""
import dataclasses

import numpy as np
import pytest

from gpu_common import log
from synthetic import TINY, make_weights

pytestmark = pytest.mark.gpu
K = 8


@pytest.fixture(scope="module")
def eng(request):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from speculative_decoding_encoder_amd.binding import Engine
    shape = dataclasses.replace(TINY, n_layers=1)
    e = Engine(shape, make_weights(shape, 5), max_batch=4, max_rows=64)
    yield e
    e.close()


def _state(eng, rs, n, n_max):
    torch = eng.torch
    n_ctx = eng.shape.n_ctx
    host = {
        "anchor": rs.integers(0, eng.shape.vocab, n),
        # a fifth of the requests within K + 2 positions of the context end
        "len": np.where(rs.random(n) < 0.2, rs.integers(n_ctx - K - 2, n_ctx + 1, n),
                        rs.integers(0, n_ctx + 1, n)),
        "emitted": rs.integers(1, n_max + 3, n),
        "done": (rs.random(n) < 0.2).astype(np.int64),
        "acc_sum": rs.integers(0, 100, n),
        "prop_sum": rs.integers(0, 100, n),
        "rounds": rs.integers(0, 50, n),
        "step": rs.integers(0, 50, n),
        "tok_sum": rs.integers(0, 100, n),
    }
    host = {k: v.astype(np.int32) for k, v in host.items()}
    host["hist"] = rs.integers(0, 20, K + 1).astype(np.int64)
    dev = {k: torch.as_tensor(v.copy(), device=eng.dev) for k, v in host.items()}
    st = eng.loop_state(*[dev[k] for k in ("anchor", "len", "emitted", "done", "acc_sum",
                                           "prop_sum", "rounds", "step", "tok_sum", "hist")])
    return host, dev, st


def _prepare_ref(h, n_max, n_ctx, table):
    R = n_max - h["emitted"].astype(np.int64)
    L = h["len"].astype(np.int64)
    k = np.maximum(0, np.minimum(np.minimum(K, R - 1), n_ctx - L - 1))
    ntok = np.where(h["done"] > 0, 0, k + 1)
    budget = np.maximum(R, 1)
    block = None
    if table is not None:
        cols = table.shape[1]
        pos = np.clip(L[:, None] + np.arange(1, K + 1)[None, :], 0, cols - 1)
        block = np.concatenate([h["anchor"][:, None], np.take_along_axis(table, pos, 1)], 1)
    return ntok, budget, block


@pytest.mark.parametrize("cols_short", [False, True])
def test_loop_prepare_against_the_rules(eng, cols_short):
    torch = eng.torch
    rs = np.random.default_rng(11 + int(cols_short))
    n, n_max, n_ctx = 300, 40, eng.shape.n_ctx
    h, d, st = _state(eng, rs, n, n_max)
    cols = 50 if cols_short else n_ctx + K + 2
    table = rs.integers(0, eng.shape.vocab, (n, cols)).astype(np.int32)
    d_table = torch.as_tensor(table, device=eng.dev)
    block = torch.full((n, K + 1), -7, dtype=torch.int32, device=eng.dev)
    ntok = torch.full((n,), -7, dtype=torch.int32, device=eng.dev)
    budget = torch.full((n,), -7, dtype=torch.int32, device=eng.dev)
    log(f"[loop] prepare n={n} K={K} n_max={n_max} table cols {cols}")
    eng.wf_loop_prepare(st, n, K, n_max, d_table, block, ntok, budget)
    r_ntok, r_budget, r_block = _prepare_ref(h, n_max, n_ctx, table)
    assert np.array_equal(ntok.cpu().numpy(), r_ntok)
    assert np.array_equal(budget.cpu().numpy(), r_budget)
    assert np.array_equal(block.cpu().numpy(), r_block)
    # without a table only n_tok and the budget are written
    block.fill_(-7)
    eng.wf_loop_prepare(st, n, K, n_max, None, block, ntok, budget)
    assert (block.cpu().numpy() == -7).all()
    assert np.array_equal(ntok.cpu().numpy(), r_ntok)
    # the state is only read
    for k, v in h.items():
        assert np.array_equal(d[k].cpu().numpy(), v), k
    # the edges occurred
    R = n_max - h["emitted"]
    assert (R <= 1).any() and (h["done"] > 0).any() and (n_ctx - h["len"] - 1 <= 0).any()


def test_loop_finish_against_the_rules(eng):
    torch = eng.torch
    rs = np.random.default_rng(23)
    n, n_max = 500, 40
    h, d, st = _state(eng, rs, n, n_max)
    ntok = rs.integers(0, K + 2, n).astype(np.int32)          # 0: inactive
    n_acc = np.array([rs.integers(0, max(t, 1)) for t in ntok], np.int32)
    nxt = rs.integers(-1, eng.shape.vocab, n).astype(np.int32)
    n_emit = (n_acc + (nxt >= 0)).astype(np.int32)
    dn = (rs.random(n) < 0.3).astype(np.int32)
    dev = [torch.as_tensor(a, device=eng.dev) for a in (ntok, n_acc, nxt, n_emit, dn)]
    log(f"[loop] finish n={n} K={K}")
    eng.wf_loop_finish(st, n, K, *dev)
    act = ntok > 0
    ref = {k: v.astype(np.int64).copy() for k, v in h.items()}
    ref["len"] += np.where(act, n_acc + 1, 0)
    ref["anchor"] = np.where(act & (nxt >= 0), nxt, ref["anchor"])
    ref["emitted"] += np.where(act, n_emit, 0)
    ref["tok_sum"] += np.where(act, n_emit, 0)
    ref["done"] = np.where(act & (dn > 0), 1, ref["done"])
    ref["acc_sum"] += np.where(act, n_acc, 0)
    ref["prop_sum"] += np.where(act, ntok - 1, 0)
    ref["rounds"] += act
    ref["step"] += act
    np.add.at(ref["hist"], np.clip(n_acc[act], 0, K), 1)
    for k in ref:
        assert np.array_equal(d[k].cpu().numpy().astype(np.int64), ref[k]), k
    assert (~act).any() and (nxt < 0).any()
