"""GPU tree verification ("Alignment Drift ...", App. E.3) through the C ABI
against the CPU oracle (oracle/tree.py).

* a one-branch tree gives the linear block's logits bit for bit;
* random trees (several requests, ragged node counts, a branch that follows
  the greedy continuation so that acceptance goes deep): every node's logits
  against the oracle's root-to-node path, argmax where the margin is clear;
* wf_accept_tree against the oracle's rule on the GPU's own argmax (integer
  logic: exact), then wf_rollback_tree and a linear block whose logits match
  the oracle request that was fed the accepted path linearly.
"""
import numpy as np
import pytest

from gpu_common import assert_argmax_where_clear, assert_logits_close, log
from oracle import decode as od
from oracle import model as om
from oracle import tree as ot
from synthetic import TINY, TURBO, WORKLOADS, make_encoder_out, make_prefixes, make_weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _engine(shape, wbits, max_batch, max_rows):
    from speculative_decoding_encoder_amd.binding import Engine
    return Engine(shape, wbits, max_batch=max_batch, max_rows=max_rows)


def _run(eng, fn, tokens, *arrays, logits=True):
    torch = eng.torch
    tokens = np.asarray(tokens, np.int32)
    n, T = tokens.shape
    am = torch.empty((n, T), dtype=torch.int32, device=eng.dev)
    lg = torch.empty((n, T, eng.shape.vocab), dtype=torch.float32, device=eng.dev) if logits else None
    fn(eng.i32(tokens), *[eng.i32(np.asarray(a, np.int32)) for a in arrays], am, lg)
    torch.cuda.synchronize()
    return am.cpu().numpy(), (lg.cpu().numpy() if logits else None)


def _prefill(eng, slots, prefixes):
    T = max(len(p) for p in prefixes)
    toks = np.zeros((len(slots), T), np.int32)
    for b, p in enumerate(prefixes):
        toks[b, :len(p)] = p
    lens = np.array([len(p) for p in prefixes], np.int32)
    am, _ = _run(eng, lambda t, nt, a, l: eng.wf_verify_block(eng.i32(slots), t, nt, a, l),
                 toks, lens, logits=False)
    eng.wf_rollback(eng.i32(slots), eng.i32(lens - 1))
    return [int(am[b, lens[b] - 1]) for b in range(len(slots))]


def _tree(g, greedy, T, V):
    """Node 0 the anchor; a greedy spine (node at depth k carries greedy[k])
    with random siblings and random subtrees hanging off it."""
    parents, toks, spine = [-1], [greedy[0]], [0]
    while len(parents) < T:
        k = len(spine)
        if k < len(greedy) and g.random() < 0.5:
            parents.append(spine[-1])
            toks.append(greedy[k])
            spine.append(len(parents) - 1)
        else:
            parents.append(int(g.integers(0, len(parents))))
            toks.append(int(g.integers(0, V - 1)))
    return parents, toks


def _greedy(m, req, L, anchor, n):
    tmp = ot.copy_request(m, req)
    out = [anchor]
    for i in range(n):
        out.append(od.argmax_lowest(m.rows(tmp, [out[-1]], L + i)[0]))
    return out


@pytest.mark.parametrize("shape_name", ["tiny", "turbo"])
def test_one_branch_tree_equals_linear_block_bitwise(torch_cuda, shape_name):
    shape = TINY if shape_name == "tiny" else TURBO
    wl = WORKLOADS[0] if shape_name == "tiny" else WORKLOADS[2]
    wbits = make_weights(shape, wl.cfg_id, ln_random=shape_name == "tiny")
    prefixes = make_prefixes(wl, 2)
    encs = np.stack([make_encoder_out(shape, wl.cfg_id, r) for r in range(2)])
    blocks = np.random.default_rng(7).integers(0, shape.vocab - 1, (2, 9)).astype(np.int32)
    chain = np.tile(np.arange(-1, 8, dtype=np.int32), (2, 1))
    outs = []
    for tree in (False, True):
        eng = _engine(shape, wbits, max_batch=2, max_rows=2 * 224)
        slots = [0, 1]
        eng.wf_encode_kv(eng.i32(slots), eng.bf16(encs))
        anchors = _prefill(eng, slots, prefixes)
        blk = blocks.copy()
        blk[:, 0] = anchors
        if tree:
            am, lg = _run(eng, lambda t, p, nt, a, l: eng.wf_verify_tree(eng.i32(slots), t, p, nt, a, l),
                          blk, chain, [9, 6])
        else:
            am, lg = _run(eng, lambda t, nt, a, l: eng.wf_verify_block(eng.i32(slots), t, nt, a, l),
                          blk, [9, 6])
        err, _ = eng.wf_device_state()
        assert (err == 0).all()
        outs.append((am, lg))
        eng.close()
    assert np.array_equal(outs[0][0], outs[1][0])
    # live rows (padding rows sit at the root's position in a tree)
    for b, k in enumerate([9, 6]):
        assert np.array_equal(outs[0][1][b, :k].view(np.uint32), outs[1][1][b, :k].view(np.uint32))


@pytest.mark.parametrize("shape_name,T", [("tiny", 14), ("tiny", 40), ("turbo", 11)])
def test_random_trees_against_the_oracle(torch_cuda, shape_name, T):
    """T = 40: three 16-row tiles, so the ancestor masks of later tiles
    reach back into earlier ones."""
    shape = TINY if shape_name == "tiny" else TURBO
    wl = WORKLOADS[0] if shape_name == "tiny" else WORKLOADS[2]
    B = 3
    wbits = make_weights(shape, wl.cfg_id, ln_random=shape_name == "tiny")
    prefixes = [p[:40] for p in make_prefixes(wl, B)]
    encs = np.stack([make_encoder_out(shape, wl.cfg_id, 10 + r) for r in range(B)])
    m = om.Model(shape, wbits)
    eng = _engine(shape, wbits, max_batch=B, max_rows=B * 64)
    slots = list(range(B))
    eng.wf_encode_kv(eng.i32(slots), eng.bf16(encs))
    anchors = _prefill(eng, slots, prefixes)
    g = np.random.default_rng(21)
    n_tok = [T, T - 3, T - 5]
    parents = np.zeros((B, T), np.int32)
    toks = np.zeros((B, T), np.int32)
    reqs, refs = [], []
    for b in range(B):
        req = m.new_request(encs[b])
        L = len(prefixes[b])
        m.rows(req, prefixes[b], 0)
        gr = _greedy(m, req, L, anchors[b], 6 if T < 20 else 12)
        p, t = _tree(g, gr, n_tok[b], shape.vocab)
        parents[b, :n_tok[b]] = p
        toks[b, :n_tok[b]] = t
        parents[b, n_tok[b]:] = 0
        reqs.append(req)
        refs.append(ot.tree_rows(m, req, t, p, L))
    log(f"tree {shape_name}: GPU verify of {B} trees")
    am, lg = _run(eng, lambda t, p, nt, a, l: eng.wf_verify_tree(eng.i32(slots), t, p, nt, a, l),
                  toks, parents, n_tok)
    for b in range(B):
        k = n_tok[b]
        assert_logits_close(lg[b, :k], refs[b], what=f"tree {shape_name} req {b}")
        assert_argmax_where_clear(am[b, :k], refs[b], what=f"tree {shape_name} req {b}")
        assert (am[b, k:] == -1).all()
    # acceptance on the GPU's own argmax: exact
    torch = eng.torch
    budget = [200, 3, 200]
    outs = [torch.empty(B, dtype=torch.int32, device=eng.dev) for _ in range(4)]
    path = torch.empty((B, T), dtype=torch.int32, device=eng.dev)
    eng.wf_accept_tree(eng.i32(toks), eng.i32(parents), eng.i32(n_tok), eng.i32(budget),
                       eng.i32(am), path, *outs)
    n_acc, nxt, n_emit, done = [o.cpu().numpy() for o in outs]
    path = path.cpu().numpy()
    for b in range(B):
        k = n_tok[b]
        a, p, em, c, dn = ot.tree_accept(toks[b, :k], parents[b, :k], am[b, :k], shape.eos_id,
                                         budget[b])
        assert n_acc[b] == a and list(path[b, :a + 1]) == p and (path[b, a + 1:] == -1).all()
        assert n_emit[b] == len(em) and nxt[b] == (c if c is not None else -1) and done[b] == dn
        log(f"tree {shape_name} req {b}: accepted {a} of depth "
            f"{max(ot.depths(list(parents[b, :k])))}, path {p}, next {nxt[b]}")
    assert n_acc.max() >= 2
    # rollback keeps the path; a linear block then matches the oracle request
    # that was fed the accepted path
    eng.wf_rollback_tree(eng.i32(slots), eng.torch.from_numpy(path).to(eng.dev), outs[0])
    err, lens = eng.wf_device_state()
    assert (err == 0).all()
    for b in range(B):
        assert lens[b] == len(prefixes[b]) + 1 + n_acc[b]
    nxt_blk = g.integers(0, shape.vocab - 1, (B, 5)).astype(np.int32)
    nxt_blk[:, 0] = np.maximum(nxt, 0)
    live = [b for b in range(B) if nxt[b] >= 0]        # a request that ended on EOS stops
    assert len(live) >= 2
    am2, lg2 = _run(eng, lambda t, nt, a, l: eng.wf_verify_block(eng.i32(slots), t, nt, a, l),
                    nxt_blk, [5 if b in live else 0 for b in range(B)])
    for b in live:
        L = len(prefixes[b])
        m.rows(reqs[b], toks[b, path[b, :n_acc[b] + 1]], L)
        ref = m.rows(reqs[b], nxt_blk[b], L + 1 + n_acc[b])
        assert_logits_close(lg2[b], ref, what=f"after tree rollback req {b}")
        assert_argmax_where_clear(am2[b], ref, what=f"after tree rollback req {b}")
    eng.close()


def test_bad_parents_flag_the_slot(torch_cuda):
    wl = WORKLOADS[0]
    wbits = make_weights(TINY, wl.cfg_id)
    eng = _engine(TINY, wbits, max_batch=2, max_rows=64)
    slots = [0, 1]
    eng.wf_encode_kv(eng.i32(slots), eng.bf16(np.stack([make_encoder_out(TINY, wl.cfg_id, r)
                                                        for r in range(2)])))
    toks = np.ones((2, 4), np.int32)
    parents = np.array([[-1, 0, 2, 1], [-1, 0, 1, 1]], np.int32)   # request 0: parents[2] = 2
    am, _ = _run(eng, lambda t, p, nt, a, l: eng.wf_verify_tree(eng.i32(slots), t, p, nt, a, l),
                 toks, parents, [4, 4], logits=False)
    err, lens = eng.wf_device_state()
    assert err[0] & 2 and err[1] == 0
    assert (am[0] == -1).all() and (am[1] >= 0).all()
    from speculative_decoding_encoder_amd.binding import WFError
    with pytest.raises(WFError):
        _run(eng, lambda t, p, nt, a, l: eng.wf_verify_tree(eng.i32(slots), t, p, nt, a, l),
             np.ones((2, 65), np.int32), np.zeros((2, 65), np.int32), [4, 4], logits=False)
    eng.close()
