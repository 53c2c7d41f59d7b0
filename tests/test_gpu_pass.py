"""The persistent verify pass (one launch for every layer and the LM head)
against the multi-kernel path and the oracle.

* every logit and argmax of a block equals the multi-kernel path bit for
  bit, at 1, 4, 32 and 96 requests (the three tile classes, M = 9 to 864
  rows, one to nine row blocks), with ragged prefixes and shuffled pages,
  and two sampled requests match the oracle within 2e-2;
* a ragged block beside an inactive request (its rows give -1, its cache
  keeps its length);
* the drafter's history taps written inside the pass: the drafter's logits
  after a round equal those of the multi-kernel path bit for bit;
* the wait limit: with a limit of 0 the pass aborts, every wait ends, the
  kernel drains, the requests' error words carry WF_DERR_TIMEOUT, and after
  wf_reset the next pass is exact again;
* the task trace covers every task of the schedule.
"""
import numpy as np
import pytest

from gpu_common import assert_argmax_where_clear, assert_logits_close, log
from oracle import model as om
from synthetic import (LARGE_V3, TURBO, WORKLOADS, make_drafter_weights, make_encoder_out,
                       make_prefixes, make_weights)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _verify(eng, slots, tokens, n_tok, logits=True):
    torch = eng.torch
    tokens = np.asarray(tokens, np.int32)
    n, T = tokens.shape
    am = torch.empty((n, T), dtype=torch.int32, device=eng.dev)
    lg = torch.empty((n, T, eng.shape.vocab), dtype=torch.float32, device=eng.dev) if logits else None
    eng.wf_verify_block(eng.i32(slots), eng.i32(tokens), eng.i32(n_tok), am, lg)
    torch.cuda.synchronize()
    return am.cpu().numpy(), (lg.cpu().numpy() if logits else None)


def _setup(B, seed=0, drafter=False):
    """Turbo engine on the persistent pass (not the library's default)."""
    from speculative_decoding_encoder_amd.binding import Engine, WF_OPT_PERSISTENT
    wl = WORKLOADS[2]
    shape = TURBO
    wbits = make_weights(shape, wl.cfg_id)
    encs = np.stack([make_encoder_out(shape, wl.cfg_id, r) for r in range(B)])
    prefixes = [p[:120] for p in make_prefixes(wl, B)]
    pps = shape.n_ctx // 16
    perm = np.random.default_rng(7 + seed).permutation(B * pps).astype(np.int32)
    eng = Engine(shape, wbits, max_batch=B, max_rows=max(B * 9, 64), page_table=perm.reshape(B, pps))
    eng.wf_set_option(WF_OPT_PERSISTENT, 1)
    slots = list(range(B))
    eng.wf_encode_kv(eng.i32(slots), eng.bf16(encs))
    return wl, shape, wbits, encs, prefixes, eng, slots


def _prefill(eng, slots, prefixes):
    """Prompts one request at a time (64-row blocks at most, so any engine
    takes them), the whole prompt kept."""
    for b, p in zip(slots, prefixes):
        for s in range(0, len(p), 64):
            piece = p[s:s + 64]
            _verify(eng, [b], piece[None], [len(piece)], logits=False)
            eng.wf_rollback(eng.i32([b]), eng.i32([len(piece) - 1]))


def _both_paths(eng, slots, blocks, n_tok, lens):
    """The block through the persistent pass, then (same state: rollback of
    the pending rows and a truncate back) through the multi-kernel path."""
    from speculative_decoding_encoder_amd.binding import WF_OPT_PERSISTENT
    eng.wf_set_option(WF_OPT_PERSISTENT, 1)
    am1, lg1 = _verify(eng, slots, blocks, n_tok)
    sched = eng.wf_pass_schedule()
    eng.wf_rollback(eng.i32(slots), eng.i32(np.zeros(len(slots), np.int32)))
    eng.wf_truncate(eng.i32(slots), eng.i32(lens))
    eng.wf_set_option(WF_OPT_PERSISTENT, 0)
    am2, lg2 = _verify(eng, slots, blocks, n_tok)
    eng.wf_rollback(eng.i32(slots), eng.i32(np.zeros(len(slots), np.int32)))
    eng.wf_truncate(eng.i32(slots), eng.i32(lens))
    eng.wf_set_option(WF_OPT_PERSISTENT, 1)
    err, _ = eng.wf_device_state()
    assert (err == 0).all(), err
    return am1, lg1, am2, lg2, sched


@pytest.mark.parametrize("B", [1, 4, 32, 96])
def test_pass_equals_multikernel_bitwise_and_oracle(torch_cuda, B):
    wl, shape, wbits, encs, prefixes, eng, slots = _setup(B)
    log(f"pass B={B}: prefill of {B} ragged prompts")
    _prefill(eng, slots, prefixes)
    lens = np.array([len(p) for p in prefixes], np.int32)
    blocks = np.random.default_rng(100 + B).integers(0, shape.vocab - 1, (B, 9)).astype(np.int32)
    am1, lg1, am2, lg2, sched = _both_paths(eng, slots, blocks, [9] * B, lens)
    log(f"pass B={B}: {sched['total']} tasks on {sched['grid']} workgroups")
    assert sched["total"] > 0 and sched["layers"] == shape.n_layers
    assert np.array_equal(am1, am2)
    assert np.array_equal(lg1.view(np.uint32), lg2.view(np.uint32))
    m = om.Model(shape, wbits)
    for b in sorted({0, B - 1}):
        req = m.new_request(encs[b])
        m.rows(req, prefixes[b], 0)
        ref = m.rows(req, blocks[b], int(lens[b]))
        assert_logits_close(lg1[b], ref, what=f"pass B={B} request {b}")
        assert_argmax_where_clear(am1[b], ref, what=f"pass B={B} request {b}")
    eng.close()


def test_pass_ragged_and_inactive_requests(torch_cuda):
    """Request 1 inactive (n_tok = 0), request 2 with 5 of 9 rows: the same
    bits on both paths, -1 past n_tok, lengths after rollback."""
    B = 20
    wl, shape, wbits, encs, prefixes, eng, slots = _setup(B, seed=3)
    _prefill(eng, slots, prefixes)
    lens = np.array([len(p) for p in prefixes], np.int32)
    blocks = np.random.default_rng(5).integers(0, shape.vocab - 1, (B, 9)).astype(np.int32)
    n_tok = np.full(B, 9, np.int32)
    n_tok[1] = 0
    n_tok[2] = 5
    am1, lg1, am2, lg2, _ = _both_paths(eng, slots, blocks, n_tok, lens)
    assert np.array_equal(am1, am2)
    assert np.array_equal(lg1[n_tok > 0].view(np.uint32), lg2[n_tok > 0].view(np.uint32))
    assert (am1[1] == -1).all() and (am1[2, 5:] == -1).all()
    m = om.Model(shape, wbits)
    req = m.new_request(encs[2])
    m.rows(req, prefixes[2], 0)
    ref = m.rows(req, blocks[2, :5], int(lens[2]))
    assert_logits_close(lg1[2, :5], ref, what="pass ragged request (5 of 9)")
    _verify(eng, slots, blocks, n_tok, logits=False)
    eng.wf_rollback(eng.i32(slots), eng.i32(np.maximum(n_tok - 1, 0)))
    err, ln = eng.wf_device_state()
    assert (err == 0).all()
    assert ln[1] == lens[1] and ln[2] == lens[2] + 5 and ln[0] == lens[0] + 9
    eng.close()


def test_pass_timeout_aborts_and_flags(torch_cuda):
    """A wait limit of 0: the first unmet wait aborts the pass; every other
    wait ends on the abort flag and the kernel drains. The requests' error
    words carry WF_DERR_TIMEOUT; after wf_reset and a normal limit the
    pass is exact again."""
    from speculative_decoding_encoder_amd.binding import WF_DERR_TIMEOUT, WF_OPT_PASS_TIMEOUT_US
    B = 8
    wl, shape, wbits, encs, prefixes, eng, slots = _setup(B, seed=5)
    _prefill(eng, slots, prefixes)
    lens = np.array([len(p) for p in prefixes], np.int32)
    blocks = np.random.default_rng(9).integers(0, shape.vocab - 1, (B, 9)).astype(np.int32)
    eng.wf_set_option(WF_OPT_PASS_TIMEOUT_US, 0)
    _verify(eng, slots, blocks, [9] * B, logits=False)
    err, _ = eng.wf_device_state()
    log(f"pass timeout: error words {err[:B]}")
    assert ((err[:B] & WF_DERR_TIMEOUT) != 0).all()
    eng.wf_set_option(WF_OPT_PASS_TIMEOUT_US, 500000)
    eng.wf_reset(eng.i32(slots))
    _prefill(eng, slots, prefixes)
    am1, lg1, am2, lg2, _ = _both_paths(eng, slots, blocks, [9] * B, lens)
    assert np.array_equal(lg1.view(np.uint32), lg2.view(np.uint32))
    eng.close()


def test_pass_trace_covers_the_schedule(torch_cuda):
    torch = torch_cuda
    B = 32
    wl, shape, wbits, encs, prefixes, eng, slots = _setup(B, seed=6)
    _prefill(eng, slots, prefixes)
    blocks = np.random.default_rng(3).integers(0, shape.vocab - 1, (B, 9)).astype(np.int32)
    buf = torch.zeros((20000, 4), dtype=torch.int64, device=eng.dev)
    eng.wf_set_trace(buf)
    _verify(eng, slots, blocks, [9] * B, logits=False)
    eng.wf_set_trace(None)
    sched = eng.wf_pass_schedule()
    assert 0 < sched["total"] <= buf.shape[0]
    tr = buf.cpu().numpy()[:sched["total"]]
    assert (tr[:, 0] > 0).all() and (tr[:, 1] >= tr[:, 0]).all() and (tr[:, 2] >= tr[:, 1]).all()
    span = (tr[:, 2].max() - tr[:, 0].min()) / 100.0
    log(f"pass trace: {sched['total']} tasks, {span:.1f} us from first start to last end")
    eng.close()


def test_pass_drafter_history_bitwise(torch_cuda):
    """32-layer large-v3 with the 2-layer drafter and taps after blocks 1, 8,
    15, 22, 29 at 3 requests: a verify round on each path, the same rollback,
    then the drafter pass: its logits (which read the history written from
    the taps of the pass) equal bit for bit."""
    from speculative_decoding_encoder_amd.binding import Engine, WF_OPT_PERSISTENT
    from synthetic import DRAFTER_TAPS
    wl = WORKLOADS[3]
    shape = LARGE_V3
    B = 3
    tw = make_weights(shape, wl.cfg_id)
    dw = make_drafter_weights(shape, wl.cfg_id)
    encs = np.stack([make_encoder_out(shape, wl.cfg_id, r) for r in range(B)])
    prefixes = [p[:30] for p in make_prefixes(wl, B)]
    rng = np.random.default_rng(21)
    blocks = rng.integers(0, shape.vocab - 1, (B, 9)).astype(np.int32)
    out = []
    for persistent in (1, 0):
        eng = Engine(shape, tw, max_batch=B, max_rows=64, drafter_bits=dw, taps=DRAFTER_TAPS)
        eng.wf_set_option(WF_OPT_PERSISTENT, persistent)
        slots = list(range(B))
        eng.wf_encode_kv(eng.i32(slots), eng.bf16(encs))
        _prefill(eng, slots, prefixes)
        am, lg = _verify(eng, slots, blocks, [9] * B)
        eng.wf_rollback(eng.i32(slots), eng.i32([3, 0, 8]))
        anchors = [int(am[0, 3]), int(am[1, 0]), int(am[2, 8])]
        torch = eng.torch
        blk = torch.empty((B, 9), dtype=torch.int32, device=eng.dev)
        dlg = torch.empty((B, 9, shape.vocab), dtype=torch.float32, device=eng.dev)
        eng.wf_draft(eng.i32(slots), eng.i32(anchors), 8, blk, dlg)
        torch.cuda.synchronize()
        err, _ = eng.wf_device_state()
        assert (err == 0).all()
        out.append((lg, blk.cpu().numpy(), dlg.cpu().numpy()))
        eng.close()
    assert np.array_equal(out[0][0].view(np.uint32), out[1][0].view(np.uint32))
    assert np.array_equal(out[0][1], out[1][1])
    assert np.array_equal(out[0][2].view(np.uint32), out[1][2].view(np.uint32))
