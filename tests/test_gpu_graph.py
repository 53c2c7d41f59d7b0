"""Graph replay of the verify step (the way bench.py times it): the step
(wf_verify_block, wf_rollback, wf_truncate) captured once in a HIP graph and
replayed several times, with eager work and synchronisations between the
replays, gives every replay the eager pass's argmax and logits bit for bit.
The kernels re-arm their own cross-workgroup counters, so nothing needs a
memset inside the graph. Batch 4 merges the cross-attention chunk groups
through scratch; batch 32 runs the tall-block GEMMs and fc2's K-group
handoff.
"""
import numpy as np
import pytest

from gpu_common import log
from synthetic import TURBO, WORKLOADS, make_encoder_out, make_prefixes, make_weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.mark.parametrize("B", [4, 32])
def test_graph_replays_equal_the_eager_step(torch_cuda, B):
    from speculative_decoding_encoder_amd.binding import Engine
    torch = torch_cuda
    wl = WORKLOADS[2]
    shape = TURBO
    wbits = make_weights(shape, wl.cfg_id)
    prefixes = make_prefixes(wl, B)
    encs = np.stack([make_encoder_out(shape, wl.cfg_id, r) for r in range(B)])
    eng = Engine(shape, wbits, max_batch=B, max_rows=B * 224)
    slots = eng.i32(list(range(B)))
    eng.wf_encode_kv(slots, eng.bf16(encs))
    T = max(len(p) for p in prefixes)
    toks = np.zeros((B, T), np.int32)
    for b, p in enumerate(prefixes):
        toks[b, :len(p)] = p
    lens = np.array([len(p) for p in prefixes], np.int32)
    am0 = torch.empty((B, T), dtype=torch.int32, device=eng.dev)
    eng.wf_verify_block(slots, eng.i32(toks), eng.i32(lens), am0)
    eng.wf_rollback(slots, eng.i32(lens - 1))
    blocks = np.random.default_rng(3).integers(0, shape.vocab - 1, (B, 9)).astype(np.int32)
    blocks[:, 0] = am0.cpu().numpy()[np.arange(B), lens - 1]
    d_blocks, d_ntok = eng.i32(blocks), eng.i32([9] * B)
    d_zero, d_lens = eng.i32([0] * B), eng.i32(lens)
    am = torch.empty((B, 9), dtype=torch.int32, device=eng.dev)
    lg = torch.empty((B, 9, shape.vocab), dtype=torch.float32, device=eng.dev)

    def step():
        eng.wf_verify_block(slots, d_blocks, d_ntok, am, lg)
        eng.wf_rollback(slots, d_zero)
        eng.wf_truncate(slots, d_lens)

    step()
    torch.cuda.synchronize()
    ref_am, ref_lg = am.cpu().numpy(), lg.cpu().numpy()
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        am.fill_(-5)
        lg.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(am.cpu().numpy(), ref_am), rep
        assert np.array_equal(lg.cpu().numpy().view(np.uint32), ref_lg.view(np.uint32)), rep
        err, ln = eng.wf_device_state()
        assert (err == 0).all() and np.array_equal(ln[:B], lens), rep
        step()                                   # eager work between the replays
        torch.cuda.synchronize()
        assert np.array_equal(am.cpu().numpy(), ref_am), rep
    log(f"graph B={B}: 4 replays equal the eager step")
    del graph
    eng.close()
