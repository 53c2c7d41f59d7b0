"""The no-allocation engine (wf_create_static) against the ordinary one.

An engine made by wf_create_static runs in the library's own static device
workspace. With the same configuration, weights and inputs it must give the
results of an engine over a caller-supplied workspace (wf_create) bit for
bit: the kernels and their launches are the same. Two static engines are
made in a row, the second with a smaller configuration (fewer requests and
rows) over the array the first one left behind; each is compared with its
own ordinary twin on a prefill, a verify block and the greedy acceptance.
Also: a configuration whose workspace exceeds the array is refused, and a
second static engine on the device is refused while the first is alive.
"""
import numpy as np
import pytest

from synthetic import TURBO, make_encoder_out, make_weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


@pytest.fixture(scope="module")
def turbo_inputs(torch_cuda):
    wbits = make_weights(TURBO, 2)
    encs = np.stack([make_encoder_out(TURBO, 2, r) for r in range(4)])
    return wbits, encs


def _round(eng, encs, lens, seed):
    """Prefill prompts of the given lengths, then verify one block of 9 per
    request and accept it greedily; returns every output as numpy arrays."""
    torch = eng.torch
    B = len(lens)
    rng = np.random.default_rng(seed)
    V, eos = eng.shape.vocab, eng.shape.eos_id
    slots = eng.i32(list(range(B)))
    eng.wf_reset(slots)
    eng.wf_encode_kv(slots, eng.bf16(encs[:B]))
    T0 = int(max(lens))
    prompt = rng.integers(0, V, (B, T0)).astype(np.int32)
    prompt[prompt == eos] = 0
    am0 = torch.empty((B, T0), dtype=torch.int32, device=eng.dev)
    lg0 = torch.empty((B, T0, V), dtype=torch.float32, device=eng.dev)
    n0 = np.asarray(lens, np.int32)
    eng.wf_verify_block(slots, eng.i32(prompt), eng.i32(n0), am0, lg0)
    eng.wf_rollback(slots, eng.i32(n0 - 1))
    a0 = am0.cpu().numpy()
    block = rng.integers(0, V, (B, 9)).astype(np.int32)
    block[block == eos] = 0
    block[:, 0] = [a0[b, n0[b] - 1] for b in range(B)]
    block[:, 1] = block[:, 0]        # some candidates repeat the anchor
    am1 = torch.empty((B, 9), dtype=torch.int32, device=eng.dev)
    lg1 = torch.empty((B, 9, V), dtype=torch.float32, device=eng.dev)
    d_block, d_ntok = eng.i32(block), eng.i32(np.full(B, 9, np.int32))
    eng.wf_verify_block(slots, d_block, d_ntok, am1, lg1)
    outs = [torch.empty(B, dtype=torch.int32, device=eng.dev) for _ in range(4)]
    eng.wf_accept(d_block, d_ntok, eng.i32(np.full(B, 50, np.int32)), am1, *outs)
    eng.wf_rollback(slots, outs[0])
    torch.cuda.synchronize()
    err, ln = eng.wf_device_state()
    return dict(am0=a0, lg0=lg0.cpu().numpy(), am1=am1.cpu().numpy(), lg1=lg1.cpu().numpy(),
                acc=[o.cpu().numpy() for o in outs], err=err, len=ln)


def _compare(ref, got, what):
    for k in ("am0", "am1", "len", "err"):
        assert np.array_equal(ref[k], got[k]), f"{what}: {k} differs"
    for k in ("lg0", "lg1"):
        assert np.array_equal(ref[k].view(np.uint32), got[k].view(np.uint32)), \
            f"{what}: {k} differs (max {np.abs(ref[k] - got[k]).max():.3e})"
    for i, (x, y) in enumerate(zip(ref["acc"], got["acc"])):
        assert np.array_equal(x, y), f"{what}: accept output {i} differs"
    assert (got["err"] == 0).all()


@pytest.mark.parametrize("B,lens", [(4, [5, 8, 3, 7])])
def test_static_engine_equals_workspace_engine_twice(torch_cuda, turbo_inputs, B, lens):
    from speculative_decoding_encoder_amd.binding import (WF_STATIC_WORKSPACE_BYTES, Engine,
                                                          workspace_bytes, make_config)
    wbits, encs = turbo_inputs
    # first engine: 4 requests, 36 rows; second: 2 requests, 18 rows
    for step, (nb, nl) in enumerate([(B, lens), (2, [6, 4])]):
        rows = nb * 9
        assert workspace_bytes(make_config(TURBO, nb, rows)) <= WF_STATIC_WORKSPACE_BYTES
        print(f"[no-alloc] call {step}: turbo, {nb} requests, max_rows {rows}", flush=True)
        ref_eng = Engine(TURBO, wbits, max_batch=nb, max_rows=rows)
        ref = _round(ref_eng, encs, nl, seed=10 + step)
        ref_eng.close()
        st_eng = Engine(TURBO, wbits, max_batch=nb, max_rows=rows, static_workspace=True)
        try:
            got = _round(st_eng, encs, nl, seed=10 + step)
        finally:
            st_eng.close()
        _compare(ref, got, f"call {step}")


def test_static_engine_limits(torch_cuda, turbo_inputs):
    from speculative_decoding_encoder_amd.binding import Engine, WFError
    wbits, _ = turbo_inputs
    with pytest.raises(WFError, match="static"):
        Engine(TURBO, wbits, max_batch=32, max_rows=32 * 200, static_workspace=True)
    first = Engine(TURBO, wbits, max_batch=2, max_rows=18, static_workspace=True)
    try:
        with pytest.raises(WFError, match="status -6"):
            Engine(TURBO, wbits, max_batch=2, max_rows=18, static_workspace=True)
    finally:
        first.close()
    # released: a new one may take the array
    again = Engine(TURBO, wbits, max_batch=2, max_rows=18, static_workspace=True)
    again.close()
