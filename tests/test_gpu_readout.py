"""GPU anchor readout ("Alignment Drift ...", Verification-Attention
Correction and App. D.2) through the C ABI against the oracle
(oracle/readout.py): the peak frame of the head-averaged cross-attention at
one layer, per verify row.

The chosen layer's cross Q and K weights are scaled by a power of two
(exact in bf16) so that attention is peaked: with the random-init weights
it is nearly uniform and every peak a near-tie. At the large-v3 width the
heads also share head 0's projections (20 random heads peak at 20 frames,
so their average has several near-equal peaks); the tiny model keeps
distinct heads. Peaks must match where the
oracle's top two are apart by more than 1% of the top; elsewhere the GPU's
frame must be within 1% of the oracle's top. Rows past n_tok give -1, the
logits do not change, and the readout turns off.
"""
import numpy as np
import pytest

from gpu_common import log
from oracle import model as om
from oracle import readout as orr
from synthetic import TINY, TURBO, WORKLOADS, make_encoder_out, make_prefixes, make_weights

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def _same_heads(bits: np.ndarray, hd: int) -> np.ndarray:
    """Every head's rows of a [d, d] projection replaced by head 0's."""
    out = bits.copy()
    for h in range(1, bits.shape[0] // hd):
        out[h * hd:(h + 1) * hd] = bits[:hd]
    return out


def _scale_bf16(bits: np.ndarray, k: int) -> np.ndarray:
    """bf16 bits times 2^k (exponent shift; the values here are normal)."""
    b = bits.astype(np.int32)
    nz = (b & 0x7fff) != 0
    return np.where(nz, b + (k << 7), b).astype(bits.dtype)


@pytest.mark.parametrize("shape_name,layer,T", [("tiny", 1, 9), ("tiny", 0, 20), ("turbo", 2, 9)])
def test_readout_against_the_oracle(torch_cuda, shape_name, layer, T):
    from speculative_decoding_encoder_amd.binding import Engine
    torch = torch_cuda
    shape = TINY if shape_name == "tiny" else TURBO
    wl = WORKLOADS[0] if shape_name == "tiny" else WORKLOADS[2]
    wbits = make_weights(shape, wl.cfg_id, ln_random=shape_name == "tiny")
    for name in ("wqc", "wkc"):
        w = _scale_bf16(wbits[f"L{layer}.{name}"], 3)
        if shape_name == "turbo":
            # 20 random heads peak at 20 different frames and their average at
            # several near-equal ones: give every head head 0's projections
            w = _same_heads(w, shape.d_model // shape.n_heads)
        wbits[f"L{layer}.{name}"] = w
    B = 3
    prefixes = [p[:40] for p in make_prefixes(wl, B)]
    encs = np.stack([make_encoder_out(shape, wl.cfg_id, 20 + r) for r in range(B)])
    eng = Engine(shape, wbits, max_batch=B, max_rows=B * 64)
    slots = list(range(B))
    eng.wf_encode_kv(eng.i32(slots), eng.bf16(encs))
    Tp = max(len(p) for p in prefixes)
    toks = np.zeros((B, Tp), np.int32)
    for b, p in enumerate(prefixes):
        toks[b, :len(p)] = p
    lens = np.array([len(p) for p in prefixes], np.int32)
    am = torch.empty((B, Tp), dtype=torch.int32, device=eng.dev)
    eng.wf_verify_block(eng.i32(slots), eng.i32(toks), eng.i32(lens), am)
    eng.wf_rollback(eng.i32(slots), eng.i32(lens - 1))
    blocks = np.random.default_rng(5).integers(0, shape.vocab - 1, (B, T)).astype(np.int32)
    blocks[:, 0] = am.cpu().numpy()[np.arange(B), lens - 1]
    n_tok = [T, 5, T]
    frame = torch.full((B * 64,), -7, dtype=torch.int32, device=eng.dev)
    outs = []
    for on in (True, False):
        eng.wf_set_readout(layer if on else -1, frame if on else None)
        am2 = torch.empty((B, T), dtype=torch.int32, device=eng.dev)
        lg = torch.empty((B, T, shape.vocab), dtype=torch.float32, device=eng.dev)
        eng.wf_verify_block(eng.i32(slots), eng.i32(blocks), eng.i32(n_tok), am2, lg)
        torch.cuda.synchronize()
        outs.append((am2.cpu().numpy(), lg.cpu().numpy(), frame.cpu().numpy().copy()))
        eng.wf_rollback(eng.i32(slots), eng.i32([0] * B))
        eng.wf_truncate(eng.i32(slots), eng.i32(lens))
        err, _ = eng.wf_device_state()
        assert (err == 0).all()
    assert np.array_equal(outs[0][1].view(np.uint32), outs[1][1].view(np.uint32))
    assert np.array_equal(outs[0][2], outs[1][2])          # off: nothing written
    got = outs[0][2][:B * T].reshape(B, T)
    assert (outs[0][2][B * T:] == -7).all()
    m = om.Model(shape, wbits)
    clear = total = 0
    for b in range(B):
        req = m.new_request(encs[b])
        m.rows(req, prefixes[b], 0)
        k = n_tok[b]
        peaks, pbar = orr.anchor_frames(m, req, blocks[b, :k], int(lens[b]), layer)
        assert (got[b, k:] == -1).all()
        for i in range(k):
            top = np.sort(pbar[i])[-2:]
            f = int(got[b, i])
            assert 0 <= f < shape.n_frames
            assert pbar[i, f] >= top[1] * 0.99, (b, i, f, int(peaks[i]), pbar[i, f], top)
            if top[1] - top[0] > 0.01 * top[1]:
                clear += 1
                assert f == peaks[i], (b, i, f, int(peaks[i]))
            total += 1
    log(f"readout {shape_name} layer {layer}: {clear} of {total} rows with a clear peak")
    assert clear >= total // 2
    eng.close()
