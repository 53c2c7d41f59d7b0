"""CPU checks of the C ABI library: it loads, exports every function that
include/wf.h declares, sizes its buffers, and rejects bad arguments before
touching a device."""
import ctypes

import pytest

from speculative_decoding_encoder_amd import binding as B
from synthetic import LARGE_V3, TINY, TURBO


@pytest.fixture(scope="module")
def lib():
    return B.load()


def test_exports_every_declared_function(lib):
    names = B.header_functions()
    assert {"wf_encode_kv", "wf_verify_block", "wf_accept", "wf_rollback"} <= set(names)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_buffer_sizes(lib):
    c = B.make_config(LARGE_V3, 32, 32 * 9)
    kv = lib.wf_kv_pool_bytes(ctypes.byref(c))
    # [layers][pages][K|V][heads][16][64] fp16
    assert kv == 32 * (32 * 28) * 2 * 20 * 16 * 64 * 2
    xkv = lib.wf_xkv_pool_bytes(ctypes.byref(c))
    assert xkv == 32 * 32 * 2 * 20 * 1504 * 64 * 2
    assert lib.wf_workspace_bytes(ctypes.byref(c)) > 0
    t = B.make_config(TURBO, 1, 9)
    assert lib.wf_kv_pool_bytes(ctypes.byref(t)) == 4 * 28 * 2 * 20 * 16 * 64 * 2


@pytest.mark.parametrize("field,value", [("head_dim", 32), ("page_size", 8), ("n_ctx", 100),
                                         ("d_ffn", 100), ("max_batch", 0), ("eos_id", 512)])
def test_bad_configs_rejected(lib, field, value):
    c = B.make_config(TINY, 2, 64)
    setattr(c, field, value)
    assert lib.wf_workspace_bytes(ctypes.byref(c)) == 0


def test_create_rejects_null_arguments(lib):
    c = B.make_config(TINY, 2, 64)
    h = ctypes.c_void_p()
    w = B.Weights()
    st = lib.wf_create(ctypes.byref(c), ctypes.byref(w), None, 0, None, 0, None, None, 0,
                       ctypes.byref(h))
    assert st == -1 and b"null" in lib.wf_last_error()
    assert lib.wf_verify_block(None, 1, None, None, 1, None, None, None, None) == -1
    assert lib.wf_accept(None, 1, None, 1, None, None, None, None, None, None, 0.0, 0,
                         None, None, None, None, None, None, None) == -1
    assert lib.wf_rollback(None, 1, None, None, None) == -1
    assert lib.wf_encode_kv(None, 1, None, None, None) == -1


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        B.load()


def _enc_config(shape, max_batch):
    return B.EncConfig(n_layers=shape.n_layers, d_model=shape.d_model, n_heads=shape.n_heads,
                       head_dim=shape.head_dim, d_ffn=shape.d_ffn, n_mels=shape.n_mels,
                       n_frames=shape.n_frames, max_batch=max_batch, ln_eps=shape.ln_eps)


def test_encoder_workspace_size(lib):
    from synthetic import ENC_LARGE_V3
    c = _enc_config(ENC_LARGE_V3, 4)
    n = lib.wf_enc_workspace_bytes(ctypes.byref(c))
    # at least the per-window activations: padded features and stem output
    # (bf16, 3002 rows), residual (fp32), LN output, q, k, v^T (1536 padded
    # frames), attention output and MLP hidden (bf16)
    per = (3002 * 128 * 2 + 3002 * 1280 * 2 + 1500 * 1280 * 4 + 1500 * 1280 * 2
           + 3 * 20 * 1536 * 64 * 2 + 1500 * 1280 * 2 + 1500 * 5120 * 2)
    assert n >= 4 * per
    assert n < 4 * per + 64 * 2 ** 20      # plus the position table and stem weights


@pytest.mark.parametrize("field,value", [("head_dim", 32), ("d_model", 1344), ("n_heads", 21),
                                         ("d_ffn", 100), ("n_mels", 300), ("n_mels", 10),
                                         ("n_frames", 0), ("max_batch", 0), ("n_layers", 0)])
def test_bad_encoder_configs_rejected(lib, field, value):
    from synthetic import ENC_SMALL
    c = _enc_config(ENC_SMALL, 2)
    assert lib.wf_enc_workspace_bytes(ctypes.byref(c)) > 0
    setattr(c, field, value)
    assert lib.wf_enc_workspace_bytes(ctypes.byref(c)) == 0


def test_encoder_calls_reject_null_arguments(lib):
    from synthetic import ENC_SMALL
    c = _enc_config(ENC_SMALL, 1)
    h = ctypes.c_void_p()
    w = B.EncWeights()
    st = lib.wf_enc_create(ctypes.byref(c), ctypes.byref(w), None, 0, ctypes.byref(h))
    assert st == -1 and b"null" in lib.wf_last_error()
    assert lib.wf_encode(None, 1, None, None, None) == -1
    assert lib.wf_enc_set_timing(None, 1) == -1
