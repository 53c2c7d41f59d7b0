"""ctypes binding of libwf.so — argument marshalling only.

Every compute step runs in the library's HIP kernels; this module turns
torch tensors into pointers, picks the current stream and raises on a
negative status. ``Engine`` additionally owns the device buffers the C ABI
expects the caller to provide (weights, KV pools, page table, workspace),
allocated with torch.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Dict, Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libwf.so")
HEADER = os.path.join(HERE, "..", "include", "wf.h")

_lib = None


class WFError(RuntimeError):
    pass


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layers", "d_model", "n_heads", "head_dim", "d_ffn", "vocab", "n_frames", "n_ctx",
        "max_batch", "max_rows", "page_size", "n_pages", "eos_id")] + [
        ("ln_eps", ctypes.c_float), ("drafter_layers", ctypes.c_int32),
        ("n_taps", ctypes.c_int32), ("tap_layers", ctypes.c_int32 * 8)]


LAYER_FIELDS = ["ln1_g", "ln1_b", "wq", "bq", "wk", "wv", "bv", "wo", "bo",
                "ln2_g", "ln2_b", "wqc", "bqc", "wkc", "wvc", "bvc", "woc", "boc",
                "ln3_g", "ln3_b", "w1", "b1", "w2", "b2"]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in LAYER_FIELDS]


class DrafterWeights(ctypes.Structure):
    _fields_ = [("layers", ctypes.POINTER(LayerWeights)), ("w_hist", ctypes.c_void_p),
                ("mask_emb", ctypes.c_void_p), ("lnd_g", ctypes.c_void_p),
                ("lnd_b", ctypes.c_void_p)]


class Weights(ctypes.Structure):
    _fields_ = [("tok_emb", ctypes.c_void_p), ("pos_emb", ctypes.c_void_p),
                ("lnf_g", ctypes.c_void_p), ("lnf_b", ctypes.c_void_p),
                ("layers", ctypes.POINTER(LayerWeights)),
                ("drafter", ctypes.POINTER(DrafterWeights))]


class LoopState(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "anchor", "len", "emitted", "done", "acc_sum", "prop_sum", "rounds", "step", "tok_sum",
        "hist")]


class EncConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layers", "d_model", "n_heads", "head_dim", "d_ffn", "n_mels", "n_frames",
        "max_batch")] + [("ln_eps", ctypes.c_float)]


ENC_LAYER_FIELDS = ["ln1_g", "ln1_b", "wq", "bq", "wk", "wv", "bv", "wo", "bo",
                    "ln2_g", "ln2_b", "w1", "b1", "w2", "b2"]


class EncLayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ENC_LAYER_FIELDS]


class EncWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("conv1_w", "conv1_b", "conv2_w", "conv2_b", "lnp_g", "lnp_b")] + [
        ("layers", ctypes.POINTER(EncLayerWeights))]


def header_functions() -> list:
    """Names of the functions include/wf.h declares."""
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(wf_[a-z_]+)\s*\(", txt)))


def load():
    """Load libwf.so; fails loudly when it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m speculative_decoding_encoder_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, SZ, VP = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
    cfgp = ctypes.POINTER(Config)
    sig = {
        "wf_kv_pool_bytes": (SZ, [cfgp]),
        "wf_xkv_pool_bytes": (SZ, [cfgp]),
        "wf_workspace_bytes": (SZ, [cfgp]),
        "wf_create": (I32, [cfgp, ctypes.POINTER(Weights), P, SZ, P, SZ, P, P, SZ,
                            ctypes.POINTER(VP)]),
        "wf_create_static": (I32, [cfgp, ctypes.POINTER(Weights), P, SZ, P, SZ, P,
                                   ctypes.POINTER(VP)]),
        "wf_destroy": (None, [P]),
        "wf_last_error": (ctypes.c_char_p, []),
        "wf_reset": (I32, [P, I32, P, P]),
        "wf_encode_kv": (I32, [P, I32, P, P, P]),
        "wf_verify_block": (I32, [P, I32, P, P, I32, P, P, P, P]),
        "wf_accept": (I32, [P, I32, P, I32, P, P, P, P, P, P, ctypes.c_float, ctypes.c_uint64,
                            P, P, P, P, P, P, P]),
        "wf_rollback": (I32, [P, I32, P, P, P]),
        "wf_verify_tree": (I32, [P, I32, P, P, I32, P, P, P, P, P]),
        "wf_set_readout": (I32, [P, I32, P]),
        "wf_accept_tree": (I32, [P, I32, P, I32, P, P, P, P, P, P, P, P, P, P]),
        "wf_rollback_tree": (I32, [P, I32, P, P, I32, P, P]),
        "wf_draft": (I32, [P, I32, P, P, I32, P, P, P]),
        "wf_truncate": (I32, [P, I32, P, P, P]),
        "wf_loop_prepare": (I32, [P, I32, ctypes.POINTER(LoopState), I32, I32, P, I32, P, P, P,
                                  P]),
        "wf_loop_finish": (I32, [P, I32, ctypes.POINTER(LoopState), I32, P, P, P, P, P, P]),
        "wf_device_state": (I32, [P, P, P, P]),
        "wf_set_timing": (I32, [P, I32]),
        "wf_get_timing": (I32, [P, I32, ctypes.POINTER(ctypes.c_double),
                                ctypes.POINTER(ctypes.c_int32)]),
        "wf_set_option": (I32, [P, I32, I32]),
        "wf_set_trace": (I32, [P, P, SZ]),
        "wf_pass_schedule": (I32, [P, ctypes.POINTER(ctypes.c_int32)]),
        "wf_enc_workspace_bytes": (SZ, [ctypes.POINTER(EncConfig)]),
        "wf_enc_create": (I32, [ctypes.POINTER(EncConfig), ctypes.POINTER(EncWeights), P, SZ,
                                ctypes.POINTER(VP)]),
        "wf_enc_destroy": (None, [P]),
        "wf_encode": (I32, [P, I32, P, P, P]),
        "wf_enc_set_timing": (I32, [P, I32]),
        "wf_enc_get_timing": (I32, [P, I32, ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_int32)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(status: int, what: str):
    if status != 0:
        msg = load().wf_last_error().decode(errors="replace")
        raise WFError(f"{what} failed with status {status}: {msg}")


def _p(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def make_config(shape, max_batch: int, max_rows: int, n_pages: Optional[int] = None,
                drafter_layers: int = 0, taps: Sequence[int] = ()) -> Config:
    pps = shape.n_ctx // 16
    tl = (ctypes.c_int32 * 8)(*list(taps)[:8])
    return Config(n_layers=shape.n_layers, d_model=shape.d_model, n_heads=shape.n_heads,
                  head_dim=shape.head_dim, d_ffn=shape.d_ffn, vocab=shape.vocab,
                  n_frames=shape.n_frames, n_ctx=shape.n_ctx, max_batch=max_batch,
                  max_rows=max_rows, page_size=16,
                  n_pages=n_pages if n_pages is not None else max_batch * pps,
                  eos_id=shape.eos_id, ln_eps=shape.ln_eps, drafter_layers=drafter_layers,
                  n_taps=len(taps), tap_layers=tl)


def workspace_bytes(cfg: Config) -> int:
    return int(load().wf_workspace_bytes(ctypes.byref(cfg)))


class Engine:
    """One engine on the current CUDA (HIP) device with its buffers.

    ``weights_bits``: name -> bf16 bit patterns (uint16 numpy arrays), the
    naming of ``synthetic.make_weights``. ``page_table``: optional int32
    numpy array [max_batch, n_ctx/16] of physical page ids.
    """

    def __init__(self, shape, weights_bits: Dict[str, np.ndarray], max_batch: int,
                 max_rows: int, page_table: Optional[np.ndarray] = None,
                 n_pages: Optional[int] = None,
                 drafter_bits: Optional[Dict[str, np.ndarray]] = None,
                 taps: Sequence[int] = (), static_workspace: bool = False,
                 share_weights: Optional["Engine"] = None):
        import torch
        self.torch = torch
        self.lib = load()
        self.shape = shape
        self.dev = torch.device("cuda", torch.cuda.current_device())
        n_dl = 0
        if drafter_bits is not None:
            n_dl = len({k.split(".")[0] for k in drafter_bits if k.startswith("D")})
        self.cfg = make_config(shape, max_batch, max_rows, n_pages, n_dl, taps)
        pps = shape.n_ctx // 16
        self.w = {}
        if share_weights is not None:
            # the same device weights as another engine (one copy in HBM)
            self.w = share_weights.w
        else:
            for k, v in list(weights_bits.items()) + list((drafter_bits or {}).items()):
                t = torch.from_numpy(np.ascontiguousarray(v).view(np.int16))
                self.w[k] = t.to(self.dev).view(torch.bfloat16)
        lw = (LayerWeights * shape.n_layers)()
        for l in range(shape.n_layers):
            for f in LAYER_FIELDS:
                setattr(lw[l], f, self.w[f"L{l}.{f}"].data_ptr())
        self._lw = lw
        dptr = None
        if n_dl:
            dlw = (LayerWeights * n_dl)()
            for l in range(n_dl):
                for f in LAYER_FIELDS:
                    setattr(dlw[l], f, self.w[f"D{l}.{f}"].data_ptr())
            self._dlw = dlw
            self._dw = DrafterWeights(dlw, self.w["w_hist"].data_ptr(),
                                      self.w["mask"].data_ptr(), self.w["lnd_g"].data_ptr(),
                                      self.w["lnd_b"].data_ptr())
            dptr = ctypes.pointer(self._dw)
        self._weights = Weights(self.w["tok_emb"].data_ptr(), self.w["pos_emb"].data_ptr(),
                                self.w["lnf_g"].data_ptr(), self.w["lnf_b"].data_ptr(), lw, dptr)
        cfgp = ctypes.byref(self.cfg)
        kvb = int(self.lib.wf_kv_pool_bytes(cfgp))
        xkvb = int(self.lib.wf_xkv_pool_bytes(cfgp))
        wsb = int(self.lib.wf_workspace_bytes(cfgp))
        if kvb == 0 or xkvb == 0 or wsb == 0:
            raise WFError("invalid configuration for libwf")
        self.kv = torch.zeros(kvb, dtype=torch.uint8, device=self.dev)
        self.xkv = torch.zeros(xkvb, dtype=torch.uint8, device=self.dev)
        # with static_workspace the library's own array serves (wf_create_static)
        self.ws = None if static_workspace else torch.zeros(wsb, dtype=torch.uint8,
                                                            device=self.dev)
        if page_table is None:
            page_table = np.arange(max_batch * pps, dtype=np.int32).reshape(max_batch, pps)
        self.page_table = torch.from_numpy(np.ascontiguousarray(page_table, dtype=np.int32)).to(self.dev)
        h = ctypes.c_void_p()
        torch.cuda.synchronize()
        if static_workspace:
            _check(self.lib.wf_create_static(cfgp, ctypes.byref(self._weights),
                                             self.kv.data_ptr(), kvb, self.xkv.data_ptr(), xkvb,
                                             self.page_table.data_ptr(), ctypes.byref(h)),
                   "wf_create_static")
        else:
            _check(self.lib.wf_create(cfgp, ctypes.byref(self._weights), self.kv.data_ptr(),
                                      kvb, self.xkv.data_ptr(), xkvb, self.page_table.data_ptr(),
                                      self.ws.data_ptr(), wsb, ctypes.byref(h)), "wf_create")
        self.h = h

    def close(self):
        if getattr(self, "h", None):
            self.lib.wf_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- thin wrappers with the C names ----------------------------------
    def wf_reset(self, slots, stream=None):
        _check(self.lib.wf_reset(self.h, slots.numel(), _p(slots), _stream(stream)), "wf_reset")

    def wf_encode_kv(self, slots, enc, stream=None):
        _check(self.lib.wf_encode_kv(self.h, slots.numel(), _p(slots), _p(enc), _stream(stream)),
               "wf_encode_kv")

    def wf_verify_block(self, slots, tokens, n_tok, argmax, logits=None, stream=None):
        n, T = tokens.shape
        _check(self.lib.wf_verify_block(self.h, n, _p(slots), _p(tokens), T, _p(n_tok),
                                        _p(argmax), _p(logits), _stream(stream)),
               "wf_verify_block")

    def wf_accept(self, tokens, n_tok, budget, argmax, n_acc, next_token, n_emit, done,
                  logits=None, q=None, suppress=None, temperature=0.0, seed=0,
                  request_id=None, step=None, stream=None):
        n, T = tokens.shape
        _check(self.lib.wf_accept(self.h, n, _p(tokens), T, _p(n_tok), _p(budget), _p(argmax),
                                  _p(logits), _p(q), _p(suppress), float(temperature), int(seed),
                                  _p(request_id), _p(step), _p(n_acc), _p(next_token),
                                  _p(n_emit), _p(done), _stream(stream)), "wf_accept")

    def wf_rollback(self, slots, n_acc, stream=None):
        _check(self.lib.wf_rollback(self.h, slots.numel(), _p(slots), _p(n_acc),
                                    _stream(stream)), "wf_rollback")

    def wf_set_readout(self, layer, frame=None):
        _check(self.lib.wf_set_readout(self.h, int(layer), _p(frame)), "wf_set_readout")

    def wf_verify_tree(self, slots, tokens, parents, n_tok, argmax, logits=None, stream=None):
        n, T = tokens.shape
        _check(self.lib.wf_verify_tree(self.h, n, _p(slots), _p(tokens), T, _p(parents),
                                       _p(n_tok), _p(argmax), _p(logits), _stream(stream)),
               "wf_verify_tree")

    def wf_accept_tree(self, tokens, parents, n_tok, budget, argmax, path, n_acc, next_token,
                       n_emit, done, stream=None):
        n, T = tokens.shape
        _check(self.lib.wf_accept_tree(self.h, n, _p(tokens), T, _p(parents), _p(n_tok),
                                       _p(budget), _p(argmax), _p(path), _p(n_acc),
                                       _p(next_token), _p(n_emit), _p(done), _stream(stream)),
               "wf_accept_tree")

    def wf_rollback_tree(self, slots, path, n_acc, stream=None):
        n, T = path.shape
        _check(self.lib.wf_rollback_tree(self.h, n, _p(slots), _p(path), T, _p(n_acc),
                                         _stream(stream)), "wf_rollback_tree")

    def wf_draft(self, slots, anchor, K, block, logits=None, stream=None):
        _check(self.lib.wf_draft(self.h, slots.numel(), _p(slots), _p(anchor), int(K), _p(block),
                                 _p(logits), _stream(stream)), "wf_draft")

    @staticmethod
    def loop_state(anchor, len, emitted, done, acc_sum, prop_sum, rounds, step, tok_sum,
                   hist) -> LoopState:
        """The device pointers of a running loop's state (torch tensors:
        int32 [n] each, hist int64 [K + 1])."""
        return LoopState(*[_p(t) for t in (anchor, len, emitted, done, acc_sum, prop_sum,
                                             rounds, step, tok_sum, hist)])

    def wf_loop_prepare(self, state: LoopState, n, K, n_max, table, block, n_tok, budget,
                        stream=None):
        cols = int(table.shape[1]) if table is not None else 0
        _check(self.lib.wf_loop_prepare(self.h, int(n), ctypes.byref(state), int(K), int(n_max),
                                        _p(table), cols, _p(block), _p(n_tok), _p(budget),
                                        _stream(stream)), "wf_loop_prepare")

    def wf_loop_finish(self, state: LoopState, n, K, n_tok, n_acc, next_token, n_emit, done,
                       stream=None):
        _check(self.lib.wf_loop_finish(self.h, int(n), ctypes.byref(state), int(K), _p(n_tok),
                                       _p(n_acc), _p(next_token), _p(n_emit), _p(done),
                                       _stream(stream)), "wf_loop_finish")

    def wf_truncate(self, slots, lens, stream=None):
        _check(self.lib.wf_truncate(self.h, slots.numel(), _p(slots), _p(lens),
                                    _stream(stream)), "wf_truncate")

    def wf_device_state(self, stream=None):
        mb = self.cfg.max_batch
        err = (ctypes.c_int32 * mb)()
        ln = (ctypes.c_int32 * mb)()
        _check(self.lib.wf_device_state(self.h, err, ln, _stream(stream)), "wf_device_state")
        return np.array(err[:], np.int32), np.array(ln[:], np.int32)

    def wf_set_timing(self, enable: bool):
        _check(self.lib.wf_set_timing(self.h, 1 if enable else 0), "wf_set_timing")

    def wf_get_timing(self, kind: int):
        ms = ctypes.c_double()
        cnt = ctypes.c_int32()
        _check(self.lib.wf_get_timing(self.h, kind, ctypes.byref(ms), ctypes.byref(cnt)),
               "wf_get_timing")
        return ms.value, cnt.value

    def wf_set_option(self, option: int, value: int):
        _check(self.lib.wf_set_option(self.h, int(option), int(value)), "wf_set_option")

    def wf_set_trace(self, buf=None):
        """buf: a device tensor (uint64 [tasks][2]) or None to stop tracing."""
        nbytes = 0 if buf is None else buf.numel() * buf.element_size()
        _check(self.lib.wf_set_trace(self.h, _p(buf), nbytes), "wf_set_trace")

    def wf_pass_schedule(self):
        """Task-list layout of the last persistent pass: dict of total,
        per_layer, layers, phase offsets (12), head offsets (3), grid."""
        info = (ctypes.c_int32 * 20)()
        _check(self.lib.wf_pass_schedule(self.h, info), "wf_pass_schedule")
        v = list(info)
        return {"total": v[0], "per_layer": v[1], "layers": v[2], "ph_off": v[3:15],
                "head_off": v[15:18], "grid": v[18]}

    # -- helpers ---------------------------------------------------------
    def i32(self, a: Sequence[int]):
        return self.torch.as_tensor(np.asarray(a, dtype=np.int32), device=self.dev)

    def bf16(self, bits: np.ndarray):
        t = self.torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
        return t.to(self.dev).view(self.torch.bfloat16)


TIMING_KINDS = ["qkv", "oproj", "cross_q", "fc1", "fc2", "lm_head", "self_attn", "cross_attn",
                "other", "encode_kv", "draft", "history", "pass"]

# wf_set_option options (include/wf.h)
WF_OPT_PERSISTENT, WF_OPT_TALL_GEMM, WF_OPT_LN_FUSION, WF_OPT_XA_CHUNKS = 1, 2, 3, 4
WF_OPT_PASS_TIMEOUT_US = 5
# device error word bits (include/wf.h)
WF_DERR_CONTEXT, WF_DERR_TOKEN, WF_DERR_STATE, WF_DERR_ACCEPT = 1, 2, 4, 8
WF_DERR_NAN, WF_DERR_PAGE, WF_DERR_SAMPLE = 16, 32, 64
WF_DERR_TIMEOUT = 128
WF_STATIC_WORKSPACE_BYTES = 64 << 20
PASS_PHASES = ["ln1", "qkv", "self_attn", "oproj", "ln2", "cross_q", "cross_attn", "oproj_c",
               "ln3", "fc1", "fc2"]


ENC_TIMING_KINDS = ["stem", "qkv", "attn", "oproj", "fc1", "fc2", "ln", "other"]


class Encoder:
    """Audio encoder through the C ABI. Owns the device copies of the
    weights (bf16 bits from ``synthetic.make_encoder_weights``) and the
    workspace, allocated with torch."""

    def __init__(self, shape, wbits: Dict[str, np.ndarray], max_batch: int, device: int = 0):
        import torch
        self.torch = torch
        self.shape = shape
        self.dev = torch.device("cuda", device)
        lib = load()
        self.cfg = EncConfig(n_layers=shape.n_layers, d_model=shape.d_model,
                             n_heads=shape.n_heads, head_dim=shape.head_dim, d_ffn=shape.d_ffn,
                             n_mels=shape.n_mels, n_frames=shape.n_frames, max_batch=max_batch,
                             ln_eps=shape.ln_eps)
        self.max_batch = max_batch
        self._bufs = {k: torch.from_numpy(v.view(np.int16).copy()).to(self.dev)
                      for k, v in wbits.items()}
        lay = (EncLayerWeights * shape.n_layers)()
        for l in range(shape.n_layers):
            for f in ENC_LAYER_FIELDS:
                setattr(lay[l], f, self._bufs[f"E{l}.{f}"].data_ptr())
        self._lay = lay
        w = EncWeights(layers=lay)
        for f in ("conv1_w", "conv1_b", "conv2_w", "conv2_b", "lnp_g", "lnp_b"):
            setattr(w, f, self._bufs[f].data_ptr())
        nb = int(lib.wf_enc_workspace_bytes(ctypes.byref(self.cfg)))
        if nb == 0:
            raise WFError("invalid encoder configuration")
        self.ws = torch.empty(nb, dtype=torch.uint8, device=self.dev)
        h = ctypes.c_void_p()
        with torch.cuda.device(self.dev):
            _check(lib.wf_enc_create(ctypes.byref(self.cfg), ctypes.byref(w), self.ws.data_ptr(),
                                     nb, ctypes.byref(h)), "wf_enc_create")
        self.h = h

    def bf16(self, bits: np.ndarray):
        return self.torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).to(self.dev)

    def wf_encode(self, d_mel, d_out, stream=None):
        n = d_mel.shape[0]
        _check(load().wf_encode(self.h, n, d_mel.data_ptr(), d_out.data_ptr(), _stream(stream)),
               "wf_encode")

    def set_timing(self, on: bool):
        _check(load().wf_enc_set_timing(self.h, 1 if on else 0), "wf_enc_set_timing")

    def timing(self) -> Dict[str, tuple]:
        out = {}
        for i, name in enumerate(ENC_TIMING_KINDS):
            ms, cnt = ctypes.c_double(), ctypes.c_int32()
            _check(load().wf_enc_get_timing(self.h, i, ctypes.byref(ms), ctypes.byref(cnt)),
                   "wf_enc_get_timing")
            out[name] = (ms.value, cnt.value)
        return out

    def close(self):
        if self.h:
            load().wf_enc_destroy(self.h)
            self.h = None
