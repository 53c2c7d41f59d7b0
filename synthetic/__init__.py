"""Seeded synthetic inputs for the Whisper-shaped block-verification path.

This module is the one piece shared by the CPU oracle and the GPU engine's
tests and benchmark. It draws numbers and rounds them to bf16; it computes
nothing of the method itself (no layer, attention, argmax or acceptance).

Recipe (every tensor is independent of every other):

* ``rng(cfg_id, tensor_id)`` is ``numpy.random.default_rng`` seeded with
  ``SeedSequence([0, cfg_id, tensor_id])`` (master seed 0).
* Weights, biases and embeddings are ``0.02 * N(0, 1)`` drawn in float32 and
  rounded to bf16 with round-to-nearest-even. Layer-norm gains are 1 and
  biases 0 (a gain drawn N(0, 0.02) would zero the network); tests may ask
  for perturbed gains ``1 + 0.1 N(0,1)`` and biases ``0.1 N(0,1)`` so that a
  kernel that ignores them is caught.
* Encoder outputs (the audio memory) are ``N(0, 1)`` with tensor id
  ``1000 + request``; prompt prefixes use ``2000 + request``; the draft table
  (Bernoulli keep-flags and uniform replacement ids per absolute position)
  uses ``3000 + request``.

The model shapes follow Whisper large-v3 (32 layers, width 1280, 20 heads of
64, MLP 5120, vocabulary 51866, 1500 encoder frames for a 30 s window) and
its 4-layer turbo variant; the 448-token decoder context is the one the
SGLang-Omni Whisper cookbook states under "Known Limitations".
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import numpy as np

__all__ = [
    "ModelShape", "Workload", "WORKLOADS", "TINY", "LARGE_V3", "TURBO",
    "rng", "f32_to_bf16_bits", "bf16_bits_to_f32", "make_weights",
    "make_encoder_out", "make_prefixes", "make_draft_table", "LAYER_TENSORS",
    "GLOBAL_TENSORS", "layer_tensor_shapes", "global_tensor_shapes", "make_drafter_weights",
    "DRAFTER_TAPS",
]

# residual streams of these target blocks (zero-based) feed the drafter's
# history (Whisper-Flash App. A.2)
DRAFTER_TAPS = (1, 8, 15, 22, 29)


@dataclasses.dataclass(frozen=True)
class ModelShape:
    n_layers: int
    d_model: int
    n_heads: int
    head_dim: int
    d_ffn: int
    vocab: int
    n_frames: int
    n_ctx: int = 448
    eos_id: int = 50257
    ln_eps: float = 1e-5


TINY = ModelShape(n_layers=2, d_model=64, n_heads=4, head_dim=16, d_ffn=256,
                  vocab=512, n_frames=100, n_ctx=448, eos_id=511)
LARGE_V3 = ModelShape(n_layers=32, d_model=1280, n_heads=20, head_dim=64,
                      d_ffn=5120, vocab=51866, n_frames=1500)
TURBO = dataclasses.replace(LARGE_V3, n_layers=4)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One of the five synthetic workloads (seeded, no datasets)."""
    cfg_id: int
    name: str
    shape: ModelShape
    batch: int
    k_draft: int
    prefix: str            # "fixed:<n>", "uniform:<lo>:<hi>", "poisson:<mean>:<lo>:<hi>"
    n_max: int             # output budget per request (tokens, incl. the first anchor)
    p_keep: float          # probability that a draft equals the greedy token
    temperature: float = 0.0
    paged_shuffle: bool = False
    drafter_layers: int = 0


WORKLOADS: Dict[int, Workload] = {
    0: Workload(0, "tiny-verify-loop", TINY, batch=1, k_draft=4,
                prefix="fixed:4", n_max=32, p_keep=0.7),
    1: Workload(1, "large-v3-verify-b1", LARGE_V3, batch=1, k_draft=8,
                prefix="fixed:64", n_max=200, p_keep=0.7),
    2: Workload(2, "turbo-loop-b32", TURBO, batch=32, k_draft=8,
                prefix="uniform:4:200", n_max=200, p_keep=0.75),
    3: Workload(3, "large-v3-drafter-b96", LARGE_V3, batch=96, k_draft=8,
                prefix="poisson:80:4:224", n_max=200, p_keep=0.0,
                paged_shuffle=True, drafter_layers=2),
    4: Workload(4, "large-v3-sampling-b32", LARGE_V3, batch=32, k_draft=8,
                prefix="uniform:4:200", n_max=200, p_keep=0.7,
                temperature=0.7),
}

# Per-layer tensors, PyTorch Linear convention: a weight is [out, in].
LAYER_TENSORS: List[str] = [
    "ln1_g", "ln1_b", "wq", "bq", "wk", "wv", "bv", "wo", "bo",
    "ln2_g", "ln2_b", "wqc", "bqc", "wkc", "wvc", "bvc", "woc", "boc",
    "ln3_g", "ln3_b", "w1", "b1", "w2", "b2",
]
GLOBAL_TENSORS: List[str] = ["tok_emb", "pos_emb", "lnf_g", "lnf_b"]


def layer_tensor_shapes(s: ModelShape) -> Dict[str, tuple]:
    d, f = s.d_model, s.d_ffn
    shp = {}
    for n in LAYER_TENSORS:
        if n.startswith("ln") or n.startswith("b"):
            shp[n] = (f,) if n == "b1" else (d,)
        elif n == "w1":
            shp[n] = (f, d)
        elif n == "w2":
            shp[n] = (d, f)
        else:
            shp[n] = (d, d)
    return shp


def global_tensor_shapes(s: ModelShape) -> Dict[str, tuple]:
    return {"tok_emb": (s.vocab, s.d_model), "pos_emb": (s.n_ctx, s.d_model),
            "lnf_g": (s.d_model,), "lnf_b": (s.d_model,)}


def rng(cfg_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([0, cfg_id, tensor_id]))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    r = (b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _tensor_id(layer: Optional[int], name: str) -> int:
    if layer is None:
        return 1 + GLOBAL_TENSORS.index(name)
    return 100 + 64 * layer + LAYER_TENSORS.index(name)


def _draw(cfg_id: int, tid: int, shape, scale: float, offset: float = 0.0) -> np.ndarray:
    x = rng(cfg_id, tid).standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    if offset != 0.0:
        x += np.float32(offset)
    return f32_to_bf16_bits(x)


def make_weights(shape: ModelShape, cfg_id: int, ln_random: bool = False,
                 n_layers: Optional[int] = None) -> Dict[str, np.ndarray]:
    """All decoder tensors as bf16 bit patterns (uint16), keyed
    ``"<name>"`` for globals and ``"L<l>.<name>"`` per layer."""
    nl = shape.n_layers if n_layers is None else n_layers
    out: Dict[str, np.ndarray] = {}
    gs = global_tensor_shapes(shape)
    for name in GLOBAL_TENSORS:
        out[name] = _ln_or_weight(cfg_id, None, name, gs[name], ln_random)
    ls = layer_tensor_shapes(shape)
    for l in range(nl):
        for name in LAYER_TENSORS:
            out[f"L{l}.{name}"] = _ln_or_weight(cfg_id, l, name, ls[name], ln_random)
    return out


def _ln_or_weight(cfg_id, layer, name, shp, ln_random):
    tid = _tensor_id(layer, name)
    if name.endswith("_g") and name.startswith("ln"):
        if ln_random:
            return _draw(cfg_id, tid, shp, 0.1, 1.0)
        return f32_to_bf16_bits(np.ones(shp, np.float32))
    if name.endswith("_b") and name.startswith("ln"):
        if ln_random:
            return _draw(cfg_id, tid, shp, 0.1)
        return np.zeros(shp, np.uint16)
    return _draw(cfg_id, tid, shp, 0.02)


def make_encoder_out(shape: ModelShape, cfg_id: int, request: int,
                     n_frames: Optional[int] = None) -> np.ndarray:
    """Audio memory for one request: bf16 bits [n_frames, d_model], N(0, 1)."""
    f = shape.n_frames if n_frames is None else n_frames
    return _draw(cfg_id, 1000 + request, (f, shape.d_model), 1.0)


def make_prefixes(wl: Workload, n: Optional[int] = None) -> List[np.ndarray]:
    """Prompt prefixes: ids uniform over [0, V) without EOS, lengths per the
    workload's distribution."""
    n = wl.batch if n is None else n
    out = []
    kind, *args = wl.prefix.split(":")
    for r in range(n):
        g = rng(wl.cfg_id, 2000 + r)
        if kind == "fixed":
            ln = int(args[0])
        elif kind == "uniform":
            ln = int(g.integers(int(args[0]), int(args[1]) + 1))
        elif kind == "poisson":
            ln = int(np.clip(g.poisson(float(args[0])), int(args[1]), int(args[2])))
        else:
            raise ValueError(wl.prefix)
        ids = g.integers(0, wl.shape.vocab - 1, size=ln)
        ids = np.where(ids >= wl.shape.eos_id, ids + 1, ids)  # skip EOS
        out.append(ids.astype(np.int32))
    return out


def make_draft_table(wl: Workload, request: int, p_keep: Optional[float] = None):
    """Per absolute sequence position: (keep flag, replacement id).

    A draft at position ``t`` is the greedy token for ``t`` when ``keep[t]``
    and ``repl[t]`` otherwise. Keying by position (not by round) gives the
    same distribution as fresh per-round draws, because positions beyond a
    rejection are never observed."""
    p = wl.p_keep if p_keep is None else p_keep
    g = rng(wl.cfg_id, 3000 + request)
    n = wl.shape.n_ctx + 1
    keep = g.random(n) < p
    repl = g.integers(0, wl.shape.vocab, size=n).astype(np.int32)
    return keep, repl


def make_drafter_weights(shape: ModelShape, cfg_id: int, n_layers: int = 2, n_taps: int = 5,
                         ln_random: bool = False) -> Dict[str, np.ndarray]:
    """Random-init parallel drafter (bf16 bits): ``"D<l>.<name>"`` layers with
    the target block's tensors (including its own cross K/V projections),
    ``w_hist`` [d, n_taps*d] (history projection, no bias), ``mask`` [d]
    (the learned mask vector) and its final norm ``lnd_g`` / ``lnd_b``."""
    out: Dict[str, np.ndarray] = {}
    ls = layer_tensor_shapes(shape)
    for l in range(n_layers):
        for name in LAYER_TENSORS:
            out[f"D{l}.{name}"] = _ln_or_weight(cfg_id, 200 + l, name, ls[name], ln_random)
    d = shape.d_model
    out["w_hist"] = _draw(cfg_id, 30001, (d, n_taps * d), 0.02)
    out["mask"] = _draw(cfg_id, 30002, (d,), 0.02)
    out["lnd_g"] = _ln_or_weight(cfg_id, None, "lnf_g", (d,), ln_random) if not ln_random \
        else _draw(cfg_id, 30003, (d,), 0.1, 1.0)
    out["lnd_b"] = np.zeros((d,), np.uint16) if not ln_random else _draw(cfg_id, 30004, (d,), 0.1)
    return out


# -- encoder (audio features -> audio memory) ---------------------------------

@dataclasses.dataclass(frozen=True)
class EncoderShape:
    """Audio encoder shape: ``n_mels`` log-mel channels over ``2 * n_frames``
    feature frames (10 ms hop) in, ``n_frames`` frames of width ``d_model``
    out (the stride-2 stem halves the frame rate)."""
    n_layers: int
    d_model: int
    n_heads: int
    head_dim: int
    d_ffn: int
    n_mels: int
    n_frames: int
    ln_eps: float = 1e-5


# Whisper large-v3 encoder (the turbo variant shares it): 32 blocks, width
# 1280, 20 heads of 64, MLP 5120, 128 mel channels, 3000 feature frames ->
# 1500 frames for a 30 s window. The small shape keeps head_dim 64.
ENC_LARGE_V3 = EncoderShape(n_layers=32, d_model=1280, n_heads=20, head_dim=64,
                            d_ffn=5120, n_mels=128, n_frames=1500)
ENC_SMALL = EncoderShape(n_layers=2, d_model=128, n_heads=2, head_dim=64,
                         d_ffn=512, n_mels=64, n_frames=100)

ENC_LAYER_TENSORS: List[str] = [
    "ln1_g", "ln1_b", "wq", "bq", "wk", "wv", "bv", "wo", "bo",
    "ln2_g", "ln2_b", "w1", "b1", "w2", "b2",
]
ENC_GLOBAL_TENSORS: List[str] = ["conv1_w", "conv1_b", "conv2_w", "conv2_b", "lnp_g", "lnp_b"]
__all__ += ["EncoderShape", "ENC_LARGE_V3", "ENC_SMALL", "ENC_LAYER_TENSORS",
            "ENC_GLOBAL_TENSORS", "make_encoder_weights", "make_mel"]


def _enc_shapes(s: EncoderShape):
    d, f = s.d_model, s.d_ffn
    g = {"conv1_w": (d, s.n_mels, 3), "conv1_b": (d,), "conv2_w": (d, d, 3), "conv2_b": (d,),
         "lnp_g": (d,), "lnp_b": (d,)}
    lay = {}
    for n in ENC_LAYER_TENSORS:
        if n in ("w1",):
            lay[n] = (f, d)
        elif n == "w2":
            lay[n] = (d, f)
        elif n == "b1":
            lay[n] = (f,)
        elif n.startswith("w"):
            lay[n] = (d, d)
        else:
            lay[n] = (d,)
    return g, lay


def make_encoder_weights(shape: EncoderShape, cfg_id: int, ln_random: bool = False,
                         n_layers: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Random-init encoder (bf16 bits): globals ``conv1_w`` [d, n_mels, 3],
    ``conv1_b``, ``conv2_w`` [d, d, 3], ``conv2_b`` (PyTorch Conv1d layout),
    the final norm ``lnp_g`` / ``lnp_b``, and ``"E<l>.<name>"`` per block.
    Same recipe as the decoder: 0.02 N(0, 1), gains 1, norm biases 0. Tensor
    ids 40000 + i (globals) and 41000 + 64 l + i (blocks)."""
    nl = shape.n_layers if n_layers is None else n_layers
    gs, ls = _enc_shapes(shape)
    out: Dict[str, np.ndarray] = {}

    def one(tid, name, shp):
        if name.startswith("ln") and name.endswith("_g"):
            return _draw(cfg_id, tid, shp, 0.1, 1.0) if ln_random \
                else f32_to_bf16_bits(np.ones(shp, np.float32))
        if name.startswith("ln") and name.endswith("_b"):
            return _draw(cfg_id, tid, shp, 0.1) if ln_random else np.zeros(shp, np.uint16)
        return _draw(cfg_id, tid, shp, 0.02)

    for i, name in enumerate(ENC_GLOBAL_TENSORS):
        out[name] = one(40000 + i, name, gs[name])
    for l in range(nl):
        for i, name in enumerate(ENC_LAYER_TENSORS):
            out[f"E{l}.{name}"] = one(41000 + 64 * l + i, name, ls[name])
    return out


def make_mel(shape: EncoderShape, cfg_id: int, request: int) -> np.ndarray:
    """Log-mel features of one request: bf16 bits [n_mels, 2 * n_frames],
    N(0, 1) (tensor id 4000 + request). They stand in for normalised
    log-mel features of a 30 s window."""
    return _draw(cfg_id, 4000 + request, (shape.n_mels, 2 * shape.n_frames), 1.0)
