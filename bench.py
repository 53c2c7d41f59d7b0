"""Benchmark of the block-verification hot path on one MI355X.

A step is one round of the running speculative loop over one batch: the
round's block (the anchor plus K = 8 candidates per request, from the
workload's drafter), wf_verify_block (every decoder layer, the tied LM head
and the per-row argmax), wf_accept, wf_rollback and the loop's state update,
all on the device and replayed from one captured HIP graph. Each timed round
verifies a new block at the positions the loop has reached, so tokens per
second come from the realized acceptance: the tokens the timed rounds emit,
sum over requests of (accepted + 1), over their time. Inputs are seeded and
synthetic (no datasets, no trained weights); weights, audio memory, prompts
and KV caches are resident in HBM before the timed region starts, and the
prompts are prefilled before it.

Workloads (``--config`` for the headline, ``--batches`` and ``--configs`` for
the rest of the line):
  1  32-layer large-v3 shape, batch 1, 64-token prefix, drafts = the greedy
     token with probability 0.7, else a uniform id (default headline)
  2  4-layer turbo shape, batch 32, prefixes uniform in [4, 200], p = 0.75,
     rounds until 200 tokens per request
  3  32-layer large-v3 shape, batch 96, prefixes Poisson(80) clipped to
     [4, 224], shuffled 16-token pages; K = 8 drafts come from the 2-layer
     random-init parallel drafter (wf_draft), timed together with the verify
  4  32-layer large-v3 shape, batch 32, prefixes uniform in [4, 200], temperature
     0.7 rejection sampling; draft distributions q_i = 0.7 p~_i + 0.3 softmax(z_i),
     z_i ~ N(0, 1), where p~_i is the target's T = 0.7 distribution at the
     drafted prefix (single-row passes, untimed, then truncated back);
     candidates are drawn from q_i. Its greedy variant (batch 32 of the
     metric) takes Bernoulli-copy drafts (p = 0.7) and greedy acceptance.
The greedy continuation that Bernoulli-copy drafts copy is the engine's own,
computed before timing. Audio seconds per second divide tokens per second by
3.5 tokens per audio second (the tokens-to-audio ratio of Whisper-Flash
Table 1).

Per workload the line also gives the fixed-block pass: one block verified
again and again from the same state (wf_truncate back after each round),
timed per step and, in a second pass, per kernel launch with HIP events.
That is the pass whose whole HBM bytes give pass_roofline_frac, and whose
dominant kernel (the largest total time) gives the roofline object.

``--encoder N`` instead times the audio encoder (wf_encode: N log-mel windows
of 30 s through the 32-block large-v3 encoder) and prints its own line in
audio seconds per second, with the bf16 MFMA roofline of its dominant kernel.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from speculative_decoding_encoder_amd.prof_summary import (  # noqa: E402
    is_encoder_workload, kernel_source_hash)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
TOKENS_PER_AUDIO_S = 3.5
METRIC = "verified tokens/sec & audio-s/sec at batch 1/32/96, K=8; % HBM roofline"
KIND_NAMES = ["qkv", "oproj", "cross_q", "fc1", "fc2", "lm_head", "self_attn",
              "cross_attn", "other", "encode_kv", "draft", "history", "pass"]
# kernel symbols (rocprofv3 name prefixes) of each timing kind: a GEMM role
# runs the register-tiled, the tall-block or the LDS-staged kernel by block
# height; the first template argument is the role
KIND_SYMBOL = {
    **{k: "|".join(f"wf::{kern}<{r}," for kern in ("gemm_rk_kernel", "gemm_tl_kernel",
                                                    "gemm_kernel"))
       for r, k in enumerate(["qkv", "oproj", "cross_q", "fc1", "fc2", "lm_head"])},
    "self_attn": "wf::self_attn_kernel<64>", "cross_attn": "wf::cross_attn_kernel<64>",
    "pass": "wf::(anonymous namespace)::pass_kernel<",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Window:
    """With --mark-timed, the host clock (CLOCK_MONOTONIC, ns; the clock of
    rocprofv3's kernel timestamps) at the start and the end of the timed
    replays of each workload's fixed-block pass (and of the calibration
    copies), printed to stderr, so that a kernel trace or a counter run can
    be cut to the steady-state dispatches (prof_summary --window)."""

    def __init__(self, on: bool = False):
        self.on = on
        self.t0 = 0

    def start(self):
        if self.on:
            self.t0 = time.monotonic_ns()

    def end(self, what: str):
        if self.on:
            log(f"[bench] timed-window {what} {self.t0} {time.monotonic_ns()}")


WINDOW = Window(False)


class Workload:
    def __init__(self, cfg_id: int, greedy: bool = False, k: int = 0, batch: int = 0,
                 readout: int = -1):
        from synthetic import (DRAFTER_TAPS, WORKLOADS, make_draft_table, make_drafter_weights,
                               make_encoder_out, make_prefixes, make_weights, rng)
        from speculative_decoding_encoder_amd.binding import Engine
        from speculative_decoding_encoder_amd.harness import prefill, run_loop
        import torch
        self.torch = torch
        self.wl = wl = WORKLOADS[cfg_id]
        self.shape = s = wl.shape
        self.B = B = batch or wl.batch
        self.K = k or wl.k_draft
        self.sampling = cfg_id == 4 and not greedy
        self.temperature = wl.temperature if self.sampling else 0.0
        self.name = wl.name if (cfg_id != 4 or self.sampling) else "large-v3-verify-b32-greedy"
        t0 = time.time()
        self.wbits = make_weights(s, wl.cfg_id)
        self.drafter = wl.drafter_layers > 0
        self.dbits = make_drafter_weights(s, wl.cfg_id, wl.drafter_layers) if self.drafter else None
        self.encs = np.stack([make_encoder_out(s, wl.cfg_id, r) for r in range(B)])
        self.prefixes = make_prefixes(wl, B)
        self.P = np.array([len(p) for p in self.prefixes], np.int32)
        log(f"[bench] inputs generated in {time.time() - t0:.1f}s")
        max_rows = max(B * (self.K + 1), B * int(self.P.max()))
        pps = s.n_ctx // 16
        page_table = None
        if wl.paged_shuffle:
            page_table = rng(wl.cfg_id, 5000).permutation(B * pps).astype(np.int32).reshape(B, pps)
        self.eng = eng = Engine(s, self.wbits, max_batch=B, max_rows=max_rows,
                                page_table=page_table, drafter_bits=self.dbits,
                                taps=DRAFTER_TAPS if self.drafter else ())
        self.slots = list(range(B))
        self.d_slots = eng.i32(self.slots)
        self.readout = readout
        if readout >= 0:
            # anchor readout at that layer in every verify pass
            self.d_frame = torch.full((max_rows,), -1, dtype=torch.int32, device=eng.dev)
            eng.wf_set_readout(readout, self.d_frame)
        d_enc = eng.bf16(self.encs)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        eng.wf_encode_kv(self.d_slots, d_enc)
        torch.cuda.synchronize()
        self.encode_kv_s = time.perf_counter() - t0
        del d_enc
        # the engine's own greedy continuation (untimed) for the drafts: the
        # whole budget, so that the running loop's table drafter can copy it
        eng.wf_reset(self.d_slots)
        if not self.drafter:
            t0 = time.time()
            g = run_loop(eng, self.slots, self.prefixes, wl.n_max, 0, None, s.eos_id)
            self.greedy = g.tokens
            eng.wf_reset(self.d_slots)
            log(f"[bench] {self.name}: greedy continuation ({wl.n_max} tokens) in "
                f"{time.time() - t0:.1f}s")
        anchors = prefill(eng, self.slots, self.prefixes)
        self.anchors = anchors
        blocks = np.zeros((B, self.K + 1), np.int32)
        for b in range(B if not self.drafter else 0):
            keep, repl = make_draft_table(wl, b)
            L = int(self.P[b])
            blocks[b, 0] = anchors[b]
            for i in range(1, self.K + 1):
                j = i  # greedy[b][i] sits at position L + i
                gt = self.greedy[b][j] if j < len(self.greedy[b]) else int(repl[L + i])
                blocks[b, i] = gt if keep[L + i] else repl[L + i]
        T = self.K + 1
        self.d_q = None
        self.d_logits = None
        if self.sampling:
            blocks = self._sampling_blocks(anchors, T)
            self.d_logits = torch.empty((B, T, s.vocab), dtype=torch.float32, device=eng.dev)
            self.d_req = eng.i32(np.arange(B, dtype=np.int32))
            self.d_step = eng.i32(np.zeros(B, np.int32))
        if self.drafter:
            self.d_anchor = eng.i32(anchors)
            self.d_tok = torch.empty((B, T), dtype=torch.int32, device=eng.dev)
            eng.wf_draft(self.d_slots, self.d_anchor, self.K, self.d_tok)
            blocks = self.d_tok.cpu().numpy()
        else:
            self.d_tok = eng.i32(blocks)
        self.blocks = blocks
        self.d_ntok = eng.i32(np.full(B, T, np.int32))
        self.d_budget = eng.i32(np.full(B, wl.n_max - 1, np.int32))
        self.d_am = torch.empty((B, T), dtype=torch.int32, device=eng.dev)
        self.outs = [torch.empty(B, dtype=torch.int32, device=eng.dev) for _ in range(4)]
        self.d_P = eng.i32(self.P)

    def _sampling_blocks(self, anchors, T):
        """Candidates drawn from q_i = 0.7 p~_i + 0.3 softmax(z_i) (untimed)."""
        from synthetic import rng
        torch, eng, s, B, K = self.torch, self.eng, self.shape, self.B, self.K
        greedy_blk = np.zeros((B, T), np.int32)
        for b in range(B):
            greedy_blk[b, 0] = anchors[b]
            greedy_blk[b, 1:] = self.greedy[b][1:T]
        lg = torch.empty((B, T, s.vocab), dtype=torch.float32, device=eng.dev)
        am = torch.empty((B, T), dtype=torch.int32, device=eng.dev)
        eng.wf_verify_block(self.d_slots, eng.i32(greedy_blk), eng.i32(np.full(B, T, np.int32)),
                            am, lg)
        eng.wf_rollback(self.d_slots, eng.i32(np.zeros(B, np.int32)))
        eng.wf_truncate(self.d_slots, eng.i32(self.P))
        z = lg.cpu().numpy()[:, :K, :] / np.float32(self.temperature)
        z -= z.max(-1, keepdims=True)
        pt = np.exp(z)
        pt /= pt.sum(-1, keepdims=True)
        q = np.empty((B, K, s.vocab), np.float32)
        blocks = np.zeros((B, T), np.int32)
        blocks[:, 0] = anchors
        for b in range(B):
            g = rng(self.wl.cfg_id, 4000 + b)
            for i in range(K):
                zz = g.standard_normal(s.vocab)
                sm = np.exp(zz - zz.max())
                qi = 0.7 * pt[b, i].astype(np.float64) + 0.3 * sm / sm.sum()
                q[b, i] = qi.astype(np.float32)
                blocks[b, i + 1] = g.choice(s.vocab, p=qi / qi.sum())
        self.q_host = q
        self.d_q = torch.from_numpy(q).to(eng.dev)
        del lg
        return blocks

    def step(self):
        e = self.eng
        if self.drafter:
            e.wf_draft(self.d_slots, self.d_anchor, self.K, self.d_tok)
        e.wf_verify_block(self.d_slots, self.d_tok, self.d_ntok, self.d_am, self.d_logits)
        if self.sampling:
            e.wf_accept(self.d_tok, self.d_ntok, self.d_budget, self.d_am, *self.outs,
                        logits=self.d_logits, q=self.d_q, temperature=self.temperature,
                        seed=0, request_id=self.d_req, step=self.d_step)
        else:
            e.wf_accept(self.d_tok, self.d_ntok, self.d_budget, self.d_am, *self.outs)
        e.wf_rollback(self.d_slots, self.outs[0])
        e.wf_truncate(self.d_slots, self.d_P)

    # algorithmic HBM bytes per launch of each kernel kind (weights and KV
    # caches; activations stay in L2 / the Infinity Cache)
    def kind_bytes(self):
        s = self.shape
        d, F, V = s.d_model, s.d_ffn, s.vocab
        T = self.K + 1
        kv_pos = 4 * d                              # fp16 K and V of one position, one layer
        self_bytes = kv_pos * float(np.sum(self.P + T))
        cross_bytes = self.B * s.n_frames * 4.0 * d
        kb = {
            "qkv": 3.0 * d * d * 2 + kv_pos * self.B * T,   # weights + K/V appended
            "oproj": d * d * 2.0, "cross_q": d * d * 2.0, "fc1": d * F * 2.0,
            "fc2": F * d * 2.0, "lm_head": V * d * 2.0, "self_attn": self_bytes,
            "cross_attn": cross_bytes,
        }
        # the persistent pass kernel: every layer and the LM head per launch
        nl = s.n_layers
        kb["pass"] = nl * (kb["qkv"] + 2 * kb["oproj"] + kb["cross_q"] + kb["fc1"] + kb["fc2"]
                           + self_bytes + cross_bytes) + kb["lm_head"]
        return kb

    def pass_bytes(self):
        """bytes_pass = N_L (45.875 MB + sum_b [7.68 MB + 5120 (L_b + n_tok_b)])
        + 132.78 MB at the large-v3 width (weights + caches)."""
        kb = self.kind_bytes()
        nl = self.shape.n_layers
        per_layer = kb["qkv"] + 2 * kb["oproj"] + kb["cross_q"] + kb["fc1"] + kb["fc2"] \
            + kb["self_attn"] + kb["cross_attn"]
        extra = 0.0
        if self.drafter:
            # drafter pass: its layers' weights, its cross K/V and history per
            # request, the LM head; history append in the verify: W_h and
            # each drafter layer's W_k, W_v
            s = self.shape
            d = s.d_model
            nd = self.wl.drafter_layers
            kb_ = self.kind_bytes()
            layer_w = kb_["qkv"] - 4 * d * self.B * (self.K + 1) + 2 * kb_["oproj"] \
                + kb_["cross_q"] + kb_["fc1"] + kb_["fc2"]
            hist = 4.0 * d * float(np.sum(self.P + self.K + 1))
            extra += nd * (layer_w + kb_["cross_attn"] + hist) + kb_["lm_head"]
            extra += 5 * d * d * 2.0 + nd * 2 * d * d * 2.0
        if self.sampling:   # logits written and read back, q read
            extra = self.B * (self.K + 1) * self.shape.vocab * 4.0 * 2 \
                + self.B * self.K * self.shape.vocab * 4.0
        return nl * per_layer + kb["lm_head"] + extra


def cpu_info() -> dict:
    """The host CPU model (/proc/cpuinfo) and the threads this process may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "threads_available": len(os.sched_getaffinity(0))}


def cpu_baseline(w: Workload, timed_s: float = 6.0, wall_s: float = 90.0, threads: int = 0,
                 dtype=np.float32):
    """The oracle, as it stands (numpy; fp32 for timing), running the same
    loop as the device on a bounded sample of the workload: request after
    request (starting over when all have been run), the prompt prefilled
    untimed, then rounds until the request is done or about ``timed_s``
    seconds of timed CPU work. Timed per round: the drafter pass (with the
    engine's drafter), the verify pass of the anchor plus k candidates
    through every layer and the LM head, the acceptance (greedy, or
    rejection sampling at the workload's temperature) and the drafter's
    history append. Built untimed per round: Bernoulli-copy candidates (the
    oracle's own greedy tokens, from single-row passes, up to the first
    replaced position; replacement ids after it, where acceptance has stopped
    either way) or, for sampling, the K single-row probe passes that give
    q_i = 0.7 p~_i + 0.3 softmax(z_i) and the candidates drawn from it.
    ``threads`` > 0 caps the BLAS threads (0: all the process may use)."""
    from oracle import decode as od
    from oracle import drafter as odr
    from oracle import model as om
    from oracle import sampling as osmp
    from synthetic import DRAFTER_TAPS, make_draft_table, rng
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except Exception:   # pragma: no cover - threadpoolctl is installed here
        threadpool_info = threadpool_limits = None
    ctx = threadpool_limits(limits=threads) if (threads and threadpool_limits) else None
    if ctx is not None:
        ctx.__enter__()
    try:
        try:
            used = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
        except Exception:
            used = threads or len(os.sched_getaffinity(0))
        s = w.shape
        K, V, eos, n_max = w.K, s.vocab, s.eos_id, w.wl.n_max
        taps = set(DRAFTER_TAPS) if w.drafter else None
        m = om.Model(s, w.wbits, dtype=dtype)
        dr = odr.Drafter(s, w.wbits, w.dbits, taps=DRAFTER_TAPS, dtype=dtype) if w.drafter else None
        toks = rounds = reqs = 0
        t_total = 0.0
        t_start = time.time()

        def budget_left():
            return t_total < timed_s and time.time() - t_start < wall_s

        n = 0
        while budget_left():
            b = n % w.B
            n += 1
            P = int(w.P[b])
            req = m.new_request(w.encs[b])
            if dr is not None:
                dreq = dr.new_request(w.encs[b])
                lg, tp = m.rows(req, w.prefixes[b], 0, taps=taps)
                dr.append_history(dreq, tp, 0)
            else:
                lg = m.rows(req, w.prefixes[b], 0)
            anchor = od.argmax_lowest(lg[-1])
            keep, repl = make_draft_table(w.wl, b)
            L, emitted, done, step = P, 1, anchor == eos or n_max <= 1, 0
            reqs += 1
            while not done and budget_left():
                R = n_max - emitted
                k = min(K, R - 1, s.n_ctx - L - 1)
                q = None
                drafts = []
                if w.sampling:
                    g = rng(w.wl.cfg_id, 4000 + 1000 * b + step)
                    q = np.empty((k, V), np.float32)
                    tok = anchor
                    for i in range(k):
                        pt = osmp.probs(m.rows(req, [tok], L + i)[0], w.temperature)
                        zz = g.standard_normal(V)
                        sm = np.exp(zz - zz.max())
                        qi = 0.7 * pt.astype(np.float64) + 0.3 * sm / sm.sum()
                        q[i] = qi.astype(np.float32)
                        tok = int(g.choice(V, p=qi / qi.sum()))
                        drafts.append(tok)
                elif dr is None:
                    tok, live = anchor, True
                    for i in range(1, k + 1):
                        live = live and bool(keep[L + i])
                        if live:
                            tok = od.argmax_lowest(m.rows(req, [tok], L + i - 1)[0])
                            drafts.append(tok)
                        else:
                            drafts.append(int(repl[L + i]))
                t0 = time.perf_counter()
                if dr is not None:
                    drafts = odr.draft_tokens(dr.block(dreq, anchor, L, K), K)[:k]
                    lg, tp = m.rows(req, [anchor] + drafts, L, taps=taps)
                else:
                    lg = m.rows(req, [anchor] + drafts, L)
                if w.sampling:
                    a, out, nxt, done = osmp.sample_round(lg.astype(np.float32), q, drafts,
                                                          w.temperature, 0, b, step, eos, R)
                else:
                    a, out, nxt, done = od.greedy_accept(
                        drafts, [od.argmax_lowest(r) for r in lg], eos, R)
                if dr is not None:
                    dr.append_history(dreq, {t: x[:a + 1] for t, x in tp.items()}, L)
                t_total += time.perf_counter() - t0
                toks += len(out)
                rounds += 1
                L += a + 1
                emitted += len(out)
                step += 1
                if nxt is not None:
                    anchor = nxt
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    what = "drafter pass + verify pass" if dr is not None else "verify pass"
    acc = "rejection sampling" if w.sampling else "greedy acceptance"
    return {"value": round(toks / t_total, 3), "unit": "tokens/s", "cores": int(used),
            "kind": "oracle",
            "sample": f"{w.name}: {rounds} rounds of the running loop ({what} of up to "
                      f"K+1 = {K + 1} rows, all {s.n_layers} layers, LM head, {acc}) over "
                      f"{reqs} request(s), {toks} tokens, tau {toks / max(rounds, 1):.2f}, "
                      f"{np.dtype(dtype).name} numpy, {t_total:.2f} s timed; cross K/V, "
                      f"prompts and candidates built untimed by the oracle itself",
            "dtype": np.dtype(dtype).name, "timed_s": round(t_total, 2)}


def _prefill(w: "Workload"):
    from speculative_decoding_encoder_amd.harness import prefill
    w.eng.wf_reset(w.d_slots)
    return prefill(w.eng, w.slots, w.prefixes)


def _fresh_loop(w: "Workload", logits: bool = False):
    """Reset the slots, prefill the prompts (untimed) and set up a device
    round loop from there: the table drafter's candidates per absolute
    position (Bernoulli-copy drafts of the greedy continuation) or the
    engine's drafter."""
    from speculative_decoding_encoder_amd.harness import DeviceLoop, draft_table
    from synthetic import make_draft_table
    s = w.shape
    anchors = _prefill(w)
    table = None
    if not w.drafter and not w.sampling:
        size = s.n_ctx + w.K + 2
        table = np.stack([draft_table(w.greedy[b], int(w.P[b]), *make_draft_table(w.wl, b),
                                      size) for b in range(w.B)])
    return DeviceLoop(w.eng, w.slots, anchors, w.P, w.wl.n_max, w.K, s.eos_id, draft_table=table,
                      drafter=w.drafter, logits=logits)


def _loop_stats(w: "Workload", c0: dict, c1: dict, rounds: int, ms: float, restarts: int) -> dict:
    toks = c1["tokens"] - c0["tokens"]
    rr = c1["request_rounds"] - c0["request_rounds"]
    acc = c1["accepted"] - c0["accepted"]
    prop = c1["proposed"] - c0["proposed"]
    hist = (c1["hist"] - c0["hist"]).astype(np.float64)
    s_k = [float(hist[k:].sum() / max(hist.sum(), 1)) for k in range(1, w.K + 1)]
    return {"rounds_timed": rounds, "ms_per_round": round(ms / rounds, 4),
            "tokens": int(toks), "tokens_per_s": round(toks / (ms * 1e-3), 2),
            "audio_s_per_s": round(toks / (ms * 1e-3) / TOKENS_PER_AUDIO_S, 2),
            "request_rounds": int(rr), "mean_active_batch": round(rr / rounds, 2),
            "tau": round(toks / max(rr, 1), 4), "alpha": round(acc / max(prop, 1), 4),
            "s_k": [round(v, 4) for v in s_k], "restarts": restarts}


def measure_loop(w: "Workload", K: int, W: int, chunk: int = 8) -> dict:
    """The real cached loop over distinct blocks: from the prompts, rounds
    of (the block from the drafter, wf_verify_block, wf_accept, wf_rollback,
    the loop's state update) captured once as a HIP graph; W untimed rounds,
    then K timed rounds, replayed back to back in chunks between HIP events.
    tokens/s counts the tokens the timed rounds emit (realized acceptance),
    tau the tokens per active request-round. When every request has
    finished, the prompts are prefilled again between chunks (untimed) and
    the loop starts over. The table drafter's gather and the state update (a
    few small kernels) are inside the timed region."""
    torch = w.torch
    loop = _fresh_loop(w)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        loop.round()            # the first round eagerly, then capture the next
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            loop.round()
    torch.cuda.synchronize()
    restarts = 0

    def run(n: int) -> float:
        nonlocal restarts
        ms, left = 0.0, n
        while left > 0:
            if loop.counters()["all_done"]:
                loop.restart(_prefill(w), w.P)
                restarts += 1
            c = min(chunk, left)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(c):
                graph.replay()
            e1.record()
            torch.cuda.synchronize()
            ms += e0.elapsed_time(e1)
            left -= c
        return ms

    run(max(W - 2, 1))
    c0 = loop.counters()
    restarts = 0
    ms = run(K)
    c1 = loop.counters()
    err, _ = w.eng.wf_device_state()
    assert (err == 0).all(), f"engine error words {err}"
    del graph
    out = _loop_stats(w, c0, c1, K, ms, restarts)
    log(f"[bench] {w.name}: loop {K} rounds {ms / K:.3f} ms/round, {out['tokens']} tokens, "
        f"tau {out['tau']}")
    return out


def measure_sampling_loop(w: "Workload", K: int, W: int) -> dict:
    """The temperature-sampling loop. Each round the untimed harness builds
    the candidates: for i = 1..K the target's T-tempered
    distribution p~_i at the drafted prefix (single-row GPU passes, kept, then
    truncated back), q_i = 0.7 p~_i + 0.3 softmax(z_i) with z_i ~ N(0, 1), and
    y_i ~ q_i (torch generators seeded by the round). The timed part is the
    round itself (wf_verify_block with the logits, wf_accept with rejection
    sampling, wf_rollback, the counters), replayed from a HIP graph between
    HIP events; the timed rounds are summed."""
    torch, eng, s = w.torch, w.eng, w.shape
    B, Kd, V, T = w.B, w.K, s.vocab, w.temperature
    loop = _fresh_loop(w, logits=True)
    q = torch.empty((B, Kd, V), dtype=torch.float32, device=eng.dev)
    req = eng.i32(np.arange(B, dtype=np.int32))
    probe_am = torch.empty((B, 1), dtype=torch.int32, device=eng.dev)
    probe_lg = torch.empty((B, 1, V), dtype=torch.float32, device=eng.dev)
    zeros = torch.zeros(B, dtype=torch.int32, device=eng.dev)
    gen = torch.Generator(device=eng.dev)
    kw = dict(logits=loop.logits, q=q, temperature=T, seed=0, request_id=req, step=loop.step)

    def harness(rnd):
        gen.manual_seed(1000 + rnd)
        R = loop.n_max - loop.emitted
        room = s.n_ctx - loop.L - 1
        k = torch.clamp(torch.minimum(torch.minimum(torch.full_like(R, Kd), R - 1), room), min=0)
        active = loop.done == 0
        loop.ntok.copy_(torch.where(active, k + 1, torch.zeros_like(k)))
        loop.budget.copy_(torch.clamp(R, min=1))
        L0 = loop.L.clone()
        tok = loop.anchor.clone()
        loop.block[:, 0].copy_(loop.anchor)
        for i in range(Kd):
            live = (active & (k > i)).to(torch.int32)
            eng.wf_verify_block(loop.d_slots, tok[:, None], live, probe_am, probe_lg)
            p = torch.softmax(probe_lg[:, 0, :] / T, dim=-1)
            z = torch.randn((B, V), generator=gen, device=eng.dev)
            qi = 0.7 * p + 0.3 * torch.softmax(z, dim=-1)
            y = torch.multinomial(qi, 1, generator=gen)[:, 0].to(torch.int32)
            q[:, i, :].copy_(qi)
            loop.block[:, i + 1].copy_(torch.where(live > 0, y, torch.zeros_like(y)))
            eng.wf_rollback(loop.d_slots, zeros)
            tok = y
        eng.wf_truncate(loop.d_slots, L0)

    def timed_round():
        loop.verify()
        loop.accept(**kw)
        loop.finish()

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    rnd = 0
    with torch.cuda.stream(stream):
        harness(rnd)
        timed_round()
        rnd += 1
        torch.cuda.synchronize()
        harness(rnd)
        with torch.cuda.graph(graph, stream=stream):
            timed_round()
        rnd += 1
    torch.cuda.synchronize()
    for _ in range(max(W - 2, 0)):
        harness(rnd)
        graph.replay()
        rnd += 1
    torch.cuda.synchronize()
    c0 = loop.counters()
    ms = 0.0
    for _ in range(K):
        harness(rnd)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        ms += e0.elapsed_time(e1)
        rnd += 1
    c1 = loop.counters()
    err, _ = eng.wf_device_state()
    assert (err == 0).all(), f"engine error words {err}"
    del graph
    out = _loop_stats(w, c0, c1, K, ms, 0)
    log(f"[bench] {w.name}: sampling loop {K} rounds {ms / K:.3f} ms/round, "
        f"{out['tokens']} tokens, tau {out['tau']}")
    return out


def measure(w: "Workload", K: int, W: int, use_graph: bool = True) -> dict:
    """Warm up, time K graph-replayed steps, then a second pass of K steps
    with HIP events around every launch for the per-kernel durations."""
    import torch
    eng = w.eng
    for _ in range(max(W, 1)):
        w.step()
    torch.cuda.synchronize()
    n_acc = w.outs[0].cpu().numpy()
    err, lens = eng.wf_device_state()
    assert (err == 0).all() and (n_acc >= 0).all(), "engine reported an error"
    tokens_per_step = int(np.sum(n_acc + 1))
    log(f"[bench] {w.name}: warm-up done")

    stream = torch.cuda.Stream()
    graph = None
    if use_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            w.step()
        torch.cuda.synchronize()
        for _ in range(W):
            graph.replay()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    WINDOW.start()
    t0 = time.perf_counter()
    evs[0].record()
    for i in range(K):
        if graph is not None:
            graph.replay()
        else:
            w.step()
        evs[i + 1].record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    WINDOW.end(w.name)
    ms_step = (t1 - t0) * 1e3 / K
    per_step = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(K)])
    n_acc2 = w.outs[0].cpu().numpy()
    assert np.array_equal(n_acc, n_acc2), "graph replay changed the round's outcome"
    used_graph = graph is not None
    del graph
    log(f"[bench] {w.name}: timed {K} steps, {ms_step:.3f} ms/step")

    # per-kernel durations from HIP events on the engine's stream (eager
    # launches of the same steps)
    eng.wf_set_timing(True)
    for _ in range(K):
        w.step()
    torch.cuda.synchronize()
    kinds = {}
    for i, name in enumerate(KIND_NAMES):
        ms, cnt = eng.wf_get_timing(i)
        if cnt:
            kinds[name] = {"total_ms_per_step": ms / K, "launches_per_step": cnt // K,
                           "avg_us": ms * 1e3 / cnt}
    eng.wf_set_timing(False)
    kb = w.kind_bytes()
    dom = max((k for k in kinds if k in kb), key=lambda k: kinds[k]["total_ms_per_step"])
    achieved = kb[dom] / (kinds[dom]["avg_us"] * 1e-6) / 1e9
    for k in kinds:
        if k in kb:
            kinds[k]["gbs"] = kb[k] / (kinds[k]["avg_us"] * 1e-6) / 1e9
    bytes_pass = w.pass_bytes()
    value = tokens_per_step / (ms_step * 1e-3)
    # acceptance of the round every step repeats: alpha = accepted / proposed
    # candidates, tau = tokens per target call, s_k = P(a >= k),
    # a_k^c = s_k / s_(k-1) (acceptance of candidate k given k - 1 accepted)
    live = n_acc[:w.B]
    s_k = [float(np.mean(live >= k)) for k in range(1, w.K + 1)]
    acc = {"alpha": round(float(live.sum()) / (w.B * w.K), 4) if w.K else None,
           "tau": round(float(np.mean(live + 1)), 4), "s_k": [round(v, 4) for v in s_k],
           "a_k_c": [round(s_k[0], 4)] + [round(s_k[k] / s_k[k - 1], 4) if s_k[k - 1] else None
                                           for k in range(1, w.K)]}
    return {
        "value": value, "ms_step": ms_step, "tokens_per_step": tokens_per_step,
        "step_ms_p10_p50_p90": [round(float(np.percentile(per_step, q)), 4) for q in (10, 50, 90)],
        "acceptance": acc,
        "accepted": [int(a) for a in n_acc[:8]], "bytes_pass": bytes_pass,
        "pass_frac": bytes_pass / (ms_step * 1e-3) / (HBM_PEAK_GBS * 1e9),
        "dom": dom, "achieved": achieved, "dom_bytes": kb[dom],
        "dom_avg_us": kinds[dom]["avg_us"], "kinds": kinds, "graph": used_graph,
    }


def pass_trace(w: "Workload") -> dict:
    """Per-phase picture of one persistent verify pass (switched on for this
    one step; the library's default is the multi-kernel path) from its task trace
    (wf_set_trace: the 100 MHz device clock at each task's start, when its
    inputs were ready, and at its end): per phase, the tasks' summed wait
    and work time over all layers, and the mean per-layer span from the
    first task's start to the last one's end; the kernel's span."""
    from speculative_decoding_encoder_amd.binding import PASS_PHASES, WF_OPT_PERSISTENT
    torch, eng = w.torch, w.eng
    buf = torch.zeros((1 << 17, 4), dtype=torch.int64, device=eng.dev)
    eng.wf_set_option(WF_OPT_PERSISTENT, 1)
    eng.wf_set_trace(buf)
    w.step()
    torch.cuda.synchronize()
    eng.wf_set_trace(None)
    eng.wf_set_option(WF_OPT_PERSISTENT, 0)
    sc = eng.wf_pass_schedule()
    total, per, nl = sc["total"], sc["per_layer"], sc["layers"]
    if total == 0 or total > buf.shape[0]:
        return {}
    tr = buf[:total].cpu().numpy().astype(np.int64)
    t0 = int(tr[:, 0].min())
    out = {"kernel_us": round((int(tr[:, 2].max()) - t0) / 100.0, 2), "tasks": total,
           "grid": sc["grid"], "phases": {}}

    def stats(seg):
        return {"wait_us": round(int((seg[:, 1] - seg[:, 0]).sum()) / 100.0, 1),
                "work_us": round(int((seg[:, 2] - seg[:, 1]).sum()) / 100.0, 1),
                "work_us_per_task": round(float((seg[:, 2] - seg[:, 1]).mean()) / 100.0, 2)}
    offs = sc["ph_off"]
    for k, name in enumerate(PASS_PHASES):
        segs, spans = [], []
        for l in range(nl):
            a, b = l * per + offs[k], l * per + offs[k + 1]
            if b <= a:
                continue
            segs.append(tr[a:b])
            spans.append(int(tr[a:b, 2].max() - tr[a:b, 0].min()))
        if not segs:
            continue
        st = stats(np.concatenate(segs))
        st.update({"tasks_per_layer": offs[k + 1] - offs[k],
                   "span_us_per_layer": round(float(np.mean(spans)) / 100.0, 2)})
        out["phases"][name] = st
    ho = sc["head_off"]
    for k, name in enumerate(["ln_final", "lm_head"]):
        a, b = nl * per + ho[k], nl * per + ho[k + 1]
        st = stats(tr[a:b])
        st.update({"tasks": b - a, "span_us": round(int(tr[a:b, 2].max() - tr[a:b, 0].min()) / 100.0, 2)})
        out["phases"][name] = st
    return out


def traffic_of(workload: str, symbol_kind: str):
    """HBM bytes per launch of a kernel from the committed rocprofv3 counter
    summary (profiles/hbm_traffic.json: FETCH_SIZE and WRITE_SIZE per
    dispatch, each scaled by the factor a copy of known size gives), or
    None when there is none for this workload and kernel, or the kernel
    sources have changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            entries = json.load(f)
    except (OSError, ValueError):
        return None
    h = kernel_source_hash(workload)
    for ent in entries:
        if ent.get("workload") == workload and ent.get("kind") == symbol_kind \
                and ent.get("source_hash") == h:
            return float(ent["hbm_bytes_per_launch"])
    return None


def expected_tau(p: float, K: int) -> float:
    """E[tokens per round] when each candidate independently equals the
    target's token with probability p and acceptance stops at the first
    miss (plus the target's own token): sum_{j=0..K} p^j."""
    return float(sum(p ** j for j in range(K + 1)))


def entry(w: "Workload", r: dict, lp: dict) -> dict:
    """One workload's figures: the running loop (tokens/s at realized
    acceptance), the fixed-block pass (its time against the whole-pass HBM
    bytes) and the dominant kernel's roofline."""
    dom = r["dom"]
    et = None
    if not (w.sampling or w.drafter):
        et = expected_tau(w.wl.p_keep, w.K)
    out = {
        "workload": w.name, "batch": w.B, "layers": w.shape.n_layers,
        "d_model": w.shape.d_model, "K": w.K, "tokens_per_s": lp["tokens_per_s"], "audio_s_per_s": lp["audio_s_per_s"],
        "ms_per_round": lp["ms_per_round"], "tau": lp["tau"], "alpha": lp["alpha"],
        "loop": lp,
        "expected_tau": round(et, 4) if et else None,
        "tokens_per_s_at_expected_tau": round(w.B * et / (r["ms_step"] * 1e-3), 2) if et else None,
        "pass_ms": round(r["ms_step"], 4), "pass_ms_p10_p50_p90": r["step_ms_p10_p50_p90"],
        "pass_bytes": r["bytes_pass"], "pass_roofline_frac": round(r["pass_frac"], 4),
        "dominant_kernel": dom, "dominant_frac": round(r["achieved"] / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "kernel": dom, "symbol": KIND_SYMBOL.get(dom, dom),
                     "achieved": round(r["achieved"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(r["achieved"] / HBM_PEAK_GBS, 4),
                     "traffic": traffic_of(w.name, dom),
                     "bytes_per_launch": r["dom_bytes"], "avg_us": round(r["dom_avg_us"], 3)},
        "kernels_avg_us": {k: round(v["avg_us"], 2) for k, v in r["kinds"].items()},
        "kernels_ms_per_pass": {k: round(v["total_ms_per_step"], 4) for k, v in r["kinds"].items()},
        "encode_kv_s": round(w.encode_kv_s, 4),
    }
    if w.sampling:
        out["temperature"] = w.temperature
    return out


# the metric's batch sizes and the other workloads: key -> (workload id, greedy acceptance)
BATCHES = {"1": (1, False), "32": (4, True), "96": (3, False)}
CONFIGS = {"2": (2, False), "4": (4, False)}


def k_sweep(args):
    """Step time at each K of --k-sweep on one workload (same prompts, weights and
    draft tables; a fresh engine per K). The pages find the verify pass nearly flat
    in K (a few candidates cost little more than one); this measures that here."""
    import torch
    rows = {}
    name = None
    for k in [int(v) for v in args.k_sweep.split(",") if v]:
        w = Workload(args.config, greedy=args.greedy, k=k, batch=args.batch,
                     readout=args.readout)
        r = measure(w, args.steps, args.warmup, use_graph=not args.no_graph)
        name = w.name
        rows[str(k)] = {"ms_per_step": round(r["ms_step"], 4),
                        "tokens_per_step": r["tokens_per_step"],
                        "tokens_per_s": round(r["value"], 2),
                        "verify_rows": w.B * (k + 1)}
        log(f"[bench] K = {k}: {r['ms_step']:.3f} ms/step")
        w.eng.close()
        del w, r
        torch.cuda.empty_cache()
    print(json.dumps({"k_sweep": rows, "workload": name, "batch": args.batch or None,
                      "readout_layer": args.readout if args.readout >= 0 else None,
                      "steps": args.steps,
                      "warmup": args.warmup, "graph": not args.no_graph}), flush=True)


def stream_bandwidth(torch, dev, gib: int = 4) -> float:
    """Device copy of a 4 GiB buffer (past the 256 MB last-level cache):
    bytes read plus written per second, best of 5, in GB/s."""
    n = gib << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    src.fill_(1)
    dst = torch.empty_like(src)
    best = None
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        t = e0.elapsed_time(e1) * 1e-3
        best = t if best is None else min(best, t)
    del src, dst
    torch.cuda.empty_cache()
    return 2 * n / best / 1e9


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, 2.5 PFLOP/s
ENC_AUDIO_S = 30.0              # one encoder window is 30 s of audio
# kernel symbols per kind: the 256 x 256 LDS-copy kernel (template argument:
# the epilogue) on grids of two or more rounds, else the register-staged one
# (epilogue, then the per-wave tile counts: 4, 8 for 128 x 256 tiles, 2, 4
# for 64 x 128)
ENC_SYMBOL = {"stem": "wf::enc::gemm_dma_kernel<0|1>|wf::enc::gemm_kernel<0|1, 4, 8>|<0|1, 2, 4>",
              "qkv": "wf::enc::gemm_dma_kernel<2>|wf::enc::gemm_kernel<2, 4, 8>|<2, 2, 4>",
              "attn": "wf::enc::attn_kernel<2>",
              "oproj": "wf::enc::gemm_dma_kernel<3>|wf::enc::gemm_kernel<3, 4, 8>|<3, 2, 4>",
              "fc1": "wf::enc::gemm_dma_kernel<4>|wf::enc::gemm_kernel<4, 4, 8>|<4, 2, 4>",
              "fc2": "wf::enc::gemm_dma_kernel<3>|wf::enc::gemm_kernel<3, 4, 8>|<3, 2, 4>",
              "ln": "wf::enc::ln_kernel", "other": "wf::enc::mel_kernel"}


def encoder_flops(s, n: int) -> dict:
    """Algorithmic flops per kind for n windows (2 per multiply-add): the two
    stem convolutions, and per block the QKV, attention (QK^T and PV), output
    and MLP products."""
    F, d, f, L, Tm = s.n_frames, s.d_model, s.d_ffn, s.n_layers, 2 * s.n_frames
    return {"stem": 2 * n * (Tm * 3 * s.n_mels * d + F * 3 * d * d),
            "qkv": 2 * n * L * F * d * 3 * d, "attn": 4 * n * L * F * F * d,
            "oproj": 2 * n * L * F * d * d, "fc1": 2 * n * L * F * d * f,
            "fc2": 2 * n * L * F * f * d}


def encoder_cpu_baseline(s, wb, timed_s: float = 12.0) -> dict:
    """The oracle encoder (fp64 numpy) on a bounded sample: the stem and as
    many blocks of one window as fit in about ``timed_s`` seconds; the
    window's time is the stem plus n_layers times the mean block time."""
    from oracle import encoder as oe
    from synthetic import bf16_bits_to_f32, make_mel
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    e = oe.Encoder(s, wb)
    mel = make_mel(s, 0, 0)
    t0 = time.perf_counter()
    x = e.stem(bf16_bits_to_f32(mel).astype(np.float64))
    t_stem = time.perf_counter() - t0
    t_blocks, nb = 0.0, 0
    while nb < s.n_layers and (nb == 0 or t_stem + t_blocks < timed_s):
        t0 = time.perf_counter()
        x = e.block(nb, x)
        t_blocks += time.perf_counter() - t0
        nb += 1
    t_window = t_stem + s.n_layers * t_blocks / nb
    return {"value": round(ENC_AUDIO_S / t_window, 4), "unit": "audio-s/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"one 30 s window: the stem and {nb} of {s.n_layers} blocks timed "
                      f"({t_stem + t_blocks:.2f} s, fp64 numpy), the window's time taken as the "
                      f"stem plus {s.n_layers} x the mean block time ({t_window:.1f} s)"}


def encoder_bench(args):
    """The audio encoder (30 s log-mel windows through the 32-block large-v3
    encoder) on --encoder windows: its own JSON line."""
    import torch
    from synthetic import ENC_LARGE_V3, make_encoder_weights, make_mel
    from speculative_decoding_encoder_amd.binding import ENC_TIMING_KINDS, Encoder
    s = ENC_LARGE_V3
    n = args.encoder
    wb = make_encoder_weights(s, 0)
    enc = Encoder(s, wb, max_batch=n)
    mel = enc.bf16(np.stack([make_mel(s, 0, r) for r in range(n)]))
    out_t = torch.empty((n, s.n_frames, s.d_model), dtype=torch.int16, device=enc.dev)
    st = torch.cuda.current_stream()
    for _ in range(args.warmup):
        enc.wf_encode(mel, out_t, st)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(args.steps):
        enc.wf_encode(mel, out_t, st)
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    log(f"[bench] encoder n = {n}: {ms:.3f} ms per call")
    # per-kind launch durations (HIP events on the launch stream), one call
    enc.set_timing(True)
    enc.wf_encode(mel, out_t, st)
    torch.cuda.synchronize()
    tk = enc.timing()
    enc.set_timing(False)
    fl = encoder_flops(s, n)
    kinds = {}
    for k in ENC_TIMING_KINDS:
        tot, cnt = tk[k]
        if cnt == 0:
            continue
        row = {"ms": round(tot, 4), "launches": cnt, "avg_us": round(tot * 1e3 / cnt, 2)}
        if k in fl and tot > 0:
            row["tflops"] = round(fl[k] / (tot * 1e-3) / 1e12, 1)
        kinds[k] = row
    dom = max((k for k in kinds if k in fl), key=lambda k: kinds[k]["ms"])
    per_launch = fl[dom] / kinds[dom]["launches"]
    achieved = per_launch / (kinds[dom]["avg_us"] * 1e-6) / 1e12
    total_flop = sum(fl.values())
    res = {
        "metric": "encoder audio-s/sec (30 s log-mel windows, 32-block large-v3 encoder); "
                  "% bf16 MFMA roofline",
        "value": round(n * ENC_AUDIO_S / (ms * 1e-3), 2), "unit": "audio-s/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "precision": "bf16 MFMA operands and activations between kernels, fp32 accumulate, "
                     "fp32 residual stream, layer norms, softmax and GELU",
        "data": "synthetic (seeded weights N(0,0.02) in bf16, log-mel features N(0,1))",
        "config": {"workload": f"large-v3 encoder, {n} x 30 s windows", "layers": s.n_layers,
                   "d_model": s.d_model, "n_mels": s.n_mels, "frames": s.n_frames, "batch": n},
        "tflops": round(total_flop / (ms * 1e-3) / 1e12, 1),
        "mfma_frac": round(total_flop / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "roofline": {"bound": "mfma", "kernel": dom, "symbol": ENC_SYMBOL[dom],
                     "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "flop_per_launch": per_launch,
                     "avg_us": kinds[dom]["avg_us"]},
        "kernels": kinds,
    }
    res["roofline"]["traffic"] = traffic_of(res["config"]["workload"], dom)
    if args.calib_copy_mib:
        nb = args.calib_copy_mib << 20
        src = torch.ones(nb, dtype=torch.uint8, device=enc.dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        res["calib_copy_bytes"] = nb
        del src, dst
    if not args.no_cpu:
        t0 = time.time()
        res["cpu_baseline"] = encoder_cpu_baseline(s, wb)
        log(f"[bench] encoder cpu baseline took {time.time() - t0:.1f}s")
    enc.close()
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=1, choices=[1, 2, 3, 4])
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--greedy", action="store_true",
                    help="config 4 with greedy acceptance instead of T = 0.7 sampling")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches")
    ap.add_argument("--batches", default="32,96",
                    help="also measure these batch sizes (32: large-v3 greedy verify, 96: "
                         "large-v3 with the parallel drafter); empty for none")
    ap.add_argument("--configs", default="2,4",
                    help="also measure these workloads (2: turbo batch 32, 4: large-v3 batch 32 "
                         "at T = 0.7); empty for none")
    ap.add_argument("--k-sweep", default="",
                    help="comma-separated K values: time the step of --config at each K "
                         "(the pass cost against the number of candidates) and print that "
                         "as the one JSON line instead")
    ap.add_argument("--readout", type=int, default=-1,
                    help="with --k-sweep: also run the verification-attention anchor "
                         "readout at this decoder layer in every verify pass")
    ap.add_argument("--batch", type=int, default=0,
                    help="with --k-sweep: this many requests instead of the workload's")
    ap.add_argument("--no-stream-bw", action="store_true",
                    help="skip the 4 GiB streaming-copy bandwidth measurement")
    ap.add_argument("--encoder", type=int, default=0,
                    help="time the audio encoder on this many 30 s windows instead (own JSON line)")
    ap.add_argument("--trace", action="store_true",
                    help="also record one persistent pass's task trace per batch and report "
                         "the per-phase busy time and spans under pass_trace")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run device-to-device copies of this size (calibrates "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE against known bytes)")
    ap.add_argument("--mark-timed", action="store_true",
                    help="print the host-clock window of each workload's timed fixed-block "
                         "replays (and of the calibration copies) for cutting a rocprofv3 trace")
    args = ap.parse_args()
    global WINDOW
    WINDOW = Window(args.mark_timed)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the verify path is built and measured on a "
              "single MI355X (requests would shard by data parallelism, with no exchange "
              "between GPUs). --gpus N > 1 is not supported.", file=sys.stderr)
        sys.exit(2)
    import torch
    torch.cuda.set_device(0)
    K, W = args.steps, args.warmup
    if args.k_sweep:
        k_sweep(args)
        return
    if args.encoder:
        encoder_bench(args)
        return
    cpu = {}
    stream_gbs = None
    results = {}
    head_key = None
    # the headline workload first, then the metric's other batch sizes and
    # the other workloads, each on its own engine
    plan = [("config", args.config, args.greedy)]
    for bkey in [b.strip() for b in args.batches.split(",") if b.strip()]:
        if bkey in BATCHES and BATCHES[bkey] != (args.config, args.greedy):
            plan.append(("batch", *BATCHES[bkey]))
    for ckey in [c.strip() for c in args.configs.split(",") if c.strip()]:
        if ckey in CONFIGS and CONFIGS[ckey] != (args.config, args.greedy):
            plan.append(("config", *CONFIGS[ckey]))
    for n, (what, cfg, greedy) in enumerate(plan):
        w = Workload(cfg, greedy=greedy)
        r = measure(w, K, W, use_graph=not args.no_graph)
        lp = measure_sampling_loop(w, K, W) if w.sampling else measure_loop(w, K, W)
        ent = entry(w, r, lp)
        ent["config_id"] = cfg
        if args.trace:
            ent["pass_trace"] = pass_trace(w)
        if n == 0:
            head_key = w.name
            if not args.no_stream_bw:
                stream_gbs = round(stream_bandwidth(torch, w.eng.dev), 1)
            if args.calib_copy_mib:
                nb = args.calib_copy_mib << 20
                src = torch.ones(nb, dtype=torch.uint8, device=w.eng.dev)
                dst = torch.empty_like(src)
                torch.cuda.synchronize()
                WINDOW.start()
                for _ in range(3):
                    dst.copy_(src)
                torch.cuda.synchronize()
                WINDOW.end("calibration-copy")
                ent["calib_copy_bytes"] = nb
                del src, dst
        if not args.no_cpu and (n == 0 or cfg in (2, 3) or w.sampling):
            t0 = time.time()
            if n == 0:
                cpu[cfg] = cpu_baseline(w, timed_s=8.0)
                cpu["threads_1"] = cpu_baseline(w, timed_s=5.0, threads=1)
            else:
                cpu[cfg] = cpu_baseline(w, timed_s=4.0)
            log(f"[bench] {w.name}: cpu baseline took {time.time() - t0:.1f}s")
        results[w.name] = (w.B, cfg, ent)
        log(f"[bench] {w.name}: pass {r['ms_step']:.3f} ms, loop {lp['ms_per_round']:.3f} "
            f"ms/round, {lp['tokens_per_s']:.1f} tokens/s")
        w.eng.close()
        del w, r
        torch.cuda.empty_cache()

    B0, cfg0, head = results[head_key]
    out = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": head["ms_per_round"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "precision": "fp16 activations and attention operands, bf16 weights (converted to "
                     "fp16 in registers), fp32 accumulate, fp32 residual stream, softmax and "
                     "layer-norm statistics",
        "data": "synthetic (seeded weights N(0,0.02) in bf16, audio memory N(0,1), "
                "Bernoulli-copy drafts of the engine's own greedy continuation)",
        "config": {"workload": head_key, "layers": head["layers"], "d_model": head["d_model"],
                   "batch": B0, "K": head["K"], "graph": not args.no_graph,
                   "step": "one round of the running loop: drafts, wf_verify_block, wf_accept, "
                           "wf_rollback, loop state"},
        "audio_s_per_s": head["audio_s_per_s"],
        "tau": head["tau"],
        "expected_tau": head["expected_tau"],
        "tokens_per_s_at_expected_tau": head["tokens_per_s_at_expected_tau"],
        "pass": {"ms": head["pass_ms"], "bytes": head["pass_bytes"],
                 "roofline_frac_of_step": head["pass_roofline_frac"]},
        "roofline": head["roofline"],
        "batches": {}, "configs": {},
    }
    if stream_gbs:
        out["stream_gbs"] = stream_gbs
        out["pass"]["stream_frac"] = round(head["pass_bytes"] / (head["pass_ms"] * 1e-3)
                                           / (stream_gbs * 1e9), 4)
    for name, (B, cfg, ent) in results.items():
        if ent is head or cfg in (1, 3) or (cfg == 4 and "greedy" in name):
            out["batches"][str(B)] = ent
        if cfg in (2, 4) and "greedy" not in name:
            out["configs"][str(cfg)] = ent
    if cpu:
        base = dict(cpu[cfg0])
        base.update(cpu_info())
        if "threads_1" in cpu:
            base["threads_1"] = {k: cpu["threads_1"][k] for k in ("value", "cores", "timed_s")}
        base["configs"] = {str(c): {k: v[k] for k in ("value", "unit", "cores", "sample")}
                           for c, v in cpu.items() if c not in (cfg0, "threads_1")}
        out["cpu_baseline"] = base
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
