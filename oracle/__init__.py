"""CPU oracle for Whisper-shaped block verification — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct numpy implementation of what the verify
path computes. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the GPU engine never
does, and the oracle imports nothing from the engine (it shares only the
seeded input generators in ``synthetic``).

Sources (page titles; sections as printed on each page):

* "Whisper-Flash: Acoustically Conditioned Parallel Drafting for Faster
  Whisper Decoding" — §3.1 (eq. 1, propose/verify/advance, rejection rule),
  §3.2 (drafter memories, eq. 2), App. A.1 (anchor, cache length L+1+a, EOS,
  budget R-1), A.2 (history taps, RoPE), A.4 (temperature sampling in FP32),
  A.5 (preallocated caches, masked rejected positions, ties).
* "Alignment Drift in Single-Model Speculative Decoding for ASR" —
  §"Speculative Loop" (s_k, a_k^c, L), App. A.4 (bf16 vs fp32 argmax flips).
* SGLang-Omni "Whisper ASR" cookbook — "Breakable Prefill CUDA Graph"
  (cross-attention K/V written once per request, then only read) and
  "Known Limitations" (448-token decoder context).

Modules: ``model`` (decoder rows, cross K/V), ``decode`` (greedy accept,
rollback, greedy / speculative / brute-force loops), ``philox``
(Philox4x64-10), ``sampling`` (temperature rejection sampling).
"""
