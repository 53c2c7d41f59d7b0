"""Shared helpers for the GPU tests: engine construction from the seeded
workloads and the comparison rules against the oracle.

Comparison protocol (tolerances of the verify path):
* logits: max |GPU - oracle| <= 2e-2 over every compared row and id;
* argmax: identical wherever the oracle's top-2 margin exceeds 5e-2;
* accepted length: identical when every position it depends on clears
  that margin.
"""
import numpy as np

LOGIT_TOL = 2e-2
MARGIN = 5e-2


def margins(logits: np.ndarray) -> np.ndarray:
    top2 = np.sort(logits, axis=-1)[..., -2:]
    return top2[..., 1] - top2[..., 0]


def assert_logits_close(gpu: np.ndarray, ref: np.ndarray, tol: float = LOGIT_TOL, what=""):
    err = float(np.abs(gpu.astype(np.float64) - ref).max())
    print(f"[parity] {what}: max |logit error| {err:.3e}", flush=True)
    assert err <= tol, f"{what}: max |logit error| {err:.3e} > {tol}"
    return err


def assert_argmax_where_clear(gpu_am: np.ndarray, ref_logits: np.ndarray, what=""):
    m = margins(ref_logits)
    ref_am = ref_logits.argmax(-1)
    clear = m > MARGIN
    bad = np.flatnonzero((gpu_am != ref_am) & clear)
    assert bad.size == 0, f"{what}: argmax differs at clear-margin rows {bad[:10]}"
    return int(clear.sum()), int(clear.size)


def oracle_accept_pinned(drafts, ref_logits, k):
    """The oracle's accepted length and next token, and whether the GPU
    must match them: every row they read (0..a) has a clear margin."""
    g = ref_logits.argmax(-1)
    a = 0
    while a < k and drafts[a] == g[a]:
        a += 1
    m = margins(ref_logits)
    # rows 0..a-1 decide the acceptance, row a gives the next token
    pinned = bool((m[:a + 1] > MARGIN).all())
    return a, int(g[a]), pinned


def log(*a):
    print(*a, flush=True)
