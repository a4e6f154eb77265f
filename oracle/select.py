"""Exact top-k over one row of scores, and the EMA threshold.

Top-k (ECHO explainer: the selection is exact, per its opening summary;
k = 2048 in "Decode: fetch above a predicted threshold"). The result has a plain
definition, so the oracle is that definition: sort the row's scores in
descending order with a stable sort (equal scores keep ascending token order,
i.e. ties go to the lower index) and keep the first min(k, len) positions.

    order  = stable argsort of -score
    S      = sorted(order[:min(k, len)])         ascending token index
    kth    = score[order[min(k, len) - 1]]        the smallest selected score

Rows with len <= k select every visible token. Output rows are padded with -1
up to k. An empty row selects nothing and has kth = NaN. -0.0 and +0.0 are
equal scores (the sort compares values). Scores must be finite.

The 256-bin histogram of the threshold-shifted score ("Prefill:
one-round histogram") is how a kernel finds this set fast; it does not change
the set, so the oracle does not model it.

Threshold (ECHO explainer, "Decode: fetch above a predicted threshold": the
predictor is an EMA with alpha = 0.5 of the previous step's k-th score).
theta is float32 state. Before the first step it is NaN (no prediction). After
a step with k-th score kth:
    theta <- kth                          if theta is NaN
    theta <- fl32(fl32(kth + theta) * 0.5) otherwise
alpha = 0.5 makes 0.5*kth + 0.5*theta = (kth + theta) * 0.5, and halving is
exact in binary floating point, so one rounding (of the sum) is the whole
arithmetic. An empty row (kth NaN) leaves theta unchanged. Because theta
decides which tokens are fetched early (score > theta), both the oracle and
the GPU keep it in float32.
"""
import numpy as np


def topk_row(scores: np.ndarray, k: int):
    """scores: 1-D float32 (the row's visible tokens). Returns (idx[k] int64
    ascending with -1 padding, kth float32)."""
    s = np.asarray(scores, dtype=np.float32)
    n = s.shape[0]
    m = min(k, n)
    idx = np.full(k, -1, dtype=np.int64)
    if m == 0:
        return idx, np.float32(np.nan)
    order = np.argsort(-s, kind='stable')
    idx[:m] = np.sort(order[:m])
    return idx, s[order[m - 1]]


def topk_rows(rows, k: int):
    """rows: sequence of 1-D float32 arrays. Returns (idx [R, k], kth [R])."""
    out = [topk_row(r, k) for r in rows]
    idx = np.stack([o[0] for o in out]) if out else np.zeros((0, k), np.int64)
    kth = np.array([o[1] for o in out], dtype=np.float32)
    return idx, kth


def theta_next(theta, kth) -> np.float32:
    theta = np.float32(theta)
    kth = np.float32(kth)
    if np.isnan(kth):
        return theta
    if np.isnan(theta):
        return kth
    return np.float32(np.float32(kth + theta) * np.float32(0.5))


def theta_rows(theta: np.ndarray, kth: np.ndarray) -> np.ndarray:
    return np.array([theta_next(t, x) for t, x in zip(theta, kth)], dtype=np.float32)
