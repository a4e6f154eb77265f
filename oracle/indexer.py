"""Lightning-indexer scores, the first stage of the path.

For a query row r with per-head query vectors q[r, h, :] (bf16) and head
weights w[r, h] (fp32), the score of cached token t is

    logit[r, t] = sum_h  w[r, h] * ReLU( q[r, h, :] . k[g, :] ),   g = tok0_r + t,

over every visible token t < len_r (ECHO explainer, "Decode: fetch above a
predicted threshold": the selection runs over indexer scores of all cached
tokens; the fused indexer kernel section names the kernel that computes them).
The formula itself is the standard lightning-indexer form; the pages do not
print it. Keys are bf16, or e4m3fn with one fp32 scale per token that
multiplies all D entries of that token's key: k[g, :] = e4m3(k8[g, :]) * s[g].
There is no other normalisation. Causal prefill is the special case
tok0_r = sequence start and len_r = (position of row r) + 1 (token t is visible
to query row r iff t <= r).

Everything is float64: decoded inputs are exact in float64, products and sums
use numpy's float64 matmul as a primitive. No blocking beyond splitting a long
row into token chunks to bound memory.
"""
from typing import Optional, Sequence

import numpy as np

from .numerics import bf16_to_f64, e4m3fn_to_f64

TOKEN_CHUNK = 1 << 16


def dequant_keys(key_bits: np.ndarray, kdtype: str, scale: Optional[np.ndarray],
                 lo: int, hi: int) -> np.ndarray:
    """Keys of tokens [lo, hi) as float64 [hi-lo, D]."""
    if kdtype == 'bf16':
        return bf16_to_f64(key_bits[lo:hi])
    if kdtype == 'fp8':
        k = e4m3fn_to_f64(key_bits[lo:hi])
        return k * np.asarray(scale[lo:hi], dtype=np.float64)[:, None]
    raise ValueError(kdtype)


def _row_scores(q64: np.ndarray, w64: np.ndarray, key_bits, kdtype, scale, g0: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    for a in range(0, n, TOKEN_CHUNK):
        b = min(n, a + TOKEN_CHUNK)
        k = dequant_keys(key_bits, kdtype, scale, g0 + a, g0 + b)   # [m, D]
        dots = q64 @ k.T                                             # [H, m]
        out[a:b] = w64 @ np.maximum(dots, 0.0)                       # [m]
    return out


def index_logits(q_bits: np.ndarray, w: np.ndarray, key_bits: np.ndarray, kdtype: str,
                 scale: Optional[np.ndarray], tok0: Sequence[int], lens: Sequence[int]) -> list:
    """Scores for R query rows. q_bits [R, H, D] bf16 bits, w [R, H] fp32,
    key_bits [P, D] (uint16 bf16 | uint8 e4m3fn), scale [P] fp32 or None,
    tok0/lens per row. Returns a list of float64 arrays, row r of length lens[r]."""
    q_bits = np.asarray(q_bits)
    R = q_bits.shape[0]
    res = []
    for r in range(R):
        q64 = bf16_to_f64(q_bits[r])
        w64 = np.asarray(w[r], dtype=np.float64)
        res.append(_row_scores(q64, w64, key_bits, kdtype, scale, int(tok0[r]), int(lens[r])))
    return res


def index_logit_at(q_bits_row: np.ndarray, w_row: np.ndarray, key_bits: np.ndarray, kdtype: str,
                   scale: Optional[np.ndarray], g: Sequence[int]) -> np.ndarray:
    """Scores of one query row at selected global token ids g (one by one)."""
    q64 = bf16_to_f64(q_bits_row)
    w64 = np.asarray(w_row, dtype=np.float64)
    out = np.empty(len(g), dtype=np.float64)
    for i, gi in enumerate(g):
        k = dequant_keys(key_bits, kdtype, scale, int(gi), int(gi) + 1)[0]
        out[i] = float(w64 @ np.maximum(q64 @ k, 0.0))
    return out
