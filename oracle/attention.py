"""Sparse attention over the selected slots of the device cache: the consumer
of ``sel_slot`` (TEST INFRASTRUCTURE ONLY; see the package docstring).

The ECHO Guide blog ("CUDA Graph Compatibility via Pre-Allocated Tensor
Pointers"; "Step 3: Implement GPU-Side Indirection Tensors") has the
attention kernel read a fixed device pool through an index tensor that the
cache step rewrites each step, so the kernel never binds new addresses; the
output is that of attention over the selected tokens held in full precision
in HBM (the method is lossless). The pages do not print the attention
itself. Reading taken: DeepSeek-V3.2-style absorbed MLA decode over
576-value rows, all 576 values forming the key and the first 512 the value;
the query of each head has 576 values; softmax over the selected tokens with
a caller-given scale; entries outside [0, C) select nothing.

Plain float64 numpy: gather, one matrix product for the scores, the
textbook softmax, one matrix product for the output.
"""
import numpy as np

from .numerics import bf16_to_f64

D_ROW = 576   # key width: 512 latent + 64 rotary values
D_V = 512     # value width: the latent part of the row


def sparse_attention(q_bits: np.ndarray, cache_bits: np.ndarray, sel_slot: np.ndarray, sm_scale: float):
    """q_bits [B, H, 576] bf16 bits; cache_bits [C, 576] bf16 bits (the
    device cache); sel_slot [B, k] slot ids, entries < 0 or >= C skipped.

    Returns out [B, H, 512] and lse [B, H] (natural log of the softmax
    denominator, scaled scores), float64; a sequence that selects nothing
    gets zeros and -inf."""
    q_bits = np.asarray(q_bits)
    B, H, _ = q_bits.shape
    C = cache_bits.shape[0]
    scale = float(np.float32(sm_scale))
    out = np.zeros((B, H, D_V))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        sl = np.asarray(sel_slot[b], np.int64)
        sl = sl[(sl >= 0) & (sl < C)]
        if len(sl) == 0:
            continue
        rows = bf16_to_f64(cache_bits[sl])           # [n, 576]
        q = bf16_to_f64(q_bits[b])                   # [H, 576]
        s = (q @ rows.T) * scale                     # [H, n]
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        den = p.sum(axis=1, keepdims=True)
        out[b] = (p @ rows[:, :D_V]) / den
        lse[b] = (m + np.log(den))[:, 0]
    return out, lse
