"""Seeded synthetic inputs for the indexer -> exact top-k -> KV-recall path.

This module only draws random inputs. It holds none of the method's
arithmetic: no indexer score, no selection, no threshold update and no slot
allocation. Both the CPU oracle (``oracle/``) and the HIP path
(``indexer_top_kv_amd``) consume what it produces, and neither is imported here.

Workload shapes follow the decode and prefill settings of the ECHO pages:
device cache sizes of 260 000, 200 000 and 110 000 slots come from the
artifact README ("Figure 13 - constrained GPU pool size" and the option tables
of the end-to-end scripts); k = 2048 and the EMA threshold come from the ECHO
explainer ("Decode: fetch above a predicted threshold"). Key/row formats (64
heads x 128 dims indexer keys, 576-bf16 KV rows of 1152 bytes) and the value
distributions are the synthetic stand-ins for DeepSeek-V3.2 and the
InfiniteBench 100K-110K requests, which are not available here.

Seeds: every array is drawn from ``numpy.random.default_rng([20261202, cfg,
stream, *extra])``; streams are 0 keys, 1 key scales, 2 q0, 3 q innovations,
4 head weights, 5 host rows, 6 lengths, 7 topic-shift draws. Large arrays are
drawn in fixed-size chunks, each with its own seed, so results do not depend on
thread count. Layer l > 0 of a workload appends 1000000 + l to the seed of
every draw except the lengths, which all layers share.

Casts to bf16 and to OCP e4m3fn use torch's round-to-nearest-even conversions
(``torch.bfloat16``, ``torch.float8_e4m3fn``); fp8 inputs are clamped to
+-448 first. Arrays are returned as raw bit patterns (uint16 for bf16, uint8
for e4m3fn) so neither side depends on a float8 numpy dtype.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Iterator, Optional

import numpy as np
import torch

SEED_ROOT = 20261202
S_KEYS, S_SCALE, S_Q0, S_QINNOV, S_W, S_ROWS, S_LENS, S_SHIFT = range(8)

H = 64          # indexer heads
D = 128         # indexer head dim
ROW_ELEMS = 576  # bf16 values per KV row
ROW_BYTES = 2 * ROW_ELEMS  # 1152
CHUNK_ROWS = 1 << 20  # rows per independently seeded chunk


def rng(cfg: int, stream: int, *extra: int) -> np.random.Generator:
    return np.random.default_rng([SEED_ROOT, cfg, stream, *extra])


def wl_rng(wl: 'Workload', stream: int, *extra: int) -> np.random.Generator:
    """The generator of one draw of a workload's layer: layer 0 uses the plain
    seed, layer l > 0 appends 1000000 + l (lengths are not drawn here: every
    layer shares them)."""
    if wl.layer == 0:
        return rng(wl.cfg, stream, *extra)
    return rng(wl.cfg, stream, *extra, 1000000 + wl.layer)


def _threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


# ---------------------------------------------------------------- casts

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_e4m3_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> OCP e4m3fn bit patterns (uint8), clamped to +-448, RNE."""
    x = np.clip(np.ascontiguousarray(x, dtype=np.float32), -448.0, 448.0)
    return torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# ---------------------------------------------------------------- configs

@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload. ``variant='dyadic'`` swaps every float draw for
    small integers / powers of two so that all scores are exact in fp32 (used
    for end-to-end bit-exact checks); shapes are unchanged."""

    name: str
    cfg: int                 # seed index
    mode: str                # 'decode' | 'prefill'
    B: int                   # sequences (prefill: 1)
    N: int                   # context length (C4: max of the length range)
    kdtype: str              # 'bf16' | 'fp8'
    C: int                   # device cache slots
    steps: int               # decode steps (prefill: 1 pass)
    k: int = 2048
    cap: int = 512           # early-fetch cap per sequence
    rho: float = 0.9         # AR(1) coefficient of q
    innov: Optional[float] = None  # innovation std; default sqrt(1 - rho^2)
    resample_p: float = 0.0  # per-sequence per-step probability of a fresh q
    len_lo: Optional[int] = None   # lengths ~ U{len_lo..N} when set
    block_rows: int = 4096   # prefill query block
    variant: str = 'normal'  # 'normal' | 'dyadic'
    layer: int = 0           # model layer: its own keys, scales, weights, queries and rows

    # ---- derived sizes
    @property
    def lens(self) -> np.ndarray:
        if self.len_lo is None:
            return np.full(self.B, self.N, dtype=np.int32)
        r = rng(self.cfg, S_LENS)
        return r.integers(self.len_lo, self.N + 1, size=self.B).astype(np.int32)

    @property
    def tok0(self) -> np.ndarray:
        lens = self.lens.astype(np.int64)
        return np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)

    @property
    def P(self) -> int:
        return int(self.lens.astype(np.int64).sum())

    @property
    def innovation(self) -> float:
        if self.innov is not None:
            return self.innov
        return float(np.sqrt(1.0 - self.rho * self.rho))

    def scaled(self, **kw) -> 'Workload':
        return dataclasses.replace(self, **kw)


CONFIGS = {
    # Single-sequence decode, bf16 keys, 4 steps, q_{s+1} = 0.9 q_s + 0.44 eps.
    'decode-1x16k-bf16': Workload('decode-1x16k-bf16', 0, 'decode', B=1, N=16384,
                                  kdtype='bf16', C=4096, steps=4, rho=0.9, innov=0.44),
    # Decode batch of 32 x 128K contexts, fp8 keys + per-token scales.
    'decode-32x128k-fp8': Workload('decode-32x128k-fp8', 1, 'decode', B=32, N=131072,
                                   kdtype='fp8', C=260000, steps=32, rho=0.9),
    # Causal prefill of one 110 000-token sequence in 4096-row query blocks.
    'prefill-110k-fp8': Workload('prefill-110k-fp8', 2, 'prefill', B=1, N=110000,
                                 kdtype='fp8', C=110000, steps=1),
    # Capacity-constrained decode: 64 x U{100000..110000}, topic shifts p=0.2.
    'decode-64x110k-fp8-capacity': Workload('decode-64x110k-fp8-capacity', 3, 'decode', B=64,
                                            N=110000, len_lo=100000, kdtype='fp8', C=110000,
                                            steps=16, rho=0.9, resample_p=0.2),
    # Long-context decode, 4 x 1M tokens, AR(1) rho = 0.95.
    'decode-4x1m-fp8': Workload('decode-4x1m-fp8', 4, 'decode', B=4, N=1048576,
                                kdtype='fp8', C=200000, steps=64, rho=0.95),
}
CONFIG_ORDER = list(CONFIGS)


def get(name: str) -> Workload:
    return CONFIGS[name]


# ---------------------------------------------------------------- draws

def _chunked(n_rows: int, fn, out: np.ndarray) -> np.ndarray:
    """Fill out[rows] chunk by chunk; fn(chunk_index, lo, hi) -> array."""
    n_chunks = (n_rows + CHUNK_ROWS - 1) // CHUNK_ROWS

    def work(c):
        lo = c * CHUNK_ROWS
        hi = min(n_rows, lo + CHUNK_ROWS)
        out[lo:hi] = fn(c, lo, hi)

    if n_chunks <= 1:
        for c in range(n_chunks):
            work(c)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(n_chunks)))
    return out


def keys(wl: Workload) -> tuple[np.ndarray, Optional[np.ndarray]]:
    """Indexer key cache for all P tokens, token-major [P, D].

    bf16: N(0,1) -> bf16 bits (uint16). fp8: N(0,1) -> e4m3fn bits (uint8)
    with a per-token fp32 scale ~ U(0.5, 2). Dyadic variant: integers in
    [-8, 8] and scales in {0.5, 1, 2}.
    """
    P = wl.P
    dyadic = wl.variant == 'dyadic'
    if wl.kdtype == 'bf16':
        out = np.empty((P, D), dtype=np.uint16)

        def f(c, lo, hi):
            r = wl_rng(wl, S_KEYS, c)
            if dyadic:
                x = r.integers(-8, 9, size=(hi - lo, D)).astype(np.float32)
            else:
                x = r.standard_normal((hi - lo, D), dtype=np.float32)
            return to_bf16_bits(x)
        return _chunked(P, f, out), None
    out = np.empty((P, D), dtype=np.uint8)

    def f8(c, lo, hi):
        r = wl_rng(wl, S_KEYS, c)
        if dyadic:
            x = r.integers(-8, 9, size=(hi - lo, D)).astype(np.float32)
        else:
            x = r.standard_normal((hi - lo, D), dtype=np.float32)
        return to_e4m3_bits(x)
    _chunked(P, f8, out)
    r = wl_rng(wl, S_SCALE)
    if dyadic:
        scale = np.array([0.5, 1.0, 2.0], dtype=np.float32)[r.integers(0, 3, size=P)]
    else:
        scale = r.uniform(0.5, 2.0, size=P).astype(np.float32)
    return out, scale


def head_weights(wl: Workload, rows: Optional[int] = None, row0: int = 0) -> np.ndarray:
    """Head weights w_h ~ U(0,1)/8 as fp32, one vector per decode sequence
    (fixed over steps) or per prefill query row. Dyadic: m/64, m in 0..8."""
    if wl.mode == 'decode':
        r = wl_rng(wl, S_W)
        if wl.variant == 'dyadic':
            return (r.integers(0, 9, size=(wl.B, H)) / 64.0).astype(np.float32)
        return (r.uniform(0.0, 1.0, size=(wl.B, H)) / 8.0).astype(np.float32)
    rows = wl.N if rows is None else rows
    out = np.empty((rows, H), dtype=np.float32)
    # prefill: one seeded stream per block of query rows
    for blk in range(row0 // wl.block_rows, (row0 + rows + wl.block_rows - 1) // wl.block_rows):
        lo = blk * wl.block_rows
        hi = min(wl.N, lo + wl.block_rows)
        r = wl_rng(wl, S_W, blk)
        if wl.variant == 'dyadic':
            wb = (r.integers(0, 9, size=(hi - lo, H)) / 64.0).astype(np.float32)
        else:
            wb = (r.uniform(0.0, 1.0, size=(hi - lo, H)) / 8.0).astype(np.float32)
        a, b = max(lo, row0), min(hi, row0 + rows)
        out[a - row0:b - row0] = wb[a - lo:b - lo]
    return out


def decode_queries(wl: Workload, steps: Optional[int] = None) -> Iterator[np.ndarray]:
    """Yield q for each decode step as bf16 bits [B, H, D].

    Normal: q_0 ~ N(0,1); q_{s+1} = rho q_s + innov eps_s with the AR state
    kept in fp32 and cast to bf16 each step; with resample_p > 0 each
    sequence draws a fresh N(0,1) q with that probability instead (topic
    shift). Dyadic: integers in [-3, 3]; each element is redrawn with
    probability 1 - rho per step (and whole sequences with resample_p).
    """
    steps = wl.steps if steps is None else steps
    shape = (wl.B, H, D)
    r0 = wl_rng(wl, S_Q0)
    dyadic = wl.variant == 'dyadic'
    if dyadic:
        state = r0.integers(-3, 4, size=shape).astype(np.float32)
    else:
        state = r0.standard_normal(shape, dtype=np.float32)
    for s in range(steps):
        yield to_bf16_bits(state)
        ri = wl_rng(wl, S_QINNOV, s)
        rs = wl_rng(wl, S_SHIFT, s)
        if dyadic:
            fresh = ri.integers(-3, 4, size=shape).astype(np.float32)
            redraw = ri.random(shape) < (1.0 - wl.rho)
            nxt = np.where(redraw, fresh, state).astype(np.float32)
        else:
            eps = ri.standard_normal(shape, dtype=np.float32)
            nxt = (np.float32(wl.rho) * state + np.float32(wl.innovation) * eps).astype(np.float32)
        if wl.resample_p > 0.0:
            shift = rs.random(wl.B) < wl.resample_p
            if shift.any():
                if dyadic:
                    new = rs.integers(-3, 4, size=(int(shift.sum()), H, D)).astype(np.float32)
                else:
                    new = rs.standard_normal((int(shift.sum()), H, D), dtype=np.float32)
                nxt[shift] = new
        state = nxt


def prefill_queries(wl: Workload, row0: int, rows: int) -> np.ndarray:
    """Prefill query rows [rows, H, D] as bf16 bits, i.i.d. N(0,1) (dyadic:
    integers in [-3, 3]), one seeded stream per query block."""
    out = np.empty((rows, H, D), dtype=np.uint16)
    for blk in range(row0 // wl.block_rows, (row0 + rows + wl.block_rows - 1) // wl.block_rows):
        lo = blk * wl.block_rows
        hi = min(wl.N, lo + wl.block_rows)
        r = wl_rng(wl, S_Q0, blk)
        if wl.variant == 'dyadic':
            x = r.integers(-3, 4, size=(hi - lo, H, D)).astype(np.float32)
        else:
            x = r.standard_normal((hi - lo, H, D), dtype=np.float32)
        a, b = max(lo, row0), min(hi, row0 + rows)
        out[a - row0:b - row0] = to_bf16_bits(x[a - lo:b - lo])
    return out


def host_rows(wl: Workload, out: Optional[np.ndarray] = None) -> np.ndarray:
    """KV rows of the host pool, [P, 576] bf16 bits ~ N(0,1), 1152 B each.
    ``out`` may be a view of pinned memory (uint16 [P, 576])."""
    P = wl.P
    if out is None:
        out = np.empty((P, ROW_ELEMS), dtype=np.uint16)
    assert out.shape == (P, ROW_ELEMS) and out.dtype == np.uint16

    def f(c, lo, hi):
        r = wl_rng(wl, S_ROWS, c)
        return to_bf16_bits(r.standard_normal((hi - lo, ROW_ELEMS), dtype=np.float32))
    return _chunked(P, f, out)


def random_logits(cfg: int, rows: int, n: int, kind: str = 'normal', seed_extra: int = 0) -> np.ndarray:
    """fp32 score rows for selection tests, drawn directly (not computed from
    keys). kinds: 'normal' N(18, 4); 'ties' integers in [0, 64); 'const' all
    equal; 'signed' N(0,1) with some exact +-0.0 entries."""
    r = rng(cfg, S_SHIFT, 1000 + seed_extra)
    if kind == 'normal':
        x = (18.0 + 4.0 * r.standard_normal((rows, n))).astype(np.float32)
    elif kind == 'ties':
        x = r.integers(0, 64, size=(rows, n)).astype(np.float32)
    elif kind == 'const':
        x = np.full((rows, n), 3.5, dtype=np.float32)
    elif kind == 'signed':
        x = r.standard_normal((rows, n)).astype(np.float32)
        z = r.random((rows, n)) < 0.05
        x[z] = np.where(r.random(int(z.sum())) < 0.5, np.float32(0.0), np.float32(-0.0))
    else:
        raise ValueError(kind)
    return x
