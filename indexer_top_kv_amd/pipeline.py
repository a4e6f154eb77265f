r"""One layer of the path, launched in order on up to three streams.

Decode step (ECHO explainer, "The top-k dependency" and "Decode: fetch above
a predicted threshold"): the recall of a step depends on its top-k; the early
fetch of tokens scoring above the predicted threshold starts before it:

    S0: ech_index_logits --> ech_topk(theta -> theta') --> FINAL maps --> FINAL recall
         \-> S1: EARLY(theta) maps -----/--> EARLY recall (PCIe) ----/

With fp8 keys the scores and the early fetch are one launch
(ech_index_logits_early): the early misses of a sequence get their slots, and
their rows start crossing PCIe, while later sequences are still being scored;
a copier on S1 takes them as they appear and, once S0 has the FINAL maps,
goes on to the FINAL rows with the link still busy:

    S0: scores + EARLY maps + band lists (one launch) --> ech_topk_early --> FINAL maps --> rest of both lists
    S1: live copier: early rows as allocated, then the FINAL rows ---------------------------/

theta is double-buffered (the early fetch reads the prediction while the
top-k writes its update). When the batch's
selections do not fit the cache at once (sum of min(k, len_b) > C),
sequences are processed in host-computed chunks, each an ECH_EARLY phase
then a FINAL phase; every selected token is resident at the end of its chunk.

Several layers (DecodeStack): one DecodeLayer per (layer, micro-batch), the
layers of a micro-batch in order, two micro-batches interleaved so that one
crosses PCIe while the other scores.

Prefill (ECHO explainer, "Prefill: one-round histogram"): query blocks are
scored one after another; the recall of block i runs on S1 while S0 scores
block i+1.

Nothing here computes: this module sizes buffers with torch, chooses the
order of the C-ABI calls and the stream events between them.
"""
from __future__ import annotations

from typing import List, Optional, Tuple

import numpy as np
import torch

from . import (ECH_EARLY, ECH_FINAL, ECH_PREFILL, LayerState, ech_cache_reset, ech_cache_step,
               ech_cache_step_ws_bytes, ech_index_logits, ech_index_logits_causal, ech_index_logits_early,
               ech_index_logits_early_ws_bytes, ech_kv_append, ech_recall, ech_recall_early_live, ech_recall_rest,
               ech_topk, ech_topk_early, ech_topk_ws_bytes)


def round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


def sequence_groups(B: int, groups: int) -> List[Tuple[int, int]]:
    """Split sequences 0..B-1 into at most `groups` consecutive ranges of
    nearly equal size."""
    g = max(1, min(int(groups), B))
    bounds = [round(i * B / g) for i in range(g + 1)]
    return [(bounds[i], bounds[i + 1]) for i in range(g) if bounds[i + 1] > bounds[i]]


def sequence_chunks(lens: np.ndarray, k: int, C: int) -> List[Tuple[int, int]]:
    """Split sequences into consecutive chunks, each the longest prefix of the
    remaining ones with sum(min(k, len_b)) <= C."""
    out, b0, acc = [], 0, 0
    for b, n in enumerate(np.asarray(lens).tolist()):
        d = min(k, int(n))
        if d > C:
            raise ValueError(f'one sequence needs {d} slots, the cache has {C}')
        if acc + d > C:
            out.append((b0, b))
            b0, acc = b, 0
        acc += d
    out.append((b0, len(lens)))
    return out


class DecodeLayer:
    """Buffers and launch order of one layer's decode step."""

    def __init__(self, kcache: torch.Tensor, kscale: Optional[torch.Tensor], w: torch.Tensor,
                 tok0: np.ndarray, lens: np.ndarray, C: int, k: int = 2048, cap: int = 512,
                 host_pool: Optional[torch.Tensor] = None, early: bool = True, topk_after_early: bool = False,
                 topk_first: Optional[bool] = None, fused: Optional[bool] = None,
                 capacity: Optional[np.ndarray] = None, device='cuda'):
        self.kcache, self.kscale, self.w = kcache, kscale, w
        self.topk_after_early = topk_after_early
        # Launch order of the two branches after the scores. A captured graph
        # keeps the branch launched first on the scores kernel's hardware
        # queue; the other starts after a cross-queue wait (~10 us). With a
        # few sequences the top-k chain is the longer branch, with many the
        # EARLY maps and their PCIe recall are.
        self.topk_first = (len(lens) <= 8) if topk_first is None else bool(topk_first)
        self.B = len(lens)
        self.lens_np = np.asarray(lens, np.int32)
        self.tok0_np = np.asarray(tok0, np.int64)
        # Growing contexts: sequence b may reach capacity[b] tokens (ech_kv_append
        # grows the device lengths); grids, buffers and chunks are sized for it.
        self.cap_np = self.lens_np.copy() if capacity is None else np.asarray(capacity, np.int32)
        if np.any(self.cap_np < self.lens_np):
            raise ValueError('capacity below the current length')
        self.max_len = int(self.cap_np.max())
        self.k, self.cap, self.C = k, cap, C
        self.early = early
        self.P = kcache.shape[0]
        dev = dict(device=device)
        self.tok0 = torch.from_numpy(self.tok0_np).to(**dev)
        self.lens = torch.from_numpy(self.lens_np).to(**dev)
        self.ld = round_up(max(self.max_len, 4), 64)
        self.logits = torch.zeros((self.B, self.ld), dtype=torch.float32, **dev)
        self.idx = torch.empty((self.B, k), dtype=torch.int32, **dev)
        self.kth = torch.empty(self.B, dtype=torch.float32, **dev)
        self.theta = [torch.full((self.B,), float('nan'), dtype=torch.float32, **dev) for _ in range(2)]
        self.parity = 0
        self.sel_slot = torch.empty((self.B, k), dtype=torch.int32, **dev)
        self.stats_early = torch.zeros((self.B, 4), dtype=torch.int32, **dev)
        self.stats_final = torch.zeros((self.B, 4), dtype=torch.int32, **dev)
        self.chunks = sequence_chunks(self.cap_np, k, C)
        self.seq_cap = torch.from_numpy(self.cap_np).to(**dev)
        cb = max(e - s for s, e in self.chunks)
        m_max = max(cb * min(k, self.max_len), cb * min(cap, self.max_len), 1)
        m_early = max(cb * min(cap, self.max_len), 1)   # the EARLY demand bound: no free slot beyond it is ranked
        self.state = LayerState.allocate(self.P, C, m_max, device, M_early=m_early)
        self.ws_topk = torch.empty(ech_topk_ws_bytes(self.B, self.max_len, k), dtype=torch.uint8, **dev)
        self.ws_early = torch.empty(ech_cache_step_ws_bytes(ECH_EARLY, cb, cb, k, self.max_len, C, m_max),
                                    dtype=torch.uint8, **dev)
        self.ws_final = torch.empty(ech_cache_step_ws_bytes(ECH_FINAL, cb, cb, k, self.max_len, C, m_max),
                                    dtype=torch.uint8, **dev)
        # Scores fused with the first chunk's early fetch: fp8 keys, a host
        # pool to copy from, and the early fetch on. By default only for
        # batches of more than 8 sequences: a sequence's early fetch starts
        # once its whole row is scored, so with a few long rows the fused
        # launch ends late (4 x 1M tokens: 261 us per step fused, 208 us
        # not), while with many rows their early rows cross PCIe under the
        # scoring (32 x 131072: 405 us vs 441 us; 64 x 110K: 2.06 vs 2.10 ms).
        can_fuse = early and host_pool is not None and kscale is not None and cap <= 4096
        self.fused = (can_fuse and self.B > 8) if fused is None else bool(fused)
        if self.fused and not can_fuse:
            raise ValueError('the fused scores + early fetch needs fp8 keys, a host pool, the early fetch and '
                             'cap <= 4096')
        if self.fused:
            # zero-filled once; every call leaves it ready for the next
            self.ws_fused = torch.zeros(ech_index_logits_early_ws_bytes(self.B, self.max_len, C, m_early),
                                        dtype=torch.uint8, **dev)
        self.host_pool = host_pool
        if host_pool is not None:
            self.dev_cache = torch.zeros((C, host_pool.shape[1]), dtype=host_pool.dtype, **dev)
        else:
            self.dev_cache = None
        self.s1 = torch.cuda.Stream(device=device)
        self.ev_fork = torch.cuda.Event()
        self.ev_logits = torch.cuda.Event()
        self.ev_early_maps = torch.cuda.Event()
        self.ev_early = torch.cuda.Event()
        ech_cache_reset(self.state)

    def reset(self) -> None:
        ech_cache_reset(self.state)
        for t in self.theta:
            t.fill_(float('nan'))
        self.parity = 0

    def _maps(self, phase: int, b0: int, b1: int, theta: torch.Tensor, stream) -> None:
        stats = self.stats_early if phase == ECH_EARLY else self.stats_final
        ech_cache_step(phase, self.state, self.tok0[b0:b1], self.lens[b0:b1], self.max_len,
                       idx=self.idx[b0:b1] if phase == ECH_FINAL else None, k=self.k,
                       logits=self.logits[b0:b1], theta=theta[b0:b1], cap=self.cap,
                       sel_slot=self.sel_slot[b0:b1] if phase == ECH_FINAL else None, stats=stats[b0:b1],
                       ws=self.ws_early if phase == ECH_EARLY else self.ws_final, stream=stream)

    def _recall(self, phase: int, stream) -> None:
        if self.host_pool is not None:
            ech_recall(self.host_pool, self.dev_cache, self.state, phase=phase, stream=stream)

    def append(self, new_rows: torch.Tensor, new_keys: torch.Tensor, new_scales: Optional[torch.Tensor] = None,
               stream=None) -> None:
        """Each sequence's decoded token joins the host pool and the key cache
        (ech_kv_append); the device lengths grow by one, up to the capacity."""
        ech_kv_append(self.host_pool, self.kcache, self.kscale, self.state, self.tok0, self.lens, self.seq_cap,
                      new_rows, new_keys, new_scales, stream=stream)

    def logits_only(self, q: torch.Tensor, stream=None) -> None:
        ech_index_logits(q, self.w, self.kcache, self.kscale, self.tok0, self.lens, self.max_len, self.logits,
                         stream=stream)

    def scores_launch(self, q: torch.Tensor, stream=None, mark=None) -> None:
        """The first launches of a step: the scores, and with the fused path
        also the first chunk's early fetch (its maps, written while the
        scoring runs) and, on S1, the live copy of its rows. `mark(name,
        stream)`, when given, records the copier's span as 'recall_live'."""
        if self.fused:
            s0 = torch.cuda.current_stream() if stream is None else stream
            self.ev_fork.record(s0)
            b0, b1 = self.chunks[0]
            ech_index_logits_early(q, self.w, self.kcache, self.kscale, self.tok0, self.lens, self.max_len,
                                   self.logits, b0, b1, self.theta[self.parity], self.cap, self.state,
                                   self.stats_early, self.ws_fused, stream=s0)
            # enqueued after the fused launch, waiting only for the step's start
            self.s1.wait_event(self.ev_fork)
            if mark is not None:
                mark('recall_live', self.s1)
            ech_recall_early_live(self.host_pool, self.dev_cache, self.state, self.ws_fused, stream=self.s1,
                                  final=True)
            if mark is not None:
                mark('recall_live', self.s1)
        else:
            self.logits_only(q, stream=stream)

    def step(self, q: Optional[torch.Tensor], marks: Optional[dict] = None,
             wait: Optional[torch.cuda.Event] = None, logits_done: Optional[torch.cuda.Event] = None,
             scores: bool = True, on_chunk=None) -> None:
        """Enqueue one decode step for query q [B, 64, 128] (bf16 bits) on the
        current stream (with S1 forked and joined inside). `marks`, when given,
        receives timing events recorded on the stream of each stage, as
        (start, end) pairs: logits, topk, final (S0: FINAL maps to the end of
        the step), early (S1: EARLY maps and recall of the first chunk), and
        early_maps, recall_early, final_maps, recall_final (one pair per
        chunk). `wait`, when given, is an event the scores wait for;
        `logits_done` is recorded once they are written (one group only).
        scores=False leaves the scores out: the caller has launched them
        (scores_launch) on the current stream already (q is then unused).

        on_chunk(b0, b1, stream), when given, is called once per sequence
        chunk, right after the chunk's FINAL recall is enqueued on `stream`:
        work the caller enqueues there (the attention over sel_slot[b0:b1])
        sees every selected token of sequences b0..b1-1 resident in the
        slot sel_slot names. When the batch's selections exceed the cache
        (several chunks), a later chunk's FINAL phase may evict an earlier
        chunk's tokens, so an earlier chunk's sel_slot rows are only valid
        until then: read them in on_chunk. With one chunk they stay valid
        until the next step."""
        s0 = torch.cuda.current_stream()
        if wait is not None:
            s0.wait_event(wait)

        def mark(name, stream):
            if marks is None:
                return None
            ev = torch.cuda.Event(enable_timing=True)
            ev.record(stream)
            marks.setdefault(name, []).append(ev)
            return ev

        th, th_next = self.theta[self.parity], self.theta[1 - self.parity]
        if scores:
            mark('logits', s0)
            self.scores_launch(q, stream=s0, mark=mark if marks is not None else None)
            mark('logits', s0)
        if logits_done is not None:
            logits_done.record(s0)
        first_b0, first_b1 = self.chunks[0]
        if self.early:
            self.ev_logits.record(s0)
        if self.fused:
            self._after_fused(th, th_next, s0, mark)   # the first chunk's FINAL recall included
        else:
            self._after_scores(th, th_next, s0, mark)
            mark('recall_final', s0)
            self._recall(ECH_FINAL, s0)
            mark('recall_final', s0)
        if on_chunk is not None:
            on_chunk(first_b0, first_b1, s0)
        for b0, b1 in self.chunks[1:]:
            for phase in ((ECH_EARLY, ECH_FINAL) if self.early else (ECH_FINAL,)):
                name = 'early' if phase == ECH_EARLY else 'final'
                mark(name + '_maps', s0)
                self._maps(phase, b0, b1, th, s0)
                mark(name + '_maps', s0)
                mark('recall_' + name, s0)
                self._recall(phase, s0)
                mark('recall_' + name, s0)
            if on_chunk is not None:
                on_chunk(b0, b1, s0)
        mark('final', s0)
        self.parity ^= 1

    def _after_fused(self, th, th_next, s0, mark) -> None:
        """First chunk after the fused launch: the top-k and the FINAL maps
        on S0, while on S1 the live copier goes on from the early rows to the
        FINAL ones as soon as S0 has completed the FINAL list. S0 then waits
        for the copier and copies what it left of both lists in one launch
        (ech_recall_rest)."""
        first_b0, first_b1 = self.chunks[0]
        mark('topk', s0)
        # from the band lists the scoring waves wrote (the scores are not read again)
        ech_topk_early(self.logits, self.lens, self.max_len, self.k, th, th_next, self.idx, self.kth, self.state,
                       self.ws_fused, stream=s0)
        mark('topk', s0)
        self.ev_early.record(self.s1)              # the copier is done
        mark('final', s0)
        mark('final_maps', s0)
        self._maps(ECH_FINAL, first_b0, first_b1, th, s0)
        mark('final_maps', s0)
        s0.wait_event(self.ev_early)
        mark('recall_final', s0)
        ech_recall_rest(self.host_pool, self.dev_cache, self.state, stream=s0)
        mark('recall_final', s0)

    def _after_scores(self, th, th_next, s0, mark) -> None:
        """First chunk after the plain scores: the EARLY maps and recall on
        S1 beside the top-k on S0, then the FINAL maps; ends with S0 waiting
        for the early rows."""
        first_b0, first_b1 = self.chunks[0]

        def early_branch():
            # S1: EARLY maps, then its rows cross PCIe while S0 carries on.
            self.s1.wait_event(self.ev_logits)
            mark('early', self.s1)
            mark('early_maps', self.s1)
            self._maps(ECH_EARLY, first_b0, first_b1, th, self.s1)
            mark('early_maps', self.s1)
            self.ev_early_maps.record(self.s1)
            mark('recall_early', self.s1)
            self._recall(ECH_EARLY, self.s1)
            mark('recall_early', self.s1)
            mark('early', self.s1)
            self.ev_early.record(self.s1)

        def topk_branch():
            # The top-k runs beside the EARLY maps (or after them, on request).
            if self.early and self.topk_after_early:
                s0.wait_event(self.ev_early_maps)
            mark('topk', s0)
            ech_topk(self.logits, self.lens, self.max_len, self.k, th, th_next, self.idx, self.kth, self.ws_topk,
                     stream=s0)
            mark('topk', s0)

        if self.early and not (self.topk_first and not self.topk_after_early):
            early_branch()
            topk_branch()
        else:
            topk_branch()
            if self.early:
                early_branch()
        mark('final', s0)
        if self.early and not self.topk_after_early:
            s0.wait_event(self.ev_early_maps)      # FINAL updates the maps EARLY left ...
        mark('final_maps', s0)
        self._maps(ECH_FINAL, first_b0, first_b1, th, s0)
        mark('final_maps', s0)
        if self.early:
            s0.wait_event(self.ev_early)           # ... but may reuse a slot EARLY is still filling

    @property
    def theta_current(self) -> torch.Tensor:
        return self.theta[self.parity]

    def capture(self, scores: bool = True) -> None:
        """Capture one decode step per threshold parity as a hipGraph that
        reads q from a static buffer (every tensor of the step has a fixed
        size and address, so the step replays unchanged). Nothing runs.
        scores=False captures the step after the scores (replay_after_scores);
        not with the fused path, whose live copier (launched with the scores)
        must precede the early rest and FINAL recalls of the same step: a
        graph of the rest alone would not wait for it."""
        if self.fused and not scores:
            raise ValueError('the fused path captures whole steps only (the scores launch starts the copier)')
        self.q_static = torch.zeros((self.B, 64, 128), dtype=torch.int16, device=self.logits.device)
        self.graphs = [None, None]
        self.graph_scores = scores
        for _ in range(2):
            p = self.parity
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self.step(self.q_static if scores else None, scores=scores)      # flips self.parity
            self.graphs[p] = g

    def replay(self, q: torch.Tensor) -> None:
        """One decode step through the captured graphs (on the current stream)."""
        if not self.graph_scores:
            raise ValueError('captured without the scores: use replay_after_scores')
        self.q_static.copy_(q, non_blocking=True)
        self.graphs[self.parity].replay()
        self.parity ^= 1

    def replay_after_scores(self) -> None:
        """The rest of a decode step through graphs captured with
        scores=False, after the caller's ech_index_logits on the current
        stream."""
        if self.graph_scores:
            raise ValueError('captured with the scores: use replay')
        self.graphs[self.parity].replay()
        self.parity ^= 1


class PrefillLayer:
    """Causal prefill of one sequence in query blocks: logits -> per-row top-k
    -> PREFILL cache step (union) -> recall of block i on S1 while S0 scores
    block i+1.

    With overlap=True the score buffer is doubled: S0 scores block i+1 into
    one buffer while S1 runs block i's top-k and cache step on the other
    (recalls on S2), so the selection work hides under the next block's
    matrix-core work."""

    def __init__(self, kcache: torch.Tensor, kscale: Optional[torch.Tensor], N: int, C: int, k: int = 2048,
                 block_rows: int = 4096, host_pool: Optional[torch.Tensor] = None, tok0: int = 0,
                 overlap: bool = False, device='cuda'):
        self.kcache, self.kscale = kcache, kscale
        self.N, self.C, self.k, self.block_rows, self.tok0 = N, C, k, block_rows, tok0
        self.overlap = overlap
        dev = dict(device=device)
        self.ld = round_up(N, 64)
        nbuf = 2 if overlap else 1
        self.logits_buf = [torch.empty((block_rows, self.ld), dtype=torch.float32, **dev) for _ in range(nbuf)]
        self.logits = self.logits_buf[0]
        self.idx = torch.empty((block_rows, k), dtype=torch.int32, **dev)
        self.kth = torch.empty(block_rows, dtype=torch.float32, **dev)
        self.theta = torch.full((block_rows,), float('nan'), dtype=torch.float32, **dev)
        self.sel_slot = torch.empty((block_rows, k), dtype=torch.int32, **dev)
        self.stats = torch.zeros((1, 4), dtype=torch.int32, **dev)
        self.m_max = min(N, block_rows * k)
        self.state = LayerState.allocate(N + tok0, C, self.m_max, device)
        self.ws_topk = torch.empty(ech_topk_ws_bytes(block_rows, N, k), dtype=torch.uint8, **dev)
        self.ws_cache = torch.empty(ech_cache_step_ws_bytes(ECH_PREFILL, 1, block_rows, k, N, C, self.m_max),
                                    dtype=torch.uint8, **dev)
        self.seq_tok0 = torch.tensor([tok0], dtype=torch.int64, **dev)
        self.seq_len = torch.tensor([N], dtype=torch.int32, **dev)
        self.row_len = torch.arange(1, block_rows + 1, dtype=torch.int32, **dev)
        self._row_lens = {}
        self.host_pool = host_pool
        self.dev_cache = (torch.zeros((C, host_pool.shape[1]), dtype=host_pool.dtype, **dev)
                          if host_pool is not None else None)
        self.s1 = torch.cuda.Stream(device=device)
        self.s2 = torch.cuda.Stream(device=device) if overlap else None
        self.ev_recall = torch.cuda.Event()
        self.ev_scored = [torch.cuda.Event() for _ in range(nbuf)]
        self.ev_used = [torch.cuda.Event() for _ in range(nbuf)]
        self.nblock = 0
        ech_cache_reset(self.state)

    def blocks(self):
        return [(r0, min(self.block_rows, self.N - r0)) for r0 in range(0, self.N, self.block_rows)]

    def reset_state(self) -> None:
        """Start the sequence again: empty cache, no threshold predictions."""
        ech_cache_reset(self.state)
        self.theta.fill_(float('nan'))
        self.nblock = 0

    def _row_len(self, row0: int, R: int) -> torch.Tensor:
        key = (row0, R)
        if key not in self._row_lens:
            self._row_lens[key] = self.row_len[:R] + row0
        return self._row_lens[key]

    def run_block(self, row0: int, q: torch.Tensor, w: torch.Tensor, first: bool, mark=None,
                  stage_marks: Optional[dict] = None) -> None:
        """q [R,64,128], w [R,64] for rows row0 .. row0+R-1, on the current
        stream. `mark`, when given, receives a (start, end) event pair around
        the scoring launch; `stage_marks`, when given, receives (start, end)
        pairs recorded on each stage's own stream under 'topk', 'cache' and
        'recall'."""

        def smark(name, stream):
            if stage_marks is not None:
                ev = torch.cuda.Event(enable_timing=True)
                ev.record(stream)
                stage_marks.setdefault(name, []).append(ev)

        s0 = torch.cuda.current_stream()
        R = q.shape[0]
        buf = self.nblock % len(self.logits_buf) if self.overlap else 0
        logits = self.logits_buf[buf][:R]
        self.logits = self.logits_buf[buf]
        row_len = self._row_len(row0, R)
        if self.overlap and self.nblock >= 2:
            s0.wait_event(self.ev_used[buf])      # the top-k two blocks back has read this buffer
        if mark is not None:
            ev = torch.cuda.Event(enable_timing=True)
            ev.record(s0)
            mark.append(ev)
        ech_index_logits_causal(q, w, self.kcache, self.kscale, self.tok0, row0, logits, stream=s0)
        if mark is not None:
            ev = torch.cuda.Event(enable_timing=True)
            ev.record(s0)
            mark.append(ev)
        self.nblock += 1
        if self.overlap:
            self.ev_scored[buf].record(s0)
            sel = self.s1
            sel.wait_event(self.ev_scored[buf])
        else:
            sel = s0
        # rows' thresholds: the EMA of the same row position in earlier blocks
        smark('topk', sel)
        ech_topk(logits, row_len, row0 + R, self.k, self.theta[:R], self.theta[:R], self.idx[:R], self.kth[:R],
                 self.ws_topk, stream=sel)
        smark('topk', sel)
        if self.overlap:
            self.ev_used[buf].record(sel)
        if not first:
            sel.wait_event(self.ev_recall)
        smark('cache', sel)
        ech_cache_step(ECH_PREFILL, self.state, self.seq_tok0, self.seq_len, self.N, idx=self.idx[:R], k=self.k,
                       sel_slot=self.sel_slot[:R], stats=self.stats, ws=self.ws_cache, stream=sel)
        smark('cache', sel)
        if self.host_pool is not None:
            rs = self.s2 if self.overlap else self.s1
            rs.wait_stream(sel)
            smark('recall', rs)
            ech_recall(self.host_pool, self.dev_cache, self.state, phase=ECH_PREFILL, stream=rs)
            smark('recall', rs)
            self.ev_recall.record(rs)
        else:
            self.ev_recall.record(sel)

    def finish(self) -> None:
        s0 = torch.cuda.current_stream()
        s0.wait_event(self.ev_recall)
        if self.overlap:
            s0.wait_stream(self.s1)


class DecodeStack:
    """One decode step over L layers for M micro-batches of the batch.

    Each (layer, micro-batch) pair is a DecodeLayer of its own: its slot map
    and device cache (the layer's cache split between the micro-batches),
    reading the layer's indexer keys and host pool at its sequences' token
    offsets. The cache is per layer because each layer's indexer selects its
    own tokens (ECHO explainer, "One layer, one step").

    Within a micro-batch the layers run in order: layer l+1 scores only after
    layer l's recall, because in the model the attention over the recalled
    rows stands between them and yields the next layer's query. The
    micro-batches are independent chains on streams of their own, started
    one score launch apart, so while one micro-batch's rows cross PCIe the
    other one scores:

        mb0: logits L0 | maps, recall L0 ............ | logits L1 | ...
        mb1:           | logits L0 | maps, recall L0 ............ | logits L1

    The queries of every layer are inputs of the step (no attention or MLP is
    computed between layers): qs[l][m] is DecodeLayer l, m's [B_m, 64, 128].
    """

    def __init__(self, layers: List[List[DecodeLayer]], device='cuda'):
        self.layers = [list(r) for r in layers]
        self.L, self.M = len(self.layers), (len(self.layers[0]) if self.layers else 0)
        if self.L == 0 or self.M == 0 or any(len(r) != self.M for r in self.layers):
            raise ValueError('layers must be a non-empty L x M list of DecodeLayer')
        # The stack launches each pair's scores itself and replays graphs of
        # the rest, which the fused path cannot split (see capture); it is
        # also slower here (4 layers x 2 micro-batches of 16 sequences: 471
        # us per layer fused, 408 us not).
        if any(d.fused for r in self.layers for d in r):
            raise ValueError('DecodeStack takes layers built with fused=False')
        # Two streams per micro-batch (scores and its chain; EARLY branch),
        # shared by its layers; micro-batch 0's chain is the caller's stream.
        # With two micro-batches these are four streams, one per hardware
        # queue at the runtime's default of four, so neither micro-batch
        # waits behind the other's work in a shared queue.
        self.streams = [None] + [torch.cuda.Stream(device=device) for _ in range(self.M - 1)]
        self.side = [torch.cuda.Stream(device=device) for _ in range(self.M)]
        for r in self.layers:
            for m, d in enumerate(r):
                d.s1 = self.side[m]
        self.ev_start = torch.cuda.Event()
        self.ev_end = [torch.cuda.Event() for _ in range(self.M)]
        self.ev_logits = [[torch.cuda.Event() for _ in range(self.M)]]

    def step(self, qs) -> None:
        """Enqueue one L-layer step on the current stream (micro-batch streams
        forked and joined inside)."""
        self._run(qs, graphs=False)

    def _run(self, qs, graphs: bool) -> None:
        # Per layer, every micro-batch's scores are enqueued before the rest
        # of any micro-batch's step, so each cross-stream wait is enqueued
        # right behind the event it waits for (the runtime can otherwise
        # resolve a wait only once later work on the recording stream has
        # been submitted and finished). Micro-batch m > 0 starts its first
        # scores after those of m - 1; from then on the chains run free, one
        # score launch apart.
        s = torch.cuda.current_stream()
        chain = [s] + self.streams[1:]          # micro-batch 0 runs on the caller's stream
        self.ev_start.record(s)
        for st in chain[1:]:
            st.wait_event(self.ev_start)
        for l in range(self.L):
            for m in range(self.M):
                st, d = chain[m], self.layers[l][m]
                if l == 0 and m > 0:
                    st.wait_event(self.ev_logits[0][m - 1])
                d.scores_launch(qs[l][m], stream=st)
                if l == 0:
                    self.ev_logits[0][m].record(st)
            for m in range(self.M):
                with torch.cuda.stream(chain[m]):
                    if graphs:
                        self.layers[l][m].replay_after_scores()
                    else:
                        self.layers[l][m].step(None, scores=False)
        for m in range(1, self.M):
            self.ev_end[m].record(chain[m])
            s.wait_event(self.ev_end[m])

    def capture(self) -> None:
        """Capture, for every (layer, micro-batch), its step after the scores
        as hipGraphs (one per threshold parity). Nothing runs. A replay then
        launches each pair's scores kernel and its graph on the micro-batch's
        stream, in the order and with the events of step()."""
        if len({d.parity for r in self.layers for d in r}) != 1:
            raise ValueError('every layer must be at the same threshold parity')
        for r in self.layers:
            for d in r:
                d.capture(scores=False)

    def replay(self, qs) -> None:
        """One L-layer step through the captured graphs (current stream)."""
        self._run(qs, graphs=True)
