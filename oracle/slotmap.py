"""Sequential per-layer slot map: free -> allocate -> recall, no write-back.

Source: ECHO explainer, "One layer, one step: free -> allocate -> recall"
(the cache is kept per layer, since layers select different tokens; an
evicted row needs no copy back, the host pool keeping all rows) and
"Five fixed-size integer tensors on the GPU" (fixed-size state, so a decode
step is one captured graph); "Decode: fetch above a predicted threshold"
(early fetch of tokens scoring above theta, up to a cap); "Prefill: one-round
histogram" (the tokens selected by a query block are fetched while the next
block is scored).

The pages give the phases but not every rule; the readings taken here:

* State: tok2slot[P] (slot of global token g, or -1), slot2tok[C] (token held
  by slot s, or -1) and a persistent ring head. The cache starts empty; every
  row lives in the host pool.
* Free is lazy: a resident token that is not selected keeps its slot (and its
  mapping) until the slot is reused, so selecting it again before then is a
  hit. Only pinned slots (the current selection's resident tokens) are
  protected in a phase.
* Allocate: misses, in the order given, take the unpinned slots in ring order
  starting at the head (head, head+1, ... mod C), one slot per miss; if that
  slot holds a token u, u is evicted (tok2slot[u] = -1; the host copy is
  untouched). After a phase that assigned anything, head = last slot + 1 mod C.
  A FINAL phase that runs out of slots is an error; an EARLY phase stops.
* Recall: for each assignment (g, p) copy host row g into device-cache slot p.
* Decode EARLY phase (only for sequences whose theta is not NaN): pins are the
  slots of resident tokens with score > theta (strict); misses are, per
  sequence in order, the first `cap` non-resident tokens with score > theta in
  ascending token order.
* Decode FINAL phase: pins are the slots of the selected tokens that are
  resident; misses are the selected non-resident tokens in ascending
  (sequence, token) order. Afterwards every selected token is resident and
  sel_slot = tok2slot[selected].
* Prefill block: one FINAL phase over the union of the block rows' selections
  (misses in ascending token order).
* Per-phase statistics per sequence: [hits, fetched, dropped, evictions] where
  hits = tokens of the phase's selection already resident, fetched = misses
  that got a slot, dropped = misses that did not (EARLY cap or no free slot),
  evictions = resident tokens evicted by this sequence's misses.
"""
from typing import Optional, Sequence

import numpy as np


class SlotMap:
    def __init__(self, P: int, C: int):
        self.P = int(P)
        self.C = int(C)
        self.tok2slot = np.full(self.P, -1, dtype=np.int64)
        self.slot2tok = np.full(self.C, -1, dtype=np.int64)
        self.head = 0

    # -------------------------------------------------------------- allocate
    def _allocate(self, pinned: np.ndarray, misses: Sequence[int], owners: Sequence[int],
                  hard: bool, nseq: int):
        """Give each miss (in order) the next unpinned slot in ring order from
        the head. Returns (assignments [(g, p)], fetched[nseq], evictions[nseq])."""
        ring = (self.head + np.arange(self.C)) % self.C
        free = ring[~pinned[ring]]
        fetched = np.zeros(nseq, dtype=np.int64)
        evictions = np.zeros(nseq, dtype=np.int64)
        assigned = []
        for i, (g, b) in enumerate(zip(misses, owners)):
            if i >= len(free):
                if hard:
                    raise RuntimeError('FINAL phase needs more slots than the cache has')
                break
            p = int(free[i])
            u = int(self.slot2tok[p])
            if u >= 0:
                self.tok2slot[u] = -1          # evict; the host row is untouched
                evictions[b] += 1
            self.slot2tok[p] = g
            self.tok2slot[g] = p
            fetched[b] += 1
            assigned.append((int(g), p))
        if assigned:
            self.head = (assigned[-1][1] + 1) % self.C
        return assigned, fetched, evictions

    # -------------------------------------------------------------- phases
    def early(self, tok0: Sequence[int], scores: Sequence[np.ndarray], theta: np.ndarray, cap: int):
        """Decode early fetch. scores[b] are the fp32 scores of sequence b's
        visible tokens, theta[b] the float32 prediction (NaN = none)."""
        B = len(tok0)
        pinned = np.zeros(self.C, dtype=bool)
        stats = np.zeros((B, 4), dtype=np.int64)
        misses, owners = [], []
        for b in range(B):
            th = np.float32(theta[b])
            if np.isnan(th):
                continue
            s = np.asarray(scores[b], dtype=np.float32)
            above = np.nonzero(s > th)[0]
            g = int(tok0[b]) + above
            slot = self.tok2slot[g]
            res = slot >= 0
            pinned[slot[res]] = True
            stats[b, 0] = int(res.sum())
            nonres = g[~res]
            take = nonres[:cap]
            stats[b, 2] = len(nonres) - len(take)
            misses.extend(int(x) for x in take)
            owners.extend([b] * len(take))
        assigned, fetched, ev = self._allocate(pinned, misses, owners, hard=False, nseq=B)
        stats[:, 1] = fetched
        # misses that did not get a slot are dropped too
        wanted = np.bincount(np.asarray(owners, dtype=np.int64), minlength=B) if owners else np.zeros(B, np.int64)
        stats[:, 2] += wanted - fetched
        stats[:, 3] = ev
        return assigned, stats

    def final(self, tok0: Sequence[int], idx: np.ndarray):
        """Decode final phase. idx [B, k] ascending token offsets, -1 padded."""
        B = len(tok0)
        pinned = np.zeros(self.C, dtype=bool)
        stats = np.zeros((B, 4), dtype=np.int64)
        misses, owners = [], []
        for b in range(B):
            t = idx[b][idx[b] >= 0]
            g = int(tok0[b]) + t
            slot = self.tok2slot[g]
            res = slot >= 0
            pinned[slot[res]] = True
            stats[b, 0] = int(res.sum())
            misses.extend(int(x) for x in g[~res])
            owners.extend([b] * int((~res).sum()))
        assigned, fetched, ev = self._allocate(pinned, misses, owners, hard=True, nseq=B)
        stats[:, 1] = fetched
        stats[:, 3] = ev
        sel_slot = self.selected_slots(tok0, idx)
        return assigned, sel_slot, stats

    def prefill_block(self, tok0: int, idx: np.ndarray):
        """Prefill: one FINAL phase over the union of the rows' selections.
        idx [R, k] token offsets within the sequence (-1 padded)."""
        t = np.unique(idx[idx >= 0])
        g = int(tok0) + t
        slot = self.tok2slot[g]
        res = slot >= 0
        pinned = np.zeros(self.C, dtype=bool)
        pinned[slot[res]] = True
        misses = [int(x) for x in g[~res]]
        assigned, fetched, ev = self._allocate(pinned, misses, [0] * len(misses), hard=True, nseq=1)
        stats = np.array([[int(res.sum()), int(fetched[0]), 0, int(ev[0])]], dtype=np.int64)
        sel_slot = np.where(idx >= 0, self.tok2slot[int(tok0) + np.maximum(idx, 0)], -1)
        return assigned, sel_slot, stats

    def selected_slots(self, tok0: Sequence[int], idx: np.ndarray) -> np.ndarray:
        out = np.full(idx.shape, -1, dtype=np.int64)
        for b in range(idx.shape[0]):
            v = idx[b] >= 0
            out[b, v] = self.tok2slot[int(tok0[b]) + idx[b][v]]
        return out

    def resident(self) -> np.ndarray:
        return np.nonzero(self.slot2tok >= 0)[0]


def recall_rows(host_pool: np.ndarray, dev_cache: np.ndarray, assigned) -> None:
    """Copy host row g into device-cache slot p for each (g, p), in order."""
    for g, p in assigned:
        dev_cache[p] = host_pool[g]
