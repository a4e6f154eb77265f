"""Slot map (free -> allocate -> recall) on the GPU against the sequential
oracle simulator, bit for bit: maps, ring head, miss list (allocation order),
sel_slot and per-sequence stats after every phase, and the recalled bytes.
Selections and scores are fed identically to both sides."""
import numpy as np
import pytest
import torch

import indexer_top_kv_amd as ech
import oracle
import workloads as wk
from gpu_util import dev, host, need_gpu

pytestmark = pytest.mark.gpu


class GpuCache:
    def __init__(self, P, C, B, k, max_len, cap=512, R=None, M_max=None):
        self.P, self.C, self.B, self.k, self.max_len, self.cap = P, C, B, k, max_len, cap
        self.R = R or B
        demand = max(B * min(k, max_len), B * min(cap, max_len), min(max_len, self.R * k))
        self.M_max = M_max or demand
        self.st = ech.LayerState.allocate(P, C, self.M_max)
        ech.ech_cache_reset(self.st)
        self.ws = {}
        for ph in (ech.ECH_EARLY, ech.ECH_FINAL, ech.ECH_PREFILL):
            n = ech.ech_cache_step_ws_bytes(ph, B if ph != ech.ECH_PREFILL else 1, self.R, k, max_len, C, self.M_max)
            self.ws[ph] = torch.empty(n, dtype=torch.uint8, device='cuda')

    def _assigned(self, phase=ech.ECH_FINAL):
        early = phase == ech.ECH_EARLY
        n = int(host(self.st.ctr)[ech.CTR_NMISS_EARLY if early else ech.CTR_NMISS])
        return [tuple(x) for x in host(self.st.miss_list(phase))[:n].tolist()]

    def final(self, tok0, lens, idx):
        sel = torch.empty((self.B, self.k), dtype=torch.int32, device='cuda')
        stats = torch.full((self.B, 4), -9, dtype=torch.int32, device='cuda')
        ech.ech_cache_step(ech.ECH_FINAL, self.st, dev(np.asarray(tok0, np.int64)), dev(np.asarray(lens, np.int32)),
                           self.max_len, idx=dev(idx.astype(np.int32)), k=self.k, sel_slot=sel, stats=stats,
                           ws=self.ws[ech.ECH_FINAL])
        torch.cuda.synchronize()
        return self._assigned(), host(sel), host(stats)

    def early(self, tok0, lens, scores, theta):
        stats = torch.full((self.B, 4), -9, dtype=torch.int32, device='cuda')
        ech.ech_cache_step(ech.ECH_EARLY, self.st, dev(np.asarray(tok0, np.int64)), dev(np.asarray(lens, np.int32)),
                           self.max_len, k=self.k, logits=dev(scores), theta=dev(np.asarray(theta, np.float32)),
                           cap=self.cap, stats=stats, ws=self.ws[ech.ECH_EARLY])
        torch.cuda.synchronize()
        return self._assigned(ech.ECH_EARLY), host(stats)

    def prefill(self, tok0, length, idx):
        sel = torch.empty(idx.shape, dtype=torch.int32, device='cuda')
        stats = torch.full((1, 4), -9, dtype=torch.int32, device='cuda')
        ech.ech_cache_step(ech.ECH_PREFILL, self.st, dev(np.array([tok0], np.int64)),
                           dev(np.array([length], np.int32)), self.max_len, idx=dev(idx.astype(np.int32)), k=self.k,
                           sel_slot=sel, stats=stats, ws=self.ws[ech.ECH_PREFILL])
        torch.cuda.synchronize()
        return self._assigned(), host(sel), host(stats)

    def compare(self, sm: oracle.SlotMap):
        np.testing.assert_array_equal(host(self.st.tok2slot), sm.tok2slot)
        np.testing.assert_array_equal(host(self.st.slot2tok), sm.slot2tok)
        ctr = host(self.st.ctr)
        assert ctr[ech.CTR_HEAD] == sm.head
        assert ctr[ech.CTR_STATUS] == 0, ctr[ech.CTR_STATUS]


def _scores(cfg, B, n, step):
    return wk.random_logits(cfg, B, n, 'normal', seed_extra=step)


def _topk_idx(scores, lens, k):
    return np.stack([oracle.topk_row(scores[b, :lens[b]], k)[0] for b in range(len(lens))])


@pytest.mark.parametrize('C', [6000, 2100, 800])
def test_final_multistep(C):
    need_gpu()
    B, k = 3, 256
    lens = np.array([5000, 2300, 4097], np.int32)
    tok0 = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    P = int(lens.sum())
    gc = GpuCache(P, C, B, k, int(lens.max()))
    sm = oracle.SlotMap(P, C)
    base = _scores(11, B, int(lens.max()), 0)
    for step in range(6):
        scores = base + 0.3 * _scores(11, B, int(lens.max()), step + 1)
        idx = _topk_idx(scores, lens, k)
        a_g, sel_g, st_g = gc.final(tok0, lens, idx)
        a_o, sel_o, st_o = sm.final(tok0, idx)
        assert a_g == a_o, step
        np.testing.assert_array_equal(sel_g, sel_o)
        np.testing.assert_array_equal(st_g, st_o)
        gc.compare(sm)


def test_early_then_final_multistep():
    need_gpu()
    B, k, cap = 4, 512, 100
    lens = np.array([8000, 8000, 3001, 6000], np.int32)
    tok0 = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    P, C = int(lens.sum()), 3000
    ld = 8000
    gc = GpuCache(P, C, B, k, ld, cap=cap)
    sm = oracle.SlotMap(P, C)
    theta = np.full(B, np.nan, np.float32)
    base = _scores(12, B, ld, 0)
    for step in range(6):
        scores = (base + 0.5 * _scores(12, B, ld, step + 1)).astype(np.float32)
        a_g, st_g = gc.early(tok0, lens, scores, theta)
        a_o, st_o = sm.early(tok0, [scores[b, :lens[b]] for b in range(B)], theta, cap)
        assert a_g == a_o, ('early', step)
        np.testing.assert_array_equal(st_g, st_o)
        gc.compare(sm)
        idx = _topk_idx(scores, lens, k)
        kth = np.array([oracle.topk_row(scores[b, :lens[b]], k)[1] for b in range(B)], np.float32)
        a_g, sel_g, st_g = gc.final(tok0, lens, idx)
        a_o, sel_o, st_o = sm.final(tok0, idx)
        assert a_g == a_o, ('final', step)
        np.testing.assert_array_equal(sel_g, sel_o)
        np.testing.assert_array_equal(st_g, st_o)
        gc.compare(sm)
        theta = oracle.theta_rows(theta, kth)


def test_early_slot_shortage_drops():
    need_gpu()
    B, k, cap = 2, 64, 400
    lens = np.array([3000, 3000], np.int32)
    tok0 = np.array([0, 3000], np.int64)
    gc = GpuCache(6000, 300, B, k, 3000, cap=cap)
    sm = oracle.SlotMap(6000, 300)
    scores = _scores(13, B, 3000, 0)
    idx = _topk_idx(scores, lens, k)
    gc.final(tok0, lens, idx)
    sm.final(tok0, idx)
    theta = np.array([17.0, 19.0], np.float32)
    a_g, st_g = gc.early(tok0, lens, scores, theta)
    a_o, st_o = sm.early(tok0, [scores[0], scores[1]], theta, cap)
    assert a_g == a_o
    np.testing.assert_array_equal(st_g, st_o)
    gc.compare(sm)
    assert st_o[:, 2].sum() > 0   # something was dropped


def test_prefill_blocks_union():
    need_gpu()
    N, k = 3000, 64
    for C, Rb in ((N, 200), (1500, 20)):
        gc = GpuCache(N, C, 1, k, N, R=Rb)
        sm = oracle.SlotMap(N, C)
        r = np.random.default_rng(14)
        for blk in range(4):
            row0 = blk * 500
            idx = np.full((Rb, k), -1, np.int64)
            for i in range(Rb):
                vis = row0 + i + 1
                m = min(k, vis)
                idx[i, :m] = np.sort(r.choice(vis, m, replace=False))
            a_g, sel_g, st_g = gc.prefill(0, N, idx)
            a_o, sel_o, st_o = sm.prefill_block(0, idx)
            assert a_g == a_o, (C, blk)
            np.testing.assert_array_equal(sel_g, sel_o)
            np.testing.assert_array_equal(st_g, st_o)
            gc.compare(sm)


def test_recall_bytes_and_no_writeback():
    need_gpu()
    B, k = 2, 128
    lens = np.array([2000, 1500], np.int32)
    tok0 = np.array([0, 2000], np.int64)
    P, C = 3500, 500
    wl = wk.CONFIGS['decode-1x16k-bf16'].scaled(N=P)
    rows = wk.host_rows(wl)
    pool = torch.empty((P, 576), dtype=torch.int16, pin_memory=True)
    pool.numpy()[:] = rows.view(np.int16)
    before = pool.numpy().copy()
    cache = torch.zeros((C, 576), dtype=torch.int16, device='cuda')
    gc = GpuCache(P, C, B, k, 2000)
    sm = oracle.SlotMap(P, C)
    ref_cache = np.zeros((C, 576), np.int16)
    recalled = 0
    for step in range(4):
        scores = _scores(15, B, 2000, step)
        idx = _topk_idx(scores, lens, k)
        a_g, _, _ = gc.final(tok0, lens, idx)
        a_o, _, _ = sm.final(tok0, idx)
        assert a_g == a_o
        recalled += len(a_o)
        ech.ech_recall(pool, cache, gc.st)
        torch.cuda.synchronize()
        oracle.recall_rows(before, ref_cache, a_o)
        np.testing.assert_array_equal(host(cache), ref_cache)
        occ = np.nonzero(sm.slot2tok >= 0)[0]
        np.testing.assert_array_equal(host(cache)[occ], before[sm.slot2tok[occ]])
    np.testing.assert_array_equal(pool.numpy(), before)
    assert int(host(gc.st.ctr)[ech.CTR_RECALLED]) == recalled


def test_bad_token_sets_status():
    need_gpu()
    gc = GpuCache(100, 50, 1, 8, 100)
    idx = np.array([[0, 5, 99, 100, 150, -1, -1, -1]], np.int64)   # 100, 150 >= len
    gc.final(np.array([0]), np.array([100]), idx)
    assert int(host(gc.st.ctr)[ech.CTR_STATUS]) & ech.ST_BADTOK


def test_deterministic_replay():
    need_gpu()
    B, k = 3, 256
    lens = np.array([4000, 4000, 4000], np.int32)
    tok0 = np.array([0, 4000, 8000], np.int64)
    outs = []
    for rep in range(2):
        gc = GpuCache(12000, 1000, B, k, 4000)
        for step in range(4):
            idx = _topk_idx(_scores(16, B, 4000, step), lens, k)
            gc.final(tok0, lens, idx)
        n = int(host(gc.st.ctr)[ech.CTR_NMISS])
        outs.append((host(gc.st.tok2slot).copy(), host(gc.st.slot2tok).copy(), host(gc.st.miss)[:n].copy(),
                     host(gc.st.ctr).copy()))
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a, b)


def test_final_large_ring_many_windows():
    """A ring of 40000 slots: the cold phase ranks 16384 free slots (several
    windows of ring positions), later phases find their free slots between
    pinned ones while the head wraps round the ring."""
    need_gpu()
    B, k = 8, 2048
    lens = np.array([30000, 21000, 30000, 9000, 30000, 25001, 30000, 17777], np.int32)
    tok0 = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    P, C = int(lens.sum()), 40000
    gc = GpuCache(P, C, B, k, int(lens.max()))
    sm = oracle.SlotMap(P, C)
    base = _scores(17, B, int(lens.max()), 0)
    wrapped = False
    for step in range(10):
        scores = base + (0.2 + 0.1 * step) * _scores(17, B, int(lens.max()), step + 1)
        idx = _topk_idx(scores, lens, k)
        head0 = sm.head
        a_g, sel_g, st_g = gc.final(tok0, lens, idx)
        a_o, sel_o, st_o = sm.final(tok0, idx)
        assert a_g == a_o, step
        np.testing.assert_array_equal(sel_g, sel_o)
        np.testing.assert_array_equal(st_g, st_o)
        gc.compare(sm)
        wrapped |= sm.head < head0
    assert wrapped


def test_early_final_large_cap_many_windows():
    """EARLY phases that want more than one window of free slots (cap 4000,
    a low theta) on a 30000-slot ring, then FINAL, over several steps."""
    need_gpu()
    B, k, cap = 4, 2048, 4000
    lens = np.array([40000, 40000, 23000, 40000], np.int32)
    tok0 = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    P, C, ld = int(lens.sum()), 30000, 40000
    gc = GpuCache(P, C, B, k, ld, cap=cap)
    sm = oracle.SlotMap(P, C)
    base = _scores(18, B, ld, 0)
    n_early = []
    for step in range(4):
        scores = (base + 0.5 * _scores(18, B, ld, step + 1)).astype(np.float32)
        theta = np.array([np.quantile(scores[b, :lens[b]], 0.85) for b in range(B)], np.float32)
        theta[2] = np.nan if step == 1 else theta[2]
        a_g, st_g = gc.early(tok0, lens, scores, theta)
        a_o, st_o = sm.early(tok0, [scores[b, :lens[b]] for b in range(B)], theta, cap)
        assert a_g == a_o, ('early', step)
        np.testing.assert_array_equal(st_g, st_o)
        gc.compare(sm)
        n_early.append(len(a_o))
        idx = _topk_idx(scores, lens, k)
        a_g, sel_g, st_g = gc.final(tok0, lens, idx)
        a_o, sel_o, st_o = sm.final(tok0, idx)
        assert a_g == a_o, ('final', step)
        np.testing.assert_array_equal(sel_g, sel_o)
        np.testing.assert_array_equal(st_g, st_o)
        gc.compare(sm)
    assert n_early[0] > 8192   # the cold phase ranks free slots over several windows


def test_prefill_large_union_many_windows():
    """Prefill blocks whose union misses span several windows of ring
    positions (64 rows x 2048 of a 60000-token sequence, 60000 slots)."""
    need_gpu()
    N, k, Rb, C = 60000, 2048, 64, 60000
    gc = GpuCache(N, C, 1, k, N, R=Rb)
    sm = oracle.SlotMap(N, C)
    r = np.random.default_rng(19)
    for blk in range(3):
        row0 = 12000 + blk * 16000
        idx = np.full((Rb, k), -1, np.int64)
        for i in range(Rb):
            vis = row0 + 211 * i + 1
            idx[i] = np.sort(r.choice(vis, k, replace=False))
        a_g, sel_g, st_g = gc.prefill(0, N, idx)
        a_o, sel_o, st_o = sm.prefill_block(0, idx)
        assert a_g == a_o, blk
        np.testing.assert_array_equal(sel_g, sel_o)
        np.testing.assert_array_equal(st_g, st_o)
        gc.compare(sm)


def test_early_cap_zero_and_an_empty_sequence():
    """EARLY with cap 0 only pins (no misses, no allocation), then FINAL, with
    an empty sequence in the batch; maps, head and stats as the oracle's."""
    need_gpu()
    B, k, cap = 3, 512, 0
    lens = np.array([5000, 0, 3001], np.int32)
    tok0 = np.array([0, 5000, 5000], np.int64)
    P, C, ld = 8001, 2000, 5000
    gc = GpuCache(P, C, B, k, ld, cap=cap)
    sm = oracle.SlotMap(P, C)
    base = _scores(20, B, ld, 0)
    theta = np.full(B, np.nan, np.float32)
    for step in range(3):
        scores = (base + 0.4 * _scores(20, B, ld, step + 1)).astype(np.float32)
        a_g, st_g = gc.early(tok0, lens, scores, theta)
        a_o, st_o = sm.early(tok0, [scores[b, :lens[b]] for b in range(B)], theta, cap)
        assert a_g == a_o == [], ('early', step)
        np.testing.assert_array_equal(st_g, st_o)
        gc.compare(sm)
        idx = np.full((B, k), -1, np.int64)
        kth = np.full(B, np.nan, np.float32)
        for b in range(B):
            if lens[b]:
                idx[b], kth[b] = oracle.topk_row(scores[b, :lens[b]], k)
        a_g, sel_g, st_g = gc.final(tok0, lens, idx)
        a_o, sel_o, st_o = sm.final(tok0, idx)
        assert a_g == a_o, ('final', step)
        np.testing.assert_array_equal(sel_g, sel_o)
        np.testing.assert_array_equal(st_g, st_o)
        gc.compare(sm)
        theta = oracle.theta_rows(theta, kth)
