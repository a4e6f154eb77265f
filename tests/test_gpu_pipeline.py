"""Whole decode steps on the GPU (two streams, early fetch overlapping the
top-k, chunked when the batch does not fit the cache) against the same steps
run by the oracle.

Dyadic inputs (small integers, power-of-two scales, head weights m/64) make
every score exact in float32 whatever the summation order, so the GPU and the
oracle see identical scores and every later stage must agree bit for bit:
idx, kth, theta, maps, head, sel_slot, stats and the recalled rows. With
normal inputs the scores agree within tolerance only, so the selections are
checked for validity against the oracle scores and the cache for its
invariants.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wk
from gpu_util import dev, host, need_gpu, TOL_BF16, TOL_FP8
from indexer_top_kv_amd.pipeline import DecodeLayer

pytestmark = pytest.mark.gpu


def oracle_chunks(lens, k, C):
    """Sequence chunks: longest prefixes with sum(min(k, len)) <= C (reading
    of the capacity-constrained decode)."""
    out, start, acc = [], 0, 0
    for b, n in enumerate(lens):
        d = min(k, int(n))
        if acc + d > C:
            out.append((start, b))
            start, acc = b, 0
        acc += d
    out.append((start, len(lens)))
    return out


class OracleDecode:
    def __init__(self, wl, keys, scale, w, pool):
        self.wl, self.keys, self.scale, self.w = wl, keys, scale, w
        self.sm = oracle.SlotMap(wl.P, wl.C)
        self.theta = np.full(wl.B, np.nan, np.float32)
        self.pool = pool
        self.cache = np.zeros((wl.C, pool.shape[1]), pool.dtype)
        self.chunks = oracle_chunks(wl.lens, wl.k, wl.C)

    def step(self, q):
        wl = self.wl
        L = [x.astype(np.float32) for x in oracle.index_logits(q, self.w, self.keys, wl.kdtype, self.scale,
                                                                 wl.tok0, wl.lens)]
        idx, kth = oracle.topk_rows(L, wl.k)
        early_stats = np.zeros((wl.B, 4), np.int64)
        final_stats = np.zeros((wl.B, 4), np.int64)
        sel = np.zeros((wl.B, wl.k), np.int64)
        for b0, b1 in self.chunks:
            a, st = self.sm.early(wl.tok0[b0:b1], L[b0:b1], self.theta[b0:b1], wl.cap)
            oracle.recall_rows(self.pool, self.cache, a)
            early_stats[b0:b1] = st
            a, s, st = self.sm.final(wl.tok0[b0:b1], idx[b0:b1])
            oracle.recall_rows(self.pool, self.cache, a)
            final_stats[b0:b1] = st
            sel[b0:b1] = s
        self.theta = oracle.theta_rows(self.theta, kth)
        return L, idx, kth, sel, early_stats, final_stats


def _setup(wl, fused=None):
    keys, scale = wk.keys(wl)
    w = wk.head_weights(wl)
    rows = wk.host_rows(wl)
    pool = torch.empty((wl.P, 576), dtype=torch.int16, pin_memory=True)
    pool.numpy()[:] = rows.view(np.int16)
    layer = DecodeLayer(dev(keys), None if scale is None else dev(scale), dev(w), wl.tok0, wl.lens, wl.C,
                        k=wl.k, cap=wl.cap, host_pool=pool, fused=fused)
    return keys, scale, w, pool, layer


def _run_bit_exact(wl, steps, fused=None):
    keys, scale, w, pool, layer = _setup(wl, fused)
    assert layer.fused == (wl.kdtype == 'fp8' if fused is None else fused)
    ref = OracleDecode(wl, keys, scale, w, pool.numpy().copy())
    copied_in_launch = 0
    for s, q in enumerate(wk.decode_queries(wl, steps)):
        layer.step(dev(q))
        torch.cuda.synchronize()
        copied_in_launch += int(host(layer.state.ctr)[10])   # early rows copied by the fused launch itself
        L, idx, kth, sel, est, fst = ref.step(q)
        for b in range(wl.B):
            np.testing.assert_array_equal(host(layer.logits)[b, :wl.lens[b]], L[b], err_msg=f'step {s} row {b}')
        np.testing.assert_array_equal(host(layer.idx), idx, err_msg=f'step {s}')
        np.testing.assert_array_equal(host(layer.kth), kth)
        np.testing.assert_array_equal(host(layer.theta_current), ref.theta)
        np.testing.assert_array_equal(host(layer.sel_slot), sel)
        np.testing.assert_array_equal(host(layer.stats_final), fst)
        np.testing.assert_array_equal(host(layer.stats_early), est)
        np.testing.assert_array_equal(host(layer.state.tok2slot), ref.sm.tok2slot)
        np.testing.assert_array_equal(host(layer.state.slot2tok), ref.sm.slot2tok)
        assert int(host(layer.state.ctr)[0]) == ref.sm.head
        assert int(host(layer.state.ctr)[5]) == 0
        np.testing.assert_array_equal(host(layer.dev_cache), ref.cache)
    np.testing.assert_array_equal(pool.numpy(), ref.pool)   # no write-back
    return layer, copied_in_launch


@pytest.mark.parametrize('fused', [True, False])
def test_dyadic_decode_fp8_batch(fused):
    """fused: the scores and the early fetch in one launch (the default for
    fp8 keys); otherwise the scores, then the EARLY phase on a second
    stream."""
    need_gpu()
    wl = wk.CONFIGS['decode-32x128k-fp8'].scaled(B=4, N=9000, C=20000, steps=5, variant='dyadic')
    _run_bit_exact(wl, 5, fused=fused)


def test_dyadic_decode_fp8_fused_slot_shortage_and_cap():
    """The fused launch with more early misses than free slots (later misses
    dropped) and sequences reaching the cap, over a ring that wraps."""
    need_gpu()
    wl = wk.CONFIGS['decode-64x110k-fp8-capacity'].scaled(B=7, N=6000, len_lo=2000, C=3600, k=512, cap=400,
                                                          steps=6, resample_p=0.5, variant='dyadic')
    layer, copied = _run_bit_exact(wl, 6, fused=True)
    assert copied > 0, 'the fused launch copied no early row itself'


@pytest.mark.parametrize('fused', [True, False])
def test_dyadic_decode_short_and_long_sequences(fused):
    """Ragged lengths from 1 token up, several no longer than k (those rows
    select every token and cannot miss the top-k), in one chunk."""
    need_gpu()
    wl = wk.CONFIGS['decode-64x110k-fp8-capacity'].scaled(B=6, N=3000, len_lo=1, C=7000, k=1024, cap=128,
                                                          steps=4, resample_p=0.0, variant='dyadic')
    assert (wl.lens <= wl.k).any() and (wl.lens > wl.k).any()
    _run_bit_exact(wl, 4, fused=fused)


def test_dyadic_decode_bf16_small_cache():
    need_gpu()
    wl = wk.CONFIGS['decode-1x16k-bf16'].scaled(N=6000, C=2100, variant='dyadic')
    _run_bit_exact(wl, 4)


@pytest.mark.parametrize('fused', [True, False])
def test_dyadic_decode_chunked_capacity(fused):
    """Batch demand above the cache: sequences run in chunks, later chunks
    evict earlier ones' tokens; topic shifts force misses. Fused: the first
    chunk's early fetch is in the scores launch, later chunks' phases follow
    one by one."""
    need_gpu()
    wl = wk.CONFIGS['decode-64x110k-fp8-capacity'].scaled(B=6, N=5000, len_lo=3000, C=5000, k=1024, cap=128,
                                                          steps=5, variant='dyadic')
    assert len(oracle_chunks(wl.lens, wl.k, wl.C)) > 1
    _run_bit_exact(wl, 5, fused=fused)


def test_normal_decode_full_size_single_sequence():
    """The bf16 single-sequence workload at its full size and step count:
    scores within tolerance of the oracle, selections valid against the oracle
    scores, and the cache invariants after every step."""
    need_gpu()
    wl = wk.CONFIGS['decode-1x16k-bf16']
    keys, scale, w, pool, layer = _setup(wl)
    for s, q in enumerate(wk.decode_queries(wl)):
        layer.step(dev(q))
        torch.cuda.synchronize()
        ref = oracle.index_logits(q, w, keys, 'bf16', scale, wl.tok0, wl.lens)[0]
        got = host(layer.logits)[0, :wl.N]
        scale_row = np.abs(ref).max()
        err = np.abs(got - ref) / np.maximum(np.abs(ref), 1e-2 * scale_row)
        assert err.max() <= TOL_BF16
        idx = host(layer.idx)[0]
        kth_ref = np.sort(ref)[-wl.k]
        mask = np.zeros(wl.N, bool)
        mask[idx] = True
        tol = TOL_BF16 * max(abs(kth_ref), 1e-2 * scale_row)
        assert ref[mask].min() >= kth_ref - tol
        assert ref[~mask].max() <= kth_ref + tol
        t2s = host(layer.state.tok2slot)
        s2t = host(layer.state.slot2tok)
        assert np.all(t2s[idx] >= 0)
        occ = np.nonzero(s2t >= 0)[0]
        assert np.all(t2s[s2t[occ]] == occ)
        np.testing.assert_array_equal(host(layer.dev_cache)[occ], pool.numpy()[s2t[occ]])
        np.testing.assert_array_equal(host(layer.sel_slot)[0], t2s[idx])


def test_cache_reset_mid_run_changes_only_residency():
    """The host pool holds every row and nothing is written back (ECHO
    explainer, "One layer, one step"), so dropping the device maps between
    two decode steps (ech_cache_reset, threshold kept) loses nothing: the
    scores, selections, k-th scores and thresholds of every later step are
    those of a run without the reset; only residency changes (the next step
    misses what was resident). The reset run is compared bit for bit with the
    oracle run reset at the same step (a fresh slot map)."""
    need_gpu()
    import indexer_top_kv_amd as ech
    wl = wk.CONFIGS['decode-32x128k-fp8'].scaled(B=4, N=9000, C=20000, steps=5, variant='dyadic')
    keys, scale, w, pool, plain = _setup(wl)
    reset = DecodeLayer(dev(keys), dev(scale), dev(w), wl.tok0, wl.lens, wl.C, k=wl.k, cap=wl.cap, host_pool=pool)
    ref = OracleDecode(wl, keys, scale, w, pool.numpy().copy())
    RESET_AT = 2
    for s, q in enumerate(wk.decode_queries(wl, 5)):
        if s == RESET_AT:
            ech.ech_cache_reset(reset.state)
            ref.sm = oracle.SlotMap(wl.P, wl.C)
        qd = dev(q)
        plain.step(qd)
        reset.step(qd)
        torch.cuda.synchronize()
        L, idx, kth, sel, est, fst = ref.step(q)
        for t in ('logits', 'idx', 'kth'):
            np.testing.assert_array_equal(host(getattr(reset, t)), host(getattr(plain, t)), err_msg=f'{t} step {s}')
        np.testing.assert_array_equal(host(reset.theta_current), host(plain.theta_current))
        np.testing.assert_array_equal(host(reset.idx), idx, err_msg=f'step {s}')
        np.testing.assert_array_equal(host(reset.sel_slot), sel, err_msg=f'step {s}')
        np.testing.assert_array_equal(host(reset.stats_early), est, err_msg=f'step {s}')
        np.testing.assert_array_equal(host(reset.stats_final), fst, err_msg=f'step {s}')
        np.testing.assert_array_equal(host(reset.state.tok2slot), ref.sm.tok2slot, err_msg=f'step {s}')
        assert int(host(reset.state.ctr)[0]) == ref.sm.head
        assert int(host(reset.state.ctr)[5]) == 0
        occ = ref.sm.resident()
        np.testing.assert_array_equal(host(reset.dev_cache)[occ], pool.numpy()[ref.sm.slot2tok[occ]])
        if s == RESET_AT:
            # nothing was resident: no early hits, and the final hits are
            # only tokens this step's early fetch brought in
            est_r, fst_r = host(reset.stats_early), host(reset.stats_final)
            assert np.all(est_r[:, 0] == 0)
            assert np.all(fst_r[:, 0] <= est_r[:, 1])
            assert host(plain.stats_final)[:, 0].sum() > fst_r[:, 0].sum()
