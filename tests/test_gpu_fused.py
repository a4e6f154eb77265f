"""The fused scores + early fetch (ech_index_logits_early) and its live
copier (ech_recall_early_live), checked against the oracle fed the launch's
own scores: scores within tolerance of the float64 oracle, and the early
phase bit for bit (maps, ring head, miss list in allocation order, stats),
then the recalled rows, over several decode steps with normal inputs (so the
thresholds fall between real scores). The copier is run in three schedules:
on a second stream beside the scoring (the normal one), on the same stream
before the fused launch (it finds no list, gives up after its patience and
leaves every row to ech_recall(ECH_EARLY)), and on the same stream after it
(the whole list is there). ECHO explainer, "Decode: fetch above a predicted
threshold" and "One layer, one step: free -> allocate -> recall"."""
import numpy as np
import pytest
import torch

import indexer_top_kv_amd as ech
import oracle
import workloads as wk
from gpu_util import TOL_FP8, dev, host, need_gpu, rel_err

pytestmark = pytest.mark.gpu


def _run(wl, schedule, steps=4, e=None):
    keys, scale = wk.keys(wl)
    w = wk.head_weights(wl)
    rows = wk.host_rows(wl)
    pool = torch.empty((wl.P, 576), dtype=torch.int16, pin_memory=True)
    pool.numpy()[:] = rows.view(np.int16)
    B, N, C, k, cap = wl.B, wl.N, wl.C, wl.k, wl.cap
    e0, e1 = e or (0, B)
    max_len = int(wl.lens.max())
    ld = (max_len + 63) // 64 * 64
    m_early = (e1 - e0) * min(cap, max_len)
    st = ech.LayerState.allocate(wl.P, C, B * min(k, max_len), M_early=m_early)
    ech.ech_cache_reset(st)
    ws = torch.zeros(ech.ech_index_logits_early_ws_bytes(B, max_len, C, m_early), dtype=torch.uint8, device='cuda')
    ws_t = torch.empty(ech.ech_topk_ws_bytes(B, max_len, k), dtype=torch.uint8, device='cuda')
    ws_f = torch.empty(ech.ech_cache_step_ws_bytes(ech.ECH_FINAL, B, B, k, max_len, C, B * min(k, max_len)),
                       dtype=torch.uint8, device='cuda')
    cache = torch.zeros((C, 576), dtype=torch.int16, device='cuda')
    kd, sd, wd = dev(keys), dev(scale), dev(w)
    t0d, lnd = dev(wl.tok0), dev(wl.lens)
    theta = torch.full((B,), float('nan'), dtype=torch.float32, device='cuda')
    sm = oracle.SlotMap(wl.P, C)
    ref_cache = np.zeros((C, 576), np.int16)
    s1 = torch.cuda.Stream()
    copied_live = 0
    for s, q in enumerate(wk.decode_queries(wl, steps)):
        qd = dev(q)
        logits = torch.zeros((B, ld), dtype=torch.float32, device='cuda')
        stats = torch.full((B, 4), -9, dtype=torch.int32, device='cuda')
        s0 = torch.cuda.current_stream()
        fused = lambda: ech.ech_index_logits_early(qd, wd, kd, sd, t0d, lnd, max_len, logits, e0, e1, theta, cap, st,
                                                   stats, ws, stream=s0)
        if schedule == 'beside':
            ev = torch.cuda.Event()
            ev.record(s0)
            fused()
            s1.wait_event(ev)
            ech.ech_recall_early_live(pool, cache, st, ws, stream=s1)
            done = torch.cuda.Event()
            done.record(s0)
            s1.wait_event(done)
            ech.ech_recall(pool, cache, st, phase=ech.ECH_EARLY, stream=s1)
            torch.cuda.synchronize()
        elif schedule == 'copier_first':
            ech.ech_recall_early_live(pool, cache, st, ws, stream=s0)
            fused()
            ech.ech_recall(pool, cache, st, phase=ech.ECH_EARLY, stream=s0)
            torch.cuda.synchronize()
        else:   # copier after the fused launch
            fused()
            ech.ech_recall_early_live(pool, cache, st, ws, stream=s0)
            ech.ech_recall(pool, cache, st, phase=ech.ECH_EARLY, stream=s0)
            torch.cuda.synchronize()
        ctr = host(st.ctr)
        assert ctr[ech.CTR_STATUS] == 0, ctr[ech.CTR_STATUS]
        assert ctr[ech.CTR_LIVE] == 0
        copied_live += int(ctr[ech.CTR_NCOPIED_EARLY])
        L = host(logits)
        # scores against the float64 oracle (two rows), then the early phase
        # bit for bit with the oracle fed the launch's scores
        for b in (0, B - 1):
            ref = oracle.index_logits(q[b:b + 1], w[b:b + 1], keys, 'fp8', scale, wl.tok0[b:b + 1],
                                      wl.lens[b:b + 1])[0]
            assert rel_err(L[b, :wl.lens[b]], ref).max() <= min(TOL_FP8, 1e-5)
        rows_l = [L[b, :wl.lens[b]] for b in range(B)]
        th = host(theta)
        a_o, st_o = sm.early(wl.tok0[e0:e1], rows_l[e0:e1], th[e0:e1], cap)
        n = int(ctr[ech.CTR_NMISS_EARLY])
        assert [tuple(x) for x in host(st.miss_early)[:n].tolist()] == a_o, f'step {s}'
        np.testing.assert_array_equal(host(stats)[e0:e1], st_o, err_msg=f'step {s}')
        np.testing.assert_array_equal(host(st.tok2slot), sm.tok2slot, err_msg=f'step {s}')
        np.testing.assert_array_equal(host(st.slot2tok), sm.slot2tok, err_msg=f'step {s}')
        assert ctr[ech.CTR_HEAD] == sm.head
        oracle.recall_rows(rows.view(np.int16), ref_cache, a_o)
        np.testing.assert_array_equal(host(cache), ref_cache, err_msg=f'step {s}')
        # the top-k and FINAL phase advance the state as a decode step does
        idx = torch.empty((B, k), dtype=torch.int32, device='cuda')
        kth = torch.empty(B, dtype=torch.float32, device='cuda')
        th_next = torch.empty(B, dtype=torch.float32, device='cuda')
        ech.ech_topk(logits, lnd, max_len, k, theta, th_next, idx, kth, ws_t)
        sel = torch.empty((B, k), dtype=torch.int32, device='cuda')
        st_f = torch.empty((B, 4), dtype=torch.int32, device='cuda')
        ech.ech_cache_step(ech.ECH_FINAL, st, t0d, lnd, max_len, idx=idx, k=k, sel_slot=sel, stats=st_f, ws=ws_f)
        ech.ech_recall(pool, cache, st, phase=ech.ECH_FINAL)
        torch.cuda.synchronize()
        idx_o, kth_o = oracle.topk_rows(rows_l, k)
        np.testing.assert_array_equal(host(idx), idx_o)
        a_f, sel_o, stf_o = sm.final(wl.tok0, idx_o)
        oracle.recall_rows(rows.view(np.int16), ref_cache, a_f)
        np.testing.assert_array_equal(host(sel), sel_o)
        np.testing.assert_array_equal(host(cache), ref_cache)
        theta.copy_(th_next)
        np.testing.assert_array_equal(host(theta), oracle.theta_rows(th, kth_o))
    np.testing.assert_array_equal(pool.numpy(), rows.view(np.int16))   # no write-back
    return copied_live


@pytest.mark.parametrize('schedule', ['beside', 'copier_first', 'copier_after'])
def test_fused_early_fetch_schedules(schedule):
    need_gpu()
    wl = wk.CONFIGS['decode-32x128k-fp8'].scaled(B=6, N=20000, C=30000, k=1024, cap=300, variant='normal')
    copied = _run(wl, schedule)
    if schedule == 'copier_first':
        assert copied == 0            # it gave up: ech_recall(ECH_EARLY) copied every row
    if schedule == 'copier_after':
        assert copied > 0


def test_fused_early_fetch_small_ring_and_a_chunk():
    """A ring smaller than one pins window with slot shortage, and the early
    fetch of a chunk of the batch (sequences 2..5 of 7): the other sequences
    are only scored."""
    need_gpu()
    wl = wk.CONFIGS['decode-64x110k-fp8-capacity'].scaled(B=7, N=6000, len_lo=2500, C=4000, k=512, cap=400,
                                                          resample_p=0.5, variant='normal')
    _run(wl, 'beside', steps=5, e=(2, 6))


def test_fused_early_fetch_ring_of_several_pin_windows():
    """A ring of 70000 slots kept nearly full by large selections, so the pins
    kernel takes windows of 16384 positions from a moving head."""
    need_gpu()
    wl = wk.CONFIGS['decode-32x128k-fp8'].scaled(B=8, N=40000, C=70000, k=4096, cap=2000, variant='normal')
    _run(wl, 'beside', steps=5)
