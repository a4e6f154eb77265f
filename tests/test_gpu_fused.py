"""The fused scores + early fetch (ech_index_logits_early) and its live
copier (ech_recall_early_live), checked against the oracle fed the launch's
own scores: scores within tolerance of the float64 oracle, and the early
phase bit for bit (maps, ring head, miss list in allocation order, stats),
then the recalled rows, over several decode steps with normal inputs (so the
thresholds fall between real scores). The copier is run in three schedules:
on a second stream beside the scoring (the normal one), on the same stream
before the fused launch (it finds no list, gives up after its patience and
leaves every row to ech_recall(ECH_EARLY)), and on the same stream after it
(the whole list is there). In the decode step's own schedule the copier
also takes the FINAL list (ech_cache_step(ECH_FINAL) on the first stream),
unless the FINAL allocation walked onto the early phase's slots. ECHO
explainer, "Decode: fetch above a predicted threshold" and "One layer, one
step: free -> allocate -> recall"."""
import numpy as np
import pytest
import torch

import indexer_top_kv_amd as ech
import oracle
import workloads as wk
from gpu_util import TOL_FP8, dev, host, need_gpu, rel_err

pytestmark = pytest.mark.gpu


def _walk(h0, h1, n, C):
    """Ring positions a phase walked from head h0 to its last allocated slot,
    h1 - 1 (0 if it allocated nothing; C if it went all the way round)."""
    if n == 0:
        return 0
    return (h1 - h0) % C or C


def _run(wl, schedule, steps=4, e=None, final_live=False, topk_early=False):
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
    copied_live = copied_final = reached = 0
    for s, q in enumerate(wk.decode_queries(wl, steps)):
        qd = dev(q)
        logits = torch.zeros((B, ld), dtype=torch.float32, device='cuda')
        stats = torch.full((B, 4), -9, dtype=torch.int32, device='cuda')
        s0 = torch.cuda.current_stream()
        fused = lambda: ech.ech_index_logits_early(qd, wd, kd, sd, t0d, lnd, max_len, logits, e0, e1, theta, cap, st,
                                                   stats, ws, stream=s0)
        idx = torch.empty((B, k), dtype=torch.int32, device='cuda')
        kth = torch.empty(B, dtype=torch.float32, device='cuda')
        th_next = torch.empty(B, dtype=torch.float32, device='cuda')
        sel = torch.empty((B, k), dtype=torch.int32, device='cuda')
        st_f = torch.empty((B, 4), dtype=torch.int32, device='cuda')

        def topk_and_final(stream):
            if topk_early:   # from the band lists the fused launch wrote
                ech.ech_topk_early(logits, lnd, max_len, k, theta, th_next, idx, kth, st, ws, stream=stream)
            else:
                ech.ech_topk(logits, lnd, max_len, k, theta, th_next, idx, kth, ws_t, stream=stream)
            ech.ech_cache_step(ech.ECH_FINAL, st, t0d, lnd, max_len, idx=idx, k=k, sel_slot=sel, stats=st_f,
                               ws=ws_f, stream=stream)

        head0 = sm.head
        if final_live and schedule == 'beside':
            # the decode step's schedule: the copier takes the FINAL rows too,
            # then one launch copies what it left of both lists
            ev = torch.cuda.Event()
            ev.record(s0)
            fused()
            s1.wait_event(ev)
            ech.ech_recall_early_live(pool, cache, st, ws, stream=s1, final=True)
            copier_done = torch.cuda.Event()
            copier_done.record(s1)
            topk_and_final(s0)
            s0.wait_event(copier_done)
            ech.ech_recall_rest(pool, cache, st, stream=s0)
            torch.cuda.synchronize()
        elif final_live:
            # the copier finds no list and gives up: every row of both lists,
            # but no early row whose slot the FINAL phase gave away, comes
            # from ech_recall_rest
            assert schedule == 'copier_first'
            ech.ech_recall_early_live(pool, cache, st, ws, stream=s0, final=True)
            fused()
            topk_and_final(s0)
            ech.ech_recall_rest(pool, cache, st, stream=s0)
            torch.cuda.synchronize()
        elif schedule == 'beside':
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
        head1 = sm.head
        if not final_live:
            np.testing.assert_array_equal(host(st.tok2slot), sm.tok2slot, err_msg=f'step {s}')
            np.testing.assert_array_equal(host(st.slot2tok), sm.slot2tok, err_msg=f'step {s}')
            assert ctr[ech.CTR_HEAD] == sm.head
            oracle.recall_rows(rows.view(np.int16), ref_cache, a_o)
            np.testing.assert_array_equal(host(cache), ref_cache, err_msg=f'step {s}')
            # the top-k and FINAL phase advance the state as a decode step does
            topk_and_final(s0)
            ech.ech_recall(pool, cache, st, phase=ech.ECH_FINAL)
            torch.cuda.synchronize()
        else:
            oracle.recall_rows(rows.view(np.int16), ref_cache, a_o)
        ctr = host(st.ctr)
        assert ctr[ech.CTR_STATUS] == 0, ctr[ech.CTR_STATUS]
        idx_o, kth_o = oracle.topk_rows(rows_l, k)
        np.testing.assert_array_equal(host(idx), idx_o)
        a_f, sel_o, stf_o = sm.final(wl.tok0, idx_o)
        oracle.recall_rows(rows.view(np.int16), ref_cache, a_f)
        n_f = int(ctr[ech.CTR_NMISS])
        assert [tuple(x) for x in host(st.miss)[:n_f].tolist()] == a_f, f'step {s}'
        np.testing.assert_array_equal(host(sel), sel_o)
        np.testing.assert_array_equal(host(st.tok2slot), sm.tok2slot, err_msg=f'step {s}')
        np.testing.assert_array_equal(host(st.slot2tok), sm.slot2tok, err_msg=f'step {s}')
        assert ctr[ech.CTR_HEAD] == sm.head
        np.testing.assert_array_equal(host(cache), ref_cache, err_msg=f'step {s}')
        # the FINAL phase's flags: its list complete, and whether its ring walk
        # (from where the early one ended) reached the early phase's slots
        w_e = _walk(head0, head1, n, C)
        w_f = _walk(head1, sm.head, n_f, C)
        assert ctr[ech.CTR_EARLY_WALK] == w_e
        reach = w_e > 0 and w_f > 0 and w_e + w_f > C
        assert ctr[ech.CTR_FINAL_READY] == (3 if reach else 1), (ctr[ech.CTR_FINAL_READY], w_e, w_f)
        if reach:
            assert ctr[ech.CTR_NCOPIED_FINAL] == 0
            reached += 1
        copied_final += int(ctr[ech.CTR_NCOPIED_FINAL])
        theta.copy_(th_next)
        np.testing.assert_array_equal(host(theta), oracle.theta_rows(th, kth_o))
    np.testing.assert_array_equal(pool.numpy(), rows.view(np.int16))   # no write-back
    return copied_live, copied_final, reached


@pytest.mark.parametrize('schedule', ['beside', 'copier_first', 'copier_after'])
def test_fused_early_fetch_schedules(schedule):
    need_gpu()
    wl = wk.CONFIGS['decode-32x128k-fp8'].scaled(B=6, N=20000, C=30000, k=1024, cap=300, variant='normal')
    copied, copied_final, _ = _run(wl, schedule)
    assert copied_final == 0          # the copier was not given the FINAL list
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


def test_fused_copier_takes_the_final_rows():
    """The decode step's schedule: the copier goes on from the early rows to
    the FINAL ones once the FINAL phase on the other stream has completed its
    list; the maps, both lists and the cache match the oracle, and the
    FINAL rows were copied by the copier."""
    need_gpu()
    wl = wk.CONFIGS['decode-32x128k-fp8'].scaled(B=6, N=20000, C=30000, k=1024, cap=300, variant='normal')
    copied, copied_final, reached = _run(wl, 'beside', final_live=True, topk_early=True)
    assert copied > 0 and copied_final > 0 and reached == 0


def test_fused_copier_final_rows_small_ring():
    """A ring barely larger than the FINAL demand (4 x 1024 of 4200 slots),
    so that in the second step the FINAL allocation walks round onto the
    slots the early phase filled: then the copier leaves every FINAL row to
    ech_recall(ECH_FINAL) (the flag checked against the oracle's ring walks
    in every step)."""
    need_gpu()
    wl = wk.CONFIGS['decode-64x110k-fp8-capacity'].scaled(B=4, N=6000, len_lo=2500, C=4200, k=1024, cap=800,
                                                          resample_p=0.5, variant='normal')
    _, _, reached = _run(wl, 'beside', steps=5, final_live=True, topk_early=True)
    assert reached >= 1


def test_recall_rest_after_a_copier_that_gave_up_small_ring():
    """The copier gives up (it runs before the fused launch), so
    ech_recall_rest copies both whole lists in one launch; in the step whose
    FINAL allocation reaches the early slots, the early rows of the slots the
    FINAL phase gave away are skipped, so each slot ends with its own
    token's row (checked against the oracle's cache)."""
    need_gpu()
    wl = wk.CONFIGS['decode-64x110k-fp8-capacity'].scaled(B=4, N=6000, len_lo=2500, C=4200, k=1024, cap=800,
                                                          resample_p=0.5, variant='normal')
    copied, copied_final, reached = _run(wl, 'copier_first', steps=3, final_live=True, topk_early=True)
    assert copied == 0 and copied_final == 0 and reached >= 1


@pytest.mark.parametrize('pred', ['near', 'high', 'low', 'nan', 'mixed', 'other'])
def test_topk_early_matches_the_oracle(pred):
    """ech_topk_early selects from the band lists the scoring waves wrote. The
    predictions steer which way it goes: near the k-th score (the lists
    decide), far above it (the band holds fewer than k tokens), far below it
    (the waves' bands overflow their slices), NaN, a mix over the rows, and a
    call with a theta other than the one the lists were made against (the
    whole row is selected). Each must give exactly the oracle's selection,
    kth and EMA update, and ech_topk's bits on the same scores.
    ECHO explainer, "Prefill: one-round histogram" and "Fused indexer kernel
    (extends DeepGEMM)"."""
    need_gpu()
    wl = wk.CONFIGS['decode-32x128k-fp8'].scaled(B=6, N=40000, C=30000, k=1024, cap=300, variant='normal')
    keys, scale = wk.keys(wl)
    w = wk.head_weights(wl)
    B, C, k, cap = wl.B, wl.C, wl.k, wl.cap
    max_len = int(wl.lens.max())
    ld = (max_len + 63) // 64 * 64
    m_early = B * min(cap, max_len)
    st = ech.LayerState.allocate(wl.P, C, B * min(k, max_len), M_early=m_early)
    ws = torch.zeros(ech.ech_index_logits_early_ws_bytes(B, max_len, C, m_early), dtype=torch.uint8, device='cuda')
    kd, sd, wd = dev(keys), dev(scale), dev(w)
    t0d, lnd = dev(wl.tok0), dev(wl.lens)
    q = next(iter(wk.decode_queries(wl, 1)))
    qd = dev(q)
    logits = torch.zeros((B, ld), dtype=torch.float32, device='cuda')
    stats = torch.zeros((B, 4), dtype=torch.int32, device='cuda')

    def fused(theta):
        ech.ech_cache_reset(st)
        ech.ech_index_logits_early(qd, wd, kd, sd, t0d, lnd, max_len, logits, 0, B, theta, cap, st, stats, ws)

    fused(torch.full((B,), float('nan'), device='cuda'))
    torch.cuda.synchronize()
    rows_l = [host(logits)[b, :wl.lens[b]] for b in range(B)]
    idx_o, kth_o = oracle.topk_rows(rows_l, k)
    kth_o = np.asarray(kth_o, np.float32)
    scale_by = {'near': 1.01, 'high': 1.6, 'low': -1.0, 'other': 1.01}
    if pred in scale_by:
        th = (kth_o * np.float32(scale_by[pred])).astype(np.float32)
    elif pred == 'nan':
        th = np.full(B, np.nan, np.float32)
    else:
        th = np.array([kth_o[b] * f for b, f in enumerate([1.0, 1.6, -1.0, np.nan, 0.99, 1.02])], np.float32)
    thd = dev(th)
    fused(thd)
    if pred == 'other':   # the selection is asked with another theta than the lists were made against
        th = (th * np.float32(1.001)).astype(np.float32)
        thd = dev(th)
    idx = torch.full((B, k), -7, dtype=torch.int32, device='cuda')
    kth = torch.empty(B, dtype=torch.float32, device='cuda')
    th_next = torch.empty(B, dtype=torch.float32, device='cuda')
    ech.ech_topk_early(logits, lnd, max_len, k, thd, th_next, idx, kth, st, ws)
    ws_t = torch.empty(ech.ech_topk_ws_bytes(B, max_len, k), dtype=torch.uint8, device='cuda')
    idx2 = torch.full((B, k), -7, dtype=torch.int32, device='cuda')
    kth2, th2 = torch.empty_like(kth), torch.empty_like(th_next)
    ech.ech_topk(logits, lnd, max_len, k, thd, th2, idx2, kth2, ws_t)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(idx), idx_o)
    np.testing.assert_array_equal(host(kth), kth_o)
    np.testing.assert_array_equal(host(th_next), oracle.theta_rows(th, kth_o))
    np.testing.assert_array_equal(host(idx), host(idx2))
    np.testing.assert_array_equal(host(kth).view(np.int32), host(kth2).view(np.int32))
    np.testing.assert_array_equal(host(th_next).view(np.int32), host(th2).view(np.int32))
