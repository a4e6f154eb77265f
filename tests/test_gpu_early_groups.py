"""The early fetch in sequence groups (ech_early_begin / ech_early_group /
ech_recall_group) against the single EARLY phase of ech_cache_step and the
oracle's early phase, on the same state and the same GPU scores.

The grouped form scores the resident tokens itself to find the pins; it must
reproduce the scores kernel bit for bit, so thresholds are set exactly to the
score of a resident token (a token scoring equal to theta is not above it: a
one-ulp difference would change the pins). Every grouping must give the same
maps, miss list, head, counters and statistics as the single phase.
"""
import numpy as np
import pytest
import torch

import indexer_top_kv_amd as ech
import oracle
from gpu_util import dev, host, need_gpu
from indexer_top_kv_amd.pipeline import sequence_groups

pytestmark = pytest.mark.gpu


def _inputs(rng, B, lens, kdtype):
    P = int(np.sum(lens))
    tok0 = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    if kdtype == 'fp8':
        keys = torch.randn(P, 128).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        scale = rng.uniform(0.5, 2.0, P).astype(np.float32)
        scale[tok0[-1]:] *= -1.0                     # one sequence with negative scales
    else:
        keys = torch.randn(P, 128).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        scale = None
    q = torch.randn(B, 64, 128).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    w = (rng.uniform(0, 1, (B, 64)) / 8).astype(np.float32)
    return P, tok0, keys, scale, q, w


def _warm_state(rng, P, C, tok0, lens, k, steps=3):
    """A lived-in slot map: a few FINAL phases over random selections."""
    sm = oracle.SlotMap(P, C)
    for _ in range(steps):
        idx = np.full((len(lens), k), -1, np.int64)
        for b, n in enumerate(lens):
            m = min(k, int(n))
            idx[b, :m] = np.sort(rng.choice(int(n), m, replace=False))
        sm.final(tok0, idx)
    return sm


def _upload(sm, P, C, M):
    st = ech.LayerState.allocate(P, C, M)
    st.tok2slot.copy_(torch.from_numpy(sm.tok2slot.astype(np.int32)))
    st.slot2tok.copy_(torch.from_numpy(sm.slot2tok.astype(np.int32)))
    st.slot_pin.zero_()
    ctr = np.zeros(ech.CTR_LEN, np.int32)
    ctr[ech.CTR_HEAD] = sm.head
    ctr[ech.CTR_EPOCH] = 7
    st.ctr.copy_(torch.from_numpy(ctr))
    st.miss_early.fill_(-9)
    return st


def _thresholds(rng, L, sm, tok0, lens, nan_rows=(), quantile=0.97):
    """theta[b] = the score of a resident token of b near the given
    percentile (so ties with theta occur on resident tokens), NaN for
    nan_rows."""
    th = np.full(len(lens), np.nan, np.float32)
    for b, n in enumerate(lens):
        if b in nan_rows:
            continue
        s = L[b]
        res = np.nonzero(sm.tok2slot[tok0[b] + np.arange(n)] >= 0)[0]
        target = np.quantile(s, quantile)
        t = res[np.argmin(np.abs(s[res] - target))] if len(res) else int(np.argmax(s))
        th[b] = s[t]
    return th


def _run_case(B, lens, C, k, cap, kdtype, groups_list, nan_rows=(), seed=0, quantile=0.97):
    need_gpu()
    rng = np.random.default_rng(seed)
    torch.manual_seed(seed)
    lens = np.asarray(lens, np.int32)
    max_len = int(lens.max())
    P, tok0, keys, scale, q, w = _inputs(rng, B, lens, kdtype)
    sm0 = _warm_state(rng, P, C, tok0, lens, k)
    M = B * min(cap, max_len)
    ld = (max_len + 63) // 64 * 64
    qd, wd, kd = dev(q), dev(w), dev(keys)
    sd = None if scale is None else dev(scale)
    t0d, lnd = dev(tok0), dev(lens)
    logits = torch.zeros((B, ld), dtype=torch.float32, device='cuda')
    ech.ech_index_logits(qd, wd, kd, sd, t0d, lnd, max_len, logits)
    torch.cuda.synchronize()
    Lh = host(logits)
    L = [Lh[b, :lens[b]].copy() for b in range(B)]
    theta = _thresholds(rng, L, sm0, tok0, lens, nan_rows, quantile)
    thd = dev(theta)

    # oracle
    sm = oracle.SlotMap(P, C)
    sm.tok2slot[:] = sm0.tok2slot
    sm.slot2tok[:] = sm0.slot2tok
    sm.head = sm0.head
    assigned, ostats = sm.early(tok0, L, theta, cap)
    omiss = np.asarray(assigned, np.int64).reshape(-1, 2)

    # single EARLY phase
    st_a = _upload(sm0, P, C, M)
    stats_a = torch.full((B, 4), -3, dtype=torch.int32, device='cuda')
    ws_a = torch.empty(ech.ech_cache_step_ws_bytes(ech.ECH_EARLY, B, B, k, max_len, C, M), dtype=torch.uint8,
                       device='cuda')
    ech.ech_cache_step(ech.ECH_EARLY, st_a, t0d, lnd, max_len, k=k, logits=logits, theta=thd, cap=cap,
                       stats=stats_a, ws=ws_a)
    torch.cuda.synchronize()
    n_a = int(host(st_a.ctr)[ech.CTR_NMISS_EARLY])
    assert n_a == len(omiss)
    np.testing.assert_array_equal(host(st_a.miss_early)[:n_a], omiss)
    np.testing.assert_array_equal(host(stats_a), ostats)
    np.testing.assert_array_equal(host(st_a.tok2slot), sm.tok2slot)
    np.testing.assert_array_equal(host(st_a.slot2tok), sm.slot2tok)
    assert int(host(st_a.ctr)[ech.CTR_HEAD]) == sm.head

    ws_g = torch.empty(ech.ech_early_ws_bytes(B, max_len, C, M), dtype=torch.uint8, device='cuda')
    for ng in groups_list:
        st_b = _upload(sm0, P, C, M)
        stats_b = torch.full((B, 4), -3, dtype=torch.int32, device='cuda')
        ech.ech_early_begin(qd, wd, kd, sd, t0d, lnd, max_len, thd, st_b, stats_b, ws_g)
        for g, (b0, b1) in enumerate(sequence_groups(B, ng)):
            ech.ech_early_group(g, b0, b1, logits, thd, cap, t0d, lnd, max_len, st_b, stats_b, ws_g)
        torch.cuda.synchronize()
        ca, cb = host(st_a.ctr), host(st_b.ctr)
        for i in (ech.CTR_HEAD, ech.CTR_NMISS_EARLY, ech.CTR_NWANT, ech.CTR_NPINNED, ech.CTR_NEVICT,
                  ech.CTR_STATUS):
            assert ca[i] == cb[i], (ng, i, ca[i], cb[i])
        assert cb[ech.CTR_TICKET] == 0
        assert cb[ech.CTR_EPOCH] == ca[ech.CTR_EPOCH]
        np.testing.assert_array_equal(host(st_b.miss_early)[:n_a], omiss, err_msg=f'groups {ng}')
        np.testing.assert_array_equal(host(stats_b), ostats, err_msg=f'groups {ng}')
        np.testing.assert_array_equal(host(st_b.tok2slot), sm.tok2slot, err_msg=f'groups {ng}')
        np.testing.assert_array_equal(host(st_b.slot2tok), sm.slot2tok, err_msg=f'groups {ng}')
        # the same pins: slot_pin equals the epoch exactly where the single phase pinned
        np.testing.assert_array_equal(host(st_b.slot_pin) == cb[ech.CTR_EPOCH],
                                      host(st_a.slot_pin) == ca[ech.CTR_EPOCH], err_msg=f'groups {ng}')
    return ostats


def test_groups_fp8_ragged():
    st = _run_case(B=5, lens=[9000, 4100, 12000, 1, 7777], C=5000, k=512, cap=64, kdtype='fp8',
                   groups_list=[1, 2, 3, 5])
    assert st[:, 0].sum() > 0 and st[:, 1].sum() > 0 and st[:, 3].sum() > 0


def test_groups_slot_shortage_and_nan_rows():
    """More early misses than unpinned slots: the later ones are dropped;
    two sequences have no prediction (no pins, no misses)."""
    st = _run_case(B=6, lens=[5000] * 6, C=3200, k=512, cap=2000, kdtype='fp8', groups_list=[1, 4, 6],
                   nan_rows=(1, 4), seed=3, quantile=0.5)
    assert st[:, 2].sum() > 0
    assert np.all(st[[1, 4]] == 0)


def test_groups_bf16_single_sequence_long():
    _run_case(B=1, lens=[70000], C=6000, k=2048, cap=512, kdtype='bf16', groups_list=[1], seed=5)


def test_groups_many_chunks_per_sequence():
    """Sequences spanning many 4096-token blocks (rank offsets carried across
    blocks and groups)."""
    _run_case(B=3, lens=[150000, 20000, 90001], C=20000, k=1024, cap=512, kdtype='fp8',
              groups_list=[1, 2, 3], seed=9)


def test_grouped_recall_rows():
    """ech_recall_group copies each group's rank range: after all groups the
    device cache holds the host rows of every early allocation."""
    need_gpu()
    rng = np.random.default_rng(11)
    torch.manual_seed(11)
    B, lens, C, k, cap = 4, np.array([6000, 6000, 3000, 8000], np.int32), 9000, 512, 128
    max_len = int(lens.max())
    P, tok0, keys, scale, q, w = _inputs(rng, B, lens, 'fp8')
    sm0 = _warm_state(rng, P, C, tok0, lens, k)
    M = B * cap
    ld = (max_len + 63) // 64 * 64
    qd, wd, kd, sd, t0d, lnd = dev(q), dev(w), dev(keys), dev(scale), dev(tok0), dev(lens)
    logits = torch.zeros((B, ld), dtype=torch.float32, device='cuda')
    ech.ech_index_logits(qd, wd, kd, sd, t0d, lnd, max_len, logits)
    torch.cuda.synchronize()
    Lh = host(logits)
    theta = _thresholds(rng, [Lh[b, :lens[b]] for b in range(B)], sm0, tok0, lens)
    st = _upload(sm0, P, C, M)
    pool = torch.empty((P, 576), dtype=torch.int16, pin_memory=True)
    pool.numpy()[:] = rng.integers(-30000, 30000, (P, 576), dtype=np.int16)
    cache = torch.full((C, 576), 5, dtype=torch.int16, device='cuda')
    stats = torch.zeros((B, 4), dtype=torch.int32, device='cuda')
    ws = torch.empty(ech.ech_early_ws_bytes(B, max_len, C, M), dtype=torch.uint8, device='cuda')
    thd = dev(theta)
    ech.ech_early_begin(qd, wd, kd, sd, t0d, lnd, max_len, thd, st, stats, ws)
    s2 = torch.cuda.Stream()
    for g, (b0, b1) in enumerate(sequence_groups(B, 4)):
        ech.ech_early_group(g, b0, b1, logits, thd, cap, t0d, lnd, max_len, st, stats, ws)
        ev = torch.cuda.Event()
        ev.record()
        s2.wait_event(ev)
        ech.ech_recall_group(g, pool, cache, st, ws, stream=s2)
    torch.cuda.current_stream().wait_stream(s2)
    torch.cuda.synchronize()
    n = int(host(st.ctr)[ech.CTR_NMISS_EARLY])
    assert n > 0
    miss = host(st.miss_early)[:n]
    c = host(cache)
    np.testing.assert_array_equal(c[miss[:, 1]], pool.numpy()[miss[:, 0]])
    untouched = np.setdiff1d(np.arange(C), miss[:, 1])
    assert np.all(c[untouched] == 5)
    assert int(host(st.ctr)[ech.CTR_RECALLED]) == n
    assert int(host(st.ctr)[ech.CTR_STATUS]) == 0
