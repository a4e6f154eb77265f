"""The decode step exactly as bench.py times it, checked against the oracle.

Workload decode-32x128k-fp8 at its full size: 32 sequences x 131072 tokens,
fp8 keys with per-token scales, k = 2048, early-fetch cap 512, a device cache
of 260000 slots, 1152-byte rows in a pinned host pool. The layer is built
with bench.py's arguments (the scores and the early fetch are one launch; a
copier on the second stream moves the early rows, then the FINAL rows). The
step is captured as hipGraphs before any step runs and every step, the cold
one included, is a replay, as in bench.py's warm-up and timed region.

Dyadic inputs (small integers, power-of-two scales, head weights m/64) make
every score exact in float32, so the oracle sees the same scores and every
stage must agree bit for bit at every step: scores, idx, kth, theta, the
EARLY and FINAL statistics, sel_slot, both maps, the ring head, both miss
lists, the status word and the whole device cache; the host pool is
unchanged (no write-back). The ECHO explainer's "Five fixed-size integer
tensors on the GPU" (a decode step is one captured graph) and "Decode: fetch
above a predicted threshold" (early fetch above the EMA threshold) define the
step."""
import numpy as np
import pytest
import torch

import indexer_top_kv_amd as ech
import workloads as wk
from gpu_util import dev, host, need_gpu
from indexer_top_kv_amd.pipeline import DecodeLayer
from test_gpu_pipeline import OracleDecode

pytestmark = pytest.mark.gpu


def _compare(layer, ref, L, idx, kth, sel, est, fst, a_early, a_final, s, wl):
    tag = f'step {s}'
    got = host(layer.logits)
    for b in range(wl.B):
        np.testing.assert_array_equal(got[b, :wl.lens[b]], L[b], err_msg=f'{tag} scores row {b}')
    np.testing.assert_array_equal(host(layer.idx), idx, err_msg=f'{tag} idx')
    np.testing.assert_array_equal(host(layer.kth), kth, err_msg=f'{tag} kth')
    np.testing.assert_array_equal(host(layer.theta_current), ref.theta, err_msg=f'{tag} theta')
    np.testing.assert_array_equal(host(layer.stats_early), est, err_msg=f'{tag} early stats')
    np.testing.assert_array_equal(host(layer.stats_final), fst, err_msg=f'{tag} final stats')
    np.testing.assert_array_equal(host(layer.sel_slot), sel, err_msg=f'{tag} sel_slot')
    np.testing.assert_array_equal(host(layer.state.tok2slot), ref.sm.tok2slot, err_msg=f'{tag} tok2slot')
    np.testing.assert_array_equal(host(layer.state.slot2tok), ref.sm.slot2tok, err_msg=f'{tag} slot2tok')
    ctr = host(layer.state.ctr)
    assert int(ctr[ech.CTR_HEAD]) == ref.sm.head, tag
    assert int(ctr[ech.CTR_STATUS]) == 0, tag
    n_e, n_f = int(ctr[ech.CTR_NMISS_EARLY]), int(ctr[ech.CTR_NMISS])
    assert [tuple(x) for x in host(layer.state.miss_early)[:n_e].tolist()] == a_early, f'{tag} early misses'
    assert [tuple(x) for x in host(layer.state.miss)[:n_f].tolist()] == a_final, f'{tag} final misses'
    np.testing.assert_array_equal(host(layer.dev_cache), ref.cache, err_msg=f'{tag} device cache')


class _Recorder(OracleDecode):
    """The oracle decode step, also keeping each phase's (g, slot) list."""

    def step(self, q):
        import oracle
        wl = self.wl
        assert len(self.chunks) == 1
        L = [x.astype(np.float32) for x in oracle.index_logits(q, self.w, self.keys, wl.kdtype, self.scale,
                                                                 wl.tok0, wl.lens)]
        idx, kth = oracle.topk_rows(L, wl.k)
        a_e, est = self.sm.early(wl.tok0, L, self.theta, wl.cap)
        oracle.recall_rows(self.pool, self.cache, a_e)
        a_f, sel, fst = self.sm.final(wl.tok0, idx)
        oracle.recall_rows(self.pool, self.cache, a_f)
        self.theta = oracle.theta_rows(self.theta, kth)
        return L, idx, kth, sel, est, fst, a_e, a_f


def test_benched_decode_step_full_size_captured_bit_exact():
    need_gpu()
    wl = wk.CONFIGS['decode-32x128k-fp8'].scaled(variant='dyadic')
    assert (wl.B, wl.N, wl.C, wl.k, wl.cap) == (32, 131072, 260000, 2048, 512)
    keys, scale = wk.keys(wl)
    w = wk.head_weights(wl)
    pool = torch.empty((wl.P, wk.ROW_ELEMS), dtype=torch.int16, pin_memory=True)
    wk.host_rows(wl, out=pool.numpy().view(np.uint16))
    pool_before = pool.numpy().copy()
    # bench.py's construction (launch order and fusion at their defaults)
    layer = DecodeLayer(dev(keys), dev(scale), dev(w), wl.tok0, wl.lens, wl.C, k=wl.k, cap=wl.cap, host_pool=pool)
    assert layer.fused and len(layer.chunks) == 1
    ref = _Recorder(wl, keys, scale, w, pool.numpy())
    qs = list(wk.decode_queries(wl, 5))
    fetched_early = 0
    layer.capture()                  # before any step, as bench.py does: every step is a replay
    for s, q in enumerate(qs):
        layer.replay(dev(q))
        torch.cuda.synchronize()
        out = ref.step(q)
        _compare(layer, ref, *out, s, wl)
        fetched_early += int(out[4][:, 1].sum())
    assert fetched_early > 0, 'the early fetch never ran'
    np.testing.assert_array_equal(pool.numpy(), pool_before)
