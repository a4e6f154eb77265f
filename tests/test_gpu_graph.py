"""The decode step captured as hipGraphs (one per threshold parity, q read
from a static buffer) replays to exactly the eager results, step after step,
with unrelated eager work and synchronisations between the replays, in both
launch orders of the two branches after the scores (top-k first, EARLY
first). The dyadic variant is also checked against the oracle (exact
scores), so the replays are pinned to the pages' definition, not only to the
eager launches."""
import numpy as np
import pytest
import torch

import workloads as wk
from gpu_util import dev, host, need_gpu
from indexer_top_kv_amd.pipeline import DecodeLayer
from test_gpu_pipeline import OracleDecode

pytestmark = pytest.mark.gpu


def _layer(wl, keys, scale, w, pool, topk_first=None):
    return DecodeLayer(dev(keys), dev(scale), dev(w), wl.tok0, wl.lens, wl.C, k=wl.k, cap=wl.cap, host_pool=pool,
                       topk_first=topk_first)


def _snap(layer):
    return [host(t).copy() for t in (layer.logits, layer.idx, layer.kth, layer.theta_current, layer.sel_slot,
                                     layer.stats_early, layer.stats_final, layer.state.tok2slot,
                                     layer.state.slot2tok, layer.state.ctr, layer.dev_cache)]


@pytest.mark.parametrize('topk_first', [True, False])
@pytest.mark.parametrize('variant', ['dyadic', 'normal'])
def test_graph_replay_matches_eager(variant, topk_first):
    need_gpu()
    wl = wk.CONFIGS['decode-32x128k-fp8'].scaled(B=3, N=7000, C=9000, k=1024, cap=200, variant=variant)
    keys, scale = wk.keys(wl)
    w = wk.head_weights(wl)
    rows = wk.host_rows(wl)
    pool = torch.empty((wl.P, 576), dtype=torch.int16, pin_memory=True)
    pool.numpy()[:] = rows.view(np.int16)
    qs_np = list(wk.decode_queries(wl, 6))
    qs = [dev(q) for q in qs_np]

    eager = _layer(wl, keys, scale, w, pool, topk_first)
    assert eager.topk_first is topk_first
    ref = []
    for q in qs:
        eager.step(q)
        torch.cuda.synchronize()
        ref.append(_snap(eager))

    g = _layer(wl, keys, scale, w, pool, topk_first)
    g.capture()
    orc = OracleDecode(wl, keys, scale, w, rows.view(np.int16).copy()) if variant == 'dyadic' else None
    for s, q in enumerate(qs):
        g.replay(q)
        torch.cuda.synchronize()
        got = _snap(g)
        for a, b in zip(got, ref[s]):
            np.testing.assert_array_equal(a, b, err_msg=f'step {s}')
        if orc is not None:
            L, idx, kth, sel, est, fst = orc.step(qs_np[s])
            for b in range(wl.B):
                np.testing.assert_array_equal(got[0][b, :wl.lens[b]], L[b], err_msg=f'step {s} row {b}')
            for a, b in zip(got[1:7], (idx, kth, orc.theta, sel, est, fst)):
                np.testing.assert_array_equal(a, b, err_msg=f'step {s}')
            np.testing.assert_array_equal(got[7], orc.sm.tok2slot, err_msg=f'step {s}')
            np.testing.assert_array_equal(got[8], orc.sm.slot2tok, err_msg=f'step {s}')
            assert int(got[9][0]) == orc.sm.head and int(got[9][5]) == 0
            np.testing.assert_array_equal(got[10], orc.cache, err_msg=f'step {s}')
        x = torch.arange(4096, device='cuda', dtype=torch.float32)   # unrelated eager work
        assert float((x * 2).sum().item()) == 4096 * 4095
        torch.cuda.synchronize()
