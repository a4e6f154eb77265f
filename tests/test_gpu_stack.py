"""A decode step over several layers and two micro-batches (DecodeStack),
eager and as captured graphs, against the oracle run layer by layer and
micro-batch by micro-batch.

Each (layer, micro-batch) pair has its own slot map and device cache and
reads its layer's keys and host pool at its sequences' token offsets; the
stack only orders the launches and the stream events between them, so with
dyadic inputs (exact scores) every result must equal the oracle's bit for
bit: scores, selections, slot maps, sel_slot, thresholds and recalled rows.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wk
from gpu_util import dev, host, need_gpu
from indexer_top_kv_amd.pipeline import DecodeLayer, DecodeStack, sequence_groups

pytestmark = pytest.mark.gpu


class OracleMicro:
    """The oracle's decode step for sequences [b0, b1) of one layer, with a
    slot map and device cache of its own (one chunk: the demand fits)."""

    def __init__(self, wl, keys, scale, w, pool, b0, b1, C):
        self.keys, self.scale, self.kdtype = keys, scale, wl.kdtype
        self.w, self.tok0, self.lens = w[b0:b1], wl.tok0[b0:b1], wl.lens[b0:b1]
        self.k, self.cap = wl.k, wl.cap
        assert int(np.minimum(self.lens, self.k).sum()) <= C
        self.sm = oracle.SlotMap(wl.P, C)
        self.theta = np.full(b1 - b0, np.nan, np.float32)
        self.pool = pool
        self.cache = np.zeros((C, pool.shape[1]), pool.dtype)

    def step(self, q):
        L = [x.astype(np.float32) for x in oracle.index_logits(q, self.w, self.keys, self.kdtype, self.scale,
                                                                 self.tok0, self.lens)]
        idx, kth = oracle.topk_rows(L, self.k)
        a, _ = self.sm.early(self.tok0, L, self.theta, self.cap)
        oracle.recall_rows(self.pool, self.cache, a)
        a, sel, _ = self.sm.final(self.tok0, idx)
        oracle.recall_rows(self.pool, self.cache, a)
        self.theta = oracle.theta_rows(self.theta, kth)
        return L, idx, sel


def _build(base, L, M, C_m, steps):
    layers, refs, qs = [], [], []
    groups = sequence_groups(base.B, M)
    for l in range(L):
        wl = base.scaled(layer=l)
        keys, scale = wk.keys(wl)
        w = wk.head_weights(wl)
        pool = torch.empty((wl.P, 576), dtype=torch.int16, pin_memory=True)
        pool.numpy()[:] = wk.host_rows(wl).view(np.int16)
        kc, ks, wd = dev(keys), dev(scale), dev(w)
        layers.append([DecodeLayer(kc, ks, wd[b0:b1], wl.tok0[b0:b1], wl.lens[b0:b1], C_m, k=wl.k, cap=wl.cap,
                                   host_pool=pool, fused=False) for b0, b1 in groups])
        refs.append([OracleMicro(wl, keys, scale, w, pool.numpy().copy(), b0, b1, C_m) for b0, b1 in groups])
        qs.append([q for q in wk.decode_queries(wl, steps)])
    return groups, layers, refs, qs


@pytest.mark.parametrize('graph,L,M', [(False, 3, 2), (True, 3, 2), (False, 2, 3), (True, 2, 3)],
                         ids=['eager-3x2', 'graph-3x2', 'eager-2x3', 'graph-2x3'])
def test_stack_matches_oracle_per_layer(graph, L, M):
    need_gpu()
    base = wk.CONFIGS['decode-64x110k-fp8-capacity'].scaled(B=5, N=7000, len_lo=3000, k=512, cap=128,
                                                            variant='dyadic', resample_p=0.3)
    C_m, steps = 1700, 4
    groups, layers, refs, qs = _build(base, L, M, C_m, steps)
    stack = DecodeStack(layers)
    if graph:
        stack.capture()
    evictions = 0
    for s in range(steps):
        q_step = [[dev(qs[l][s])[b0:b1] for b0, b1 in groups] for l in range(L)]
        (stack.replay if graph else stack.step)(q_step)
        torch.cuda.synchronize()
        for l in range(L):
            for m, (b0, b1) in enumerate(groups):
                d, o = layers[l][m], refs[l][m]
                Lo, idx, sel = o.step(qs[l][s][b0:b1])
                tag = f'step {s} layer {l} micro-batch {m}'
                for b in range(b1 - b0):
                    np.testing.assert_array_equal(host(d.logits)[b, :o.lens[b]], Lo[b], err_msg=tag)
                np.testing.assert_array_equal(host(d.idx), idx, err_msg=tag)
                np.testing.assert_array_equal(host(d.sel_slot), sel, err_msg=tag)
                np.testing.assert_array_equal(host(d.theta_current), o.theta, err_msg=tag)
                np.testing.assert_array_equal(host(d.state.tok2slot), o.sm.tok2slot, err_msg=tag)
                np.testing.assert_array_equal(host(d.state.slot2tok), o.sm.slot2tok, err_msg=tag)
                np.testing.assert_array_equal(host(d.dev_cache), o.cache, err_msg=tag)
                ctr = host(d.state.ctr)
                assert int(ctr[0]) == o.sm.head and int(ctr[5]) == 0, tag
                evictions += int(host(d.stats_final)[:, 3].sum()) + int(host(d.stats_early)[:, 3].sum())
        # unrelated eager work between steps
        x = torch.arange(4096, device='cuda', dtype=torch.float32)
        assert float((x * 2).sum().item()) == 4096 * 4095
    assert evictions > 0                  # the small caches were under pressure
    for l in range(L):
        for m in range(M):
            np.testing.assert_array_equal(layers[l][m].host_pool.numpy(), refs[l][m].pool)   # no write-back


def test_stack_rejects_bad_shapes():
    need_gpu()
    with pytest.raises(ValueError):
        DecodeStack([])
    base = wk.CONFIGS['decode-32x128k-fp8'].scaled(B=2, N=3000, C=5000, k=256, cap=64, variant='dyadic')
    keys, scale = wk.keys(base)
    w = dev(wk.head_weights(base))
    mk = lambda: DecodeLayer(dev(keys), dev(scale), w, base.tok0, base.lens, base.C, k=base.k, cap=base.cap)
    with pytest.raises(ValueError):
        DecodeStack([[mk(), mk()], [mk()]])
    # the fused path: its scores launch starts the live copier, which a graph
    # of the rest of the step would not wait for
    pool = torch.zeros((base.P, 576), dtype=torch.int16, pin_memory=True)
    fused = DecodeLayer(dev(keys), dev(scale), w, base.tok0, base.lens, base.C, k=base.k, cap=base.cap,
                        host_pool=pool, fused=True)
    with pytest.raises(ValueError):
        DecodeStack([[fused]])
    with pytest.raises(ValueError):
        fused.capture(scores=False)
