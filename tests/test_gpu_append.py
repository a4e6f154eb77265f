"""Growing contexts: ech_kv_append against the oracle's append, and decode
steps with a token appended to every sequence between them against the
oracle run the same way (dyadic inputs: exact scores, so every stage agrees
bit for bit), up to a sequence reaching its capacity."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wk
from gpu_util import dev, host, need_gpu
import indexer_top_kv_amd as ech
from indexer_top_kv_amd.pipeline import DecodeLayer

pytestmark = pytest.mark.gpu


def _dyadic(r, lens, cap, kdtype):
    tok0 = np.concatenate([[0], np.cumsum(cap)[:-1]]).astype(np.int64)
    P = int(np.sum(cap))
    x = r.integers(-8, 9, (P, 128)).astype(np.float32)
    if kdtype == 'fp8':
        keys = wk.to_e4m3_bits(x)
        scale = np.array([0.5, 1.0, 2.0], np.float32)[r.integers(0, 3, P)]
    else:
        keys = wk.to_bf16_bits(x)
        scale = None
    rows = wk.to_bf16_bits(r.standard_normal((P, 576)).astype(np.float32))
    return tok0, P, keys, scale, rows


@pytest.mark.parametrize('kdtype', ['fp8', 'bf16'])
def test_append_kernel_against_oracle(kdtype):
    need_gpu()
    r = np.random.default_rng(1 if kdtype == 'fp8' else 2)
    cap = np.array([5, 3, 8, 1, 4], np.int32)
    lens = np.array([2, 3, 0, 1, 3], np.int32)              # sequences 1 and 3 are full
    tok0, P, keys, scale, rows = _dyadic(r, lens, cap, kdtype)
    B = len(cap)
    st = ech.LayerState.allocate(P, 16, 16)
    ech.ech_cache_reset(st)
    t2s = r.integers(-1, 16, P).astype(np.int32)
    st.tok2slot.copy_(torch.from_numpy(t2s))
    pool = torch.empty((P, 576), dtype=torch.int16, pin_memory=True)
    pool.numpy()[:] = rows.view(np.int16)
    kc = dev(keys)
    ks = dev(scale) if scale is not None else None
    ld = dev(lens)
    new_rows = wk.to_bf16_bits(r.standard_normal((B, 576)).astype(np.float32))
    new_keys = keys[:B].copy() * 0 + (wk.to_e4m3_bits(r.integers(-8, 9, (B, 128)).astype(np.float32)) if kdtype == 'fp8'
                                      else wk.to_bf16_bits(r.integers(-8, 9, (B, 128)).astype(np.float32)))
    new_sc = np.array([2.0, 0.5, 1.0, 1.0, 0.5], np.float32) if kdtype == 'fp8' else None
    ech.ech_kv_append(pool, kc, ks, st, dev(tok0), ld, dev(cap), dev(new_rows), dev(new_keys),
                      dev(new_sc) if new_sc is not None else None)
    torch.cuda.synchronize()
    o_pool, o_keys, o_t2s, o_lens = rows.copy(), keys.copy(), t2s.copy(), lens.copy()
    o_sc = scale.copy() if scale is not None else None
    full = oracle.kv_append(o_pool, o_keys, o_sc, o_t2s, tok0, o_lens, cap, new_rows, new_keys, new_sc)
    assert full
    np.testing.assert_array_equal(pool.numpy().view(np.uint16), o_pool)
    np.testing.assert_array_equal(host(kc).view(o_keys.dtype), o_keys)
    if o_sc is not None:
        np.testing.assert_array_equal(host(ks), o_sc)
    np.testing.assert_array_equal(host(st.tok2slot), o_t2s)
    np.testing.assert_array_equal(host(ld), o_lens)
    assert int(host(st.ctr)[ech.CTR_STATUS]) & ech.ST_FULL


def test_growing_decode_against_oracle():
    need_gpu()
    r = np.random.default_rng(7)
    lens0 = np.array([3000, 5000, 700], np.int32)
    cap = lens0 + np.array([6, 2, 6], np.int32)              # sequence 1 fills up after two appends
    tok0, P, keys, scale, rows = _dyadic(r, lens0, cap, 'fp8')
    B, C, k, kcap, steps = 3, 2500, 512, 96, 5
    w = (r.integers(0, 9, (B, 64)) / 64.0).astype(np.float32)
    pool = torch.empty((P, 576), dtype=torch.int16, pin_memory=True)
    pool.numpy()[:] = rows.view(np.int16)
    layer = DecodeLayer(dev(keys), dev(scale), dev(w), tok0, lens0, C, k=k, cap=kcap, host_pool=pool, capacity=cap)
    o_keys, o_sc, o_pool = keys.copy(), scale.copy(), rows.copy()
    sm = oracle.SlotMap(P, C)
    cache = np.zeros((C, 576), np.uint16)
    theta = np.full(B, np.nan, np.float32)
    lens = lens0.copy()
    q = r.integers(-3, 4, (B, 64, 128)).astype(np.float32)
    for s in range(steps):
        qb = wk.to_bf16_bits(q)
        layer.step(dev(qb))
        torch.cuda.synchronize()
        L = [x.astype(np.float32) for x in oracle.index_logits(qb, w, o_keys, 'fp8', o_sc, tok0, lens)]
        idx, kth = oracle.topk_rows(L, k)
        a, _ = sm.early(tok0, L, theta, kcap)
        oracle.recall_rows(o_pool, cache, a)
        a, sel, _ = sm.final(tok0, idx)
        oracle.recall_rows(o_pool, cache, a)
        theta = oracle.theta_rows(theta, kth)
        tag = f'step {s}'
        for b in range(B):
            np.testing.assert_array_equal(host(layer.logits)[b, :lens[b]], L[b], err_msg=tag)
        np.testing.assert_array_equal(host(layer.idx), idx, err_msg=tag)
        np.testing.assert_array_equal(host(layer.sel_slot), sel, err_msg=tag)
        np.testing.assert_array_equal(host(layer.state.tok2slot), sm.tok2slot, err_msg=tag)
        np.testing.assert_array_equal(host(layer.dev_cache).view(np.uint16), cache, err_msg=tag)
        # the decoded token of each sequence joins the layer
        nr = wk.to_bf16_bits(r.standard_normal((B, 576)).astype(np.float32))
        nk = wk.to_e4m3_bits(r.integers(-8, 9, (B, 128)).astype(np.float32))
        ns = np.array([0.5, 1.0, 2.0], np.float32)[r.integers(0, 3, B)]
        layer.append(dev(nr), dev(nk), dev(ns))
        torch.cuda.synchronize()
        full = oracle.kv_append(o_pool, o_keys, o_sc, sm.tok2slot, tok0, lens, cap, nr, nk, ns)
        np.testing.assert_array_equal(host(layer.lens), lens, err_msg=tag)
        assert bool(int(host(layer.state.ctr)[ech.CTR_STATUS]) & ech.ST_FULL) == (full or s >= 2), tag
        np.testing.assert_array_equal(pool.numpy().view(np.uint16), o_pool, err_msg=tag)
        q = np.clip(q + r.integers(-1, 2, q.shape), -3, 3).astype(np.float32)
    assert lens[1] == cap[1] and lens[0] == lens0[0] + steps
