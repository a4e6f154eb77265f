"""Parity at the full sizes of the decode and prefill workloads, in the launch
configuration the benchmark uses.

- 4 x 1M fp8 decode: oracle scores of all tokens (float64, cast to fp32) fed
  to the GPU top-k and slot map for two steps; everything bit-exact; GPU
  scores within tolerance of the oracle on every token of one row.
- 64 x 100K-110K capacity-constrained decode (chunked): dyadic inputs, so
  the whole pipeline is compared bit for bit with the oracle over 3 steps.
- 110K-token causal prefill, all 27 query blocks: GPU scores of all 4096
  rows of block 1 and of 16 sampled rows of every other block against the
  oracle, the exact-top-k property of every row of every block
  (checked on the GPU scores), and the union slot map against first-touch
  order after every block (the cache is as large as the sequence).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wk
from gpu_util import TOL_FP8, dev, host, need_gpu, rel_err
from test_gpu_pipeline import _run_bit_exact

import indexer_top_kv_amd as ech
from indexer_top_kv_amd.pipeline import PrefillLayer

pytestmark = pytest.mark.gpu


def test_long_context_decode_full_size():
    need_gpu()
    wl = wk.CONFIGS['decode-4x1m-fp8']
    keys, scale = wk.keys(wl)
    w = wk.head_weights(wl)
    qs = list(wk.decode_queries(wl, 2))
    kd, sd = dev(keys), dev(scale)
    tok0, lens = dev(wl.tok0), dev(wl.lens)
    # scores of one full row on the GPU against the oracle
    out = torch.zeros((wl.B, wl.N), dtype=torch.float32, device='cuda')
    ech.ech_index_logits(dev(qs[0]), dev(w), kd, sd, tok0, lens, wl.N, out)
    torch.cuda.synchronize()
    ref0 = oracle.index_logits(qs[0][:1], w[:1], keys, 'fp8', scale, wl.tok0[:1], wl.lens[:1])[0]
    assert rel_err(host(out)[0], ref0).max() <= min(TOL_FP8, 1e-5)
    # top-k and slot map at the launch shape, fed the oracle's scores
    gc_state = ech.LayerState.allocate(wl.P, wl.C, wl.B * wl.k)
    ech.ech_cache_reset(gc_state)
    ws_t = torch.empty(ech.ech_topk_ws_bytes(wl.B, wl.N, wl.k), dtype=torch.uint8, device='cuda')
    ws_e = torch.empty(ech.ech_cache_step_ws_bytes(ech.ECH_EARLY, wl.B, wl.B, wl.k, wl.N, wl.C, wl.B * wl.k),
                       dtype=torch.uint8, device='cuda')
    ws_f = torch.empty(ech.ech_cache_step_ws_bytes(ech.ECH_FINAL, wl.B, wl.B, wl.k, wl.N, wl.C, wl.B * wl.k),
                       dtype=torch.uint8, device='cuda')
    sm = oracle.SlotMap(wl.P, wl.C)
    theta = np.full(wl.B, np.nan, np.float32)
    for s, q in enumerate(qs):
        L = np.stack(oracle.index_logits(q, w, keys, 'fp8', scale, wl.tok0, wl.lens)).astype(np.float32)
        Ld = dev(L)
        th_in = dev(theta)
        th_out = torch.empty(wl.B, dtype=torch.float32, device='cuda')
        idx = torch.empty((wl.B, wl.k), dtype=torch.int32, device='cuda')
        kth = torch.empty(wl.B, dtype=torch.float32, device='cuda')
        ech.ech_topk(Ld, lens, wl.N, wl.k, th_in, th_out, idx, kth, ws_t)
        st_e = torch.empty((wl.B, 4), dtype=torch.int32, device='cuda')
        ech.ech_cache_step(ech.ECH_EARLY, gc_state, tok0, lens, wl.N, k=wl.k, logits=Ld, theta=th_in, cap=wl.cap,
                           stats=st_e, ws=ws_e)
        torch.cuda.synchronize()
        ref_idx, ref_kth = oracle.topk_rows(list(L), wl.k)
        np.testing.assert_array_equal(host(idx), ref_idx)
        np.testing.assert_array_equal(host(kth), ref_kth)
        a_o, st_o = sm.early(wl.tok0, list(L), theta, wl.cap)
        n = int(host(gc_state.ctr)[ech.CTR_NMISS_EARLY])
        assert [tuple(x) for x in host(gc_state.miss_early)[:n].tolist()] == a_o
        np.testing.assert_array_equal(host(st_e), st_o)
        sel = torch.empty((wl.B, wl.k), dtype=torch.int32, device='cuda')
        st_f = torch.empty((wl.B, 4), dtype=torch.int32, device='cuda')
        ech.ech_cache_step(ech.ECH_FINAL, gc_state, tok0, lens, wl.N, idx=idx, k=wl.k, sel_slot=sel, stats=st_f,
                           ws=ws_f)
        torch.cuda.synchronize()
        a_o, sel_o, st_o = sm.final(wl.tok0, ref_idx)
        n = int(host(gc_state.ctr)[ech.CTR_NMISS])
        assert [tuple(x) for x in host(gc_state.miss)[:n].tolist()] == a_o
        np.testing.assert_array_equal(host(sel), sel_o)
        np.testing.assert_array_equal(host(st_f), st_o)
        np.testing.assert_array_equal(host(gc_state.tok2slot), sm.tok2slot)
        np.testing.assert_array_equal(host(gc_state.slot2tok), sm.slot2tok)
        theta = oracle.theta_rows(theta, ref_kth)
        np.testing.assert_array_equal(host(th_out), theta)


def test_capacity_decode_full_size_dyadic_bit_exact():
    need_gpu()
    wl = wk.CONFIGS['decode-64x110k-fp8-capacity'].scaled(steps=3, variant='dyadic')
    _run_bit_exact(wl, 3)


def _check_exact_topk(row, idx, k):
    """idx is exactly the top-k of row (ties to the lower index)."""
    n = len(row)
    m = min(k, n)
    sel = idx[idx >= 0]
    assert len(sel) == m and np.all(np.diff(sel) > 0)
    if m == n:
        return
    mask = np.zeros(n, bool)
    mask[sel] = True
    kth = row[sel].min()
    assert np.all(row[~mask] <= kth)
    eq_out = np.nonzero(~mask & (row == kth))[0]
    eq_in = np.nonzero(mask & (row == kth))[0]
    if len(eq_out):
        assert eq_in.max() < eq_out.min()


def test_prefill_full_size_all_blocks():
    need_gpu()
    wl = wk.CONFIGS['prefill-110k-fp8']
    keys, scale = wk.keys(wl)
    layer = PrefillLayer(dev(keys), dev(scale), wl.N, wl.C, k=wl.k, block_rows=wl.block_rows)
    order = []            # first-touch order of tokens
    touched = np.zeros(wl.N, bool)
    rng = np.random.default_rng(3)
    for bi, (r0, R) in enumerate(layer.blocks()):
        q = wk.prefill_queries(wl, r0, R)
        w = wk.head_weights(wl, rows=R, row0=r0)
        layer.run_block(r0, dev(q), dev(w), first=(bi == 0))
        layer.finish()
        torch.cuda.synchronize()
        L = host(layer.logits[:R])
        idx = host(layer.idx[:R])
        for i in range(R):
            _check_exact_topk(L[i, :r0 + i + 1], idx[i], wl.k)
        # every row of block 1 against the oracle, 16 sampled rows of the others
        rows = np.arange(R) if bi == 1 else rng.choice(R, 16, replace=False)
        refs = oracle.index_logits(q[rows], w[rows], keys, 'fp8', scale, [0] * len(rows), r0 + rows + 1)
        for i, ref in zip(rows, refs):
            assert rel_err(L[i, :r0 + i + 1], ref).max() <= min(TOL_FP8, 1e-5), f'block {bi} row {i}'
        # union slot map: C = N, so slot = first-touch rank
        new = np.setdiff1d(np.unique(idx[idx >= 0]), np.nonzero(touched)[0])
        order.extend(new.tolist())
        touched[new] = True
        t2s = host(layer.state.tok2slot)
        np.testing.assert_array_equal(t2s[np.array(order)], np.arange(len(order)))
        assert np.all(t2s[~touched] == -1)
        np.testing.assert_array_equal(host(layer.sel_slot[:R]), np.where(idx >= 0, t2s[np.maximum(idx, 0)], -1))
        assert int(host(layer.state.ctr)[ech.CTR_STATUS]) == 0


def test_prefill_overlapped_matches_serial():
    """The double-buffered prefill (block i's top-k and slot-map step on a
    second stream while block i+1 is scored, recalls on a third) against the
    serial one, with no synchronisation between blocks: every block's
    selection, the final maps and the device cache are identical."""
    need_gpu()
    wl = wk.CONFIGS['prefill-110k-fp8']
    keys, scale = wk.keys(wl)
    rows = torch.from_numpy(np.random.default_rng(5).integers(-30000, 30000, (wl.N, 64), dtype=np.int16))
    pool = torch.empty((wl.N, 64), dtype=torch.int16, pin_memory=True)
    pool.copy_(rows)
    kd, sd = dev(keys), dev(scale)
    blocks = None
    results = []
    for overlap in (False, True):
        layer = PrefillLayer(kd, sd, wl.N, wl.C, k=wl.k, block_rows=wl.block_rows, host_pool=pool, overlap=overlap)
        blocks = layer.blocks()
        qs = [dev(wk.prefill_queries(wl, r0, R)) for r0, R in blocks]
        ws = [dev(wk.head_weights(wl, rows=R, row0=r0)) for r0, R in blocks]
        torch.cuda.synchronize()
        saved = []
        for bi, (r0, R) in enumerate(blocks):
            layer.run_block(r0, qs[bi], ws[bi], first=(bi == 0))
            sel_stream = layer.s1 if overlap else torch.cuda.current_stream()
            with torch.cuda.stream(sel_stream):
                saved.append(layer.idx[:R].clone())
        layer.finish()
        torch.cuda.synchronize()
        results.append((saved, layer.state.tok2slot.clone(), layer.state.slot2tok.clone(), layer.dev_cache.clone(),
                        int(host(layer.state.ctr)[ech.CTR_STATUS])))
    (sa, t2a, s2a, ca, sta), (sb, t2b, s2b, cb, stb) = results
    for bi in range(len(blocks)):
        assert torch.equal(sa[bi], sb[bi]), f'block {bi}'
    assert torch.equal(t2a, t2b) and torch.equal(s2a, s2b) and torch.equal(ca, cb)
    assert sta == 0 and stb == 0
    occ = host(s2b)
    occ_slots = np.nonzero(occ >= 0)[0]
    np.testing.assert_array_equal(host(cb)[occ_slots], pool.numpy()[occ[occ_slots]])
