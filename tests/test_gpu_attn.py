"""Sparse attention over sel_slot (ech_sparse_attn) against the oracle.

Tolerance: the scores are exact bf16 products summed in fp32, the softmax
weights enter the value product rounded to bf16 (relative error <= 2^-9
each) while the denominator sums them unrounded, so an output may be off by
a few 2^-9 of the largest |output| of its head; the bound used is
|gpu - oracle| <= 5e-3 * max_c |oracle[b, h, c]| + 1e-6, and lse within
1e-4 (fp32 sums of exp). Lossless: attention through the device cache equals,
bit for bit, the same kernel over the rows held in full in HBM.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wk
from gpu_util import dev, host, need_gpu
import indexer_top_kv_amd as ech

pytestmark = pytest.mark.gpu


def _run(q, cache, sel, scale):
    B, H = q.shape[0], q.shape[1]
    out = torch.full((B, H, 512), 7.0, dtype=torch.float32, device='cuda')
    lse = torch.full((B, H), 7.0, dtype=torch.float32, device='cuda')
    ws = torch.empty(ech.ech_sparse_attn_ws_bytes(B, H, sel.shape[1]), dtype=torch.uint8, device='cuda')
    ech.ech_sparse_attn(q, cache, sel, scale, out, lse, ws)
    torch.cuda.synchronize()
    return host(out), host(lse)


def _check(o_gpu, l_gpu, o_ref, l_ref, tag=''):
    bound = 5e-3 * np.abs(o_ref).max(axis=2, keepdims=True) + 1e-6
    err = np.abs(o_gpu - o_ref)
    assert np.all(err <= bound), (tag, float((err / bound).max()))
    fin = np.isfinite(l_ref)
    np.testing.assert_array_equal(np.isfinite(l_gpu), fin, err_msg=tag)
    assert np.all(np.abs(l_gpu[fin] - l_ref[fin]) <= 1e-4 * np.maximum(1.0, np.abs(l_ref[fin]))), tag
    assert np.all(o_gpu[~fin] == 0), tag


def _case(seed, B, H, C, k, pad_max, q_scale=1.0):
    r = np.random.default_rng(seed)
    q = wk.to_bf16_bits((q_scale * r.standard_normal((B, H, 576))).astype(np.float32))
    cache = wk.to_bf16_bits(r.standard_normal((C, 576)).astype(np.float32))
    sel = np.stack([r.choice(C, k, replace=False) for _ in range(B)]).astype(np.int32)
    for b in range(B):
        npad = int(r.integers(0, pad_max + 1))
        if npad:
            sel[b, k - npad:] = -1
    if k > 3:
        sel[0, 2] = C + 5                  # out of range: selects nothing
        sel[-1, 1] = -7
    return q, cache, sel


@pytest.mark.parametrize('B,H,k,pad', [(3, 16, 37, 10), (2, 48, 64, 64), (4, 128, 2048, 1500), (1, 128, 5, 0),
                                       (5, 64, 300, 299),
                                       # few sequences: the heads of a span split over 2-4 workgroups
                                       # (3 for 48 heads above), several spans and tiles each
                                       (1, 128, 2048, 0), (2, 128, 1024, 100), (4, 128, 2048, 7), (1, 64, 999, 3),
                                       # two token lanes per workgroup: 8 waves as 4 x 2 (16, 8 sequences),
                                       # spans ending on one tile of a step (33 tiles), 7 waves (112 heads)
                                       # with one lane
                                       (16, 128, 2048, 40), (8, 128, 1056, 0), (32, 128, 1056, 31),
                                       (3, 112, 700, 20)])
def test_random_against_oracle(B, H, k, pad):
    need_gpu()
    q, cache, sel = _case(B * 100 + H + k, B, H, 4000, k, pad)
    scale = 1.0 / np.sqrt(192.0)
    o, l = _run(dev(q), dev(cache), dev(sel), scale)
    ro, rl = oracle.sparse_attention(q, cache, sel, scale)
    _check(o, l, ro, rl, f'B{B} H{H} k{k}')


def test_many_spans_merged_in_groups():
    """One sequence of 8192 selected rows: 64 spans, more than one merge group
    of 32 (the other merge forms cover up to 32 spans)."""
    need_gpu()
    q, cache, sel = _case(7, 1, 32, 10000, 8192, 50)
    scale = 1.0 / np.sqrt(192.0)
    o, l = _run(dev(q), dev(cache), dev(sel), scale)
    ro, rl = oracle.sparse_attention(q, cache, sel, scale)
    _check(o, l, ro, rl, 'k8192')


def test_peaked_and_flat_softmax():
    """Large scores (one token dominates) and a zero query (uniform weights)."""
    need_gpu()
    q, cache, sel = _case(3, 2, 32, 1000, 256, 0, q_scale=4.0)
    o, l = _run(dev(q), dev(cache), dev(sel), 0.5)
    ro, rl = oracle.sparse_attention(q, cache, sel, 0.5)
    _check(o, l, ro, rl, 'peaked')
    q0 = np.zeros_like(q)
    o, l = _run(dev(q0), dev(cache), dev(sel), 0.5)
    ro, rl = oracle.sparse_attention(q0, cache, sel, 0.5)
    _check(o, l, ro, rl, 'flat')


def test_degenerate_selections():
    need_gpu()
    q, cache, sel = _case(4, 3, 16, 500, 40, 0)
    sel[0, :] = -1                         # nothing selected
    sel[1, :] = -1
    sel[1, 17] = 123                       # one valid slot: its row, exactly
    sel[2, :] = 499                        # one slot selected 40 times
    o, l = _run(dev(q), dev(cache), dev(sel), 0.09)
    ro, rl = oracle.sparse_attention(q, cache, sel, 0.09)
    assert np.all(o[0] == 0) and np.all(np.isneginf(l[0]))
    from oracle.numerics import bf16_to_f64
    np.testing.assert_array_equal(o[1], np.broadcast_to(bf16_to_f64(cache[123, :512]).astype(np.float32), (16, 512)))
    np.testing.assert_array_equal(o[2], np.broadcast_to(bf16_to_f64(cache[499, :512]).astype(np.float32), (16, 512)))
    _check(o, l, ro, rl, 'degenerate')


def test_bad_arguments():
    need_gpu()
    q = torch.zeros((2, 24, 576), dtype=torch.int16, device='cuda')          # H not a multiple of 16
    cache = torch.zeros((10, 576), dtype=torch.int16, device='cuda')
    sel = torch.zeros((2, 8), dtype=torch.int32, device='cuda')
    out = torch.zeros((2, 24, 512), dtype=torch.float32, device='cuda')
    ws = torch.empty(1 << 20, dtype=torch.uint8, device='cuda')
    with pytest.raises(ech.EchError):
        ech.ech_sparse_attn(q, cache, sel, 0.1, out, None, ws)
    assert ech.ech_sparse_attn_ws_bytes(2, 24, 8) == 0
    assert ech.ech_sparse_attn_ws_bytes(2, 144, 8) == 0


def test_full_size_decode_batch():
    """32 sequences x 128 heads x 2048 selected of a 260000-slot cache, the
    launch the benchmark times; every sequence checked against the oracle."""
    need_gpu()
    r = np.random.default_rng(99)
    B, H, k, C = 32, 128, 2048, 260000
    cache_t = torch.randn((C, 576), device='cuda').to(torch.bfloat16).view(torch.int16)
    sel = np.stack([r.choice(C, k, replace=False) for _ in range(B)]).astype(np.int32)
    sel[5, 1000:] = -1
    q = wk.to_bf16_bits(r.standard_normal((B, H, 576)).astype(np.float32))
    o, l = _run(dev(q), cache_t, dev(sel), 1.0 / np.sqrt(192.0))
    cache = host(cache_t).view(np.uint16)
    ro, rl = oracle.sparse_attention(q, cache, sel, 1.0 / np.sqrt(192.0))
    _check(o, l, ro, rl, 'full size')


def test_lossless_through_the_cache():
    """After decode steps, attention through dev_cache[sel_slot] equals, bit
    for bit, attention over the host pool's rows of the selected tokens held
    whole in HBM: the offloaded cache holds exactly the right rows."""
    need_gpu()
    from indexer_top_kv_amd.pipeline import DecodeLayer
    wl = wk.CONFIGS['decode-64x110k-fp8-capacity'].scaled(B=4, N=9000, len_lo=1500, C=6000, k=1024, cap=128,
                                                          resample_p=0.3)
    keys, scale = wk.keys(wl)
    w = wk.head_weights(wl)
    rows = wk.host_rows(wl)
    pool = torch.empty((wl.P, 576), dtype=torch.int16, pin_memory=True)
    pool.numpy()[:] = rows.view(np.int16)
    layer = DecodeLayer(dev(keys), dev(scale), dev(w), wl.tok0, wl.lens, wl.C, k=wl.k, cap=wl.cap, host_pool=pool)
    full = dev(rows)                                  # every row, resident
    r = np.random.default_rng(5)
    for s, qi in enumerate(wk.decode_queries(wl, 3)):
        layer.step(dev(qi))
        qa = dev(wk.to_bf16_bits(r.standard_normal((wl.B, 128, 576)).astype(np.float32)))
        idx = host(layer.idx)
        g = np.where(idx >= 0, idx + wl.tok0[:, None], -1).astype(np.int32)
        o1, l1 = _run(qa, layer.dev_cache, layer.sel_slot, 0.07)
        o2, l2 = _run(qa, full, dev(g), 0.07)
        np.testing.assert_array_equal(o1, o2, err_msg=f'step {s}')
        np.testing.assert_array_equal(l1, l2, err_msg=f'step {s}')
        assert np.all(np.isfinite(l1))


def test_lossless_through_the_cache_chunked():
    """A batch whose selections exceed the cache runs in sequence chunks,
    and a later chunk may evict an earlier chunk's tokens. The consumer reads
    each chunk's sel_slot rows right after that chunk's FINAL recall
    (DecodeLayer.step's on_chunk): there every selected token is resident in
    the slot sel_slot names (slot2tok[sel_slot] == the selected token), and
    attention through the device cache equals, bit for bit, attention over
    the selected rows held whole in HBM."""
    need_gpu()
    from indexer_top_kv_amd.pipeline import DecodeLayer
    wl = wk.CONFIGS['decode-64x110k-fp8-capacity'].scaled(B=6, N=5000, len_lo=3000, C=5000, k=1024, cap=128,
                                                          resample_p=0.4)
    keys, scale = wk.keys(wl)
    w = wk.head_weights(wl)
    rows = wk.host_rows(wl)
    pool = torch.empty((wl.P, 576), dtype=torch.int16, pin_memory=True)
    pool.numpy()[:] = rows.view(np.int16)
    layer = DecodeLayer(dev(keys), dev(scale), dev(w), wl.tok0, wl.lens, wl.C, k=wl.k, cap=wl.cap, host_pool=pool)
    assert len(layer.chunks) > 1
    full = dev(rows)
    r = np.random.default_rng(8)
    H = 64
    tok0_d = dev(wl.tok0)
    for s, qi in enumerate(wk.decode_queries(wl, 4)):
        qa = dev(wk.to_bf16_bits(r.standard_normal((wl.B, H, 576)).astype(np.float32)))
        outs = {}

        def consume(b0, b1, stream):
            with torch.cuda.stream(stream):
                sel = layer.sel_slot[b0:b1]
                n = b1 - b0
                o = torch.empty((n, H, 512), dtype=torch.float32, device='cuda')
                l = torch.empty((n, H), dtype=torch.float32, device='cuda')
                ws = torch.empty(ech.ech_sparse_attn_ws_bytes(n, H, wl.k), dtype=torch.uint8, device='cuda')
                ech.ech_sparse_attn(qa[b0:b1], layer.dev_cache, sel, 0.07, o, l, ws, stream=stream)
                # residency of what the consumer read, at the time it read it
                held = torch.where(sel >= 0, layer.state.slot2tok[sel.clamp(min=0).long()], -1)
                want = torch.where(layer.idx[b0:b1] >= 0, layer.idx[b0:b1] + tok0_d[b0:b1, None], -1)
                outs[(b0, b1)] = (o, l, held.clone(), want.clone(), layer.idx[b0:b1].clone())

        layer.step(dev(qi), on_chunk=consume)
        torch.cuda.synchronize()
        assert sorted(outs) == layer.chunks
        for (b0, b1), (o, l, held, want, idx_c) in outs.items():
            np.testing.assert_array_equal(host(held), host(want), err_msg=f'step {s} chunk {b0}:{b1}')
            idx = host(idx_c)
            g = np.where(idx >= 0, idx + wl.tok0[b0:b1, None], -1).astype(np.int32)
            o2, l2 = _run(qa[b0:b1], full, dev(g), 0.07)
            np.testing.assert_array_equal(host(o), o2, err_msg=f'step {s} chunk {b0}:{b1}')
            np.testing.assert_array_equal(host(l), l2, err_msg=f'step {s} chunk {b0}:{b1}')


def test_captured_attention_follows_the_index_tensor():
    """The attention captured once in a hipGraph keeps reading the fixed
    pool through sel_slot: after the selection and the cache rows change in
    place (as decode steps change them), every replay equals an eager call,
    with unrelated eager work between the replays."""
    need_gpu()
    r = np.random.default_rng(21)
    B, H, k, C = 3, 64, 512, 3000
    q = dev(wk.to_bf16_bits(r.standard_normal((B, H, 576)).astype(np.float32)))
    cache = dev(wk.to_bf16_bits(r.standard_normal((C, 576)).astype(np.float32)))
    sel = dev(np.stack([r.choice(C, k, replace=False) for _ in range(B)]).astype(np.int32))
    out = torch.zeros((B, H, 512), dtype=torch.float32, device='cuda')
    lse = torch.zeros((B, H), dtype=torch.float32, device='cuda')
    ws = torch.empty(ech.ech_sparse_attn_ws_bytes(B, H, k), dtype=torch.uint8, device='cuda')
    ech.ech_sparse_attn(q, cache, sel, 0.08, out, lse, ws)     # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ech.ech_sparse_attn(q, cache, sel, 0.08, out, lse, ws)
    for step in range(4):
        new_sel = np.stack([r.choice(C, k, replace=False) for _ in range(B)]).astype(np.int32)
        new_sel[step % B, k - 100:] = -1
        sel.copy_(torch.from_numpy(new_sel))
        rows = r.choice(C, 200, replace=False)
        cache[torch.from_numpy(rows).cuda()] = dev(wk.to_bf16_bits(r.standard_normal((200, 576)).astype(np.float32)))
        g.replay()
        torch.cuda.synchronize()
        got_o, got_l = host(out).copy(), host(lse).copy()
        ref_o, ref_l = _run(q, cache, sel, 0.08)
        np.testing.assert_array_equal(got_o, ref_o, err_msg=f'replay {step}')
        np.testing.assert_array_equal(got_l, ref_l, err_msg=f'replay {step}')
        x = torch.arange(4096, device='cuda', dtype=torch.float32)    # unrelated eager work
        assert float((x * 2).sum().item()) == 4096 * 4095
