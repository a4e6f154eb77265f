"""Indexer scores on the GPU against the CPU oracle (float64).

Tolerances: rel 1e-3 for bf16 keys and 2e-2 for fp8 keys, elementwise as
|g - o| <= tol * max(|o|, 1e-2 * max_t |o_t|) per row. The kernels form every
product exactly (bf16 x bf16, fp8 widened exactly to bf16) and round only in
the fp32 sums, so a much tighter bound (1e-5) is also asserted: the stated
tolerances would hide small systematic mistakes. Dyadic inputs make every
score exact in fp32, so those must match bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wk
from gpu_util import TOL_BF16, TOL_FP8, need_gpu, rel_err, run_logits, dev, host
import indexer_top_kv_amd as ech

pytestmark = pytest.mark.gpu
ARITH_BOUND = 1e-5


def _case(name, **kw):
    wl = wk.CONFIGS[name].scaled(**kw)
    keys, scale = wk.keys(wl)
    q = next(wk.decode_queries(wl))
    w = wk.head_weights(wl)
    return wl, keys, scale, q, w


def _compare(wl, keys, scale, q, w, tok0, lens, tol):
    got = run_logits(q, w, keys, scale, tok0, lens)
    ref = oracle.index_logits(q, w, keys, wl.kdtype, scale, tok0, lens)
    worst = 0.0
    for r in range(len(lens)):
        n = int(lens[r])
        e = rel_err(got[r, :n], ref[r])
        if n:
            worst = max(worst, float(e.max()))
        assert np.all(e <= tol), (r, float(e.max()))
        assert np.all(np.isnan(got[r, n:])), 'wrote past the row length'
    assert worst <= ARITH_BOUND, worst
    return worst


def test_bf16_single_sequence_ragged():
    need_gpu()
    wl, keys, scale, q, w = _case('decode-1x16k-bf16', N=3001)
    _compare(wl, keys, scale, q, w, wl.tok0, wl.lens, TOL_BF16)


def test_bf16_full_size_decode():
    need_gpu()
    wl, keys, scale, q, w = _case('decode-1x16k-bf16')
    _compare(wl, keys, scale, q, w, wl.tok0, wl.lens, TOL_BF16)


def test_fp8_ragged_batch():
    need_gpu()
    wl, keys, scale, q, w = _case('decode-32x128k-fp8', B=4, N=6000)
    lens = np.array([6000, 4097, 1, 17], np.int32)
    tok0 = wl.tok0
    _compare(wl, keys, scale, q, w, tok0, lens, TOL_FP8)


def test_fp8_empty_rows_untouched():
    need_gpu()
    wl, keys, scale, q, w = _case('decode-32x128k-fp8', B=3, N=500)
    lens = np.array([0, 500, 0], np.int32)
    got = run_logits(q, w, keys, scale, wl.tok0, lens)
    assert np.all(np.isnan(got[0])) and np.all(np.isnan(got[2]))
    assert not np.isnan(got[1, :500]).any()


def test_fp8_negative_scales():
    need_gpu()
    wl, keys, scale, q, w = _case('decode-32x128k-fp8', B=2, N=999)
    scale = scale.copy()
    scale[::3] *= -1.0
    _compare(wl, keys, scale, q, w, wl.tok0, wl.lens, TOL_FP8)


@pytest.mark.parametrize('kdtype', ['fp8', 'bf16'])
def test_dyadic_scores_bit_exact(kdtype):
    need_gpu()
    name = 'decode-32x128k-fp8' if kdtype == 'fp8' else 'decode-1x16k-bf16'
    wl, keys, scale, q, w = _case(name, B=3 if kdtype == 'fp8' else 1, N=2500, variant='dyadic')
    got = run_logits(q, w, keys, scale, wl.tok0, wl.lens)
    ref = oracle.index_logits(q, w, keys, kdtype, scale, wl.tok0, wl.lens)
    for r in range(wl.B):
        np.testing.assert_array_equal(got[r, :wl.N].astype(np.float64), ref[r])


def test_fp8_full_size_decode_sampled():
    """32 x 131072 fp8 at the launch shape the bench uses: two full rows and
    4096 sampled (row, token) scores against the oracle."""
    need_gpu()
    wl = wk.CONFIGS['decode-32x128k-fp8']
    keys, scale = wk.keys(wl)
    q = next(wk.decode_queries(wl))
    w = wk.head_weights(wl)
    got = run_logits(q, w, keys, scale, wl.tok0, wl.lens)
    for r in (0, 31):
        ref = oracle.index_logits(q[r:r + 1], w[r:r + 1], keys, 'fp8', scale, wl.tok0[r:r + 1], wl.lens[r:r + 1])[0]
        e = rel_err(got[r, :wl.N], ref)
        assert e.max() <= min(TOL_FP8, ARITH_BOUND), float(e.max())
    rng = np.random.default_rng(5)
    rows = rng.integers(0, wl.B, 4096)
    ts = rng.integers(0, wl.N, 4096)
    for r in np.unique(rows):
        sel = ts[rows == r]
        ref = oracle.index_logit_at(q[r], w[r], keys, 'fp8', scale, wl.tok0[r] + sel)
        full_ref_scale = np.abs(got[r, :wl.N]).max()
        e = np.abs(got[r, sel] - ref) / np.maximum(np.abs(ref), 1e-2 * full_ref_scale)
        assert e.max() <= min(TOL_FP8, ARITH_BOUND), (r, float(e.max()))


def test_fp8_ragged_at_full_launch_shape():
    """32 rows of the 32 x 131072 launch shape (2048 tokens per workgroup,
    512 per wave) with ragged lengths ending inside a tile, on tile, wave and
    workgroup edges and after one token, and key offsets that are not
    multiples of 8 rows: every row's first and last 64 scores, the scores
    around each 512-token wave edge and 2048 sampled ones against the
    oracle; nothing past a row's end is written."""
    need_gpu()
    wl = wk.CONFIGS['decode-32x128k-fp8']
    keys, scale = wk.keys(wl)
    q = next(wk.decode_queries(wl))
    w = wk.head_weights(wl)
    rng = np.random.default_rng(17)
    edge = [1, 15, 16, 17, 511, 512, 513, 2047, 2048, 2049, 4095, 131072, 131071, 100003]
    lens = np.concatenate([edge, rng.integers(1, wl.N + 1, wl.B - len(edge))]).astype(np.int32)
    lens[wl.B - 1] = wl.N                          # keeps max_len (and so the launch shape) at 131072
    P = keys.shape[0]
    tok0 = np.array([min(int(wl.tok0[r]) + 37 * r + 3, P - int(lens[r])) for r in range(wl.B)], np.int64)
    got = run_logits(q, w, keys, scale, tok0, lens)
    for r in range(wl.B):
        n = int(lens[r])
        assert np.all(np.isnan(got[r, n:])), r
        sel = np.unique(np.concatenate([np.arange(min(n, 64)), np.arange(max(0, n - 64), n),
                                        np.array([t for e in range(512, n, 512) for t in (e - 1, e) if t < n], np.int64),
                                        rng.integers(0, n, 64)]).astype(np.int64))
        ref = oracle.index_logit_at(q[r], w[r], keys, 'fp8', scale, tok0[r] + sel)
        scale_r = max(np.abs(ref).max(), np.abs(got[r, :n]).max())
        e = np.abs(got[r, sel] - ref) / np.maximum(np.abs(ref), 1e-2 * scale_r)
        assert e.max() <= min(TOL_FP8, ARITH_BOUND), (r, n, float(e.max()))


def _causal(wl, keys, scale, row0, R):
    q = wk.prefill_queries(wl, row0, R)
    w = wk.head_weights(wl, rows=R, row0=row0)
    ld = ((row0 + R + 3) // 4) * 4
    out = torch.full((R, ld), float('nan'), dtype=torch.float32, device='cuda')
    ech.ech_index_logits_causal(dev(q), dev(w), dev(keys), None if scale is None else dev(scale), 0, row0, out)
    torch.cuda.synchronize()
    return q, w, host(out)


@pytest.mark.parametrize('row0,R', [(0, 300), (1000, 257), (4093, 70)])
def test_causal_prefill_block(row0, R):
    need_gpu()
    wl = wk.CONFIGS['prefill-110k-fp8'].scaled(N=5000, block_rows=512)
    keys, scale = wk.keys(wl)
    q, w, got = _causal(wl, keys, scale, row0, R)
    lens = row0 + np.arange(R) + 1
    ref = oracle.index_logits(q, w, keys, 'fp8', scale, np.zeros(R, np.int64), lens)
    for r in range(R):
        n = int(lens[r])
        e = rel_err(got[r, :n], ref[r])
        assert e.max() <= min(TOL_FP8, ARITH_BOUND), (r, float(e.max()))
        assert np.all(np.isnan(got[r, n:])), 'causal mask violated'


def test_causal_prefill_dyadic_bit_exact():
    need_gpu()
    wl = wk.CONFIGS['prefill-110k-fp8'].scaled(N=3000, block_rows=512, variant='dyadic')
    keys, scale = wk.keys(wl)
    q, w, got = _causal(wl, keys, scale, 2000, 100)
    lens = 2000 + np.arange(100) + 1
    ref = oracle.index_logits(q, w, keys, 'fp8', scale, np.zeros(100, np.int64), lens)
    for r in range(100):
        np.testing.assert_array_equal(got[r, :lens[r]].astype(np.float64), ref[r])
