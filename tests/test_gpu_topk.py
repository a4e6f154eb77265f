"""Exact top-k on the GPU against the oracle's stable sort, bit for bit.

Both sides get the same float32 score rows (drawn by the generator or computed
by the oracle), so idx, kth and the EMA threshold must match exactly. The
threshold only steers speed; every theta (none, exact, off by a little, far
off so the boundary bin overflows its list) must give the same set.
"""
import numpy as np
import pytest

import oracle
import workloads as wk
from gpu_util import need_gpu, run_topk

pytestmark = pytest.mark.gpu


def _check(scores, lens, k, theta=None):
    idx, kth, th_out = run_topk(scores, lens, k, theta)
    for r, n in enumerate(lens):
        ref_idx, ref_kth = oracle.topk_row(scores[r, :n], k)
        np.testing.assert_array_equal(idx[r], ref_idx, err_msg=f'row {r} len {n}')
        if np.isnan(ref_kth):
            assert np.isnan(kth[r])
        else:
            assert kth[r] == ref_kth, (r, kth[r], ref_kth)
        th_in = np.float32(np.nan) if theta is None else np.float32(theta[r])
        want = oracle.theta_next(th_in, ref_kth)
        if np.isnan(want):
            assert np.isnan(th_out[r])
        else:
            assert th_out[r] == want, (r, th_out[r], want)
    return idx, kth


def _pad(x, ld):
    out = np.zeros((x.shape[0], ld), np.float32)
    out[:, :x.shape[1]] = x
    return out


@pytest.mark.parametrize('kind', ['normal', 'ties', 'const', 'signed'])
def test_kinds_ragged_lengths(kind):
    need_gpu()
    n = 20000
    x = wk.random_logits(1, 6, n, kind)
    lens = [20000, 2048, 2049, 1, 0, 12345]
    _check(_pad(x, 20000), lens, 2048)


@pytest.mark.parametrize('k', [1, 7, 2048, 4096])
def test_various_k(k):
    need_gpu()
    x = wk.random_logits(2, 3, 30001, 'normal')
    _check(_pad(x, 30004), [30001, 9000, 4100], k)


def test_theta_exact_and_offsets():
    need_gpu()
    x = wk.random_logits(3, 8, 65536, 'normal')
    lens = [65536] * 8
    kth = np.array([oracle.topk_row(x[r], 2048)[1] for r in range(8)], np.float32)
    offs = np.array([0.0, 1e-6, -1e-6, 0.01, -0.01, 0.3, -0.3, np.nan], np.float32)
    _check(x, lens, 2048, kth + offs)


def test_theta_far_off_overflows_candidate_list():
    need_gpu()
    x = wk.random_logits(4, 4, 200000, 'normal')
    theta = np.array([-100.0, 100.0, 18.0, 1e30], np.float32)
    _check(_pad(x, 200000), [200000] * 4, 2048, theta)


def test_ties_at_the_boundary_with_theta():
    need_gpu()
    x = wk.random_logits(5, 4, 50000, 'ties')   # integers 0..63: huge tie groups
    theta = np.array([np.nan, 62.0, 61.5, 63.0], np.float32)
    _check(x, [50000] * 4, 2048, theta)


def test_oracle_scores_full_row_decode_shape():
    """fp32 casts of oracle scores for a 32 x 131072 fp8 decode batch, with
    the previous step's k-th scores as theta."""
    need_gpu()
    wl = wk.CONFIGS['decode-32x128k-fp8'].scaled(B=4)
    keys, scale = wk.keys(wl)
    qs = wk.decode_queries(wl, 2)
    w = wk.head_weights(wl)
    q0, q1 = next(qs), next(qs)
    s0 = np.stack(oracle.index_logits(q0, w, keys, 'fp8', scale, wl.tok0, wl.lens)).astype(np.float32)
    s1 = np.stack(oracle.index_logits(q1, w, keys, 'fp8', scale, wl.tok0, wl.lens)).astype(np.float32)
    _, kth0 = _check(s0, list(wl.lens), 2048)
    _check(s1, list(wl.lens), 2048, kth0)


def test_long_rows():
    need_gpu()
    x = wk.random_logits(6, 2, 1 << 20, 'normal')
    kth = np.array([oracle.topk_row(x[0], 2048)[1], np.nan], np.float32)
    _check(x, [1 << 20, (1 << 20) - 3], 2048, kth + np.float32(0.05))


def test_many_rows_prefill_shape():
    """4096 rows with causal lengths (row r sees r + 1 + offset tokens)."""
    need_gpu()
    R, off = 512, 3000
    x = wk.random_logits(7, R, off + R, 'normal')
    lens = [off + r + 1 for r in range(R)]
    ld = ((off + R + 3) // 4) * 4
    _check(_pad(x, ld), lens, 2048)


def test_many_rows_theta_far_above_refined():
    """More than 256 rows (the many-rows path) with predictions far above the
    true k-th score, so the boundary is the lumped bin: rows whose refined
    boundary fits the list (theta = 1.5 x kth) and rows where it does not
    (2 x kth on N(18, 4) scores, constant rows, tied integers) must all give
    the oracle's set; the others take no, exact or near predictions."""
    need_gpu()
    R, k = 320, 2048
    lens = [12000 + (r * 877) % 28000 for r in range(R)]
    ld = ((max(lens) + 3) // 4) * 4
    x = wk.random_logits(8, R, ld, 'normal')
    ties = wk.random_logits(9, R, ld, 'ties')
    for r in range(R):
        if r % 16 == 3:
            x[r] = 3.5
        elif r % 16 == 11:
            x[r] = ties[r]
    kth = np.array([oracle.topk_row(x[r, :lens[r]], k)[1] for r in range(R)], np.float32)
    factor = np.array([1.5, 2.0, 1.1, np.nan, 1.0], np.float32)[np.arange(R) % 5]
    theta = (kth * factor).astype(np.float32)
    theta[np.arange(R) % 16 == 3] = np.float32(14.0)       # constant rows: 4 x the score
    _check(x, lens, k, theta)


def test_rows_longer_than_one_rowsel_pass():
    """Rows whose chunk histograms take the row select more than one pass:
    over 256 chunks of 4096 (1M tokens) with a few rows, over 64 chunks
    (262144 tokens) with more than 256 rows. Predictions exact, absent and far
    above the k-th score (a wide boundary bin)."""
    need_gpu()
    k = 2048
    lens = [1_500_007, 1_100_000, 1_300_000]
    x = wk.random_logits(12, 3, 1_500_008, 'normal')
    kth = np.array([oracle.topk_row(x[r, :lens[r]], k)[1] for r in range(3)], np.float32)
    theta = np.array([kth[0], np.nan, 3.0 * kth[2]], np.float32)
    _check(x, lens, k, theta)

    R = 260
    lens = [3000 + 7 * r for r in range(R)]
    lens[0], lens[100], lens[259] = 300_000, 400_003, 270_001
    ld = ((max(lens) + 3) // 4) * 4
    x = wk.random_logits(13, R, ld, 'normal')
    kth = np.array([oracle.topk_row(x[r, :lens[r]], k)[1] for r in range(R)], np.float32)
    factor = np.array([1.0, np.nan, 1.5, 3.0], np.float32)[np.arange(R) % 4]
    _check(x, lens, k, (kth * factor).astype(np.float32))


@pytest.mark.parametrize('kind', ['normal', 'ties', 'const', 'signed'])
def test_short_rows_one_launch(kind):
    """A few rows of at most 16384 tokens take the one-launch path (one
    workgroup per row, the row in LDS): ragged lengths around k, empty and
    one-token rows, with no, exact, near, far-above and far-below predictions."""
    need_gpu()
    n = 16384
    lens = [16384, 2048, 2049, 2047, 1, 0, 9999, 16383]
    R = len(lens)
    x = wk.random_logits(14, R, n, kind)
    kth = np.array([oracle.topk_row(x[r, :lens[r]], 2048)[1] if lens[r] else np.nan for r in range(R)], np.float32)
    _check(x, lens, 2048)
    for th in (kth, kth + np.float32(1e-3), kth * np.float32(3.0) + np.float32(5.0), kth - np.float32(40.0)):
        _check(x, lens, 2048, th)
    mixed = kth.copy()
    mixed[::3] = np.nan
    _check(x, lens, 2048, mixed)


@pytest.mark.parametrize('k', [1, 7, 2048, 4096])
def test_short_rows_various_k(k):
    need_gpu()
    x = wk.random_logits(15, 5, 16384, 'normal')
    lens = [16384, 5000, 4097, 4096, 4095]
    kth = np.array([oracle.topk_row(x[r, :lens[r]], k)[1] for r in range(5)], np.float32)
    _check(x, lens, k, kth * np.float32(1.01))


def test_short_rows_most_rows_and_many_rows():
    """256 rows of 16384 (the most the one-launch path takes) and 300 short
    rows (more than that: the multi-kernel path)."""
    need_gpu()
    x = wk.random_logits(16, 256, 16384, 'normal')
    kth = np.array([oracle.topk_row(x[r], 2048)[1] for r in range(256)], np.float32)
    _check(x, [16384] * 256, 2048, kth)
    lens = [100 + (r * 977) % 16285 for r in range(300)]
    y = wk.random_logits(17, 300, 16384, 'ties')
    _check(y, lens, 2048)


@pytest.mark.parametrize('kind', ['normal', 'signed', 'ties'])
def test_one_pass_predictions_and_ragged_rows(kind):
    """A few long rows (the one-pass launch: one read of the scores, the last
    workgroup of a row selecting from the chunks' lists): predictions inside
    the band (exact, 1% and 3% off), below it (the chunks' lists capped by
    their slices), above it so far that the lists miss b* (the whole-row
    selection), absent and mixed; rows of one chunk, empty rows and rows no
    longer than k in the same call."""
    need_gpu()
    ld = 131076
    lens = [131076, 131073, 100000, 16385, 16384, 5000, 0, 2048, 40000, 65536]
    R = len(lens)
    x = wk.random_logits(18, R, ld, kind)
    kth = np.array([oracle.topk_row(x[r, :lens[r]], 2048)[1] if lens[r] else np.nan for r in range(R)],
                   np.float32)
    _check(x, lens, 2048)
    for f in (1.0, 1.01, 0.97, 1.03, 0.5, 1.3):
        _check(x, lens, 2048, (kth * np.float32(f)).astype(np.float32))
    mixed = kth.copy()
    mixed[::3] = np.nan
    mixed[1::3] *= np.float32(2.0)
    _check(x, lens, 2048, mixed)


def test_one_pass_wide_boundary_bin_in_the_lists():
    """More tokens tie at the k-th score than the LDS selection holds (5000
    at one value, 1000 above it): the boundary is selected by rounds over the
    listed entries, and the ties are taken in token order."""
    need_gpu()
    n = 131072
    x = wk.random_logits(19, 2, n, 'normal')
    r = np.random.default_rng(19)
    for row in range(2):
        order = np.argsort(-x[row], kind='stable')
        v = x[row, order[1000]]
        below = order[1001:]
        x[row, r.choice(below, 5000, replace=False)] = v
    kth = np.array([oracle.topk_row(x[row], 2048)[1] for row in range(2)], np.float32)
    _check(x, [n, n - 4], 2048, kth)
    _check(x, [n, n - 4], 4096, kth)


def test_one_pass_workspace_reused_across_shapes():
    """One workspace for calls of different shapes in a row: nothing a call
    leaves behind steers the next."""
    need_gpu()
    import torch
    from gpu_util import dev, host
    import indexer_top_kv_amd as ech
    # (rows, row stride, tokens per row, k)
    shapes = [(6, 200000, 200000, 2048), (2, 40000, 39999, 7), (9, 131072, 131072, 4096), (1, 16388, 16385, 2048)]
    ws = torch.empty(max(ech.ech_topk_ws_bytes(R, n, k) for R, _, n, k in shapes), dtype=torch.uint8,
                     device='cuda')
    for i, (R, ld, n, k) in enumerate(shapes):
        x = wk.random_logits(20, R, ld, 'normal', seed_extra=i)
        kth = np.array([oracle.topk_row(x[row, :n], k)[1] for row in range(R)], np.float32)
        th = (kth * np.float32(1.01)).astype(np.float32)
        idx = torch.full((R, k), -7, dtype=torch.int32, device='cuda')
        kt = torch.empty(R, dtype=torch.float32, device='cuda')
        to = torch.empty(R, dtype=torch.float32, device='cuda')
        ech.ech_topk(dev(x), dev(np.full(R, n, np.int32)), n, k, dev(th), to, idx, kt, ws)
        torch.cuda.synchronize()
        for row in range(R):
            ref_idx, ref_kth = oracle.topk_row(x[row, :n], k)
            np.testing.assert_array_equal(host(idx)[row], ref_idx, err_msg=f'shape {i} row {row}')
            assert host(kt)[row] == ref_kth
            assert host(to)[row] == oracle.theta_next(th[row], ref_kth)
