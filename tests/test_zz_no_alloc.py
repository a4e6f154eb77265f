"""ech_topk_noalloc (the top-k with the library's static per-GPU scratch
array as its workspace, for callers that cannot allocate) against ech_topk
with a caller workspace: idx, kth and the threshold update bit for bit, on
calls in a row on one GPU, each smaller than the one before, so that every
call starts from the scratch contents the previous, larger one left."""
import numpy as np
import pytest
import torch

import indexer_top_kv_amd as ech
import workloads as wk
from gpu_util import dev, host, need_gpu

pytestmark = pytest.mark.gpu


def _both(L, lens, max_len, k, theta):
    R = L.shape[0]
    out = []
    for noalloc in (False, True):
        idx = torch.full((R, k), -7, dtype=torch.int32, device='cuda')
        kth = torch.full((R,), 123.0, dtype=torch.float32, device='cuda')
        th_out = torch.full((R,), -5.0, dtype=torch.float32, device='cuda')
        if noalloc:
            ech.ech_topk_noalloc(L, lens, max_len, k, theta, th_out, idx, kth)
        else:
            ws = torch.empty(ech.ech_topk_ws_bytes(R, max_len, k), dtype=torch.uint8, device='cuda')
            ech.ech_topk(L, lens, max_len, k, theta, th_out, idx, kth, ws)
        torch.cuda.synchronize()
        out.append((host(idx), host(kth), host(th_out)))
    return out


def test_noalloc_matches_workspace_variant_on_shrinking_calls():
    need_gpu()
    calls = [
        # (rows, tokens per row, k, ragged): the decode launch shape, then smaller ones
        (32, 131072, 2048, False),
        (7, 50000, 1024, True),
        (300, 9000, 512, True),    # many rows: the refinement path
        (3, 5000, 256, True),      # short rows: one launch, scratch unused
    ]
    for i, (R, N, k, ragged) in enumerate(calls):
        assert ech.ech_topk_ws_bytes(R, N, k) <= ech._native.ECH_TOPK_SCRATCH_BYTES
        x = wk.random_logits(1, R, N, 'normal' if i % 2 == 0 else 'ties', seed_extra=i)
        lens = np.full(R, N, np.int32)
        if ragged:
            lens = np.random.default_rng(i).integers(0, N + 1, R).astype(np.int32)
            lens[0] = N
        ld = (N + 63) // 64 * 64
        L = torch.zeros((R, ld), dtype=torch.float32, device='cuda')
        L[:, :N] = dev(x)
        # thresholds: exact k-th scores for some rows, off or missing for others
        kth_true = np.array([np.sort(x[r, :lens[r]])[-k] if lens[r] >= k else np.nan for r in range(R)],
                            np.float32)
        th = kth_true * np.where(np.arange(R) % 3 == 0, 1.0, 0.97).astype(np.float32)
        th[np.arange(R) % 5 == 4] = np.nan
        (i1, k1, t1), (i2, k2, t2) = _both(L, dev(lens), N, k, dev(th))
        np.testing.assert_array_equal(i2, i1, err_msg=f'call {i} idx')
        np.testing.assert_array_equal(k2, k1, err_msg=f'call {i} kth')
        np.testing.assert_array_equal(t2, t1, err_msg=f'call {i} theta')


def test_noalloc_rejects_more_than_the_scratch_holds():
    need_gpu()
    R, N, k = 4096, 110000, 2048
    assert ech.ech_topk_ws_bytes(R, N, k) > ech._native.ECH_TOPK_SCRATCH_BYTES
    L = torch.zeros((R, 110016), dtype=torch.float32, device='cuda')
    lens = torch.full((R,), N, dtype=torch.int32, device='cuda')
    idx = torch.empty((R, k), dtype=torch.int32, device='cuda')
    kth = torch.empty(R, dtype=torch.float32, device='cuda')
    with pytest.raises(ech.EchError) as e:
        ech.ech_topk_noalloc(L, lens, N, k, None, None, idx, kth)
    assert e.value.code == ech._native.ECH_ESCRATCH
