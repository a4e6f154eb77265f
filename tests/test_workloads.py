"""Seeded generators: determinism, shapes, encodings and the AR(1) process."""
import numpy as np
import pytest

import workloads as wk
from oracle.numerics import bf16_to_f64, e4m3fn_to_f64


def test_configs_shapes():
    c = wk.CONFIGS
    assert c['decode-32x128k-fp8'].P == 32 * 131072
    assert c['decode-4x1m-fp8'].P == 4 * 1048576
    assert c['decode-1x16k-bf16'].P == 16384
    lens = c['decode-64x110k-fp8-capacity'].lens
    assert lens.min() >= 100000 and lens.max() <= 110000 and len(lens) == 64
    assert np.array_equal(lens, c['decode-64x110k-fp8-capacity'].lens)  # seeded
    t0 = c['decode-64x110k-fp8-capacity'].tok0
    assert t0[0] == 0 and np.all(np.diff(t0) == lens[:-1])


def test_keys_deterministic_and_encoded():
    wl = wk.CONFIGS['decode-32x128k-fp8'].scaled(B=2, N=3000)
    a, sa = wk.keys(wl)
    b, sb = wk.keys(wl)
    assert a.dtype == np.uint8 and a.shape == (6000, 128)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(sa, sb)
    v = e4m3fn_to_f64(a)
    assert not np.isnan(v).any()
    assert abs(v.std() - 1.0) < 0.05
    assert sa.min() >= 0.5 and sa.max() <= 2.0


def test_bf16_keys_normal():
    wl = wk.CONFIGS['decode-1x16k-bf16'].scaled(N=4000)
    k, s = wk.keys(wl)
    assert s is None and k.dtype == np.uint16
    v = bf16_to_f64(k)
    assert abs(v.mean()) < 0.02 and abs(v.std() - 1) < 0.02


def test_ar1_variance_stationary():
    wl = wk.CONFIGS['decode-32x128k-fp8'].scaled(B=4, steps=30)
    qs = [bf16_to_f64(q) for q in wk.decode_queries(wl)]
    for q in qs[::10]:
        assert abs(q.std() - 1.0) < 0.05
    # lag-1 correlation close to rho
    c = np.corrcoef(qs[10].ravel(), qs[11].ravel())[0, 1]
    assert abs(c - 0.9) < 0.02


def test_resample_topic_shift():
    wl = wk.CONFIGS['decode-64x110k-fp8-capacity'].scaled(steps=6)
    qs = [bf16_to_f64(q) for q in wk.decode_queries(wl)]
    corr = [np.corrcoef(qs[1][b].ravel(), qs[2][b].ravel())[0, 1] for b in range(64)]
    shifted = sum(c < 0.5 for c in corr)
    assert 3 <= shifted <= 25   # ~0.2 * 64


def test_dyadic_variant_integers():
    wl = wk.CONFIGS['decode-32x128k-fp8'].scaled(B=2, N=500, variant='dyadic')
    k, s = wk.keys(wl)
    v = e4m3fn_to_f64(k)
    assert np.all(v == np.round(v)) and np.abs(v).max() <= 8
    assert set(np.unique(s).tolist()) <= {0.5, 1.0, 2.0}
    q = bf16_to_f64(next(wk.decode_queries(wl)))
    assert np.all(q == np.round(q)) and np.abs(q).max() <= 3
    w = wk.head_weights(wl)
    assert np.all(w * 64 == np.round(w * 64))


def test_host_rows_chunk_seeding():
    wl = wk.CONFIGS['decode-1x16k-bf16'].scaled(N=3000)
    a = wk.host_rows(wl)
    b = wk.host_rows(wl)
    np.testing.assert_array_equal(a, b)
    assert a.shape == (3000, 576)
    v = bf16_to_f64(a[:100])
    assert abs(v.std() - 1) < 0.05


def test_prefill_blocks_consistent():
    wl = wk.CONFIGS['prefill-110k-fp8'].scaled(N=700, block_rows=256)
    whole = wk.prefill_queries(wl, 0, 700)
    part = wk.prefill_queries(wl, 200, 300)
    np.testing.assert_array_equal(whole[200:500], part)
    w = wk.head_weights(wl)
    np.testing.assert_array_equal(w[200:500], wk.head_weights(wl, rows=300, row0=200))


def test_layers_share_lengths_and_draw_their_own_values():
    base = wk.CONFIGS['decode-64x110k-fp8-capacity'].scaled(B=3, N=3000, len_lo=1000)
    l0, l1, l2 = base, base.scaled(layer=1), base.scaled(layer=2)
    np.testing.assert_array_equal(l0.lens, l1.lens)
    np.testing.assert_array_equal(l0.tok0, l2.tok0)
    k0, s0 = wk.keys(l0)
    k1, s1 = wk.keys(l1)
    k0b, _ = wk.keys(base.scaled(layer=0))
    np.testing.assert_array_equal(k0, k0b)              # layer 0 keeps the plain seeds
    assert not np.array_equal(k0, k1) and not np.array_equal(s0, s1)
    assert not np.array_equal(wk.head_weights(l0), wk.head_weights(l1))
    assert not np.array_equal(next(wk.decode_queries(l1, 1)), next(wk.decode_queries(l2, 1)))
    assert not np.array_equal(wk.host_rows(l0)[:4], wk.host_rows(l1)[:4])
