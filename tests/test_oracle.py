"""The CPU oracle against its pins (closed forms, hand-worked fixtures, brute
force by a different algorithm, library routines, invariants)."""
import numpy as np
import pytest
import torch

import oracle
import pins
from oracle.numerics import bf16_to_f64, e4m3fn_table


def test_e4m3fn_closed_form_matches_torch_all_codes():
    tab = e4m3fn_table()
    lib = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(tab)
    np.testing.assert_array_equal(nan, np.isnan(lib))
    np.testing.assert_array_equal(tab[~nan], lib[~nan])
    assert nan.sum() == 2


def test_e4m3fn_hand_codes():
    g = pins.golden('e4m3fn_codes.json')
    tab = e4m3fn_table()
    for code, val in g['codes'].items():
        assert tab[int(code)] == val, code
    for c in g['nan_codes']:
        assert np.isnan(tab[c])
    z = tab[g['negative_zero_code']]
    assert z == 0.0 and np.signbit(z)


def test_bf16_decode():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x4049, 0x0001], np.uint16)
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(bf16_to_f64(bits), lib)
    assert bf16_to_f64(np.array([0x3F80], np.uint16))[0] == 1.0


@pytest.mark.parametrize('pin', pins.INDEXER_PINS, ids=lambda p: p.__name__)
def test_indexer_pins(pin):
    pin(oracle.index_logits)


def test_index_logit_at_agrees_with_rows():
    q, w, kb, sc = pins._rand_case(9, R=1, P=64)
    rows = oracle.index_logits(q, w, kb, 'fp8', sc, [0], [64])[0]
    g = [0, 5, 63, 17]
    at = oracle.index_logit_at(q[0], w[0], kb, 'fp8', sc, g)
    np.testing.assert_allclose(at, rows[g], rtol=1e-14)


@pytest.mark.parametrize('pin', pins.TOPK_PINS, ids=lambda p: p.__name__)
def test_topk_pins(pin):
    pin(oracle.topk_row)


def test_topk_hypothesis():
    hyp = pytest.importorskip('hypothesis')
    from hypothesis import given, settings, strategies as st

    @settings(max_examples=200, deadline=None)
    @given(st.lists(st.integers(-3, 3), min_size=0, max_size=30), st.integers(1, 10))
    def run(vals, k):
        s = np.array(vals, dtype=np.float32)
        idx, kth = oracle.topk_row(s, k)
        want = pins.brute_topk(s, k)
        np.testing.assert_array_equal(idx[:len(want)], want)
    run()


def test_theta_pins():
    pins.pin_theta(oracle.theta_next)


@pytest.mark.parametrize('pin', pins.SLOTMAP_PINS, ids=lambda p: p.__name__)
def test_slotmap_pins(pin):
    pin(oracle.SlotMap)


def test_final_overflow_is_error():
    sm = oracle.SlotMap(10, 2)
    with pytest.raises(RuntimeError):
        sm.final([0], np.array([[0, 1, 2]], np.int64))


@pytest.mark.parametrize('pin', pins.ATTN_PINS, ids=lambda f: f.__name__)
def test_attention_pins(pin):
    pin(oracle.sparse_attention)


@pytest.mark.parametrize('pin', pins.APPEND_PINS, ids=lambda f: f.__name__)
def test_append_pins(pin):
    pin(oracle.kv_append)
