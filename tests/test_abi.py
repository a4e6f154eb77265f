"""The C ABI without a GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

import indexer_top_kv_amd as ech
from indexer_top_kv_amd import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, 'include', 'ech.h')


def declared_symbols():
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r'/\*.*?\*/', '', text, flags=re.S)
    return sorted(set(re.findall(r'\b(ech_[a-z_0-9]+)\s*\(', text)))


def test_header_declares_entry_points():
    syms = declared_symbols()
    for name in ['ech_index_logits', 'ech_index_logits_causal', 'ech_topk', 'ech_topk_ws_bytes',
                 'ech_cache_step', 'ech_cache_step_ws_bytes', 'ech_cache_reset', 'ech_recall',
                 'ech_early_ws_bytes', 'ech_early_begin', 'ech_early_group', 'ech_recall_group',
                 'ech_status_str', 'ech_version']:
        assert name in syms


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_native.LIB_PATH)
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert set(declared_symbols()) == set(_native.SIGNATURES)


def test_status_strings_and_version():
    lib = ech.lib()
    assert lib.ech_version() == 101
    assert lib.ech_status_str(0) == b'ok'
    for code in (-1, -2, -3, -4):
        assert b'unknown' not in lib.ech_status_str(code)


def test_ws_sizes_monotone():
    lib = ech.lib()
    a = lib.ech_topk_ws_bytes(32, 131072, 2048)
    b = lib.ech_topk_ws_bytes(64, 131072, 2048)
    assert 0 < a < b
    assert lib.ech_topk_ws_bytes(0, 10, 10) == 0
    c = lib.ech_cache_step_ws_bytes(1, 32, 32, 2048, 131072, 260000, 65536)
    assert c >= 32 * 2048 * 8          # FINAL: room to list every selected token as a miss (8 B each)
    assert lib.ech_cache_step_ws_bytes(1, 64, 64, 2048, 131072, 260000, 131072) > c
    assert lib.ech_cache_step_ws_bytes(7, 1, 1, 1, 1, 1, 1) == 0


FAKE = 1 << 20  # never dereferenced: validation fails before any HIP call


def test_index_logits_rejects_bad_args():
    lib = ech.lib()
    ok = dict(q=FAKE, w=FAKE, k=FAKE, dt=1, sc=FAKE, t0=FAKE, ln=FAKE, R=2, H=64, D=128, ml=100, out=FAKE, ld=100)

    def call(**kw):
        a = dict(ok, **kw)
        return lib.ech_index_logits(a['q'], a['w'], a['k'], a['dt'], a['sc'], a['t0'], a['ln'], a['R'], a['H'],
                                    a['D'], a['ml'], a['out'], a['ld'], None)
    assert call(q=None) == -1
    assert call(H=32) == -1
    assert call(D=64) == -1
    assert call(R=0) == -1
    assert call(ld=50) == -1
    assert call(dt=7) == -3
    assert call(sc=None) == -1          # fp8 needs scales
    assert call(q=FAKE + 4) == -1        # misaligned
    assert call(ml=0) == 0               # nothing to do, nothing launched


def test_topk_rejects_bad_args():
    lib = ech.lib()
    ws = lib.ech_topk_ws_bytes(4, 1000, 64)

    def call(k=64, ld=1000, ml=1000, wsb=ws, ptr=FAKE, wsp=FAKE):
        return lib.ech_topk(ptr, ld, FAKE, 4, ml, k, None, None, FAKE, FAKE, wsp, wsb, None)
    assert call(k=0) == -1
    assert call(k=5000) == -1
    assert call(ld=999) == -1
    assert call(ld=1002) == -1           # rows must stay 16-byte aligned
    assert call(wsb=ws - 1) == -1
    assert call(ptr=FAKE + 4) == -1
    assert call(wsp=FAKE + 16) == -1     # workspace must be 256-byte aligned
    assert call(ml=1 << 24) == -1


def test_cache_step_rejects_bad_args():
    lib = ech.lib()

    def call(phase=1, B=2, R=2, k=64, ml=1000, C=1000, M=128, cap=8, P=4000, wsb=None, idx=FAKE):
        wsz = lib.ech_cache_step_ws_bytes(phase, B, R, k, ml, C, M) if wsb is None else wsb
        return lib.ech_cache_step(phase, FAKE, P, FAKE, FAKE, C, FAKE, M, FAKE, FAKE, FAKE, B, ml, idx, R, k,
                                  FAKE, 1000, FAKE, cap, FAKE, FAKE, FAKE, wsz, None)
    assert call(phase=5) == -1
    assert call(C=100) == -2             # FINAL demand 2*64 > 100
    assert call(phase=2, B=1, R=4, C=200) == -2   # PREFILL demand min(1000, 256) > 200
    assert call(M=100) == -1             # miss list smaller than the demand
    assert call(P=1 << 31) == -1
    assert call(idx=None) == -1
    assert call(phase=2, B=2) == -1      # PREFILL is one sequence
    assert call(wsb=16) == -1
    assert call(phase=0, M=15) == -1     # EARLY needs B*cap entries


def test_recall_rejects_bad_args():
    lib = ech.lib()
    assert lib.ech_recall(1, FAKE, 10, 1150, FAKE, 10, FAKE, FAKE, 4, None) == -1   # row_bytes % 16
    assert lib.ech_recall(1, None, 10, 1152, FAKE, 10, FAKE, FAKE, 4, None) == -1
    assert lib.ech_recall(1, FAKE, 0, 1152, FAKE, 10, FAKE, FAKE, 4, None) == -1
    assert lib.ech_recall(9, FAKE, 10, 1152, FAKE, 10, FAKE, FAKE, 4, None) == -1   # no such phase


def test_early_group_calls_reject_bad_args():
    lib = ech.lib()
    assert lib.ech_early_ws_bytes(0, 10, 10, 10) == 0
    a = lib.ech_early_ws_bytes(4, 131072, 260000, 2048)
    b = lib.ech_early_ws_bytes(32, 131072, 260000, 16384)
    assert 0 < a < b
    ws = lib.ech_early_ws_bytes(2, 1000, 500, 64)

    def begin(q=FAKE, dt=1, sc=FAKE, B=2, ml=1000, C=500, M=64, wsb=ws, wsp=FAKE):
        return lib.ech_early_begin(q, FAKE, FAKE, dt, sc, FAKE, FAKE, B, ml, FAKE, FAKE, 4000, FAKE, C, FAKE, M,
                                   FAKE, wsp, wsb, None)
    assert begin(q=None) == -1
    assert begin(dt=5) == -3
    assert begin(sc=None) == -1
    assert begin(q=FAKE + 8) == -1
    assert begin(B=2000) == -1
    assert begin(wsb=ws - 1) == -1
    assert begin(wsp=FAKE + 64) == -1

    def group(g=0, b0=0, b1=2, B=2, cap=32, M=64, ld=1000, lg=FAKE, wsb=ws):
        return lib.ech_early_group(g, b0, b1, lg, ld, FAKE, cap, FAKE, FAKE, B, 1000, FAKE, 4000, FAKE, FAKE, 500,
                                   FAKE, M, FAKE, FAKE, FAKE, wsb, None)
    assert group(g=-1) == -1
    assert group(g=96) == -1
    assert group(b0=1, b1=1) == -1
    assert group(b1=3) == -1
    assert group(cap=33) == -1            # early miss list smaller than B * cap
    assert group(ld=999) == -1
    assert group(lg=FAKE + 4) == -1
    assert group(wsb=16) == -1
    assert lib.ech_recall_group(0, FAKE, 10, 1150, FAKE, 10, FAKE, 4, FAKE, FAKE, None) == -1   # row_bytes % 16
    assert lib.ech_recall_group(99, FAKE, 10, 1152, FAKE, 10, FAKE, 4, FAKE, FAKE, None) == -1
    assert lib.ech_recall_group(0, FAKE, 10, 1152, FAKE, 10, FAKE, 4, FAKE, FAKE + 16, None) == -1
