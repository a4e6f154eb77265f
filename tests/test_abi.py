"""The C ABI without a GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

import indexer_top_kv_amd as ech
from indexer_top_kv_amd import _native

import abi_checks

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
                 'ech_index_logits_early', 'ech_index_logits_early_ws_bytes', 'ech_recall_early_live',
                 'ech_recall_rest', 'ech_topk_early', 'ech_topk_noalloc',
                 'ech_status_str', 'ech_version']:
        assert name in syms


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_native.LIB_PATH)
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert set(declared_symbols()) == set(_native.SIGNATURES)


def test_status_strings_and_version():
    lib = ech.lib()
    assert lib.ech_version() == 300
    assert lib.ech_status_str(0) == b'ok'
    for code in (-1, -2, -3, -4, -5):
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


def test_argument_checks():
    for fn in abi_checks.CHECKS:
        fn(ech.lib())


def _clang_rt(name):
    import glob
    hits = sorted(glob.glob(f'/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.{name}-x86_64.so'))
    return hits[-1] if hits else None


def test_argument_checks_under_asan_ubsan():
    """The host code of every entry point (argument validation, workspace
    sizing, status strings) built with AddressSanitizer and UBSan on the host
    side, and run through the same checks: no sanitizer report."""
    import subprocess
    import sys
    from indexer_top_kv_amd import build as b
    rt = _clang_rt('asan')
    if rt is None or not os.path.exists(os.environ.get('HIPCC', '/opt/rocm/bin/hipcc')):
        pytest.skip('no hipcc or sanitizer runtime')
    lib = b.build_sanitized()
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS='detect_leaks=0:abort_on_error=1',
               UBSAN_OPTIONS='halt_on_error=1:print_stacktrace=1',
               LD_LIBRARY_PATH=os.path.dirname(rt) + ':' + os.environ.get('LD_LIBRARY_PATH', ''))
    r = subprocess.run([sys.executable, os.path.join(ROOT, 'tests', 'abi_checks.py'), lib], env=env,
                       capture_output=True, text=True, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert 'abi checks ok' in r.stdout
    assert 'AddressSanitizer' not in out and 'runtime error' not in out, out[-4000:]
