"""Host-side argument checks of the C ABI, written against a bare ctypes
handle so that they run both on the built library (tests/test_abi.py) and on
a build whose host code is instrumented with AddressSanitizer and UBSan (run as a
script, in a process with the sanitizer runtime preloaded):

    python tests/abi_checks.py PATH_TO_LIBRARY

Every call here fails validation (or has nothing to do) before any HIP call
or kernel launch, so no GPU is needed; no pointer is dereferenced.
"""
import ctypes
import importlib.util
import os
import sys

FAKE = 1 << 20  # never dereferenced: validation fails before any HIP call


def check_index_logits_rejects_bad_args(lib):
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


def check_topk_rejects_bad_args(lib):
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


def check_cache_step_rejects_bad_args(lib):

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


def check_recall_rejects_bad_args(lib):
    assert lib.ech_recall(1, FAKE, 10, 1150, FAKE, 10, FAKE, FAKE, 4, None) == -1   # row_bytes % 16
    assert lib.ech_recall(1, None, 10, 1152, FAKE, 10, FAKE, FAKE, 4, None) == -1
    assert lib.ech_recall(1, FAKE, 0, 1152, FAKE, 10, FAKE, FAKE, 4, None) == -1
    assert lib.ech_recall(9, FAKE, 10, 1152, FAKE, 10, FAKE, FAKE, 4, None) == -1   # no such phase


def check_index_logits_early_rejects_bad_args(lib):
    assert lib.ech_index_logits_early_ws_bytes(0, 10, 10, 10) == 0
    a = lib.ech_index_logits_early_ws_bytes(4, 131072, 260000, 2048)
    b = lib.ech_index_logits_early_ws_bytes(32, 131072, 260000, 16384)
    assert 0 < a < b
    ws = lib.ech_index_logits_early_ws_bytes(4, 1000, 500, 64)

    def call(q=FAKE, dt=1, sc=FAKE, R=4, ml=1000, ld=1000, e0=0, e1=4, cap=16, P=4000, C=500, M=64, wsb=ws,
             wsp=FAKE, miss=FAKE):
        return lib.ech_index_logits_early(q, FAKE, FAKE, dt, sc, FAKE, FAKE, R, 64, 128, ml, FAKE, ld, e0, e1, FAKE,
                                          cap, FAKE, P, FAKE, FAKE, C, miss, M, FAKE, FAKE, wsp, wsb, None)
    assert call(q=None) == -1
    assert call(dt=0) == -3              # bf16 keys: not fused
    assert call(sc=None) == -1
    assert call(R=2000) == -1
    assert call(ld=999) == -1
    assert call(e0=2, e1=2) == -1
    assert call(e1=5) == -1
    assert call(cap=5000) == -1
    assert call(cap=17) == -1            # early miss list smaller than (e1 - e0) * cap
    assert call(P=1 << 31) == -1
    assert call(wsb=ws - 1) == -1
    assert call(wsp=FAKE + 64) == -1
    assert call(q=FAKE + 8) == -1
    assert call(miss=FAKE + 4) == -1

    def live(pool=FAKE, rb=1152, miss=FAKE, wsp=FAKE, M=64, mf=None, Mf=0):
        return lib.ech_recall_early_live(pool, 4000, rb, FAKE, 500, miss, M, mf, Mf, FAKE, wsp, None)
    assert live(pool=None) == -1
    assert live(rb=1150) == -1
    assert live(rb=65536) == -1
    assert live(miss=FAKE + 4) == -1
    assert live(wsp=FAKE + 64) == -1
    assert live(M=-1) == -1
    assert live(mf=FAKE + 4) == -1       # FINAL list not 8-byte aligned
    assert live(mf=FAKE, Mf=-1) == -1

    def rest(pool=FAKE, rb=1152, me=FAKE, mf=FAKE, s2t=FAKE, Me=64, Mf=64):
        return lib.ech_recall_rest(pool, 4000, rb, FAKE, 500, me, Me, mf, Mf, s2t, FAKE, None)
    assert rest(pool=None) == -1
    assert rest(rb=1150) == -1
    assert rest(me=None) == -1
    assert rest(mf=None) == -1
    assert rest(s2t=None) == -1
    assert rest(Me=-1) == -1
    assert rest(pool=FAKE + 8) == -1

    wse = lib.ech_index_logits_early_ws_bytes(8, 20000, 500, 64)

    def early_topk(k=64, ld=20032, ml=20000, th=FAKE, wsp=FAKE, wsb=wse, R=8):
        return lib.ech_topk_early(FAKE, ld, FAKE, R, ml, k, th, None, FAKE, FAKE, wsp, wsb, 500, 64, None)
    assert early_topk(th=None) == -1          # the theta the scores call took is required
    assert early_topk(k=0) == -1
    assert early_topk(k=4097) == -1
    assert early_topk(ld=19999) == -1
    assert early_topk(ld=20002) == -1         # rows 16-byte aligned
    assert early_topk(wsp=FAKE + 128) == -1
    assert early_topk(wsb=wse - 1) == -1
    assert early_topk(R=0) == -1
    assert early_topk(ml=(1 << 20) + 1, ld=(1 << 20) + 64, wsb=1 << 40) == -1   # more than 4096 waves per row


def check_topk_noalloc_rejects_bad_args(lib):
    def call(R=4, ml=1000, k=64, ld=1000, ptr=FAKE):
        return lib.ech_topk_noalloc(ptr, ld, FAKE, R, ml, k, None, None, FAKE, FAKE, None)
    assert call(k=0) == -1
    assert call(k=5000) == -1
    assert call(ld=999) == -1
    assert call(ptr=FAKE + 4) == -1
    assert call(ptr=None) == -1
    # a 4096-row prefill block needs more than the static array: -5, before any HIP call
    assert lib.ech_topk_ws_bytes(4096, 110000, 2048) > (16 << 20)
    assert call(R=4096, ml=110000, k=2048, ld=110016) == -5
    assert lib.ech_topk_ws_bytes(32, 131072, 2048) <= (16 << 20)



CHECKS = [v for k, v in sorted(globals().items()) if k.startswith('check_')]


def load(path):
    """ctypes handle with the signatures of indexer_top_kv_amd/_native.py
    (loaded by file path: the package itself imports torch)."""
    here = os.path.dirname(os.path.abspath(__file__))
    spec = importlib.util.spec_from_file_location(
        '_ech_native', os.path.join(os.path.dirname(here), 'indexer_top_kv_amd', '_native.py'))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.load(path)


if __name__ == '__main__':
    lib = load(sys.argv[1])
    for fn in CHECKS:
        fn(lib)
    print(f'abi checks ok: {len(CHECKS)}', flush=True)
