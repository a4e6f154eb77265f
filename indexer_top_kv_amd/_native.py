"""ctypes loader and signatures for libech.so (the C ABI in include/ech.h).

Loading fails loudly when the library is missing: there is no fallback
implementation of any step.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, 'libech.so')

ECH_OK = 0
ECH_EINVAL = -1
ECH_ENOSPC = -2
ECH_EUNSUPPORTED = -3
ECH_EHIP = -4
ECH_ESCRATCH = -5
ECH_TOPK_SCRATCH_BYTES = 16 << 20

ECH_KEY_BF16 = 0
ECH_KEY_FP8 = 1

ECH_EARLY = 0
ECH_FINAL = 1
ECH_PREFILL = 2

(CTR_HEAD, CTR_EPOCH, CTR_NMISS, CTR_NEVICT, CTR_RECALLED, CTR_STATUS, CTR_NWANT, CTR_NPINNED,
 CTR_NMISS_EARLY, CTR_TICKET, CTR_NCOPIED_EARLY, CTR_LIVE, CTR_NCOPIED_FINAL, CTR_FINAL_READY, CTR_FINAL_DONE,
 CTR_EARLY_WALK) = range(16)
CTR_LEN = 16

ST_OVERFLOW = 1
ST_BADTOK = 2
ST_BADMISS = 4
ST_FULL = 8
ST_TIMEOUT = 16

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t

SIGNATURES = {
    'ech_status_str': (ctypes.c_char_p, [ctypes.c_int]),
    'ech_version': (ctypes.c_int, []),
    'ech_index_logits': (ctypes.c_int, [_p, _p, _p, ctypes.c_int, _p, _p, _p, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_int, ctypes.c_int, _p, _i64, _p]),
    'ech_index_logits_causal': (ctypes.c_int, [_p, _p, _p, ctypes.c_int, _p, _i64, _i64, ctypes.c_int,
                                               ctypes.c_int, ctypes.c_int, _p, _i64, _p]),
    'ech_topk_ws_bytes': (_sz, [ctypes.c_int, ctypes.c_int, ctypes.c_int]),
    'ech_topk': (ctypes.c_int, [_p, _i64, _p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _p, _p, _p, _p, _p, _sz,
                                _p]),
    'ech_topk_noalloc': (ctypes.c_int, [_p, _i64, _p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _p, _p, _p, _p,
                                        _p]),
    'ech_cache_reset': (ctypes.c_int, [_p, _i64, _p, _p, _i32, _p, _p]),
    'ech_cache_step_ws_bytes': (_sz, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _i32,
                                      _i32]),
    'ech_cache_step': (ctypes.c_int, [ctypes.c_int, _p, _i64, _p, _p, _i32, _p, _i32, _p, _p, _p, ctypes.c_int,
                                      ctypes.c_int, _p, ctypes.c_int, ctypes.c_int, _p, _i64, _p, ctypes.c_int, _p,
                                      _p, _p, _sz, _p]),
    'ech_recall': (ctypes.c_int, [ctypes.c_int, _p, _i64, _i64, _p, _i32, _p, _p, _i32, _p]),
    'ech_index_logits_early_ws_bytes': (_sz, [ctypes.c_int, ctypes.c_int, _i32, _i32]),
    'ech_index_logits_early': (ctypes.c_int, [_p, _p, _p, ctypes.c_int, _p, _p, _p, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int, _p, _i64, ctypes.c_int, ctypes.c_int, _p,
                                              ctypes.c_int, _p, _i64, _p, _p, _i32, _p, _i32, _p, _p, _p, _sz, _p]),
    'ech_recall_early_live': (ctypes.c_int, [_p, _i64, _i64, _p, _i32, _p, _i32, _p, _i32, _p, _p, _p]),
    'ech_recall_rest': (ctypes.c_int, [_p, _i64, _i64, _p, _i32, _p, _i32, _p, _i32, _p, _p, _p]),
    'ech_topk_early': (ctypes.c_int, [_p, _i64, _p, ctypes.c_int, ctypes.c_int, ctypes.c_int, _p, _p, _p, _p, _p, _sz,
                                      _i32, _i32, _p]),
    'ech_kv_append': (ctypes.c_int, [_p, _i64, _i64, _p, ctypes.c_int, _p, _p, _p, _p, _p, ctypes.c_int, _p, _p, _p,
                                     _p, _p]),
    'ech_sparse_attn_ws_bytes': (_sz, [ctypes.c_int, ctypes.c_int, ctypes.c_int]),
    'ech_sparse_attn': (ctypes.c_int, [_p, _p, _i32, _p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                       _p, _p, _p, _sz, _p]),
}

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f'{path} is missing: build it with `python -m indexer_top_kv_amd.build` '
                          '(there is no fallback implementation)')
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
