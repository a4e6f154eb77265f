"""Python binding of libech: the MI355X (gfx950) indexer -> exact top-k ->
KV-recall path of ECHO-style lossless KV offloading.

Each function takes torch tensors (device memory, or pinned host memory for
the host pool), passes their pointers and sizes to the C ABI of the same name
(include/ech.h) and raises EchError on a non-zero return code. Nothing is
computed here; every step runs in the library's HIP kernels. Calls are
asynchronous on the given stream (default: torch's current stream).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

from . import _native
from ._native import (ECH_EARLY, ECH_FINAL, ECH_PREFILL, ECH_KEY_BF16, ECH_KEY_FP8,  # noqa: F401
                      CTR_HEAD, CTR_EPOCH, CTR_NMISS, CTR_NEVICT, CTR_RECALLED, CTR_STATUS, CTR_NWANT,
                      CTR_NPINNED, CTR_NMISS_EARLY, CTR_TICKET, CTR_NCOPIED_EARLY, CTR_LIVE,
                      CTR_NCOPIED_FINAL, CTR_FINAL_READY, CTR_FINAL_DONE, CTR_EARLY_WALK, CTR_LEN, ST_OVERFLOW, ST_BADTOK,
                      ST_BADMISS, ST_FULL, ST_TIMEOUT)

__all__ = ['ech_kv_append', 'ech_sparse_attn', 'ech_sparse_attn_ws_bytes', 'ech_index_logits', 'ech_index_logits_causal', 'ech_topk', 'ech_topk_noalloc', 'ech_topk_ws_bytes', 'ech_cache_reset',
           'ech_cache_step', 'ech_cache_step_ws_bytes', 'ech_recall', 'ech_index_logits_early',
           'ech_index_logits_early_ws_bytes', 'ech_recall_early_live', 'ech_recall_rest', 'ech_topk_early', 'EchError', 'LayerState',
           'lib']


class EchError(RuntimeError):
    def __init__(self, fn: str, code: int):
        self.code = code
        msg = lib().ech_status_str(code).decode()
        super().__init__(f'{fn} failed: {msg} ({code})')


def lib():
    return _native.load()


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise EchError(fn, rc)


def _key_dtype(kcache: torch.Tensor) -> int:
    if kcache.dtype in (torch.uint8, torch.float8_e4m3fn):
        return ECH_KEY_FP8
    if kcache.dtype in (torch.int16, torch.uint16, torch.bfloat16):
        return ECH_KEY_BF16
    raise TypeError(f'unsupported key dtype {kcache.dtype}')


# ------------------------------------------------------------------ stage 1
def ech_index_logits(q, w, kcache, kscale, row_tok0, row_len, max_len: int, logits, stream=None) -> None:
    """Decode indexer scores: q [R,H,D] bf16, w [R,H] f32, kcache [P,D] (uint8
    e4m3fn or bf16), kscale [P] f32 or None, row_tok0 [R] i64, row_len [R] i32,
    logits [R, ld] f32."""
    R, H, D = q.shape
    _check('ech_index_logits', lib().ech_index_logits(
        _ptr(q), _ptr(w), _ptr(kcache), _key_dtype(kcache), _ptr(kscale), _ptr(row_tok0), _ptr(row_len),
        R, H, D, int(max_len), _ptr(logits), logits.stride(0), _stream(stream)))


def ech_index_logits_causal(q, w, kcache, kscale, tok0: int, row0: int, logits, stream=None) -> None:
    """Prefill indexer scores for query rows at positions row0 .. row0+R-1 of
    the sequence starting at global token tok0 (row r sees t <= row0 + r)."""
    R, H, D = q.shape
    _check('ech_index_logits_causal', lib().ech_index_logits_causal(
        _ptr(q), _ptr(w), _ptr(kcache), _key_dtype(kcache), _ptr(kscale), int(tok0), int(row0), R, H, D,
        _ptr(logits), logits.stride(0), _stream(stream)))


# ------------------------------------------------------------------ stage 2
def ech_topk_ws_bytes(R: int, max_len: int, k: int) -> int:
    return int(lib().ech_topk_ws_bytes(R, max_len, k))


def ech_topk(logits, row_len, max_len: int, k: int, theta_in, theta_out, idx, kth, ws, stream=None) -> None:
    """Exact top-k of each row of logits [R, ld]; idx [R,k] i32 (ascending, -1
    padded), kth [R] f32, theta_in/theta_out [R] f32 or None, ws uint8."""
    R = logits.shape[0]
    _check('ech_topk', lib().ech_topk(
        _ptr(logits), logits.stride(0), _ptr(row_len), R, int(max_len), int(k), _ptr(theta_in), _ptr(theta_out),
        _ptr(idx), _ptr(kth), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def ech_topk_noalloc(logits, row_len, max_len: int, k: int, theta_in, theta_out, idx, kth, stream=None) -> None:
    """ech_topk with the library's static per-GPU scratch array as its
    workspace (allocates nothing; calls on one GPU must not overlap)."""
    R = logits.shape[0]
    _check('ech_topk_noalloc', lib().ech_topk_noalloc(
        _ptr(logits), logits.stride(0), _ptr(row_len), R, int(max_len), int(k), _ptr(theta_in), _ptr(theta_out),
        _ptr(idx), _ptr(kth), _stream(stream)))


# ------------------------------------------------------------------ stage 3
@dataclasses.dataclass
class LayerState:
    """The fixed-size int32 tensors of one layer's slot map, on the device:
    the two maps, the epoch pins, the miss list (FINAL/PREFILL; EARLY phases
    write their own list so their rows can still be in flight while FINAL
    updates the maps) and the control counters."""
    tok2slot: torch.Tensor   # [P]
    slot2tok: torch.Tensor   # [C]
    slot_pin: torch.Tensor   # [C]
    miss: torch.Tensor       # [M_max, 2]
    ctr: torch.Tensor        # [CTR_LEN]
    miss_early: Optional[torch.Tensor] = None   # [M_early, 2]

    @property
    def P(self) -> int:
        return self.tok2slot.numel()

    @property
    def C(self) -> int:
        return self.slot2tok.numel()

    @property
    def M_max(self) -> int:
        return self.miss.shape[0]

    def miss_list(self, phase: int) -> torch.Tensor:
        return self.miss_early if phase == ECH_EARLY else self.miss

    @staticmethod
    def allocate(P: int, C: int, M_max: int, device='cuda', M_early: Optional[int] = None) -> 'LayerState':
        i32 = dict(dtype=torch.int32, device=device)
        M_early = M_max if M_early is None else M_early
        st = LayerState(torch.empty(P, **i32), torch.empty(C, **i32), torch.empty(C, **i32),
                        torch.empty((max(M_max, 1), 2), **i32), torch.empty(CTR_LEN, **i32),
                        torch.empty((max(M_early, 1), 2), **i32))
        return st


def ech_cache_reset(state: LayerState, stream=None) -> None:
    _check('ech_cache_reset', lib().ech_cache_reset(
        _ptr(state.tok2slot), state.P, _ptr(state.slot2tok), _ptr(state.slot_pin), state.C, _ptr(state.ctr),
        _stream(stream)))


def ech_cache_step_ws_bytes(phase: int, B: int, R: int, k: int, max_len: int, C: int, M_max: int) -> int:
    return int(lib().ech_cache_step_ws_bytes(phase, B, R, k, max_len, C, M_max))


def ech_cache_step(phase: int, state: LayerState, seq_tok0, seq_len, max_len: int, idx=None, k: int = 2048,
                   logits=None, theta=None, cap: int = 0, sel_slot=None, stats=None, ws=None,
                   stream=None) -> None:
    """One phase (ECH_EARLY / ECH_FINAL / ECH_PREFILL) of the slot map."""
    B = seq_tok0.shape[0]
    R = idx.shape[0] if idx is not None else B
    ld = logits.stride(0) if logits is not None else 0
    miss = state.miss_list(phase)
    _check('ech_cache_step', lib().ech_cache_step(
        phase, _ptr(state.tok2slot), state.P, _ptr(state.slot2tok), _ptr(state.slot_pin), state.C,
        _ptr(miss), miss.shape[0], _ptr(state.ctr), _ptr(seq_tok0), _ptr(seq_len), B, int(max_len),
        _ptr(idx), R, int(k), _ptr(logits), ld, _ptr(theta), int(cap), _ptr(sel_slot), _ptr(stats), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))


def ech_recall(host_pool, dev_cache, state: LayerState, phase: int = ECH_FINAL, stream=None) -> None:
    """Copy the rows missed by the last phase of this kind: host_pool
    [P, row_bytes] pinned (uint8/uint16), dev_cache [C, row_bytes] on the
    device."""
    row_bytes = host_pool.shape[1] * host_pool.element_size()
    miss = state.miss_list(phase)
    _check('ech_recall', lib().ech_recall(
        phase, _ptr(host_pool), host_pool.shape[0], row_bytes, _ptr(dev_cache), dev_cache.shape[0], _ptr(miss),
        _ptr(state.ctr), miss.shape[0], _stream(stream)))


# ------------------------------------------------------------------ stages 1 and 3 fused (decode, fp8 keys)
def ech_index_logits_early_ws_bytes(R: int, max_len: int, C: int, M_early: int) -> int:
    return int(lib().ech_index_logits_early_ws_bytes(R, max_len, C, M_early))


def ech_index_logits_early(q, w, kcache, kscale, row_tok0, row_len, max_len: int, logits, e0: int, e1: int, theta,
                           cap: int, state: 'LayerState', stats, ws, stream=None) -> None:
    """Decode scores of every row fused with the early fetch of sequences
    [e0, e1) (maps and early miss list, written while the scoring runs).
    ws: uint8, zero-filled before the first call."""
    R = q.shape[0]
    _check('ech_index_logits_early', lib().ech_index_logits_early(
        _ptr(q), _ptr(w), _ptr(kcache), _key_dtype(kcache), _ptr(kscale), _ptr(row_tok0), _ptr(row_len), R,
        q.shape[1], q.shape[2], int(max_len), _ptr(logits), logits.stride(0), int(e0), int(e1), _ptr(theta),
        int(cap), _ptr(state.tok2slot), state.P, _ptr(state.slot2tok), _ptr(state.slot_pin), state.C,
        _ptr(state.miss_early), state.miss_early.shape[0], _ptr(state.ctr), _ptr(stats), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))


def ech_recall_early_live(host_pool, dev_cache, state: 'LayerState', ws, stream=None, final: bool = False) -> None:
    """Copy early rows as ech_index_logits_early allocates them (enqueue on a
    second stream right after it; ech_recall(ECH_EARLY) afterwards copies the
    rest). final=True: then the rows of the FINAL phase that follows in the
    same step (state.miss), once that phase has completed its list;
    ech_recall(ECH_FINAL) afterwards copies what it left."""
    row_bytes = host_pool.shape[1] * host_pool.element_size()
    _check('ech_recall_early_live', lib().ech_recall_early_live(
        _ptr(host_pool), host_pool.shape[0], row_bytes, _ptr(dev_cache), dev_cache.shape[0], _ptr(state.miss_early),
        state.miss_early.shape[0], _ptr(state.miss) if final else None, state.miss.shape[0] if final else 0,
        _ptr(state.ctr), _ptr(ws), _stream(stream)))


def ech_topk_early(logits, row_len, max_len: int, k: int, theta_in, theta_out, idx, kth, state: 'LayerState', ws,
                   stream=None) -> None:
    """ech_topk for the rows of the last ech_index_logits_early call on ws,
    from the band lists its scoring waves wrote (theta_in: that call's)."""
    R = logits.shape[0]
    _check('ech_topk_early', lib().ech_topk_early(
        _ptr(logits), logits.stride(0), _ptr(row_len), R, int(max_len), int(k), _ptr(theta_in), _ptr(theta_out),
        _ptr(idx), _ptr(kth), _ptr(ws), ws.numel() * ws.element_size(), state.C, state.miss_early.shape[0],
        _stream(stream)))


def ech_recall_rest(host_pool, dev_cache, state: 'LayerState', stream=None) -> None:
    """What ech_recall_early_live left of the step's early and FINAL lists, in
    one launch (after the FINAL phase and the copier)."""
    row_bytes = host_pool.shape[1] * host_pool.element_size()
    _check('ech_recall_rest', lib().ech_recall_rest(
        _ptr(host_pool), host_pool.shape[0], row_bytes, _ptr(dev_cache), dev_cache.shape[0], _ptr(state.miss_early),
        state.miss_early.shape[0], _ptr(state.miss), state.miss.shape[0], _ptr(state.slot2tok), _ptr(state.ctr),
        _stream(stream)))


# ------------------------------------------------------------------ consumer
def ech_sparse_attn_ws_bytes(B: int, H: int, k: int) -> int:
    return int(lib().ech_sparse_attn_ws_bytes(B, H, k))


def ech_sparse_attn(q, dev_cache, sel_slot, sm_scale: float, out, lse=None, ws=None, stream=None) -> None:
    """Attention of each head over the rows its sequence selects: q [B, H, 576]
    bf16 bits (int16/uint16), dev_cache [C, 576] bf16 bits, sel_slot [B, k]
    int32 -> out [B, H, 512] fp32, lse [B, H] fp32 (optional)."""
    B, H = q.shape[0], q.shape[1]
    k = sel_slot.shape[1]
    _check('ech_sparse_attn', lib().ech_sparse_attn(
        _ptr(q), _ptr(dev_cache), dev_cache.shape[0], _ptr(sel_slot), B, H, k, float(sm_scale), _ptr(out),
        _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


# ------------------------------------------------------------------ growing contexts
def ech_kv_append(host_pool, kcache, kscale, state: LayerState, seq_tok0, seq_len, seq_cap, new_rows, new_keys,
                  new_scales=None, stream=None) -> None:
    """Each sequence's decoded token joins the host pool (pinned [P, row])
    and the key cache; seq_len (device int32) grows in place."""
    row_bytes = host_pool.shape[1] * host_pool.element_size()
    _check('ech_kv_append', lib().ech_kv_append(
        _ptr(host_pool), host_pool.shape[0], row_bytes, _ptr(kcache), _key_dtype(kcache), _ptr(kscale),
        _ptr(state.tok2slot), _ptr(seq_tok0), _ptr(seq_len), _ptr(seq_cap), seq_tok0.shape[0], _ptr(new_rows),
        _ptr(new_keys), _ptr(new_scales), _ptr(state.ctr), _stream(stream)))
