"""Plant plausible mistakes in copies of the oracle (on the CPU) and check
that the pins catch every one. A pin set that lets a mutant through would not
be pinning the oracle."""
import numpy as np
import pytest

import oracle
import pins
from oracle import indexer as ix
from oracle import select as sel
from oracle import slotmap as sm
from oracle.numerics import bf16_to_f64


def _fails(pin_list, impl):
    for p in pin_list:
        try:
            p(impl)
        except AssertionError:
            return True
        except Exception:
            return True
    return False


# ------------------------------------------------------------------ indexer

def _logits_with(core):
    def f(q_bits, w, key_bits, kdtype, scale, tok0, lens):
        out = []
        for r in range(q_bits.shape[0]):
            q64 = bf16_to_f64(q_bits[r])
            w64 = np.asarray(w[r], np.float64)
            out.append(core(q64, w64, key_bits, kdtype, scale, int(tok0[r]), int(lens[r])))
        return out
    return f


def _m_no_relu(q, w, kb, kd, sc, g0, n):
    return w @ (q @ ix.dequant_keys(kb, kd, sc, g0, g0 + n).T)


def _m_relu_after_sum(q, w, kb, kd, sc, g0, n):
    return np.maximum(w @ (q @ ix.dequant_keys(kb, kd, sc, g0, g0 + n).T), 0)


def _m_unweighted(q, w, kb, kd, sc, g0, n):
    return np.maximum(q @ ix.dequant_keys(kb, kd, sc, g0, g0 + n).T, 0).sum(0)


def _m_off_by_one(q, w, kb, kd, sc, g0, n):
    lo = min(g0 + 1, kb.shape[0] - n)
    return w @ np.maximum(q @ ix.dequant_keys(kb, kd, sc, lo, lo + n).T, 0)


def _m_reversed_dims(q, w, kb, kd, sc, g0, n):
    return w @ np.maximum(q @ ix.dequant_keys(kb, kd, sc, g0, g0 + n)[:, ::-1].T, 0)


def _m_scale_added(q, w, kb, kd, sc, g0, n):
    if kd == 'fp8':
        from oracle.numerics import e4m3fn_to_f64
        k = e4m3fn_to_f64(kb[g0:g0 + n]) + np.asarray(sc[g0:g0 + n], np.float64)[:, None]
    else:
        k = ix.dequant_keys(kb, kd, sc, g0, g0 + n)
    return w @ np.maximum(q @ k.T, 0)


def _m_scale_after_relu_abs(q, w, kb, kd, sc, g0, n):
    # scale factored out of the ReLU with its magnitude only (wrong for negative scales)
    if kd == 'fp8':
        from oracle.numerics import e4m3fn_to_f64
        k = e4m3fn_to_f64(kb[g0:g0 + n])
        s = np.abs(np.asarray(sc[g0:g0 + n], np.float64))
        return s * (w @ np.maximum(q @ k.T, 0))
    return w @ np.maximum(q @ ix.dequant_keys(kb, kd, sc, g0, g0 + n).T, 0)


INDEXER_MUTANTS = [_m_no_relu, _m_relu_after_sum, _m_unweighted, _m_off_by_one, _m_reversed_dims,
                   _m_scale_added, _m_scale_after_relu_abs]


@pytest.mark.parametrize('core', INDEXER_MUTANTS, ids=lambda f: f.__name__)
def test_indexer_mutant_caught(core):
    assert _fails(pins.INDEXER_PINS, _logits_with(core))


def test_indexer_unmutated_passes():
    assert not _fails(pins.INDEXER_PINS, _logits_with(ix._row_scores))


# ------------------------------------------------------------------ top-k

def _t_ties_high(s, k):
    s = np.asarray(s, np.float32)
    n = len(s)
    m = min(k, n)
    idx = np.full(k, -1, np.int64)
    if m == 0:
        return idx, np.float32(np.nan)
    order = (n - 1) - np.argsort(-s[::-1], kind='stable')
    idx[:m] = np.sort(order[:m])
    return idx, s[order[m - 1]]


def _t_kth_max(s, k):
    idx, kth = sel.topk_row(s, k)
    m = int((idx >= 0).sum())
    return idx, (np.asarray(s, np.float32)[idx[:m]].max() if m else kth)


def _t_k_minus_one(s, k):
    return sel.topk_row(s, max(0, k - 1)) if k > 1 else sel.topk_row(s, k)


def _t_zero_pad(s, k):
    idx, kth = sel.topk_row(s, k)
    return np.where(idx < 0, 0, idx), kth


def _t_score_order(s, k):
    s = np.asarray(s, np.float32)
    m = min(k, len(s))
    idx = np.full(k, -1, np.int64)
    if m == 0:
        return idx, np.float32(np.nan)
    order = np.argsort(-s, kind='stable')
    idx[:m] = order[:m]
    return idx, s[order[m - 1]]


def _t_signed_zero(s, k):
    # orders by raw bit pattern key, which puts -0.0 below +0.0
    s = np.asarray(s, np.float32)
    u = s.view(np.uint32).astype(np.int64)
    key = np.where(u >= 0x80000000, -(u - 0x80000000) - 1, u)
    m = min(k, len(s))
    idx = np.full(k, -1, np.int64)
    if m == 0:
        return idx, np.float32(np.nan)
    order = np.argsort(-key, kind='stable')
    idx[:m] = np.sort(order[:m])
    return idx, s[order[m - 1]]


TOPK_MUTANTS = [_t_ties_high, _t_kth_max, _t_k_minus_one, _t_zero_pad, _t_score_order, _t_signed_zero]


@pytest.mark.parametrize('impl', TOPK_MUTANTS, ids=lambda f: f.__name__)
def test_topk_mutant_caught(impl):
    assert _fails(pins.TOPK_PINS, impl)


# ------------------------------------------------------------------ theta

def _th_two_roundings(theta, kth):
    theta, kth = np.float32(theta), np.float32(kth)
    if np.isnan(kth):
        return theta
    if np.isnan(theta):
        return kth
    return np.float32(theta + np.float32(0.5) * np.float32(kth - theta))


def _th_init_zero(theta, kth):
    theta = np.float32(0.0) if np.isnan(theta) else theta
    return sel.theta_next(theta, kth)


def _th_alpha_quarter(theta, kth):
    theta, kth = np.float32(theta), np.float32(kth)
    if np.isnan(kth):
        return theta
    if np.isnan(theta):
        return kth
    return np.float32(np.float32(0.25) * kth + np.float32(0.75) * theta)


def _th_empty_poisons(theta, kth):
    if np.isnan(kth):
        return np.float32(np.nan)
    return sel.theta_next(theta, kth)


@pytest.mark.parametrize('impl', [_th_two_roundings, _th_init_zero, _th_alpha_quarter, _th_empty_poisons],
                         ids=lambda f: f.__name__)
def test_theta_mutant_caught(impl):
    assert _fails([pins.pin_theta], impl)


# ------------------------------------------------------------------ slot map

class HeadReset(sm.SlotMap):
    def _allocate(self, *a, **k):
        out = super()._allocate(*a, **k)
        self.head = 0
        return out


class NoUnmap(sm.SlotMap):
    def _allocate(self, pinned, misses, owners, hard, nseq):
        saved = self.tok2slot.copy()
        out = super()._allocate(pinned, misses, owners, hard, nseq)
        # restore evicted tokens' stale mappings
        stale = (saved >= 0) & (self.tok2slot < 0)
        self.tok2slot[stale] = saved[stale]
        return out


class IgnorePins(sm.SlotMap):
    def _allocate(self, pinned, *a, **k):
        return super()._allocate(np.zeros_like(pinned), *a, **k)


class DescendingMisses(sm.SlotMap):
    def _allocate(self, pinned, misses, owners, hard, nseq):
        return super()._allocate(pinned, list(misses)[::-1], list(owners)[::-1], hard, nseq)


class EagerFree(sm.SlotMap):
    def final(self, tok0, idx):
        keep = set()
        for b in range(idx.shape[0]):
            keep |= set((int(tok0[b]) + idx[b][idx[b] >= 0]).tolist())
        for s in range(self.C):
            u = int(self.slot2tok[s])
            if u >= 0 and u not in keep:
                self.slot2tok[s] = -1
                self.tok2slot[u] = -1
        return super().final(tok0, idx)


class HeadFromFirst(sm.SlotMap):
    def _allocate(self, *a, **k):
        out = super()._allocate(*a, **k)
        if out[0]:
            self.head = (out[0][0][1] + 1) % self.C
        return out


class EarlyNonStrict(sm.SlotMap):
    def early(self, tok0, scores, theta, cap):
        th = np.array([np.nextafter(np.float32(t), np.float32(-np.inf)) for t in theta], np.float32)
        return super().early(tok0, scores, th, cap)


class EarlyCapCountsResident(sm.SlotMap):
    def early(self, tok0, scores, theta, cap):
        B = len(tok0)
        capped = []
        for b in range(B):
            s = np.asarray(scores[b], np.float32).copy()
            th = np.float32(theta[b])
            if not np.isnan(th):
                above = np.nonzero(s > th)[0]
                drop = above[cap:]
                s[drop] = -np.inf
            capped.append(s)
        return super().early(tok0, capped, theta, cap)


SLOTMAP_MUTANTS = [HeadReset, NoUnmap, IgnorePins, DescendingMisses, EagerFree, HeadFromFirst,
                   EarlyNonStrict, EarlyCapCountsResident]


@pytest.mark.parametrize('cls', SLOTMAP_MUTANTS, ids=lambda c: c.__name__)
def test_slotmap_mutant_caught(cls):
    assert _fails(pins.SLOTMAP_PINS, cls)


def test_unmutated_oracle_passes_all():
    assert not _fails(pins.TOPK_PINS, oracle.topk_row)
    assert not _fails([pins.pin_theta], oracle.theta_next)
    assert not _fails(pins.SLOTMAP_PINS, oracle.SlotMap)


# ------------------------------------------------------------------ sparse attention

def _attn_with(core):
    """An attention oracle whose per-sequence core (q [H,576], rows [n,576],
    scale) -> (out, lse) is replaced; slot filtering as in the oracle unless
    the core takes the raw slot list."""
    def f(q_bits, cache_bits, sel_slot, sm_scale):
        B, H, _ = q_bits.shape
        out = np.zeros((B, H, 512))
        lse = np.full((B, H), -np.inf)
        C = cache_bits.shape[0]
        for b in range(B):
            sl = np.asarray(sel_slot[b], np.int64)
            sl = core.get('filter', lambda s: s[(s >= 0) & (s < C)])(sl)
            if len(sl) == 0:
                continue
            o, l = core['fn'](bf16_to_f64(q_bits[b]), bf16_to_f64(cache_bits[sl]), float(np.float32(sm_scale)))
            out[b], lse[b] = o, l
        return out, lse
    return f


def _softmax_core(s, v):
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    den = p.sum(axis=1, keepdims=True)
    return (p @ v) / den, (m + np.log(den))[:, 0]


ATTN_MUTANTS = {
    'no_scale': dict(fn=lambda q, r, sc: _softmax_core(q @ r.T, r[:, :512])),
    'value_is_rope_end': dict(fn=lambda q, r, sc: _softmax_core(q @ r.T * sc, r[:, 64:])),
    'key_without_rope': dict(fn=lambda q, r, sc: _softmax_core(q[:, :512] @ r[:, :512].T * sc, r[:, :512])),
    'softmax_over_heads': dict(fn=lambda q, r, sc: (
        (np.exp(q @ r.T * sc - (q @ r.T * sc).max(0)) / np.exp(q @ r.T * sc - (q @ r.T * sc).max(0)).sum(0)) @ r[:, :512],
        np.log(np.exp(q @ r.T * sc).sum(1)))),
    'lse_log2': dict(fn=lambda q, r, sc: (_softmax_core(q @ r.T * sc, r[:, :512])[0],
                                          _softmax_core(q @ r.T * sc, r[:, :512])[1] / np.log(2.0))),
    'unnormalised': dict(fn=lambda q, r, sc: (np.exp(q @ r.T * sc - (q @ r.T * sc).max(1, keepdims=True)) @ r[:, :512],
                                              _softmax_core(q @ r.T * sc, r[:, :512])[1])),
    'negative_slot_wraps': dict(filter=lambda s: s[s < 10 ** 9], fn=lambda q, r, sc: _softmax_core(q @ r.T * sc,
                                                                                               r[:, :512])),
    'last_slot_dropped': dict(filter=lambda s: s[(s >= 0) & (s < s.max())] if len(s) else s,
                              fn=lambda q, r, sc: _softmax_core(q @ r.T * sc, r[:, :512])),
}


def _attn_negative_slot_wraps(q_bits, cache_bits, sel_slot, sm_scale):
    # -1 indexes the last slot (numpy negative indexing) instead of selecting nothing
    return _attn_with(ATTN_MUTANTS['negative_slot_wraps'])(q_bits, cache_bits,
                                                           np.where(np.asarray(sel_slot) >= cache_bits.shape[0], -1,
                                                                    sel_slot), sm_scale)


@pytest.mark.parametrize('name', list(ATTN_MUTANTS))
def test_attention_mutants_are_caught(name):
    impl = (_attn_negative_slot_wraps if name == 'negative_slot_wraps' else _attn_with(ATTN_MUTANTS[name]))
    assert _fails(pins.ATTN_PINS, impl), name


def test_attention_unmutated_core_passes():
    for p in pins.ATTN_PINS:
        p(_attn_with(dict(fn=lambda q, r, sc: _softmax_core(q @ r.T * sc, r[:, :512]))))


# ------------------------------------------------------------------ append

def _append_mutant(kind):
    def f(host_pool, kcache, kscale, tok2slot, tok0, lens, cap, new_rows, new_keys, new_scales):
        full = False
        for b in range(len(lens)):
            if kind != 'ignores_cap' and lens[b] >= cap[b]:
                full = True
                continue
            if kind == 'ignores_cap' and lens[b] >= cap[b]:
                full = True
            g = int(tok0[b]) + int(lens[b]) - (1 if kind == 'off_by_one' else 0)
            if kind == 'ignores_cap' and g >= host_pool.shape[0]:
                continue
            host_pool[g] = new_rows[b]
            kcache[g] = new_keys[b]
            if kscale is not None:
                kscale[g if kind != 'scale_next' else min(g + 1, len(kscale) - 1)] = new_scales[b]
            if kind != 'keeps_slot':
                tok2slot[g] = -1
            if kind != 'no_grow':
                lens[b] += 1
        return full
    return f


@pytest.mark.parametrize('kind', ['off_by_one', 'ignores_cap', 'scale_next', 'keeps_slot', 'no_grow'])
def test_append_mutants_are_caught(kind):
    assert _fails(pins.APPEND_PINS, _append_mutant(kind)), kind


def test_append_unmutated_passes():
    for p in pins.APPEND_PINS:
        p(_append_mutant('none'))
