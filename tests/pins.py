"""Pins of the CPU oracle against facts other than itself.

Each ``pin_*`` takes the implementation under test and raises AssertionError
when it disagrees with a hand-worked fixture (tests/golden), a closed form, a
brute-force definition computed by a different algorithm, a library routine,
or an invariant. The oracle tests call them on the oracle; the mutation tests
call them on copies of the oracle with a plausible mistake planted, and expect
them to fail.
"""
import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), 'golden')


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def bf16_bits(x):
    import torch
    t = torch.tensor(np.asarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------------ indexer

def pin_indexer_hand(index_logits):
    g = golden('indexer_hand.json')
    q = bf16_bits(np.array(g['q'])[None])
    w = np.array([g['w']], dtype=np.float32)
    kb = bf16_bits(np.array(g['bf16_keys']))
    out = index_logits(q, w, kb, 'bf16', None, [0], [2])[0]
    np.testing.assert_array_equal(out, g['bf16_expected'])
    k8 = np.array(g['fp8_codes'], dtype=np.uint8)
    out = index_logits(q, w, k8, 'fp8', np.array(g['fp8_scale'], np.float32), [0], [2])[0]
    np.testing.assert_array_equal(out, g['fp8_expected'])
    k8n = np.array(g['neg_scale_codes'], dtype=np.uint8)
    out = index_logits(q, w, k8n, 'fp8', np.array(g['neg_scale'], np.float32), [0], [1])[0]
    np.testing.assert_array_equal(out, g['neg_scale_expected'])


def _rand_case(seed, R=2, H=8, D=16, P=40, kdtype='fp8'):
    import workloads as wk
    r = np.random.default_rng(seed)
    q = wk.to_bf16_bits(r.standard_normal((R, H, D)).astype(np.float32))
    w = (r.uniform(0, 1, (R, H)) / 8).astype(np.float32)
    if kdtype == 'fp8':
        kb = wk.to_e4m3_bits(r.standard_normal((P, D)).astype(np.float32))
        sc = r.uniform(0.5, 2.0, P).astype(np.float32)
    else:
        kb = wk.to_bf16_bits(r.standard_normal((P, D)).astype(np.float32))
        sc = None
    return q, w, kb, sc


def pin_indexer_basis(index_logits):
    """One-hot head weight and a basis query: the score of token t is
    ReLU(k[t, d] * s[t]) exactly (catches transposed operands, wrong dims,
    a dropped scale or ReLU)."""
    from oracle.numerics import e4m3fn_to_f64
    q, w, kb, sc = _rand_case(1, R=1, H=4, D=8, P=30)
    for h0, d0 in [(0, 0), (2, 5), (3, 7)]:
        w1 = np.zeros((1, 4), np.float32)
        w1[0, h0] = 1.0
        q1 = q.copy()
        q1[0, h0] = bf16_bits(np.eye(8)[d0])
        out = index_logits(q1, w1, kb, 'fp8', sc, [0], [30])[0]
        want = np.maximum(e4m3fn_to_f64(kb[:, d0]) * sc.astype(np.float64), 0.0)
        np.testing.assert_array_equal(out, want)


def pin_indexer_linear(index_logits):
    """ReLU(x) - ReLU(-x) = x, so score(q) - score(-q) = (w^T Q) . k_t, a
    linear form computed here by a different route (catches a missing or
    misplaced ReLU and wrong head weighting)."""
    from oracle.numerics import bf16_to_f64, e4m3fn_to_f64
    q, w, kb, sc = _rand_case(2, R=2, H=8, D=16, P=50)
    neg = q ^ np.uint16(0x8000)
    a = index_logits(q, w, kb, 'fp8', sc, [0, 10], [50, 40])
    b = index_logits(neg, w, kb, 'fp8', sc, [0, 10], [50, 40])
    K = e4m3fn_to_f64(kb) * sc.astype(np.float64)[:, None]
    for r, (t0, n) in enumerate([(0, 50), (10, 40)]):
        v = w[r].astype(np.float64) @ bf16_to_f64(q[r])       # [D]
        lin = K[t0:t0 + n] @ v
        np.testing.assert_allclose(a[r] - b[r], lin, rtol=1e-12, atol=1e-12)


def pin_indexer_scale(index_logits):
    """A positive per-token scale factors out of the score; token ranges
    (tok0, len) select the right keys (catches off-by-one segments)."""
    q, w, kb, sc = _rand_case(3, R=1, P=64)
    ones = np.ones_like(sc)
    a = index_logits(q, w, kb, 'fp8', sc, [0], [64])[0]
    b = index_logits(q, w, kb, 'fp8', ones, [0], [64])[0]
    np.testing.assert_allclose(a, b * sc.astype(np.float64), rtol=1e-13)
    c = index_logits(q, w, kb, 'fp8', sc, [17], [20])[0]
    np.testing.assert_array_equal(c, a[17:37])


def pin_indexer_permutation(index_logits):
    """Permuting heads (q rows with w) or dims (q columns with key columns)
    leaves every score unchanged up to summation order; permuting tokens
    permutes the scores."""
    q, w, kb, sc = _rand_case(4, R=1, H=8, D=16, P=32, kdtype='bf16')
    base = index_logits(q, w, kb, 'bf16', None, [0], [32])[0]
    ph = np.random.default_rng(5).permutation(8)
    pd = np.random.default_rng(6).permutation(16)
    pt = np.random.default_rng(7).permutation(32)
    h = index_logits(q[:, ph], w[:, ph], kb, 'bf16', None, [0], [32])[0]
    d = index_logits(q[:, :, pd], w, kb[:, pd], 'bf16', None, [0], [32])[0]
    t = index_logits(q, w, kb[pt], 'bf16', None, [0], [32])[0]
    np.testing.assert_allclose(h, base, rtol=1e-12)
    np.testing.assert_allclose(d, base, rtol=1e-12)
    np.testing.assert_allclose(t, base[pt], rtol=1e-12)


INDEXER_PINS = [pin_indexer_hand, pin_indexer_basis, pin_indexer_linear, pin_indexer_scale,
                pin_indexer_permutation]


# ------------------------------------------------------------------ top-k

def brute_topk(s, k):
    """Rank-count definition, O(n^2): t is selected iff fewer than k tokens
    beat it, where u beats t when s_u > s_t, or s_u == s_t and u < t."""
    s = np.asarray(s, dtype=np.float32).astype(np.float64)
    n = len(s)
    sel = []
    for t in range(n):
        beats = int(np.sum(s > s[t])) + int(np.sum(s[:t] == s[t]))
        if beats < k:
            sel.append(t)
    return np.array(sel, dtype=np.int64)


def pin_topk_bruteforce(topk_row):
    r = np.random.default_rng(11)
    for trial in range(60):
        n = int(r.integers(0, 40))
        k = int(r.integers(1, 12))
        kind = trial % 3
        if kind == 0:
            s = r.integers(0, 5, n).astype(np.float32)           # many ties
        elif kind == 1:
            s = r.standard_normal(n).astype(np.float32)
        else:
            s = np.where(r.random(n) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
        idx, kth = topk_row(s, k)
        want = brute_topk(s, k)
        m = min(k, n)
        np.testing.assert_array_equal(idx[:m], want)
        assert np.all(idx[m:] == -1)
        if m:
            assert kth == s[want].min()
        else:
            assert np.isnan(kth)


def pin_topk_special(topk_row):
    # all equal -> the first k indices
    idx, kth = topk_row(np.full(50, 2.5, np.float32), 7)
    np.testing.assert_array_equal(idx, np.arange(7))
    assert kth == np.float32(2.5)
    # n <= k -> everything, padded
    idx, kth = topk_row(np.array([3, 1, 2], np.float32), 5)
    np.testing.assert_array_equal(idx, [0, 1, 2, -1, -1])
    assert kth == np.float32(1)
    # distinct -> same set as numpy's argpartition (a library routine)
    s = np.random.default_rng(12).permutation(1000).astype(np.float32)
    idx, kth = topk_row(s, 100)
    want = np.sort(np.argpartition(-s, 99)[:100])
    np.testing.assert_array_equal(idx, want)
    assert kth == np.float32(900)
    # -0.0 and +0.0 are equal scores: lower index wins
    idx, _ = topk_row(np.array([-0.0, 0.0, -1.0], np.float32), 1)
    np.testing.assert_array_equal(idx, [0])
    idx, _ = topk_row(np.array([0.0, -0.0, -1.0], np.float32), 1)
    np.testing.assert_array_equal(idx, [0])


TOPK_PINS = [pin_topk_bruteforce, pin_topk_special]


def pin_theta(theta_next):
    g = golden('theta_trace.json')
    for seq in g['sequences']:
        th = np.float32(np.nan)
        for kth, want in zip(seq['kth'], seq['theta']):
            th = theta_next(th, np.float32(kth))
            assert th == np.float32(want), (seq, th)
    o = g['one_rounding']
    assert theta_next(np.float32(o['theta']), np.float32(o['kth'])) == np.float32(o['expected'])
    e = g['empty_row']
    assert theta_next(np.float32(e['theta']), np.float32(np.nan)) == np.float32(e['expected'])
    # constant k-th score: theta equals it from the first step on
    th = np.float32(np.nan)
    for _ in range(5):
        th = theta_next(th, np.float32(7.25))
        assert th == np.float32(7.25)
    # 0, 1, 1, 1, ... -> 1 - 2^-n (closed form of the alpha = 0.5 EMA)
    th = theta_next(np.float32(np.nan), np.float32(0.0))
    for n in range(1, 20):
        th = theta_next(th, np.float32(1.0))
        assert th == np.float32(1.0 - 2.0 ** -n)


# ------------------------------------------------------------------ slot map

def pin_slotmap_trace(SlotMap):
    g = golden('slotmap_trace.json')
    sm = SlotMap(g['P'], g['C'])
    for st in g['steps']:
        idx = np.array([st['selected']], dtype=np.int64)
        assigned, sel, stats = sm.final([0], idx)
        assert [list(a) for a in assigned] == st['assigned'], (st, assigned)
        assert sm.head == st['head']
        np.testing.assert_array_equal(sm.slot2tok, st['slot2tok'])
        np.testing.assert_array_equal(sel[0], st['sel_slot'])
        np.testing.assert_array_equal(stats[0], st['stats'])
    np.testing.assert_array_equal(sm.tok2slot, g['final_tok2slot'])


def pin_slotmap_early(SlotMap):
    g = golden('early_hand.json')
    for case in g['cases']:
        sm = SlotMap(g['P'], case['C'])
        sm.final([0], np.array([g['setup_final_selected']], np.int64))
        scores = np.array(g['scores'], np.float32)
        assigned, stats = sm.early([0], [scores], np.array([g['theta']], np.float32), g['cap'])
        assert [list(a) for a in assigned] == case['assigned'], (case, assigned)
        assert sm.head == case['head']
        np.testing.assert_array_equal(stats[0], case['stats'])
        if 'then_final' in case:
            tf = case['then_final']
            assigned, sel, stats = sm.final([0], np.array([tf['selected']], np.int64))
            assert [list(a) for a in assigned] == tf['assigned']
            assert sm.head == tf['head']
            np.testing.assert_array_equal(sel[0], tf['sel_slot'])
            np.testing.assert_array_equal(stats[0], tf['stats'])
    # NaN theta: no early fetch at all
    sm = SlotMap(8, 4)
    assigned, stats = sm.early([0], [np.arange(8, dtype=np.float32)], np.array([np.nan], np.float32), 4)
    assert assigned == [] and not stats.any()


def _random_selections(r, n, k, steps, keep=0.7):
    sels = []
    cur = np.sort(r.choice(n, k, replace=False))
    for _ in range(steps):
        sels.append(cur)
        stay = cur[r.random(len(cur)) < keep]
        new = r.choice(np.setdiff1d(np.arange(n), stay), k - len(stay), replace=False)
        cur = np.sort(np.concatenate([stay, new]))
    return sels


def pin_slotmap_large_cache(SlotMap):
    """C >= P: nothing is ever evicted and the misses of a step are exactly
    the selected tokens never selected before (first-touch set algebra)."""
    r = np.random.default_rng(21)
    sm = SlotMap(60, 60)
    seen = set()
    for S in _random_selections(r, 60, 9, 12):
        assigned, _, stats = sm.final([0], S[None])
        want = sorted(set(S.tolist()) - seen)
        assert [a[0] for a in assigned] == want
        assert stats[0, 3] == 0
        seen |= set(S.tolist())


def pin_slotmap_exact_cache(SlotMap):
    """C = k, one sequence, no early fetch: after each step the resident set
    is exactly the selection."""
    r = np.random.default_rng(22)
    sm = SlotMap(80, 10)
    for S in _random_selections(r, 80, 10, 15, keep=0.5):
        sm.final([0], S[None])
        assert set(sm.slot2tok.tolist()) == set(S.tolist())


def pin_slotmap_fifo(SlotMap):
    """Selections disjoint from everything resident pin nothing, so slots are
    reused in ring order: evictions follow first-in first-out order (checked
    against a deque model)."""
    from collections import deque
    sm = SlotMap(200, 7)
    q = deque()
    r = np.random.default_rng(23)
    perm = r.permutation(200)
    pos = 0
    for step in range(20):
        m = int(r.integers(1, 6))
        S = np.sort(perm[pos:pos + m])
        pos += m
        evicted_model = []
        for g in S.tolist():
            if len(q) == 7:
                evicted_model.append(q.popleft())
            q.append(g)
        before = set(sm.slot2tok.tolist())
        sm.final([0], S[None])
        after = set(sm.slot2tok.tolist())
        evicted = sorted((before - after) - {-1})
        assert evicted == sorted(evicted_model), (step, evicted, evicted_model)
        assert after - {-1} == set(q)


def pin_slotmap_prefill_first_touch(SlotMap):
    """Prefill with C = N: slot of token g = its first-touch rank (blocks in
    order, ascending tokens within a block)."""
    r = np.random.default_rng(24)
    N = 50
    sm = SlotMap(N, N)
    order = []
    for blk in range(4):
        idx = np.full((3, 6), -1, np.int64)
        for row in range(3):
            c = np.sort(r.choice(N, int(r.integers(1, 7)), replace=False))
            idx[row, :len(c)] = c
        for g in np.unique(idx[idx >= 0]).tolist():
            if g not in order:
                order.append(g)
        sm.prefill_block(0, idx)
    for rank, g in enumerate(order):
        assert sm.tok2slot[g] == rank


def check_invariants(sm, selected_global, pinned_before=None):
    """Invariants the pages fix: every selected token is resident after a
    FINAL phase; tok2slot and slot2tok are inverse maps; at most C tokens are
    resident."""
    occ = np.nonzero(sm.slot2tok >= 0)[0]
    assert np.all(sm.tok2slot[sm.slot2tok[occ]] == occ)
    res_tok = np.nonzero(sm.tok2slot >= 0)[0]
    assert np.all(sm.slot2tok[sm.tok2slot[res_tok]] == res_tok)
    assert len(res_tok) == len(occ) <= sm.C
    assert np.all(sm.tok2slot[np.asarray(selected_global, dtype=np.int64)] >= 0)
    if pinned_before is not None:
        for s, t in pinned_before.items():
            assert sm.slot2tok[s] == t


def pin_slotmap_invariants(SlotMap):
    """Random multi-sequence runs with early fetch: invariants hold, pinned
    slots keep their tokens, and recalled rows match the host pool (no
    write-back: the pool is never modified)."""
    from oracle.slotmap import recall_rows
    r = np.random.default_rng(25)
    B, n, k, C = 3, 40, 6, 24
    P = B * n
    tok0 = [b * n for b in range(B)]
    sm = SlotMap(P, C)
    pool = r.integers(0, 1 << 16, size=(P, 4), dtype=np.uint16)
    pool0 = pool.copy()
    cache = np.zeros((C, 4), np.uint16)
    theta = np.full(B, np.nan, np.float32)
    for step in range(10):
        scores = [r.standard_normal(n).astype(np.float32) for _ in range(B)]
        a, _ = sm.early(tok0, scores, theta, cap=3)
        recall_rows(pool, cache, a)
        idx = np.stack([np.sort(np.argsort(-s, kind='stable')[:k]) for s in scores])
        pinned_before = {int(sm.tok2slot[tok0[b] + t]): int(tok0[b] + t)
                         for b in range(B) for t in idx[b] if sm.tok2slot[tok0[b] + t] >= 0}
        a, sel, _ = sm.final(tok0, idx)
        recall_rows(pool, cache, a)
        gsel = np.concatenate([tok0[b] + idx[b] for b in range(B)])
        check_invariants(sm, gsel, pinned_before)
        np.testing.assert_array_equal(sel, sm.tok2slot[np.array(tok0)[:, None] + idx])
        occ = np.nonzero(sm.slot2tok >= 0)[0]
        np.testing.assert_array_equal(cache[occ], pool[sm.slot2tok[occ]])
        theta = np.array([np.sort(s)[-k] for s in scores], np.float32)
    np.testing.assert_array_equal(pool, pool0)


SLOTMAP_PINS = [pin_slotmap_trace, pin_slotmap_early, pin_slotmap_large_cache, pin_slotmap_exact_cache,
                pin_slotmap_fifo, pin_slotmap_prefill_first_touch, pin_slotmap_invariants]


# ------------------------------------------------------------------ sparse attention

def _attn_case(seed, B=2, H=4, C=50, k=12, pad=3):
    import workloads as wk
    r = np.random.default_rng(seed)
    q = wk.to_bf16_bits(r.standard_normal((B, H, 576)).astype(np.float32))
    cache = wk.to_bf16_bits(r.standard_normal((C, 576)).astype(np.float32))
    sel = np.stack([r.choice(C, k, replace=False) for _ in range(B)]).astype(np.int32)
    sel[:, k - pad:] = -1                       # padding at the end (short sequences)
    sel[0, 1] = C + 7                           # out of range: selects nothing
    return q, cache, sel


def pin_attn_library(sparse_attention):
    """Against torch's scaled_dot_product_attention in float64 on the CPU,
    over the valid slots gathered by hand (keys = the 576-value rows, values
    = their first 512), and torch.logsumexp for the denominator."""
    import torch
    from oracle.numerics import bf16_to_f64
    for seed in range(3):
        q, cache, sel = _attn_case(seed)
        scale = 0.0721
        out, lse = sparse_attention(q, cache, sel, scale)
        for b in range(q.shape[0]):
            ok = [s for s in sel[b] if 0 <= s < cache.shape[0]]
            rows = torch.from_numpy(bf16_to_f64(cache[ok]))
            qq = torch.from_numpy(bf16_to_f64(q[b]))
            sc = float(np.float32(scale))
            ref = torch.nn.functional.scaled_dot_product_attention(qq[None], rows[None], rows[None, :, :512],
                                                                   scale=sc)[0]
            np.testing.assert_allclose(out[b], ref.numpy(), rtol=1e-10, atol=1e-12)
            np.testing.assert_allclose(lse[b], torch.logsumexp(qq @ rows.T * sc, dim=1).numpy(), rtol=1e-12)


def pin_attn_closed_forms(sparse_attention):
    r = np.random.default_rng(7)
    import workloads as wk
    from oracle.numerics import bf16_to_f64
    C = 9
    cache = wk.to_bf16_bits(r.standard_normal((C, 576)).astype(np.float32))
    q = wk.to_bf16_bits(r.standard_normal((1, 3, 576)).astype(np.float32))
    row = bf16_to_f64(cache)
    # every selected slot holds the same row: the weights sum to one
    same = cache.copy()
    same[:] = cache[4]
    out, lse = sparse_attention(q, same, np.array([[0, 2, 5, -1, 8]]), 0.05)
    np.testing.assert_allclose(out[0], np.broadcast_to(row[4, :512], (3, 512)), rtol=1e-13, atol=1e-14)
    s = bf16_to_f64(q[0]) @ row[4] * float(np.float32(0.05))
    np.testing.assert_allclose(lse[0], s + np.log(4.0), rtol=1e-12)
    # a zero query weighs every selected row equally
    out, lse = sparse_attention(np.zeros_like(q), cache, np.array([[1, 3, 6]]), 0.3)
    np.testing.assert_allclose(out[0], np.broadcast_to(row[[1, 3, 6], :512].mean(0), (3, 512)), rtol=1e-12,
                               atol=1e-14)
    np.testing.assert_allclose(lse[0], np.log(3.0), rtol=1e-14)
    # one valid slot: its value row, unchanged
    out, lse = sparse_attention(q, cache, np.array([[-1, 7, C, -5]]), 1.0)
    np.testing.assert_array_equal(out[0], np.broadcast_to(row[7, :512], (3, 512)))
    np.testing.assert_allclose(lse[0], bf16_to_f64(q[0]) @ row[7], rtol=1e-12)
    # nothing selected
    out, lse = sparse_attention(q, cache, np.array([[-1, -1, C]]), 1.0)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def pin_attn_bruteforce(sparse_attention):
    """Pure-Python loops with math.exp, one head and token at a time."""
    import math
    from oracle.numerics import bf16_to_f64
    q, cache, sel = _attn_case(11, B=1, H=2, C=10, k=5, pad=1)
    scale = 0.11
    out, lse = sparse_attention(q, cache, sel, scale)
    sc = float(np.float32(scale))
    rows = bf16_to_f64(cache)
    qq = bf16_to_f64(q[0])
    for h in range(2):
        sc_list = []
        for s in sel[0]:
            if 0 <= s < 10:
                sc_list.append((sum(qq[h, d] * rows[s, d] for d in range(576)) * sc, s))
        mx = max(v for v, _ in sc_list)
        den = sum(math.exp(v - mx) for v, _ in sc_list)
        for c in (0, 1, 255, 511):
            num = sum(math.exp(v - mx) * rows[s, c] for v, s in sc_list)
            assert abs(out[0, h, c] - num / den) <= 1e-12 * max(1.0, abs(num / den))
        assert abs(lse[0, h] - (mx + math.log(den))) <= 1e-12 * abs(mx + math.log(den))


def pin_attn_permutation(sparse_attention):
    q, cache, sel = _attn_case(5, B=1, k=20, pad=0)
    out, lse = sparse_attention(q, cache, sel, 0.07)
    perm = np.random.default_rng(1).permutation(20)
    out2, lse2 = sparse_attention(q, cache, sel[:, perm], 0.07)
    np.testing.assert_allclose(out2, out, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, rtol=1e-13)


ATTN_PINS = [pin_attn_library, pin_attn_closed_forms, pin_attn_bruteforce, pin_attn_permutation]


# ------------------------------------------------------------------ append

def pin_append_hand(kv_append):
    """Two sequences laid out [0, 4) and [4, 7) (capacities 4 and 3), worked
    by hand: sequence 0 (length 2) gets token 2, sequence 1 (length 3) is
    full."""
    pool = np.zeros((7, 2), np.int16)
    keys = np.zeros((7, 3), np.uint8)
    scale = np.zeros(7, np.float32)
    t2s = np.array([5, 1, 9, -1, 0, 2, 3], np.int32)
    lens = np.array([2, 3], np.int32)
    full = kv_append(pool, keys, scale, t2s, np.array([0, 4]), lens, np.array([4, 3]),
                     np.array([[11, 12], [21, 22]], np.int16), np.array([[1, 2, 3], [4, 5, 6]], np.uint8),
                     np.array([0.5, 2.0], np.float32))
    assert full
    np.testing.assert_array_equal(lens, [3, 3])
    np.testing.assert_array_equal(pool, [[0, 0], [0, 0], [11, 12], [0, 0], [0, 0], [0, 0], [0, 0]])
    np.testing.assert_array_equal(keys[2], [1, 2, 3])
    assert keys[[0, 1, 3, 4, 5, 6]].sum() == 0
    np.testing.assert_array_equal(scale, [0, 0, 0.5, 0, 0, 0, 0])
    np.testing.assert_array_equal(t2s, [5, 1, -1, -1, 0, 2, 3])
    # bf16 keys carry no scale; appending again fills the last free id of sequence 0
    full = kv_append(pool, keys, None, t2s, np.array([0, 4]), lens, np.array([4, 3]),
                     np.array([[31, 32], [41, 42]], np.int16), np.array([[7, 8, 9], [1, 1, 1]], np.uint8), None)
    assert full
    np.testing.assert_array_equal(lens, [4, 3])
    np.testing.assert_array_equal(pool[3], [31, 32])
    np.testing.assert_array_equal(keys[3], [7, 8, 9])


def pin_append_invariants(kv_append):
    """Random layouts: only the ids tok0 + old length change, each to its
    sequence's new row; nothing is written for full sequences."""
    r = np.random.default_rng(3)
    for _ in range(20):
        B = int(r.integers(1, 6))
        cap = r.integers(1, 6, B)
        tok0 = np.concatenate([[0], np.cumsum(cap)[:-1]])
        P = int(cap.sum())
        lens = np.array([int(r.integers(0, c + 1)) for c in cap], np.int32)
        pool = r.integers(-100, 100, (P, 3)).astype(np.int16)
        keys = r.integers(0, 255, (P, 2)).astype(np.uint8)
        t2s = r.integers(-1, 9, P).astype(np.int32)
        rows = r.integers(-100, 100, (B, 3)).astype(np.int16)
        nk = r.integers(0, 255, (B, 2)).astype(np.uint8)
        p0, k0, t0, l0 = pool.copy(), keys.copy(), t2s.copy(), lens.copy()
        full = kv_append(pool, keys, None, t2s, tok0, lens, cap, rows, nk, None)
        assert full == bool((l0 >= cap).any())
        changed = set()
        for b in range(B):
            if l0[b] < cap[b]:
                g = tok0[b] + l0[b]
                changed.add(int(g))
                assert lens[b] == l0[b] + 1
                np.testing.assert_array_equal(pool[g], rows[b])
                np.testing.assert_array_equal(keys[g], nk[b])
                assert t2s[g] == -1
            else:
                assert lens[b] == l0[b]
        rest = [i for i in range(P) if i not in changed]
        np.testing.assert_array_equal(pool[rest], p0[rest])
        np.testing.assert_array_equal(keys[rest], k0[rest])
        np.testing.assert_array_equal(t2s[rest], t0[rest])


APPEND_PINS = [pin_append_hand, pin_append_invariants]
