#!/usr/bin/env python3
"""Benchmark of one layer of the indexer -> exact top-k -> KV-recall path on
one MI355X.

Default workload: decode, 32 sequences x 131072 tokens, fp8 indexer keys
(64 heads x 128) with per-token scales, k = 2048, early-fetch cap 512, device
cache 260000 slots, host pool of 4.19M rows x 1152 B in pinned memory, q from
an AR(1) process (rho 0.9). A step is one full pass of the path for the
batch: indexer scores, exact top-k + threshold update, early fetch (second
stream), final slot-map step and recall. Inputs are resident in HBM (and the
pinned pool) before the timed region; F fill steps (from the cold device
cache: the first step misses every selected row, and the resident set takes
about ten steps to settle) and W warm-up steps are untimed, then exactly K
steps are timed between two device synchronisations.

Prints one JSON line (stdout). Progress goes to stderr.

  python bench.py [--steps K] [--warmup W] [--fill F] [--config NAME] [--no-cpu-baseline]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0           # MI355X HBM3E, vendor figure
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA, vendor figure


def log(*a):
    print('[bench]', *a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument('--gpus', type=int, default=1)
    p.add_argument('--steps', type=int, default=30)
    p.add_argument('--warmup', type=int, default=2)
    p.add_argument('--fill', type=int, default=8,
                   help='decode: untimed steps before the warm-up ones, from the cold device cache until the '
                        'resident set has converged (the steady state of a serving layer)')
    p.add_argument('--config', default='decode-32x128k-fp8')
    p.add_argument('--no-cpu-baseline', action='store_true')
    p.add_argument('--no-early', action='store_true', help='disable the early fetch (ablation)')
    p.add_argument('--eager', action='store_true', help='time eager launches instead of graph replays')
    p.add_argument('--topk-after-early', action='store_true', help='start the top-k after the EARLY maps')
    p.add_argument('--no-fused', action='store_true',
                   help='decode: the plain scores kernel, then the EARLY phase on a second stream (ablation of the '
                        'fused scores + early-fetch launch)')
    p.add_argument('--prefill-serial', action='store_true',
                   help='prefill: one score buffer, top-k after each block on the same stream (ablation)')
    p.add_argument('--cpu-seqs', type=int, default=32, help='sequences in the oracle sample')
    p.add_argument('--cpu-steps', type=int, default=5, help='decode steps in the oracle sample')
    p.add_argument('--topk-first', choices=['auto', 'on', 'off'], default='auto',
                   help='decode: launch the top-k before the EARLY maps (auto: batches of at most 8 sequences)')
    p.add_argument('--layers', type=int, default=1,
                   help='decode: layers per step, each with its own keys, slot maps, cache and host pool')
    p.add_argument('--micro-batches', type=int, default=1,
                   help='decode with --layers: micro-batches, interleaved so one recalls while another scores')
    p.add_argument('--calibrate-copy', action='store_true',
                   help='only run a plain 1 GiB device copy 5 times (reference for HBM byte counters)')
    return p.parse_args()


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, 'indexer_top_kv_amd', 'csrc', n), 'rb') as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key, src_hash, field='bytes_per_launch'):
    """HBM bytes per launch (or per pass) from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, 'profiles', 'hbm_traffic.json')
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    e = d.get(kernel_key)
    if not e or e.get('source_hash') != src_hash:
        return None
    return e.get(field)


def cpu_cores():
    try:
        from threadpoolctl import threadpool_info
        n = max([i.get('num_threads', 1) for i in threadpool_info()] or [1])
    except Exception:
        n = 1
    return int(n)


# ---------------------------------------------------------------------------- decode
def bench_decode(args, wl):
    import numpy as np
    import torch
    import workloads as wk
    from indexer_top_kv_amd.pipeline import DecodeLayer

    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x.view(np.int16) if x.dtype == np.uint16 else x)).cuda()
    t = time.time()
    keys, scale = wk.keys(wl)
    w = wk.head_weights(wl)
    log(f'keys {keys.shape} generated in {time.time() - t:.1f}s')
    t = time.time()
    pool = torch.empty((wl.P, wk.ROW_ELEMS), dtype=torch.int16, pin_memory=True)
    wk.host_rows(wl, out=pool.numpy().view(np.uint16))
    log(f'host pool {wl.P} rows x {wk.ROW_BYTES} B pinned in {time.time() - t:.1f}s')
    n_stage = 4                                       # extra eager steps for the stage breakdown
    pre = args.fill + args.warmup                # untimed steps before the timed ones
    total_steps = pre + args.steps + n_stage
    qs = np.stack(list(wk.decode_queries(wl, total_steps)))
    kc, ks, wd = dev(keys), (dev(scale) if scale is not None else None), dev(w)
    qd = dev(qs)
    layer = DecodeLayer(kc, ks, wd, wl.tok0, wl.lens, wl.C, k=wl.k, cap=wl.cap, host_pool=pool,
                        early=not args.no_early, topk_after_early=args.topk_after_early,
                        topk_first={'auto': None, 'on': True, 'off': False}[args.topk_first],
                        fused=False if (args.no_fused or args.no_early) else None)
    torch.cuda.synchronize()
    log(f'chunks {layer.chunks}; {args.fill} fill + {args.warmup} warm-up steps')
    if not args.eager:
        layer.capture()          # nothing runs; the warm-up steps are replays of the timed path
        torch.cuda.synchronize()
    for s in range(pre):
        if args.eager:
            layer.step(qd[s])
        else:
            layer.replay(qd[s])
    torch.cuda.synchronize()
    recalled0 = int(layer.state.ctr[4].item())
    log(f'timing {args.steps} steps ({"eager launches" if args.eager else "hipGraph replay per step"})')
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        if args.eager:
            layer.step(qd[pre + s])
        else:
            layer.replay(qd[pre + s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    recalled = int(layer.state.ctr[4].item()) - recalled0
    stats_final = layer.stats_final.cpu().numpy()
    stats_early = layer.stats_early.cpu().numpy()

    s0 = torch.cuda.current_stream()
    # The plain scores kernel, timed with HIP events on its launch stream: K
    # launches back to back (the step's queries) between one pair of events,
    # so no event sits between launches; the average launch is the span / K.
    # Without the fused path this is the roofline kernel; with it, the same
    # stream alone, for comparison with the fused launch inside the step.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    layer.logits_only(qd[pre], stream=s0)
    ev0.record(s0)
    for s in range(args.steps):
        layer.logits_only(qd[pre + s], stream=s0)
    ev1.record(s0)
    torch.cuda.synchronize()
    logits_runs = [ev0.elapsed_time(ev1) / args.steps]

    # The top-k alone: K calls back to back on the last step's scores with its
    # prediction, into scratch outputs (the layer's state is left as it is).
    # With the fused path the step's top-k selects from the band lists the
    # last scores launch wrote with the theta it took (theta[1 - parity] once
    # the step is over).
    import indexer_top_kv_amd as ech_m
    th_a = layer.theta[1 - layer.parity if layer.fused else layer.parity].clone()
    th_b, idx_b = torch.empty_like(th_a), torch.empty_like(layer.idx)
    kth_b, ws_b = torch.empty_like(layer.kth), torch.zeros_like(layer.ws_topk)
    if layer.fused:
        topk_call = lambda: ech_m.ech_topk_early(layer.logits, layer.lens, layer.max_len, layer.k, th_a, th_b, idx_b,
                                                 kth_b, layer.state, layer.ws_fused, stream=s0)
    else:
        topk_call = lambda: ech_m.ech_topk(layer.logits, layer.lens, layer.max_len, layer.k, th_a, th_b, idx_b,
                                           kth_b, ws_b, stream=s0)
    topk_call()
    ev0.record(s0)
    for s in range(args.steps):
        topk_call()
    ev1.record(s0)
    torch.cuda.synchronize()
    topk_alone_us = ev0.elapsed_time(ev1) / args.steps * 1e3

    # Stage breakdown from eager steps with events on each stage's stream.
    # With the fused launch these also time the roofline launch inside the
    # step (beside the live copier), on its own stream.
    marks = {}
    for s in range(n_stage):
        layer.step(qd[pre + args.steps + s], marks)
    torch.cuda.synchronize()

    def avg_ms(name):
        """Time per step of a stage (summed over the chunks of a step)."""
        ev = marks.get(name, [])
        if not ev:
            return None
        d = [ev[i].elapsed_time(ev[i + 1]) for i in range(0, len(ev), 2)]
        return float(np.sum(d)) / n_stage

    # The consumer of sel_slot: sparse attention (128 heads, 576-value rows)
    # over the step's selections in the device cache, K launches between one
    # pair of events.
    import indexer_top_kv_amd as ech
    Ha = 128
    qa = torch.randn((wl.B, Ha, 576), device='cuda').to(torch.bfloat16).view(torch.int16)
    out_a = torch.empty((wl.B, Ha, 512), dtype=torch.float32, device='cuda')
    lse_a = torch.empty((wl.B, Ha), dtype=torch.float32, device='cuda')
    # a chunk of fewer sequences splits each into more spans: size for the largest need
    ws_a = torch.empty(max(ech.ech_sparse_attn_ws_bytes(b1 - b0, Ha, wl.k) for b0, b1 in [(0, wl.B)] + layer.chunks),
                       dtype=torch.uint8, device='cuda')
    sm = 1.0 / float(np.sqrt(192.0))
    if len(layer.chunks) == 1:
        ech.ech_sparse_attn(qa, layer.dev_cache, layer.sel_slot, sm, out_a, lse_a, ws_a)
        ea0, ea1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ea0.record(s0)
        for _ in range(args.steps):
            ech.ech_sparse_attn(qa, layer.dev_cache, layer.sel_slot, sm, out_a, lse_a, ws_a)
        ea1.record(s0)
        torch.cuda.synchronize()
        attn_us = ea0.elapsed_time(ea1) / args.steps * 1e3
        n_sel = int((layer.sel_slot >= 0).sum().item())
        attn_note = 'the consumer of sel_slot, after the timed steps; not part of the step time'
    else:
        # Several chunks: a later chunk may evict an earlier chunk's tokens, so
        # each chunk's attention runs inside the step, right after that
        # chunk's FINAL recall (on_chunk), timed with events around it.
        att_ev, n_sel_c = [], []

        def consume(b0, b1, stream):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            ech.ech_sparse_attn(qa[b0:b1], layer.dev_cache, layer.sel_slot[b0:b1], sm, out_a[b0:b1],
                                lse_a[b0:b1], ws_a, stream=stream)
            e1.record(stream)
            att_ev.append((e0, e1))
            n_sel_c.append((layer.sel_slot[b0:b1] >= 0).sum())

        n_att = 2
        for s in range(n_att):
            layer.step(qd[pre + args.steps + s], on_chunk=consume)
        torch.cuda.synchronize()
        attn_us = sum(a.elapsed_time(b) for a, b in att_ev) / n_att * 1e3
        n_sel = int(sum(int(x.item()) for x in n_sel_c) / n_att)
        attn_note = ('the consumer of sel_slot, per sequence chunk right after its FINAL recall (a later chunk '
                     'may evict an earlier chunk\'s tokens), in eager steps after the timed ones; not part of '
                     'the step time')

    # Growing contexts: ech_kv_append of one decoded token per sequence, on a
    # scratch layout of the same batch (B sequences with room for K tokens)
    # so the layer's own data stays as the steps left it.
    Ka = args.steps
    Ps = wl.B * (Ka + 1)
    pool_s = torch.empty((Ps, 576), dtype=torch.int16, pin_memory=True)
    kc_s = torch.zeros((Ps, 128), dtype=torch.uint8, device='cuda')
    ks_s = torch.zeros(Ps, dtype=torch.float32, device='cuda')
    st_s = ech.LayerState.allocate(Ps, 16, 16)
    ech.ech_cache_reset(st_s)
    t0_s = torch.arange(wl.B, dtype=torch.int64, device='cuda') * (Ka + 1)
    len_s = torch.zeros(wl.B, dtype=torch.int32, device='cuda')
    cap_s = torch.full((wl.B,), Ka + 1, dtype=torch.int32, device='cuda')
    rows_s = torch.zeros((wl.B, 576), dtype=torch.int16, device='cuda')
    keys_s = torch.zeros((wl.B, 128), dtype=torch.uint8, device='cuda')
    sc_s = torch.ones(wl.B, dtype=torch.float32, device='cuda')
    ech.ech_kv_append(pool_s, kc_s, ks_s, st_s, t0_s, len_s, cap_s, rows_s, keys_s, sc_s)
    eb0, eb1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    eb0.record(s0)
    for _ in range(Ka - 1):
        ech.ech_kv_append(pool_s, kc_s, ks_s, st_s, t0_s, len_s, cap_s, rows_s, keys_s, sc_s)
    eb1.record(s0)
    torch.cuda.synchronize()
    append_us = eb0.elapsed_time(eb1) / max(Ka - 1, 1) * 1e3
    assert int(len_s.min().item()) == Ka and int(st_s.ctr[5].item()) == 0

    wall = t1 - t0
    tokens = int(wl.lens.astype(np.int64).sum())
    value = tokens * args.steps / wall
    plain_ms = float(np.mean(logits_runs))
    logits_ms = avg_ms('logits') if layer.fused else plain_ms
    kbytes = 128 + 4 if wl.kdtype == 'fp8' else 256
    per_token = kbytes + 4                                   # key (+scale) read, score written
    per_launch = tokens * per_token + wl.B * (64 * 128 * 2 + 64 * 4)
    achieved = per_launch / (logits_ms * 1e-3) / 1e9
    flops = tokens * 2 * 64 * 128
    src = source_hash('fused.hip', 'decode.hpp', 'score.hpp', 'bins.hpp') if layer.fused else \
        source_hash('logits.hip', 'decode.hpp', 'score.hpp')
    traffic = measured_traffic(('fused_' if layer.fused else 'logits_decode_') + wl.name, src)
    out = {
        'metric': 'decode tokens scored/s (indexer logits + exact top-k + early/final slot-map step + recall), '
                  '1 layer',
        'value': value,
        'unit': 'tokens/s',
        'n_gpus': 1,
        'steps': args.steps,
        'warmup': args.warmup,
        'fill_steps': args.fill,
        'ms_per_step': wall / args.steps * 1e3,
        'higher_is_better': True,
        'scaling': 'weak',
        'vs_baseline': None,
        'dtype': 'fp8-e4m3 keys, bf16 q, bf16 MFMA with fp32 accumulation',
        'data': 'synthetic, seeded',
        'config': {'workload': wl.name, 'B': wl.B, 'context': wl.N, 'k': wl.k, 'heads': 64, 'head_dim': 128,
                   'key_dtype': wl.kdtype, 'cache_slots': wl.C, 'early_fetch_cap': wl.cap,
                   'early_fetch': not args.no_early, 'fused_scores_early_fetch': layer.fused, 'row_bytes': 1152,
                   'launch': 'eager' if args.eager else 'hipGraph replay per step',
                   'topk_first': layer.topk_first},
        'roofline': {'bound': 'hbm',
                     'kernel': ('ech_index_logits_early (fused_pins_kernel + fused_kernel: scores, pins, EARLY '
                                'allocation), inside the step beside the live copier') if layer.fused else
                     ('logits_decode_fp8_kernel' if wl.kdtype == 'fp8' else 'logits_decode_kernel'),
                     'achieved': achieved,
                     'peak': PEAK_HBM_GBS, 'unit': 'GB/s', 'frac': achieved / PEAK_HBM_GBS,
                     'traffic': traffic, 'algorithmic_bytes_per_launch': per_launch,
                     'avg_launch_us': logits_ms * 1e3,
                     'timing': ('HIP events on the scores stream around the fused launch in eager steps '
                                '(the PCIe copier runs beside it on the other stream)'
                                if layer.fused else 'HIP events around K back-to-back launches on its stream'),
                     'mfma_bf16_frac': flops / (logits_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                     'plain_scores_kernel_alone': {
                         'kernel': 'logits_decode_fp8_kernel' if wl.kdtype == 'fp8' else 'logits_decode_kernel',
                         'avg_launch_us': plain_ms * 1e3,
                         'achieved': per_launch / (plain_ms * 1e-3) / 1e9,
                         'frac': per_launch / (plain_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         'traffic': measured_traffic('logits_decode_' + wl.name,
                                                     source_hash('logits.hip', 'decode.hpp', 'score.hpp')),
                         'timing': 'HIP events around K back-to-back launches on its stream'}},
        'stages_us_eager': {k: (avg_ms(k) or 0.0) * 1e3
                            for k in ('logits', 'recall_live', 'topk', 'early', 'early_maps', 'recall_early',
                                      'final', 'final_maps', 'recall_final')},
        'recall': {'rows_per_step': recalled / args.steps, 'bytes_per_step': recalled * 1152 / args.steps},
        'last_step': {'final_hits': int(stats_final[:, 0].sum()), 'final_misses': int(stats_final[:, 1].sum()),
                      'early_fetched': int(stats_early[:, 1].sum()), 'evictions':
                      int(stats_final[:, 3].sum() + stats_early[:, 3].sum())},
        'logits_source': src,
    }
    st = out['stages_us_eager']
    topk_bytes = tokens * 4 + wl.B * wl.k * 4
    rec_us = st['recall_live'] + st['recall_early'] + st['recall_final']
    one_pass = wl.B <= 256 and layer.max_len > 16384
    if layer.fused:
        topk_stage = {'kernel': 'ech_topk_early (topk_lists_kernel: the selection from the band lists the scores '
                                'launch wrote as it scored)',
                      'bound': 'latency', 'us': st['topk'], 'alone_us': topk_alone_us,
                      'traffic': measured_traffic('topk_lists_' + wl.name, source_hash('topk.hip', 'bins.hpp')),
                      'note': 'one workgroup per row reads its band lists (a few thousand entries) and writes its k '
                              'indices; the scores are not read again (rows the lists cannot decide take one pass '
                              'over the row). us: in eager steps, alone_us: K calls back to back'}
    out['stage_rooflines'] = {
        'topk': topk_stage if layer.fused else {'bound': 'hbm', 'algorithmic_bytes': topk_bytes, 'us': st['topk'],
                 'achieved_GBs': topk_bytes / (st['topk'] * 1e-6) / 1e9 if st['topk'] else None,
                 'peak_GBs': PEAK_HBM_GBS,
                 'frac': topk_bytes / (st['topk'] * 1e-6) / 1e9 / PEAK_HBM_GBS if st['topk'] else None,
                 'alone_us': topk_alone_us,
                 'alone_frac': topk_bytes / (topk_alone_us * 1e-6) / 1e9 / PEAK_HBM_GBS,
                 'traffic': (measured_traffic('topk_one_' + wl.name, source_hash('topk.hip', 'bins.hpp'))
                             if one_pass else None),
                 'note': ('one read of the scores plus the index output; us: in eager steps, alone_us: K calls '
                          'back to back; ' + ('one pass (a reset and the pass kernel)' if one_pass else
                                              'one launch (rows of at most 16384 tokens)'))},
        'recall': {'bound': 'pcie', 'bytes_per_step': out['recall']['bytes_per_step'], 'us': rec_us,
                   'achieved_GBs': out['recall']['bytes_per_step'] / (rec_us * 1e-6) / 1e9 if rec_us else None,
                   'note': ('the recall kernels of eager steps: the live copier (early rows beside the scoring, '
                            'then the FINAL rows) and the rest of both lists (ech_recall_rest); denominator: '
                            'pcie.h2d_memcpy_GBs' if layer.fused else
                            'the recall kernels of eager steps (EARLY, FINAL); denominator: pcie.h2d_memcpy_GBs')},
        'attention': {'kernel': 'ech_sparse_attn (span + merge launches)', 'heads': Ha, 'rows_attended': n_sel,
                      'us': attn_us,
                      'bound': 'hbm',
                      'algorithmic_bytes': n_sel * 1152 + wl.B * Ha * (576 * 2 + 512 * 4 + 4),
                      'achieved_GBs': (n_sel * 1152 + wl.B * Ha * (576 * 2 + 512 * 4 + 4)) / (attn_us * 1e-6) / 1e9,
                      'peak_GBs': PEAK_HBM_GBS,
                      'frac': (n_sel * 1152 + wl.B * Ha * (576 * 2 + 512 * 4 + 4)) / (attn_us * 1e-6) / 1e9
                      / PEAK_HBM_GBS,
                      'mfma_bf16_frac': n_sel * Ha * (576 + 512) * 2 / (attn_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS,
                      'note': attn_note},
        'append': {'kernel': 'ech_kv_append', 'sequences': wl.B, 'us': append_us,
                   'bytes_per_call': wl.B * (1152 + 128 + 4),
                   'note': 'one decoded token per sequence: its row written over PCIe into the pinned pool, '
                           'its fp8 key and scale into the key cache; latency-bound'},
        'allocator': {'early_maps_us': st['early_maps'], 'final_maps_us': st['final_maps'],
                      'note': ('FINAL maps (count, place) in eager steps, beside the live copier; the EARLY maps '
                               'are part of the fused launch' if layer.fused else
                               'slot-map phases in eager steps (count, place), run beside '
                               'the top-k (EARLY) and beside the EARLY recall (FINAL)')},
    }
    return out, dict(wl=wl, pool=pool, qs=qs, w=w, keys=keys, scale=scale)


def bench_stack(args, wl):
    """Decode steps over `--layers` layers in `--micro-batches` micro-batches
    (DecodeStack): every (layer, micro-batch) has its own slot map and a
    1/M share of the layer's device cache; each layer its own keys, scales,
    head weights, queries and host pool (seeded per layer). Times graph
    replays of the whole L-layer step."""
    import numpy as np
    import torch
    import workloads as wk
    from indexer_top_kv_amd.pipeline import DecodeLayer, DecodeStack, sequence_groups

    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x.view(np.int16) if x.dtype == np.uint16 else x)).cuda()
    L, M = args.layers, args.micro_batches
    groups = sequence_groups(wl.B, M)
    C_m = wl.C // len(groups)
    pre = args.fill + args.warmup                # untimed steps before the timed ones
    total_steps = pre + args.steps
    layers, qs, pools = [], [], []
    ctx0 = None
    for l in range(L):
        t = time.time()
        wll = wl.scaled(layer=l)
        keys, scale = wk.keys(wll)
        pool = torch.empty((wll.P, wk.ROW_ELEMS), dtype=torch.int16, pin_memory=True)
        wk.host_rows(wll, out=pool.numpy().view(np.uint16))
        w_np = wk.head_weights(wll)
        kc, ks, wd = dev(keys), (dev(scale) if scale is not None else None), dev(w_np)
        layers.append([DecodeLayer(kc, ks, wd[b0:b1], wll.tok0[b0:b1], wll.lens[b0:b1], C_m, k=wll.k,
                                   cap=wll.cap, host_pool=pool, fused=False)
                       for b0, b1 in groups])
        q_np = np.stack(list(wk.decode_queries(wll, total_steps)))
        qs.append(dev(q_np))
        pools.append(pool)
        if l == 0:   # layer 0's inputs for the CPU oracle baseline
            ctx0 = dict(keys=keys, scale=scale, w=w_np, pool=pool, qs=q_np)
        else:
            del keys, scale
        log(f'layer {l}: keys, {wll.P} host rows and queries in {time.time() - t:.1f}s')
    stack = DecodeStack(layers)
    step_q = lambda s: [[qs[l][s, b0:b1] for b0, b1 in groups] for l in range(L)]
    if not args.eager:
        stack.capture()          # nothing runs; the warm-up steps are replays of the timed path
    torch.cuda.synchronize()
    for s in range(pre):
        (stack.step if args.eager else stack.replay)(step_q(s))
    torch.cuda.synchronize()
    rec0 = sum(int(d.state.ctr[4].item()) for r in layers for d in r)
    launch = ('eager launches' if args.eager
              else 'per (layer, micro-batch): scores kernel + hipGraph replay of the rest of its step')
    log(f'timing {args.steps} steps of {L} layers x {len(groups)} micro-batches ({launch})')
    t0 = time.perf_counter()
    for s in range(args.steps):
        (stack.step if args.eager else stack.replay)(step_q(pre + s))
    t_host = time.perf_counter() - t0                  # host time to enqueue the K steps
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    recalled = sum(int(d.state.ctr[4].item()) for r in layers for d in r) - rec0
    tokens = int(wl.lens.astype(np.int64).sum())
    step_ms = wall / args.steps * 1e3
    rec_bytes = recalled * 1152 / args.steps
    # Roofline: every (layer, micro-batch)'s plain scores kernel, K rounds of
    # L x M launches back to back on one stream between one pair of HIP
    # events (the step's own queries); per layer = span / (K x L).
    s0 = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(s0)
    for s in range(args.steps):
        for l in range(L):
            for m, (b0, b1) in enumerate(groups):
                layers[l][m].logits_only(qs[l][pre + s, b0:b1], stream=s0)
    ev1.record(s0)
    torch.cuda.synchronize()
    layer_ms = ev0.elapsed_time(ev1) / (args.steps * L)
    per_layer = tokens * (128 + 4 + 4) + wl.B * (64 * 128 * 2 + 64 * 4)
    return {
        'metric': f'decode tokens scored/s over a {L}-layer step (indexer logits + exact top-k + early/final '
                  f'slot-map step + recall per layer)',
        'value': tokens * L * args.steps / wall,
        'unit': 'tokens/s',
        'n_gpus': 1, 'steps': args.steps, 'warmup': args.warmup, 'fill_steps': args.fill,
        'ms_per_step': step_ms,
        'higher_is_better': True, 'scaling': 'weak', 'vs_baseline': None,
        'dtype': 'fp8-e4m3 keys, bf16 q, bf16 MFMA with fp32 accumulation' if wl.kdtype == 'fp8' else 'bf16',
        'data': 'synthetic, seeded per layer',
        'config': {'workload': wl.name, 'layers': L, 'micro_batches': len(groups),
                   'micro_batch_sequences': [b1 - b0 for b0, b1 in groups], 'cache_slots_per_micro_batch': C_m,
                   'fused_scores_early_fetch': layers[0][0].fused,
                   'B': wl.B, 'context': wl.N, 'k': wl.k, 'early_fetch_cap': wl.cap,
                   'launch': launch},
        'us_per_layer': step_ms * 1e3 / L,
        'host_enqueue_ms_per_step': t_host / args.steps * 1e3,
        'recall': {'rows_per_step': recalled / args.steps, 'bytes_per_step': rec_bytes,
                   'GBs_over_step': rec_bytes / (step_ms * 1e-3) / 1e9},
        'roofline': {'bound': 'hbm', 'kernel': 'logits_decode_fp8_kernel (every layer and micro-batch)',
                     'achieved': per_layer / (layer_ms * 1e-3) / 1e9, 'peak': PEAK_HBM_GBS, 'unit': 'GB/s',
                     'frac': per_layer / (layer_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 'traffic': None,
                     'algorithmic_bytes_per_layer': per_layer, 'avg_us_per_layer': layer_ms * 1e3,
                     'timing': 'HIP events around K rounds of the L x M scores launches back to back on one '
                               'stream'},
        'cpu_baseline': None,
    }, pools, ctx0


def pcie_check(pool, C, rows=16384, reps=5):
    """Host->device bandwidth two ways on this machine: a pinned 256 MiB
    hipMemcpyAsync (DMA engines; the denominator) and the recall gather kernel
    copying `rows` random rows of the pinned pool into a scratch cache through a
    synthetic miss list (separate buffers; the layer's state is untouched)."""
    import numpy as np
    import torch
    import indexer_top_kv_amd as ech

    src = torch.empty(256 << 20, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(256 << 20, dtype=torch.uint8, device='cuda')
    best = 0.0
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src, non_blocking=True)
        b.record()
        torch.cuda.synchronize()
        best = max(best, src.numel() / (a.elapsed_time(b) * 1e-3) / 1e9)
    del src, dst
    P = pool.shape[0]
    rows = min(rows, C, P)
    rng = np.random.default_rng(7)
    g = rng.choice(P, rows, replace=False).astype(np.int32)
    p = rng.permutation(C).astype(np.int32)[:rows]
    st = ech.LayerState.allocate(P, C, rows)
    st.miss.copy_(torch.from_numpy(np.stack([g, p], 1)))
    ctr = np.zeros(ech.CTR_LEN, np.int32)
    ctr[ech.CTR_NMISS] = rows
    st.ctr.copy_(torch.from_numpy(ctr))
    cache = torch.empty((C, pool.shape[1]), dtype=pool.dtype, device='cuda')
    t = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        ech.ech_recall(pool, cache, st)
        b.record()
        torch.cuda.synchronize()
        t.append(a.elapsed_time(b))
    gather = rows * pool.shape[1] * pool.element_size() / (min(t) * 1e-3) / 1e9
    return {'h2d_memcpy_GBs': best, 'recall_gather_GBs': gather, 'gather_rows': rows,
            'frac_of_memcpy': gather / best}


def cpu_baseline_decode(args, wl, ctx):
    """The oracle as it stands, on a bounded sample of the same workload: the
    first `cpu_seqs` sequences for `cpu_steps` decode steps (scores, top-k,
    threshold, early and final slot-map phases, recall)."""
    import numpy as np
    import oracle
    import workloads as wk

    S, T = min(args.cpu_seqs, wl.B), args.cpu_steps
    lens, tok0 = wl.lens[:S], wl.tok0[:S]
    P = int(tok0[-1] + lens[-1])
    keys = ctx['keys'][:P]
    scale = None if ctx['scale'] is None else ctx['scale'][:P]
    w = ctx['w'][:S]
    pool = ctx['pool'].numpy()
    C = min(wl.C, P)
    sm = oracle.SlotMap(P, C)
    cache = np.zeros((C, pool.shape[1]), pool.dtype)
    theta = np.full(S, np.nan, np.float32)
    t0 = time.perf_counter()
    for s in range(T):
        q = ctx['qs'][s][:S]
        L = [x.astype(np.float32) for x in oracle.index_logits(q, w, keys, wl.kdtype, scale, tok0, lens)]
        idx, kth = oracle.topk_rows(L, wl.k)
        a, _ = sm.early(tok0, L, theta, wl.cap)
        oracle.recall_rows(pool, cache, a)
        a, _, _ = sm.final(tok0, idx)
        oracle.recall_rows(pool, cache, a)
        theta = oracle.theta_rows(theta, kth)
    dt = time.perf_counter() - t0
    tokens = int(lens.astype(np.int64).sum()) * T
    return {'value': tokens / dt, 'unit': 'tokens/s', 'cores': cpu_cores(), 'kind': 'oracle',
            'sample': f'first {S} of {wl.B} sequences x {T} decode steps ({tokens} tokens scored), '
                      f'{dt:.1f} s; label: CPU oracle - reported baseline',
            'seconds': dt, 'host_cpus': len(os.sched_getaffinity(0))}


def cpu_baseline_prefill(args, wl, ctx):
    """The oracle as it stands, on a bounded sample of the prefill pass: the
    first 128 rows of three query blocks (early, middle, last) - scores of
    every visible token, exact top-k of each row, one union slot-map phase per
    sampled block, recall of its rows. Scaled to (row, token) pairs per
    second."""
    import numpy as np
    import oracle
    import workloads as wk

    keys, scale, pool = ctx['keys'], ctx['scale'], ctx['pool'].numpy()
    nblk = (wl.N + wl.block_rows - 1) // wl.block_rows
    blocks = sorted({1 % nblk, nblk // 2, nblk - 1})
    rows_per = min(128, wl.block_rows)
    sm = oracle.SlotMap(wl.N, wl.C)
    cache = np.zeros((wl.C, pool.shape[1]), pool.dtype)
    pairs = 0
    t0 = time.perf_counter()
    for bi in blocks:
        r0 = bi * wl.block_rows
        R = min(rows_per, wl.N - r0)
        q = wk.prefill_queries(wl, r0, R)
        w = wk.head_weights(wl, rows=R, row0=r0)
        vis = r0 + 1 + np.arange(R)
        L = [x.astype(np.float32) for x in oracle.index_logits(q, w, keys, wl.kdtype, scale, [0] * R, vis)]
        idx, _ = oracle.topk_rows(L, wl.k)
        a, _, _ = sm.prefill_block(0, idx)
        oracle.recall_rows(pool, cache, a)
        pairs += int(vis.sum())
    dt = time.perf_counter() - t0
    return {'value': pairs / dt, 'unit': 'pairs/s', 'cores': cpu_cores(), 'kind': 'oracle',
            'sample': f'first {rows_per} rows of query blocks {blocks} ({pairs} (row, token) pairs scored, '
                      f'selected and made resident), {dt:.1f} s; label: CPU oracle - reported baseline',
            'seconds': dt, 'host_cpus': len(os.sched_getaffinity(0))}


# ---------------------------------------------------------------------------- prefill
def bench_prefill(args, wl):
    import numpy as np
    import torch
    import workloads as wk
    import indexer_top_kv_amd as ech
    from indexer_top_kv_amd.pipeline import PrefillLayer

    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x.view(np.int16) if x.dtype == np.uint16 else x)).cuda()
    keys, scale = wk.keys(wl)
    pool = torch.empty((wl.P, wk.ROW_ELEMS), dtype=torch.int16, pin_memory=True)
    wk.host_rows(wl, out=pool.numpy().view(np.uint16))
    layer = PrefillLayer(dev(keys), dev(scale), wl.N, wl.C, k=wl.k, block_rows=wl.block_rows, host_pool=pool,
                         overlap=not args.prefill_serial)
    blocks = layer.blocks()
    q = [dev(wk.prefill_queries(wl, r0, R)) for r0, R in blocks]
    w = [dev(wk.head_weights(wl, rows=R, row0=r0)) for r0, R in blocks]
    log(f'{len(blocks)} query blocks staged')
    marks = []
    stage_marks = {}

    def one_pass(timed):
        layer.reset_state()
        for i, (r0, R) in enumerate(blocks):
            layer.run_block(r0, q[i], w[i], first=(i == 0), mark=marks if timed else None,
                            stage_marks=stage_marks if timed else None)
        layer.finish()

    for _ in range(args.warmup):
        one_pass(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        one_pass(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pairs = sum(sum(r0 + i + 1 for i in range(R)) for r0, R in blocks)
    lg = [marks[i].elapsed_time(marks[i + 1]) for i in range(0, len(marks), 2)]
    logits_ms_total = float(np.sum(lg)) / args.steps
    flops = pairs * 2 * 64 * 128
    tflops = flops / (logits_ms_total * 1e-3) / 1e12

    def stage_ms(name):
        ev = stage_marks.get(name, [])
        return float(np.sum([ev[i].elapsed_time(ev[i + 1]) for i in range(0, len(ev), 2)])) / args.steps

    # top-k: one read of every visible score plus the index output, per pass
    topk_bytes = pairs * 4 + sum(R for _, R in blocks) * wl.k * 4
    topk_ms = stage_ms('topk')
    recalled = int(layer.state.ctr[ech.CTR_RECALLED].item())   # counted since the pass's reset
    recall_ms = stage_ms('recall')
    h2d = pcie_check(pool, wl.C)['h2d_memcpy_GBs']
    stages = {
        'topk': {'bound': 'hbm', 'algorithmic_bytes_per_pass': topk_bytes, 'ms_per_pass': topk_ms,
                 'achieved_GBs': topk_bytes / (topk_ms * 1e-3) / 1e9 if topk_ms else None, 'peak_GBs': PEAK_HBM_GBS,
                 'frac': topk_bytes / (topk_ms * 1e-3) / 1e9 / PEAK_HBM_GBS if topk_ms else None,
                 'note': 'one read of the visible scores plus the index output; the five top-k launches of each '
                         'block, timed on their stream' + ('' if args.prefill_serial else
                                                           ' (beside the next block\'s scoring)')},
        'cache_step_ms_per_pass': stage_ms('cache'),
        'recall': {'bound': 'pcie', 'ms_per_pass': recall_ms, 'h2d_memcpy_GBs': h2d,
                   'rows_per_pass': recalled,
                   'achieved_GBs': recalled * 1152 / (recall_ms * 1e-3) / 1e9 if recalled and recall_ms else None,
                   'frac_of_memcpy': recalled * 1152 / (recall_ms * 1e-3) / 1e9 / h2d if recalled and recall_ms
                   else None},
    }
    return {
        'metric': 'prefill (row, token) pairs scored/s (causal indexer logits + per-row exact top-k + '
                  'union slot-map step + overlapped recall), 1 layer',
        'value': pairs * args.steps / wall, 'unit': 'pairs/s', 'n_gpus': 1, 'steps': args.steps,
        'warmup': args.warmup, 'ms_per_step': wall / args.steps * 1e3, 'higher_is_better': True,
        'scaling': 'weak', 'vs_baseline': None, 'dtype': 'fp8-e4m3 keys, bf16 q, bf16 MFMA fp32 accumulation',
        'data': 'synthetic, seeded',
        'config': {'workload': wl.name, 'N': wl.N, 'block_rows': wl.block_rows, 'k': wl.k, 'cache_slots': wl.C,
                   'selection_beside_next_block': not args.prefill_serial},
        'roofline': {'bound': 'mfma', 'kernel': 'logits_causal_kernel', 'achieved': tflops,
                     'peak': PEAK_BF16_TFLOPS, 'unit': 'TFLOP/s', 'frac': tflops / PEAK_BF16_TFLOPS,
                     'traffic': measured_traffic('logits_causal_' + wl.name, source_hash('logits.hip', 'score.hpp'),
                                                 'bytes_per_pass'),
                     'traffic_unit': 'bytes per pass (27 launches)',
                     'algorithmic_flops_per_pass': flops, 'logits_ms_per_pass': logits_ms_total},
        'stage_rooflines': stages,
    }, dict(keys=keys, scale=scale, pool=pool)


def main():
    args = parse()
    world = int(os.environ.get('WORLD_SIZE', '1'))
    if args.gpus != 1 or world != 1:
        print('bench.py runs on one GPU only: this path is a per-layer, per-GPU kernel pipeline with no '
              'inter-GPU exchange (sequences shard across GPUs with no communication); run with --gpus 1.',
              file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads as wk
    import indexer_top_kv_amd as ech
    ech.lib()
    assert torch.cuda.is_available(), 'no GPU'
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        src = torch.ones(1 << 30, dtype=torch.uint8, device='cuda')
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({'copy_bytes_read_per_launch': src.numel(), 'copy_bytes_written_per_launch': src.numel(),
                          'launches': 5}), flush=True)
        return
    wl = wk.CONFIGS[args.config]
    log(f'{wl.name} on {torch.cuda.get_device_name(0)}')
    if wl.mode == 'decode' and (args.layers > 1 or args.micro_batches > 1):
        out, pools, ctx0 = bench_stack(args, wl)
        out['pcie'] = pcie_check(pools[0], wl.C)
        out['recall']['frac_of_memcpy'] = out['recall']['GBs_over_step'] / out['pcie']['h2d_memcpy_GBs']
        if not args.no_cpu_baseline:
            log('timing the CPU oracle on a sample of layer 0')
            cb = cpu_baseline_decode(args, wl, ctx0)
            cb['sample'] += ' (layer 0; every layer costs the oracle the same, so the rate is per token-layer)'
            out['cpu_baseline'] = cb
    elif wl.mode == 'decode':
        out, ctx = bench_decode(args, wl)
        out['pcie'] = pcie_check(ctx['pool'], wl.C)
        r = out['stage_rooflines']['recall']
        if r['achieved_GBs']:
            r['frac_of_memcpy'] = r['achieved_GBs'] / out['pcie']['h2d_memcpy_GBs']
        if not args.no_cpu_baseline:
            log('timing the CPU oracle on a sample')
            out['cpu_baseline'] = cpu_baseline_decode(args, wl, ctx)
        else:
            out['cpu_baseline'] = None
    else:
        out, ctx = bench_prefill(args, wl)
        if not args.no_cpu_baseline:
            log('timing the CPU oracle on a sample')
            out['cpu_baseline'] = cpu_baseline_prefill(args, wl, ctx)
        else:
            out['cpu_baseline'] = None
    print(json.dumps(out), flush=True)


if __name__ == '__main__':
    main()
