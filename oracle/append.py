"""Appending the newly decoded token of each sequence (TEST INFRASTRUCTURE
ONLY; see the package docstring).

The ECHO explainer ("One layer, one step") keeps every KV row in the host
copy, which is per model, and never writes back on eviction; a decoded
token's row therefore goes to the host pool once, when it is produced, and
its indexer key joins the key cache that every later step scores. Reading
taken (the pages give no append step): sequence b owns the global token ids
[tok0[b], tok0[b] + cap[b]); its new token gets id tok0[b] + lens[b], is not
resident (tok2slot = -1: the next steps' recall brings it in if selected),
and lens[b] grows by one. A sequence already at its capacity gets nothing
written and raises the "full" flag.
"""
import numpy as np


def kv_append(host_pool, kcache, kscale, tok2slot, tok0, lens, cap, new_rows, new_keys, new_scales):
    """In place on numpy arrays: host_pool [P, row], kcache [P, key], kscale
    [P] or None, tok2slot [P], lens [B]; tok0, cap [B]; new_rows [B, row],
    new_keys [B, key], new_scales [B] or None. Returns True if some sequence
    was full."""
    full = False
    for b in range(len(lens)):
        if lens[b] >= cap[b]:
            full = True
            continue
        g = int(tok0[b]) + int(lens[b])
        host_pool[g] = new_rows[b]
        kcache[g] = new_keys[b]
        if kscale is not None:
            kscale[g] = new_scales[b]
        tok2slot[g] = -1
        lens[b] += 1
    return full
