"""CPU oracle for the indexer -> exact top-k -> KV-recall path.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from here. The HIP
path (``indexer_top_kv_amd``) never imports, links or runs this package, and
this package imports nothing from the HIP path: the two share no code. Inputs
come from ``workloads`` (seeded draws only).

Plain numpy, float64 for floating point, written for a reader to check by eye
against the pages:

- ``numerics``  - bf16 and OCP e4m3fn decoding (closed forms).
- ``indexer``   - lightning-indexer scores sum_h w_h ReLU(q_h . k_t).
- ``select``    - exact top-k by full stable sort; EMA threshold.
- ``slotmap``   - sequential per-layer slot-map simulator (free -> allocate ->
                  recall, no write-back) and the recall byte copy.
- ``append``    - the decoded token of each sequence joins the host pool and
                  the key cache (growing contexts).
- ``attention`` - softmax attention of each head over the rows its sequence
                  selects through sel_slot (the consumer of the path).

Sources: the ECHO explainer page ("One layer, one step: free -> allocate ->
recall", "Decode: fetch above a predicted threshold", "Prefill: one-round
histogram", "Five fixed-size integer tensors on the GPU") and the ECHO artifact
README. The indexer formula itself is not printed on the pages; the oracle
takes the standard lightning-indexer form.

Every function is pinned by ``tests/test_oracle_*.py`` against closed forms,
brute force on tiny inputs, library routines and invariants; none is marked
"parity unpinned".
"""
from . import numerics, indexer, select, slotmap, attention, append  # noqa: F401
from .numerics import bf16_to_f64, e4m3fn_to_f64, e4m3fn_table  # noqa: F401
from .indexer import index_logits, index_logit_at, dequant_keys  # noqa: F401
from .select import topk_row, topk_rows, theta_next, theta_rows  # noqa: F401
from .slotmap import SlotMap, recall_rows  # noqa: F401
from .attention import sparse_attention  # noqa: F401
from .append import kv_append  # noqa: F401
