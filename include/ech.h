/*
 * ech.h - C ABI of the MI355X (gfx950) indexer -> exact top-k -> KV-recall path
 * of ECHO-style lossless KV-cache offloading for native-sparse-attention models.
 *
 * The path, per layer and step (ECHO explainer page, sections "The top-k
 * dependency", "Decode: fetch above a predicted threshold", "Prefill: one-round
 * histogram", "One layer, one step: free -> allocate -> recall", "Five
 * fixed-size integer tensors on the GPU"):
 *   1. ech_index_logits / ech_index_logits_causal: indexer score of every
 *      cached token, logit[r,t] = sum_h w[r,h] * ReLU(q[r,h,:] . k[g,:]).
 *   2. ech_topk: exact top-k of each row (ties to the lower token index) found
 *      with a 256-bin histogram keyed by the high byte of (score - theta), theta
 *      being an EMA (alpha = 0.5) of the previous step's k-th score.
 *   3. ech_cache_step: GPU-resident per-layer slot map. EARLY (decode): fetch
 *      tokens scoring above theta, up to a cap, before the top-k is known
 *      (ech_index_logits_early: fused with the scores, for fp8 keys).
 *      FINAL: pin the selected resident tokens, give every selected miss a
 *      slot in ring order (evicting lazily freed tokens, no write-back).
 *      PREFILL: FINAL over the union of a query block's selections.
 *   4. ech_recall: copy the missed KV rows from pinned host memory into their
 *      device-cache slots.
 *   5. ech_sparse_attn (the consumer): attention of each head over the rows
 *      its sequence selects, through sel_slot.
 *   6. ech_kv_append: each sequence's decoded token joins the host pool and
 *      the key cache (growing contexts).
 *
 * Conventions
 *  - Ownership: the caller owns every buffer (device memory, the pinned host
 *    pool, workspaces) and the stream. The library allocates nothing, keeps no
 *    global state and is re-entrant; per-layer state is a set of caller
 *    buffers, so L layers are L buffer sets. The one exception is
 *    ech_topk_noalloc, whose workspace is a static per-GPU array inside the
 *    library (for callers that cannot allocate).
 *  - Pointers are device pointers unless stated. bf16 = uint16 bit patterns;
 *    fp8 = OCP e4m3fn bytes. Row-major throughout.
 *  - Asynchrony: every call only enqueues kernels on `stream` (a hipStream_t,
 *    NULL = the default stream). It never synchronises, never allocates,
 *    never prints and never issues hipMemset, so a whole step can be captured
 *    in a hipGraph. Grids are sized from host-known maxima; data-dependent
 *    counts stay in device memory (the `ctr` tensor).
 *  - Errors: calls return ECH_OK or a negative code. Arguments are checked on
 *    the host before any launch; on an error nothing is enqueued. Problems only
 *    the device can see (a token index out of range, a miss list that would
 *    overflow) set sticky bits in ctr[ECH_CTR_STATUS], which the caller reads
 *    after its own synchronisation.
 */
#ifndef ECH_H
#define ECH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes */
#define ECH_OK            0
#define ECH_EINVAL       -1   /* bad sizes, NULL pointer, misalignment, unsupported H/D/k */
#define ECH_ENOSPC       -2   /* host-known FINAL demand exceeds the cache size C */
#define ECH_EUNSUPPORTED -3   /* key dtype or device architecture not supported */
#define ECH_EHIP         -4   /* a HIP call or kernel launch failed */
#define ECH_ESCRATCH     -5   /* the call needs more than the library's static scratch array holds */

/* ---- key dtypes */
#define ECH_KEY_BF16 0        /* keys [P, D] bf16, no scale */
#define ECH_KEY_FP8  1        /* keys [P, D] OCP e4m3fn, one fp32 scale per token */

/* ---- cache-step phases */
#define ECH_EARLY   0         /* decode: fetch tokens scoring above theta, up to cap */
#define ECH_FINAL   1         /* decode: make every selected token resident */
#define ECH_PREFILL 2         /* prefill: FINAL over the union of R rows of one sequence */

/* ---- the control tensor ctr[ECH_CTR_LEN] (int32, device), one per layer */
#define ECH_CTR_HEAD      0   /* ring head: next slot the allocator looks at */
#define ECH_CTR_EPOCH     1   /* phase counter; slot s is pinned in a phase iff slot_pin[s] == epoch */
#define ECH_CTR_NMISS     2   /* entries written to the miss list by the last FINAL/PREFILL phase */
#define ECH_CTR_NEVICT    3   /* resident tokens evicted by the last phase */
#define ECH_CTR_RECALLED  4   /* rows copied by ech_recall since reset (wraps at 2^31) */
#define ECH_CTR_STATUS    5   /* sticky ECH_ST_* bits */
#define ECH_CTR_NWANT     6   /* misses the last phase wanted (before cap / slot limits) */
#define ECH_CTR_NPINNED   7   /* slots pinned by the last phase */
#define ECH_CTR_NMISS_EARLY 8 /* entries written to the miss list by the last EARLY phase */
#define ECH_CTR_TICKET    9   /* reserved: stays 0 */
#define ECH_CTR_NCOPIED_EARLY 10 /* leading EARLY miss-list entries already copied (by ech_recall_early_live) */
#define ECH_CTR_LIVE     11   /* 1 while ech_index_logits_early is writing the early list; ech_recall(EARLY) clears it */
#define ECH_CTR_NCOPIED_FINAL 12 /* leading FINAL miss-list entries already copied (by ech_recall_early_live) */
#define ECH_CTR_FINAL_READY 13 /* bit 0: the FINAL phase's miss list is complete; bit 1: its allocation walked
                                  onto slots the EARLY phase before it allocated (cleared by each FINAL phase
                                  and by ech_index_logits_early) */
#define ECH_CTR_FINAL_DONE 14 /* internal: FINAL placing workgroups finished */
#define ECH_CTR_EARLY_WALK 15 /* ring positions the last EARLY phase walked, head to last slot it allocated (0: none) */
#define ECH_CTR_LEN      16

/* ---- sticky status bits in ctr[ECH_CTR_STATUS] */
#define ECH_ST_OVERFLOW   1   /* a FINAL/PREFILL phase found fewer unpinned slots than misses */
#define ECH_ST_BADTOK     2   /* a selected token offset was outside [0, len) */
#define ECH_ST_BADMISS    4   /* ech_recall saw a miss entry with g >= P or slot >= C */
#define ECH_ST_FULL       8   /* ech_kv_append found a sequence at its capacity */
#define ECH_ST_TIMEOUT   16   /* a bounded wait inside ech_index_logits_early ran out (results invalid) */

/* Human-readable name of a return code. */
const char* ech_status_str(int code);

/* Library ABI version (major*100 + minor); 200: the grouped early-fetch calls gave way to
   ech_index_logits_early; ech_topk_noalloc. 300: ech_recall_early_live also takes the FINAL list;
   ech_recall_rest; ech_topk_early. */
int ech_version(void);

/*
 * ech_index_logits - decode indexer scores (one query row per sequence).
 *
 * Computes, for r < R and t < row_len[r],
 *     logits[r*ld + t] = sum_h w[r*H+h] * ReLU( sum_d q[(r*H+h)*D+d] * k(g, d) ),
 *     g = row_tok0[r] + t,
 * with k(g,d) = bf16 key, or e4m3fn key * kscale[g] (the scale multiplies the
 * whole key; any sign is allowed). Indexer scores of every cached token:
 * ECHO explainer, "Decode: fetch above a predicted threshold" and "Fused
 * indexer kernel (extends DeepGEMM)"; the formula is the lightning-indexer form.
 *
 *  q         [R, H, D] bf16, device.        w       [R, H] fp32, device.
 *  kcache    [P, D] bf16 or e4m3fn, device, token-major (row g = token g).
 *  kdtype    ECH_KEY_BF16 or ECH_KEY_FP8.   kscale  [P] fp32 (FP8) or NULL (BF16).
 *  row_tok0  [R] int64, row_len [R] int32 (0 <= row_len[r] <= max_len), device.
 *  logits    [R, ld] fp32, device, ld >= max_len; entries t >= row_len[r] are
 *            not written.
 *  Requires H == 64, D == 128, R >= 1, max_len >= 0, 16-byte aligned q/kcache.
 *  Arithmetic: bf16 x bf16 products (fp8 keys widen exactly to bf16) summed in
 *  fp32 on the matrix cores; ReLU, head weights and the per-token scale in fp32.
 */
int ech_index_logits(const void* q, const float* w, const void* kcache, int kdtype,
                     const float* kscale, const int64_t* row_tok0, const int32_t* row_len,
                     int R, int H, int D, int max_len, float* logits, int64_t ld, void* stream);

/*
 * ech_index_logits_causal - prefill indexer scores for a block of R query rows
 * of one sequence (ECHO explainer, "Prefill: one-round histogram": query
 * blocks are scored one after another). Row r is the query at position
 * row0 + r and sees tokens t = 0 .. row0 + r (inclusive) of the sequence
 * whose first token is tok0:
 *     logits[r*ld + t] = sum_h w[r*H+h] * ReLU(q[r,h,:] . k(tok0 + t, :)).
 * Entries t > row0 + r are not written. ld >= row0 + R. Same dtypes and
 * limits as ech_index_logits.
 */
int ech_index_logits_causal(const void* q, const float* w, const void* kcache, int kdtype,
                            const float* kscale, int64_t tok0, int64_t row0, int R, int H, int D,
                            float* logits, int64_t ld, void* stream);

/*
 * ech_topk - exact top-k of each score row, ascending token order.
 *
 * For each row r (its first row_len[r] scores), idx[r*k + j] lists the tokens
 * t whose (score, -t) is among the k largest, in ascending t, padded with -1
 * when row_len[r] < k; ties go to the lower token index. kth[r] is the
 * smallest selected score (NaN for an empty row). The selection is exact, as
 * the ECHO explainer's opening summary requires; it is found with 256 bins over
 * the high byte of each score minus the predicted threshold ("Prefill:
 * one-round histogram"), then the boundary bin is resolved exactly.
 *
 *  theta_in  [R] fp32 or NULL: predicted threshold per row; NaN or NULL means
 *            no prediction (the histogram is unshifted). It only steers speed:
 *            the result is the same for any theta.
 *  theta_out [R] fp32 or NULL: receives the EMA update (ECHO explainer,
 *            "Decode: fetch above a predicted threshold", alpha = 0.5):
 *            kth if theta_in is NaN/NULL, else fl32(fl32(kth + theta_in) * 0.5);
 *            unchanged copy of theta_in for an empty row. May alias theta_in
 *            only when nothing else reads theta_in concurrently.
 *  Scores must be finite; -0.0 and +0.0 are equal.
 *  Requires 1 <= k <= 4096, R >= 1, ld >= max_len, 0 <= row_len[r] <= max_len.
 *  ws: device workspace of ech_topk_ws_bytes(R, max_len, k) bytes, 256-byte
 *  aligned; contents need not be initialised.
 */
size_t ech_topk_ws_bytes(int R, int max_len, int k);
int ech_topk(const float* logits, int64_t ld, const int32_t* row_len, int R, int max_len, int k,
             const float* theta_in, float* theta_out, int32_t* idx, float* kth,
             void* ws, size_t ws_bytes, void* stream);

/*
 * ech_topk_noalloc - ech_topk for callers that cannot allocate device memory
 * (code under hipGraph capture, tight serving loops, harnesses that forbid
 * allocation). Same arguments, results and errors as ech_topk, without ws:
 * the workspace is a static device array of ECH_TOPK_SCRATCH_BYTES inside the
 * library, one copy per GPU, held until the process ends. Its device address
 * is looked up once per device, on the first call with that device current;
 * no call allocates or frees memory. Contents left by earlier calls do not
 * matter (nothing needs to start at zero).
 *  ECH_ESCRATCH if ech_topk_ws_bytes(R, max_len, k) > ECH_TOPK_SCRATCH_BYTES
 *  (16 MiB: enough for 64 rows of 131072 tokens or 4 rows of 1M tokens at
 *  k = 2048; a 4096-row prefill block needs ech_topk with a workspace).
 *  Every call on one GPU uses the same array: calls on one GPU that may
 *  overlap in time (different streams without ordering between them) race
 *  and give wrong results; order them.
 */
#define ECH_TOPK_SCRATCH_BYTES (16u << 20)
int ech_topk_noalloc(const float* logits, int64_t ld, const int32_t* row_len, int R, int max_len, int k,
                     const float* theta_in, float* theta_out, int32_t* idx, float* kth, void* stream);

/*
 * ech_cache_reset - clear one layer's slot-map state: tok2slot[0..P) = -1,
 * slot2tok[0..C) = -1, slot_pin[0..C) = 0, ctr[0..ECH_CTR_LEN) = 0. Uses fill
 * kernels (no hipMemset), so it may be captured. The cache starts empty; every
 * row lives in the host pool.
 */
int ech_cache_reset(int32_t* tok2slot, int64_t P, int32_t* slot2tok, int32_t* slot_pin, int32_t C,
                    int32_t* ctr, void* stream);

/*
 * ech_cache_step - one phase of the per-layer slot map (ECHO explainer, "One
 * layer, one step: free -> allocate -> recall"; "Five fixed-size integer
 * tensors on the GPU"). The five tensors, all int32 on the device:
 *   tok2slot [P]        slot of global token g, or -1
 *   slot2tok [C]        token held by slot s, or -1
 *   slot_pin [C]        epoch stamp; slot s is pinned in a phase iff it equals
 *                       that phase's epoch (no clearing pass). Pins are the
 *                       phase's resident selection; slots it allocates are
 *                       not stamped.
 *   miss     [M_max,2]  (g, slot) pairs allocated by the phase, in
 *                       allocation order; consumed by ech_recall. EARLY
 *                       phases should get their own buffer (count in
 *                       ctr[ECH_CTR_NMISS_EARLY]) so that a FINAL phase can
 *                       update the maps while the early rows are still being
 *                       copied; FINAL/PREFILL counts go to ctr[ECH_CTR_NMISS].
 *   ctr      [ECH_CTR_LEN] ring head, epoch, counts, status (ECH_CTR_*)
 *
 * Free is lazy: unselected resident tokens keep their slot until it is reused.
 * Allocation: misses, in ascending (sequence, token) order, take the unpinned
 * slots in ring order from ctr[HEAD] (head, head+1, ... mod C); a slot's old
 * token is unmapped (tok2slot = -1) and nothing is written back, the host
 * pool holding every row. Afterwards head = last allocated slot + 1 mod C.
 *
 * phase ECH_EARLY (decode, B sequences): for each b with theta[b] not NaN,
 *   pin the slots of resident tokens t < seq_len[b] with logits[b*ld+t] >
 *   theta[b] (strict) and allocate the first `cap` non-resident ones in
 *   ascending t; when slots run out, later misses are dropped. idx unused.
 * phase ECH_FINAL (decode): idx [B, k] ascending token offsets (-1 padded, as
 *   ech_topk writes them); pin selected resident tokens, allocate every
 *   selected miss; sel_slot[b*k+j] = slot of token idx[b*k+j] (-1 for pads).
 *   The sequences' token ranges [seq_tok0, seq_tok0+seq_len) must not overlap.
 * phase ECH_PREFILL: B must be 1; idx [R, k] rows of one sequence; the union
 *   of their tokens is made resident (misses in ascending token order);
 *   sel_slot [R, k].
 *
 *  stats [B, 4] int32 (PREFILL: [1, 4]) receives, for this phase and
 *   sequence, {hits, fetched, dropped, evictions}: selection tokens already
 *   resident, misses given a slot, misses not given one, tokens evicted.
 *  Host-checked: FINAL demand B*min(k, max_len) (PREFILL: min(max_len, R*k))
 *   must be <= C (else ECH_ENOSPC); M_max must be >= that demand (EARLY:
 *   B*cap); P < 2^31; C >= 1.
 *  ws: ech_cache_step_ws_bytes(...) bytes, 256-byte aligned, uninitialised OK.
 *  Calls on the same layer state must be ordered (same stream or events).
 */
size_t ech_cache_step_ws_bytes(int phase, int B, int R, int k, int max_len, int32_t C, int32_t M_max);
int ech_cache_step(int phase, int32_t* tok2slot, int64_t P, int32_t* slot2tok, int32_t* slot_pin,
                   int32_t C, int32_t* miss, int32_t M_max, int32_t* ctr,
                   const int64_t* seq_tok0, const int32_t* seq_len, int B, int max_len,
                   const int32_t* idx, int R, int k,
                   const float* logits, int64_t ld, const float* theta, int cap,
                   int32_t* sel_slot, int32_t* stats, void* ws, size_t ws_bytes, void* stream);

/*
 * ech_recall - copy missed KV rows host -> device (ECHO explainer, "One layer,
 * one step: free -> allocate -> recall"; the host pool holds every row).
 * For m < n: dev_cache[miss[2m+1]] = host_pool[miss[2m]], row_bytes each,
 * where n = ctr[ECH_CTR_NMISS_EARLY] for phase ECH_EARLY and ctr[ECH_CTR_NMISS]
 * otherwise; `miss` is the list that phase wrote. Phase ECH_EARLY starts at
 * m = ctr[ECH_CTR_NCOPIED_EARLY] (rows ech_index_logits_early already
 * copied; 0 after ech_cache_step). Rows are read directly over
 * PCIe by a gather kernel (zero-copy). Phase ECH_FINAL starts at
 * m = ctr[ECH_CTR_NCOPIED_FINAL] (rows ech_recall_early_live already copied;
 * 0 after ech_cache_step(ECH_FINAL)). A FINAL recall must be ordered after
 * the EARLY recall of the same step (it may reuse a slot the EARLY phase
 * filled).
 *  host_pool  [P, row_bytes] pinned host memory (hipHostMalloc / torch
 *             pin_memory), host pointer; ECH_EINVAL if it is not device-mapped.
 *  dev_cache  [C, row_bytes] device memory.
 *  row_bytes  multiple of 16 (1152 for 576 bf16 values); both buffers 16-byte
 *             aligned. Adds the rows copied to ctr[ECH_CTR_RECALLED].
 */
int ech_recall(int phase, const void* host_pool, int64_t P, int64_t row_bytes, void* dev_cache, int32_t C,
               const int32_t* miss, int32_t* ctr, int32_t M_max, void* stream);

/*
 * ech_index_logits_early - decode scores fused with the early fetch (ECHO
 * explainer, "Decode: fetch above a predicted threshold": tokens scoring above
 * the predicted threshold are fetched before the exact top-k is known, hiding
 * the recall's dependency on the top-k; "Fused indexer kernel (extends
 * DeepGEMM)": the scores and the prefetch in one kernel).
 *
 * Results: exactly those of ech_index_logits(q, ..., logits, ld) followed by
 * ech_cache_step(ECH_EARLY) over sequences [e0, e1) with the same scores,
 * theta and cap (maps, early miss list, ctr, stats[e0..e1); ctr[NPINNED]
 * counts the resident tokens above theta). The early misses of a sequence get
 * their slots, and appear in the early miss list, while later sequences are
 * still being scored, so ech_recall_early_live on another stream can copy
 * their rows meanwhile.
 *
 *  q, w, kcache, kscale, row_tok0, row_len, R, H, D, max_len, logits, ld:
 *            as ech_index_logits (R sequences, one query row each); fp8 keys
 *            only (ECH_EUNSUPPORTED otherwise); R <= 1024.
 *  e0, e1    the sequences whose early fetch runs (0 <= e0 < e1 <= R): a
 *            chunk of the batch when its selections do not fit the cache.
 *  theta [R], cap (<= 4096), tok2slot, P, slot2tok, slot_pin, C, ctr, stats [R, 4]:
 *            as ech_cache_step(ECH_EARLY), indexed by absolute sequence.
 *  miss_early [M_early, 2], M_early >= (e1 - e0) * min(cap, max_len); 8-byte
 *            aligned; rewritten ((-1, -1) where unused).
 *  ws        ech_index_logits_early_ws_bytes(R, max_len, C, M_early) bytes,
 *            256-byte aligned, zero-filled before the first call; the calls
 *            keep it ready for the next one (after ECH_ST_TIMEOUT, zero it
 *            again). Calls with the same ws must be ordered.
 * The launch's workgroups wait on one another within the launch, with bounded
 * waits: if one runs out, ECH_ST_TIMEOUT is set in ctr[ECH_CTR_STATUS] and the
 * results of the call are not valid.
 */
size_t ech_index_logits_early_ws_bytes(int R, int max_len, int32_t C, int32_t M_early);
int ech_index_logits_early(const void* q, const float* w, const void* kcache, int kdtype, const float* kscale,
                           const int64_t* row_tok0, const int32_t* row_len, int R, int H, int D, int max_len,
                           float* logits, int64_t ld, int e0, int e1, const float* theta, int cap,
                           int32_t* tok2slot, int64_t P, int32_t* slot2tok, int32_t* slot_pin, int32_t C,
                           int32_t* miss_early, int32_t M_early, int32_t* ctr, int32_t* stats, void* ws,
                           size_t ws_bytes, void* stream);

/*
 * ech_topk_early - ech_topk for the rows of the last ech_index_logits_early
 * call on ws (ECHO explainer, "Fused indexer kernel (extends DeepGEMM)" and
 * "Prefill: one-round histogram": the scores kernel also emits what the
 * selection needs). Each scoring wave of that launch listed, as it scored,
 * its tokens in the band its row's theta implies (the bins from the bin of
 * theta - |theta|/8 up); this selects from those lists, one workgroup per
 * row, without reading the scores again, and takes the whole row where the
 * lists cannot decide (NaN theta, a wave whose band did not fit its 64
 * entries, or a band holding fewer than k tokens). Results exactly those of
 * ech_topk(logits, ld, row_len, R, max_len, k, theta_in, ...).
 *  logits, ld, row_len, R, max_len: those of the ech_index_logits_early call
 *            (its output scores, unchanged since).
 *  theta_in  [R]: the theta that call took (not NULL; a row whose theta_in
 *            differs from it bit for bit is selected from the whole row:
 *            slower, same result); theta_out, idx, kth, k (<= 4096) as
 *            ech_topk.
 *  ws, ws_bytes, C, M_early: that call's workspace and sizes; read only.
 *  max_len at most 1048576.
 */
int ech_topk_early(const float* logits, int64_t ld, const int32_t* row_len, int R, int max_len, int k,
                   const float* theta_in, float* theta_out, int32_t* idx, float* kth, const void* ws,
                   size_t ws_bytes, int32_t C, int32_t M_early, void* stream);

/*
 * ech_recall_early_live - copy the early rows while ech_index_logits_early
 * allocates them (ECHO explainer, "Decode: fetch above a predicted
 * threshold": the early fetch's transfer overlaps the scoring). Enqueue it on
 * a second stream right after ech_index_logits_early is enqueued (with no
 * wait on it); it copies dev_cache[slot] = host_pool[g] for the early
 * miss-list entries as they appear, leaving ctr[ECH_CTR_NCOPIED_EARLY] = the
 * length of the copied prefix (added to ctr[ECH_CTR_RECALLED]). Then enqueue
 * ech_recall(ECH_EARLY) on that stream, ordered after ech_index_logits_early
 * (an event): it copies the rest and ends the step's early list.
 * The copier never depends on being scheduled beside the scoring: it waits
 * for the list to start and for each entry with a bounded patience (1 ms
 * without progress) and otherwise leaves the rows to ech_recall(ECH_EARLY).
 *
 * With miss_final (the list of the ech_cache_step(ECH_FINAL) call that
 * follows in the same step, on another stream, for the same sequences), the
 * copier goes on to the FINAL rows once it has copied the whole early list:
 * it waits, with the same patience, for that phase to complete its list
 * (ctr[ECH_CTR_FINAL_READY] bit 0) and copies its entries in order, leaving
 * ctr[ECH_CTR_NCOPIED_FINAL] = the copied prefix; ech_recall(ECH_FINAL) or
 * ech_recall_rest, ordered after both, copies the rest. It copies no FINAL
 * row when the FINAL allocation walked onto slots the early phase allocated
 * (bit 1): those rows must land after the early ones.
 *  host_pool [P, row_bytes] pinned, device-mapped (host pointer); dev_cache
 *  [C, row_bytes]; row_bytes a multiple of 16, at most 32768; miss_early,
 *  M_early, ctr and ws: those of the ech_index_logits_early call.
 *  miss_final [M_final, 2], 8-byte aligned, or NULL (early rows only).
 */
int ech_recall_early_live(const void* host_pool, int64_t P, int64_t row_bytes, void* dev_cache, int32_t C,
                          const int32_t* miss_early, int32_t M_early, const int32_t* miss_final, int32_t M_final,
                          int32_t* ctr, void* ws, void* stream);

/*
 * ech_recall_rest - what ech_recall_early_live left of a step's two lists, in
 * one launch (ECHO explainer, "One layer, one step: free -> allocate ->
 * recall"): the early entries m >= ctr[ECH_CTR_NCOPIED_EARLY] (m <
 * ctr[ECH_CTR_NMISS_EARLY]) whose slot still holds their token
 * (slot2tok[slot] == g: a slot the FINAL phase gave to another token gets
 * that token's row from the FINAL list instead), and the FINAL entries
 * m >= ctr[ECH_CTR_NCOPIED_FINAL] (m < ctr[ECH_CTR_NMISS]); so no two rows of
 * the launch go to one slot. The same rows as ech_recall(ECH_EARLY) followed
 * by ech_recall(ECH_FINAL). Enqueue it after the FINAL phase and after the
 * copier; it ends the step's early list (ctr[ECH_CTR_LIVE] = 0) and adds the
 * rows it copies to ctr[ECH_CTR_RECALLED].
 *  host_pool [P, row_bytes] pinned, device-mapped (host pointer); dev_cache
 *  [C, row_bytes]; row_bytes a multiple of 16; both 16-byte aligned.
 *  miss_early [M_early, 2], miss [M_max, 2]: the lists of the step's EARLY
 *  and FINAL phases; slot2tok [C] the layer's map after the FINAL phase.
 */
int ech_recall_rest(const void* host_pool, int64_t P, int64_t row_bytes, void* dev_cache, int32_t C,
                    const int32_t* miss_early, int32_t M_early, const int32_t* miss, int32_t M_max,
                    const int32_t* slot2tok, int32_t* ctr, void* stream);

/*
 * ech_sparse_attn - the consumer of sel_slot: softmax attention of each head
 * over the rows its sequence selects, read from the fixed device cache through
 * the index tensor (ECHO Guide blog, "CUDA Graph Compatibility via
 * Pre-Allocated Tensor Pointers": the attention binds no new addresses as the
 * selection changes). Rows are absorbed-MLA rows of 576 bf16 values: all 576
 * are the key, the first 512 the value. For sequence b and head h, over the
 * valid entries j of sel_slot[b, :] (0 <= slot < C):
 *   s_j = sm_scale * q[b,h,:] . dev_cache[slot_j, :]
 *   out[b,h,:] = sum_j softmax(s)_j * dev_cache[slot_j, 0:512]
 *   lse[b,h] = log sum_j exp(s_j)
 * Entries < 0 or >= C select nothing (padding of short sequences); a sequence
 * that selects nothing gets out = 0 and lse = -inf. Scores accumulate in fp32
 * on bf16 matrix cores; the softmax weights enter the value product as bf16.
 *  q          [B, H, 576] bf16, 16-byte aligned; H a multiple of 16, <= 128.
 *  dev_cache  [C, 576] bf16 (the layer's device cache), 16-byte aligned.
 *  sel_slot   [B, k] int32 (what ech_cache_step FINAL writes), 1 <= k <= 65536.
 *  out        [B, H, 512] fp32, 16-byte aligned; lse [B, H] fp32 or NULL.
 *  ws         ech_sparse_attn_ws_bytes(B, H, k) bytes, 256-byte aligned
 *             (per-span partial results; uninitialised OK).
 *  ECH_EINVAL for NULLs, bad sizes or alignment, a NaN sm_scale.
 */
size_t ech_sparse_attn_ws_bytes(int B, int H, int k);
int ech_sparse_attn(const void* q, const void* dev_cache, int32_t C, const int32_t* sel_slot, int B, int H, int k,
                    float sm_scale, float* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * ech_kv_append - each sequence's newly decoded token joins the layer's data
 * (growing contexts). The host copy holds every KV row and is per model (ECHO
 * explainer, "One layer, one step"), so the row is written once, here, over
 * PCIe into the pinned host pool; the key cache gets the token's indexer key.
 * Sequence b owns global token ids [seq_tok0[b], seq_tok0[b] + seq_cap[b]);
 * its new token g = seq_tok0[b] + seq_len[b]:
 *   host_pool[g] = new_rows[b]   (row_bytes)
 *   kcache[g] = new_keys[b]      (128 B fp8 or 256 B bf16), kscale[g] = new_scales[b] (fp8)
 *   tok2slot[g] = -1             (not resident; a later recall brings it in)
 *   seq_len[b] += 1              (device, in place)
 * A sequence with seq_len[b] >= seq_cap[b] (or g outside [0, P)) gets nothing
 * written and sets ECH_ST_FULL in ctr[ECH_CTR_STATUS].
 *  host_pool  [P, row_bytes] pinned host memory (host pointer, device-mapped).
 *  new_rows   [B, row_bytes] and new_keys [B, key bytes] device, 16-byte aligned;
 *             new_scales [B] fp32 (fp8 keys; NULL for bf16).
 *  Order it after the step that scores the old length and before the next.
 */
int ech_kv_append(void* host_pool, int64_t P, int64_t row_bytes, void* kcache, int kdtype, float* kscale,
                  int32_t* tok2slot, const int64_t* seq_tok0, int32_t* seq_len, const int32_t* seq_cap, int B,
                  const void* new_rows, const void* new_keys, const float* new_scales, int32_t* ctr, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* ECH_H */
