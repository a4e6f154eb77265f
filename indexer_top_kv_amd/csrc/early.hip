// Decode early fetch in sequence groups (ECHO explainer, "Decode: fetch above
// a predicted threshold": tokens scoring above the predicted threshold are
// fetched before the exact top-k is known; "One layer, one step: free ->
// allocate -> recall").
//
// The result is the one of a single EARLY phase over the whole batch (the
// ECH_EARLY phase of ech_cache_step): pins = slots of resident tokens scoring
// above theta; misses = per sequence, the first `cap` non-resident tokens
// above theta in ascending token order; misses in ascending (sequence, token)
// order take the unpinned slots in ring order from the head. It is computed
// in an order that lets the rows of the first sequences cross PCIe while the
// scores of later sequences are still being computed:
//
//   begin   (needs no scores)
//     pin       grid (chunks, B): compact the chunk's resident tokens, score
//               them with the same MFMA tile and epilogue as the scores kernel
//               (bit-identical values), pin those above theta, count hits.
//     free      grid (slot blocks): unpinned slots per block in ring order;
//               the last block to finish scans the counts (free-slot rank of
//               every block), sums the hits per sequence and advances the epoch.
//     freelist  grid (slot blocks): slot of every free rank below the early
//               demand bound, in ring order from the head.
//   group [b0, b1), in ascending b0, once that group's scores are written
//     want      grid (chunks, b1-b0): non-resident tokens above theta per
//               block; the last block gives every sequence its rank range
//               (continuing the ranks of earlier groups, capped per sequence).
//     apply     grid (chunks, b1-b0): recompute the same flags in order; miss
//               of rank m takes freelist[m] (evicting its old token, no
//               write-back) and is written to the miss list at m.
//   recall per group: the rows of the group's rank range.
//
// Only the pins depend on the whole batch, and they involve resident tokens
// only, which the begin step scores itself; the free-slot ranking is then
// fixed for the step, and a group's misses are not changed by earlier groups
// (an earlier group evicts only unpinned slots, i.e. resident tokens at or
// below theta, and maps only its own tokens). So any grouping gives the same
// maps, miss list and statistics as the single phase.
//
// "Last block" steps use a ticket counter in ctr[ECH_CTR_TICKET]: every block
// takes one ticket with atomicInc after a release fence; the block that draws
// the last one wraps the counter back to 0 and runs the step. No block waits
// for another.

#include <algorithm>

#include "score.hpp"

namespace {

constexpr int kT = 256;
constexpr int kPer = 16;
constexpr int kBlk = kT * kPer;   // tokens or slots per block
constexpr int kMaxGroups = 96;
constexpr int kMaxB = 1024;

enum { E_EP = 0, E_NFREE = 1, E_RUN = 2, E_HEAD0 = 3, E_NSC = 16 };

struct EWs {
  int* sc;        // [E_NSC] scalars
  int* grp;       // [2 * kMaxGroups] (begin, end) rank range of each group's allocations
  int* hitblk;    // [B * nch]
  int* want;      // [B * nch]
  int* off;       // [B * nch] rank of the block's first miss
  int* lim;       // [B] rank limit of the sequence (cap)
  int* seqd;      // [B] rank of a sequence's first miss minus its raw want prefix
  int* nfree;     // [ns]
  int* soff;      // [ns]
  int* freelist;  // [M_early]
  int nch, ns;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t early_layout(int B, int max_len, int32_t C, int32_t M_early, EWs* w, char* base) {
  const int nch = std::max(1, (max_len + kBlk - 1) / kBlk);
  const int ns = (int)((C + kBlk - 1) / kBlk);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  const size_t o_sc = take(4 * E_NSC), o_grp = take(4 * 2 * kMaxGroups);
  const size_t o_hit = take(4 * (size_t)B * nch), o_want = take(4 * (size_t)B * nch),
               o_off = take(4 * (size_t)B * nch), o_lim = take(4 * (size_t)B), o_sd = take(4 * (size_t)B),
               o_nf = take(4 * (size_t)ns),
               o_so = take(4 * (size_t)ns), o_fl = take(4 * (size_t)std::max(M_early, 1));
  if (w && base) {
    w->sc = reinterpret_cast<int*>(base + o_sc);
    w->grp = reinterpret_cast<int*>(base + o_grp);
    w->hitblk = reinterpret_cast<int*>(base + o_hit);
    w->want = reinterpret_cast<int*>(base + o_want);
    w->off = reinterpret_cast<int*>(base + o_off);
    w->lim = reinterpret_cast<int*>(base + o_lim);
    w->seqd = reinterpret_cast<int*>(base + o_sd);
    w->nfree = reinterpret_cast<int*>(base + o_nf);
    w->soff = reinterpret_cast<int*>(base + o_so);
    w->freelist = reinterpret_cast<int*>(base + o_fl);
    w->nch = nch;
    w->ns = ns;
  }
  return o;
}

// ------------------------------------------------------------------ begin: pin
// grid (nch, B), 4 waves. Chunk c of sequence b covers tokens [c*kBlk, +kBlk).
template <int KDT>
__global__ __launch_bounds__(kT) void early_pin_kernel(const uint16_t* __restrict__ q, const float* __restrict__ w,
                                                       const uint8_t* __restrict__ kc, const float* __restrict__ ksc,
                                                       const int64_t* __restrict__ tok0,
                                                       const int32_t* __restrict__ lens,
                                                       const float* __restrict__ theta,
                                                       const int32_t* __restrict__ tok2slot, int64_t P, int32_t C,
                                                       int32_t* __restrict__ slot_pin, const int32_t* ctr, EWs ws) {
  constexpr int kRowB = (KDT == ECH_KEY_FP8) ? kD : 2 * kD;
  __shared__ uint4 qs[kH * kD * 2 / 16];
  __shared__ int rt[kBlk];          // resident token offsets of the chunk, ascending
  __shared__ int scr[kT / 64];
  const int b = blockIdx.y, c = blockIdx.x;
  const int len = lens[b];
  const float th = theta[b];
  const int lo = c * kBlk;
  int* out = ws.hitblk + (size_t)b * ws.nch + c;
  if (th != th || lo >= len) {
    if (threadIdx.x == 0) *out = 0;
    return;
  }
  const int64_t g0 = tok0[b];
  const int ep = ctr[ECH_CTR_EPOCH] + 1;
  // 1. ordered compaction of the chunk's resident tokens
  const int t_first = lo + threadIdx.x * kPer;
  bool res[kPer];
  int n = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int t = t_first + i;
    res[i] = false;
    if (t < len && g0 + t < P) {
      const int sl = tok2slot[g0 + t];
      res[i] = sl >= 0 && sl < C;
    }
    n += res[i];
  }
  int nres;
  int pos = ech::block_excl_scan<kT>(n, scr, &nres);
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (res[i]) rt[pos++] = t_first + i;
  int hits = 0;
  if (nres > 0) {   // block-uniform
    // 2. score them: the scores kernel's tile, one 16-token tile per wave step
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    bf16x8_t a[4][4];
    float wv[4][4];
    load_query<KDT>(q + (size_t)b * kH * kD, w + (size_t)b * kH, qs, a, wv, col, grp);   // syncs rt too
    const uint8_t* kbase = kc + (size_t)g0 * kRowB;
    const int ntile = (nres + 15) / 16;
    for (int j = wave; j < ntile; j += kT / 64) {
      const int e = 16 * j + col;
      const int t = rt[min(e, nres - 1)];
      KeyFrag<KDT> f;
      load_key<KDT>(f, kbase + (size_t)t * kRowB, grp);
      const float sc = (KDT == ECH_KEY_FP8) ? ksc[g0 + t] : 1.f;
      bf16x8_t kb[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) kb[s] = key_step<KDT>(f, s);
      const float v = tile_score(a, wv, kb, sc);
      if (grp == 0 && e < nres && v > th) {
        slot_pin[tok2slot[g0 + t]] = ep;
        ++hits;
      }
    }
  }
  const int tot = ech::block_sum<kT>(hits, scr);
  if (threadIdx.x == 0) *out = tot;
}

// ------------------------------------------------------------------ begin: free
__device__ __forceinline__ void free_flags(const int32_t* __restrict__ slot_pin, int32_t C, int head, int ep,
                                           int i0, bool (&fr)[kPer], int* n) {
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int pos = i0 + i;
    fr[i] = false;
    if (pos < C) {
      int p = head + pos;
      if (p >= C) p -= C;
      fr[i] = slot_pin[p] != ep;
    }
    cnt += fr[i];
  }
  *n = cnt;
}

__global__ __launch_bounds__(kT) void early_free_kernel(const int32_t* __restrict__ slot_pin, int32_t C, int B,
                                                        int32_t* ctr, int32_t* __restrict__ stats, EWs ws) {
  __shared__ int scr[kT / 64];
  const int head = ctr[ECH_CTR_HEAD];
  const int ep = ctr[ECH_CTR_EPOCH] + 1;
  bool fr[kPer];
  int n;
  free_flags(slot_pin, C, head, ep, blockIdx.x * kBlk + threadIdx.x * kPer, fr, &n);
  const int tot = ech::block_sum<kT>(n, scr);
  if (threadIdx.x == 0) ws.nfree[blockIdx.x] = tot;
  if (!ech::last_block(ctr, gridDim.x)) return;
  // free-slot rank of every block (ring order), total
  int run = 0;
  for (int b0 = 0; b0 < ws.ns; b0 += kT) {
    const int i = b0 + threadIdx.x;
    const int v = i < ws.ns ? ws.nfree[i] : 0;
    int t;
    const int ex = ech::block_excl_scan<kT>(v, scr, &t);
    if (i < ws.ns) ws.soff[i] = run + ex;
    run += t;
  }
  for (int b = threadIdx.x; b < B; b += kT) {
    int h = 0;
    for (int c = 0; c < ws.nch; ++c) h += ws.hitblk[(size_t)b * ws.nch + c];
    int32_t* s = stats + 4 * b;
    s[0] = h;
    s[1] = 0;
    s[2] = 0;
    s[3] = 0;
  }
  if (threadIdx.x == 0) {
    ws.sc[E_EP] = ep;
    ws.sc[E_NFREE] = run;
    ws.sc[E_RUN] = 0;
    ws.sc[E_HEAD0] = head;
    ctr[ECH_CTR_EPOCH] = ep;
    ctr[ECH_CTR_NPINNED] = C - run;
    ctr[ECH_CTR_NEVICT] = 0;
    ctr[ECH_CTR_NWANT] = 0;
    ctr[ECH_CTR_NMISS_EARLY] = 0;
  }
}

__global__ __launch_bounds__(kT) void early_freelist_kernel(const int32_t* __restrict__ slot_pin, int32_t C,
                                                            int32_t M_early, EWs ws) {
  __shared__ int scr[kT / 64];
  const int base = ws.soff[blockIdx.x];
  const int lim = min(ws.sc[E_NFREE], M_early);
  if (base >= lim) return;   // block-uniform
  const int head = ws.sc[E_HEAD0], ep = ws.sc[E_EP];
  const int i0 = blockIdx.x * kBlk + threadIdx.x * kPer;
  bool fr[kPer];
  int n;
  free_flags(slot_pin, C, head, ep, i0, fr, &n);
  int tot;
  int rank = base + ech::block_excl_scan<kT>(n, scr, &tot);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (!fr[i]) continue;
    if (rank < lim) {
      int p = head + i0 + i;
      if (p >= C) p -= C;
      ws.freelist[rank] = p;
    }
    ++rank;
  }
}

// ------------------------------------------------------------------ group
// Miss flags of 16 consecutive tokens of sequence b: non-resident, score above
// theta (strict), inside the row.
__device__ __forceinline__ void miss_flags(const float* __restrict__ row, int t, int len, float th, int64_t g0,
                                           int64_t P, const int32_t* __restrict__ tok2slot, bool (&m)[kPer],
                                           int* n) {
  int cnt = 0;
  float v[kPer];
  if (t + kPer <= len) {
#pragma unroll
    for (int i = 0; i < kPer / 4; ++i) {
      const float4 x = reinterpret_cast<const float4*>(row + t)[i];
      v[4 * i] = x.x;
      v[4 * i + 1] = x.y;
      v[4 * i + 2] = x.z;
      v[4 * i + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kPer; ++i) v[i] = (t + i < len) ? row[t + i] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    m[i] = t + i < len && v[i] > th && g0 + t + i < P && tok2slot[g0 + t + i] < 0;
    cnt += m[i];
  }
  *n = cnt;
}

// grid (nch, b1 - b0)
__global__ __launch_bounds__(kT) void early_want_kernel(int group, int b0, const float* __restrict__ logits,
                                                        int64_t ld, const float* __restrict__ theta, int cap,
                                                        const int64_t* __restrict__ tok0,
                                                        const int32_t* __restrict__ lens,
                                                        const int32_t* __restrict__ tok2slot, int64_t P,
                                                        int32_t* ctr, int32_t* __restrict__ stats, EWs ws) {
  __shared__ int scr[kT / 64];
  const int b = b0 + blockIdx.y, c = blockIdx.x;
  const int len = lens[b];
  const float th = theta[b];
  const int t = c * kBlk + threadIdx.x * kPer;
  int n = 0;
  if (th == th && t < len) {
    bool m[kPer];
    miss_flags(logits + (size_t)b * ld, t, len, th, tok0[b], P, tok2slot, m, &n);
  }
  const int tot = ech::block_sum<kT>(n, scr);
  if (threadIdx.x == 0) ws.want[(size_t)b * ws.nch + c] = tot;
  if (!ech::last_block(ctr, gridDim.x * gridDim.y)) return;
  // Rank ranges of the group's sequences, continuing earlier groups.
  // (a) exclusive prefix of the want counts over the group's blocks in
  //     (sequence, chunk) order, stored in off[]
  const int nb = gridDim.y, nch = ws.nch;
  const int E = nb * nch;
  int* off = ws.off + (size_t)b0 * nch;
  const int* want = ws.want + (size_t)b0 * nch;
  int run = 0;
  for (int e0 = 0; e0 < E; e0 += kT) {
    const int e = e0 + threadIdx.x;
    const int v = e < E ? want[e] : 0;
    int t_tot;
    const int ex = ech::block_excl_scan<kT>(v, scr, &t_tot);
    if (e < E) off[e] = run + ex;
    run += t_tot;
  }
  const int want_all = run;
  __syncthreads();
  // (b) per sequence: capped take, rank of its first miss, statistics; the
  //     shift from the raw prefix to the rank goes to seqd[]
  const int start = ws.sc[E_RUN], nfree = ws.sc[E_NFREE];
  int rank_run = start;
  for (int j0 = 0; j0 < nb; j0 += kT) {
    const int j = j0 + threadIdx.x;
    int want_b = 0, raw0 = 0;
    if (j < nb) {
      raw0 = off[j * nch];
      want_b = (j + 1 < nb ? off[(j + 1) * nch] : want_all) - raw0;
    }
    const int take = min(cap, want_b);
    int t_tot;
    const int seq_off = rank_run + ech::block_excl_scan<kT>(j < nb ? take : 0, scr, &t_tot);
    if (j < nb) {
      const int bb = b0 + j;
      ws.seqd[bb] = seq_off - raw0;
      ws.lim[bb] = seq_off + take;
      const int fetched = max(0, min(nfree - seq_off, take));
      stats[4 * bb + 1] = fetched;
      stats[4 * bb + 2] = want_b - fetched;
    }
    rank_run += t_tot;
  }
  __syncthreads();
  // (c) ranks of the blocks' first misses
  for (int e = threadIdx.x; e < E; e += kT) off[e] += ws.seqd[b0 + e / nch];
  if (threadIdx.x == 0) {
    ws.sc[E_RUN] = rank_run;
    ws.grp[2 * group] = min(start, nfree);
    ws.grp[2 * group + 1] = min(rank_run, nfree);
    ctr[ECH_CTR_NWANT] += rank_run - start;
    ctr[ECH_CTR_NMISS_EARLY] = min(rank_run, nfree);
  }
}

// grid (nch, b1 - b0)
__global__ __launch_bounds__(kT) void early_apply_kernel(int group, int b0, const float* __restrict__ logits,
                                                         int64_t ld, const float* __restrict__ theta,
                                                         const int64_t* __restrict__ tok0,
                                                         const int32_t* __restrict__ lens,
                                                         int32_t* __restrict__ tok2slot, int64_t P,
                                                         int32_t* __restrict__ slot2tok,
                                                         int32_t* __restrict__ slot_pin, int32_t C,
                                                         int32_t* __restrict__ miss, int32_t M_early, int32_t* ctr,
                                                         int32_t* __restrict__ stats, EWs ws) {
  __shared__ int scr[kT / 64];
  const int b = b0 + blockIdx.y, c = blockIdx.x;
  const int len = lens[b];
  const float th = theta[b];
  const int t = c * kBlk + threadIdx.x * kPer;
  const int base = ws.off[(size_t)b * ws.nch + c];
  const int lim = min(ws.lim[b], min(ws.grp[2 * group + 1], M_early));
  if (!(th == th) || c * kBlk >= len || base >= lim) return;   // block-uniform
  const int64_t g0 = tok0[b];
  bool m[kPer];
  int n = 0;
  if (t < len) miss_flags(logits + (size_t)b * ld, t, len, th, g0, P, tok2slot, m, &n);
  else
#pragma unroll
    for (int i = 0; i < kPer; ++i) m[i] = false;
  int tot;
  int rank = base + ech::block_excl_scan<kT>(n, scr, &tot);
  const int ep = ws.sc[E_EP];
  const int last = ws.grp[2 * group + 1] - 1;
  int nev = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (m[i] && rank < lim) {
      const int g = (int)(g0 + t + i);
      const int p = ws.freelist[rank];
      if (p < 0 || p >= C) {
        atomicOr(&ctr[ECH_CTR_STATUS], ECH_ST_OVERFLOW);   // unreachable unless counts and ranks disagree
      } else {
        const int u = slot2tok[p];
        if (u >= 0 && u < P) {
          tok2slot[u] = -1;   // evict; the host row stays where it is
          ++nev;
        }
        slot2tok[p] = g;
        tok2slot[g] = p;
        slot_pin[p] = ep;
        miss[2 * rank] = g;
        miss[2 * rank + 1] = p;
        if (rank == last) ctr[ECH_CTR_HEAD] = (p + 1 == C) ? 0 : p + 1;
      }
    }
    rank += m[i] ? 1 : 0;
  }
  // One eviction count per wave (the block serves one sequence b).
  const int wev = ech::wave_sum(nev);
  if (wev > 0 && ech::lane_id() == 0) {
    atomicAdd(&ctr[ECH_CTR_NEVICT], wev);
    atomicAdd(&stats[4 * b + 3], wev);
  }
}

// ------------------------------------------------------------------ recall of a group
constexpr int kRecallUnroll = 8;
constexpr int kRecallBlocks = 48;
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kT) void recall_range_kernel(const v4u* __restrict__ host, int64_t P, int row16,
                                                          v4u* __restrict__ dev, int32_t C,
                                                          const int32_t* __restrict__ miss, int32_t M_max,
                                                          const int* __restrict__ range, int32_t* ctr) {
  const int m0 = max(0, range[0]);
  const int m1 = min(range[1], M_max);
  const int n = max(0, m1 - m0);
  const int64_t total = (int64_t)n * row16;
  const int64_t stride = (int64_t)gridDim.x * kT * kRecallUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kT * kRecallUnroll + threadIdx.x; base < total; base += stride) {
    v4u v[kRecallUnroll];
    int64_t dst[kRecallUnroll];
#pragma unroll
    for (int u = 0; u < kRecallUnroll; ++u) {
      const int64_t i = base + (int64_t)u * kT;
      dst[u] = -1;
      if (i < total) {
        const int m = m0 + (int)(i / row16);
        const int c = (int)(i % row16);
        const int g = miss[2 * m], p = miss[2 * m + 1];
        if (g >= 0 && g < P && p >= 0 && p < C) {
          v[u] = __builtin_nontemporal_load(host + (int64_t)g * row16 + c);
          dst[u] = (int64_t)p * row16 + c;
        } else if (c == 0) {
          atomicOr(&ctr[ECH_CTR_STATUS], ECH_ST_BADMISS);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kRecallUnroll; ++u)
      if (dst[u] >= 0) __builtin_nontemporal_store(v[u], dev + dst[u]);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) atomicAdd(&ctr[ECH_CTR_RECALLED], n);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool ws_ok(void* ws, size_t ws_bytes, int B, int max_len, int32_t C, int32_t M_early) {
  return ws && !(reinterpret_cast<uintptr_t>(ws) & 255u) &&
         ws_bytes >= early_layout(B, max_len, C, M_early, nullptr, nullptr);
}

}  // namespace

extern "C" size_t ech_early_ws_bytes(int B, int max_len, int32_t C, int32_t M_early) {
  if (B < 1 || max_len < 0 || C < 1 || M_early < 0) return 0;
  return early_layout(B, max_len, C, M_early, nullptr, nullptr);
}

extern "C" int ech_early_begin(const void* q, const float* w, const void* kcache, int kdtype, const float* kscale,
                               const int64_t* seq_tok0, const int32_t* seq_len, int B, int max_len,
                               const float* theta, const int32_t* tok2slot, int64_t P, int32_t* slot_pin, int32_t C,
                               int32_t* ctr, int32_t M_early, int32_t* stats, void* ws, size_t ws_bytes,
                               void* stream) {
  if (!q || !w || !kcache || !seq_tok0 || !seq_len || !theta || !tok2slot || !slot_pin || !ctr || !stats)
    return ECH_EINVAL;
  if (kdtype != ECH_KEY_BF16 && kdtype != ECH_KEY_FP8) return ECH_EUNSUPPORTED;
  if (kdtype == ECH_KEY_FP8 && !kscale) return ECH_EINVAL;
  if (!aligned16(q) || !aligned16(kcache)) return ECH_EINVAL;
  if (B < 1 || B > kMaxB || max_len < 0 || P < 1 || P >= INT32_MAX || C < 1 || C > (1 << 30) || M_early < 0)
    return ECH_EINVAL;
  if (!ws_ok(ws, ws_bytes, B, max_len, C, M_early)) return ECH_EINVAL;
  EWs e;
  early_layout(B, max_len, C, M_early, &e, static_cast<char*>(ws));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const dim3 gp(e.nch, B);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint8_t* kk = static_cast<const uint8_t*>(kcache);
  if (kdtype == ECH_KEY_FP8)
    hipLaunchKernelGGL(early_pin_kernel<ECH_KEY_FP8>, gp, dim3(kT), 0, s, qq, w, kk, kscale, seq_tok0, seq_len,
                       theta, tok2slot, P, C, slot_pin, ctr, e);
  else
    hipLaunchKernelGGL(early_pin_kernel<ECH_KEY_BF16>, gp, dim3(kT), 0, s, qq, w, kk, kscale, seq_tok0, seq_len,
                       theta, tok2slot, P, C, slot_pin, ctr, e);
  ECH_LAUNCH_CHECK();
  hipLaunchKernelGGL(early_free_kernel, dim3(e.ns), dim3(kT), 0, s, slot_pin, C, B, ctr, stats, e);
  ECH_LAUNCH_CHECK();
  hipLaunchKernelGGL(early_freelist_kernel, dim3(e.ns), dim3(kT), 0, s, slot_pin, C, M_early, e);
  ECH_LAUNCH_CHECK();
  return ECH_OK;
}

extern "C" int ech_early_group(int group, int b0, int b1, const float* logits, int64_t ld, const float* theta,
                               int cap, const int64_t* seq_tok0, const int32_t* seq_len, int B, int max_len,
                               int32_t* tok2slot, int64_t P, int32_t* slot2tok, int32_t* slot_pin, int32_t C,
                               int32_t* miss_early, int32_t M_early, int32_t* ctr, int32_t* stats, void* ws,
                               size_t ws_bytes, void* stream) {
  if (!logits || !theta || !seq_tok0 || !seq_len || !tok2slot || !slot2tok || !slot_pin || !miss_early || !ctr ||
      !stats)
    return ECH_EINVAL;
  if (group < 0 || group >= kMaxGroups || b0 < 0 || b1 <= b0 || b1 > B) return ECH_EINVAL;
  if (B < 1 || B > kMaxB || max_len < 0 || P < 1 || P >= INT32_MAX || C < 1 || C > (1 << 30) || cap < 0)
    return ECH_EINVAL;
  if (ld < max_len || ld % 4 != 0 || !aligned16(logits)) return ECH_EINVAL;
  if ((int64_t)M_early < (int64_t)B * std::min(cap, max_len)) return ECH_EINVAL;
  if (!ws_ok(ws, ws_bytes, B, max_len, C, M_early)) return ECH_EINVAL;
  EWs e;
  early_layout(B, max_len, C, M_early, &e, static_cast<char*>(ws));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const dim3 gg(e.nch, b1 - b0);
  hipLaunchKernelGGL(early_want_kernel, gg, dim3(kT), 0, s, group, b0, logits, ld, theta, cap, seq_tok0, seq_len,
                     tok2slot, P, ctr, stats, e);
  ECH_LAUNCH_CHECK();
  hipLaunchKernelGGL(early_apply_kernel, gg, dim3(kT), 0, s, group, b0, logits, ld, theta, seq_tok0, seq_len,
                     tok2slot, P, slot2tok, slot_pin, C, miss_early, M_early, ctr, stats, e);
  ECH_LAUNCH_CHECK();
  return ECH_OK;
}

extern "C" int ech_recall_group(int group, const void* host_pool, int64_t P, int64_t row_bytes, void* dev_cache,
                                int32_t C, const int32_t* miss_early, int32_t M_early, int32_t* ctr, const void* ws,
                                void* stream) {
  if (!host_pool || !dev_cache || !miss_early || !ctr || !ws || P < 1 || C < 1 || M_early < 0) return ECH_EINVAL;
  if (group < 0 || group >= kMaxGroups) return ECH_EINVAL;
  if (row_bytes <= 0 || row_bytes % 16 != 0 || row_bytes / 16 > INT32_MAX) return ECH_EINVAL;
  if (!aligned16(host_pool) || !aligned16(dev_cache) || (reinterpret_cast<uintptr_t>(ws) & 255u))
    return ECH_EINVAL;
  void* dptr = nullptr;
  if (hipHostGetDevicePointer(&dptr, const_cast<void*>(host_pool), 0) != hipSuccess || !dptr) {
    (void)hipGetLastError();
    return ECH_EINVAL;
  }
  if (M_early == 0) return ECH_OK;
  // the group ranges sit at a fixed place at the start of the workspace
  EWs e;
  early_layout(1, 0, 1, 0, &e, static_cast<char*>(const_cast<void*>(ws)));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int row16 = (int)(row_bytes / 16);
  const int64_t work = (int64_t)M_early * row16;
  const int blocks = (int)std::max<int64_t>(
      1, std::min<int64_t>(kRecallBlocks, (work + kT * kRecallUnroll - 1) / (kT * kRecallUnroll)));
  hipLaunchKernelGGL(recall_range_kernel, dim3(blocks), dim3(kT), 0, s, static_cast<const v4u*>(dptr), P, row16,
                     static_cast<v4u*>(dev_cache), C, miss_early, M_early, e.grp + 2 * group, ctr);
  ECH_LAUNCH_CHECK();
  return ECH_OK;
}
