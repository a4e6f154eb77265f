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
//     alloc     one workgroup: hits per sequence; the unpinned slots in ring
//               order from the head, as far as the early demand bound needs
//               (window by window), into the free list; advances the epoch.
//   group [b0, b1), in ascending b0, once that group's scores are written
//     want      grid (chunks, b1-b0): each block lists its non-resident tokens
//               above theta, in order.
//     rank      one workgroup: every sequence's rank range (continuing the
//               ranks of earlier groups, capped per sequence) and every
//               block's first rank.
//     apply     grid (chunks, b1-b0): a listed miss of rank m takes
//               freelist[m] (evicting its old token, no write-back) and is
//               written to the miss list at m.
//   recall per group: the rows of the group's rank range.
//
// Only the pins depend on the whole batch, and they involve resident tokens
// only, which the begin step scores itself; the free-slot ranking is then
// fixed for the step, and a group's misses are not changed by earlier groups
// (an earlier group evicts only unpinned slots, i.e. resident tokens at or
// below theta, and maps only its own tokens). So any grouping gives the same
// maps, miss list and statistics as the single phase.

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
  int* want;      // [B * nch] misses per block (all of them)
  int* off;       // [B * nch] rank of the block's first miss
  int* lim;       // [B] rank limit of the sequence (cap)
  int* freelist;  // [M_early]
  int* lmiss;     // [B * nch][kBlk] the block's missed token ids, in order
  int nch;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// sc and grp come first: ech_recall_group finds them without the sizes.
size_t early_layout(int B, int max_len, int32_t C, int32_t M_early, EWs* w, char* base) {
  (void)C;
  const int nch = std::max(1, (max_len + kBlk - 1) / kBlk);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  const size_t o_sc = take(4 * E_NSC), o_grp = take(4 * 2 * kMaxGroups);
  const size_t o_hit = take(4 * (size_t)B * nch), o_want = take(4 * (size_t)B * nch),
               o_off = take(4 * (size_t)B * nch), o_lim = take(4 * (size_t)B),
               o_fl = take(4 * (size_t)std::max(M_early, 1)), o_lm = take(4 * (size_t)B * nch * kBlk);
  if (w && base) {
    w->sc = reinterpret_cast<int*>(base + o_sc);
    w->grp = reinterpret_cast<int*>(base + o_grp);
    w->hitblk = reinterpret_cast<int*>(base + o_hit);
    w->want = reinterpret_cast<int*>(base + o_want);
    w->off = reinterpret_cast<int*>(base + o_off);
    w->lim = reinterpret_cast<int*>(base + o_lim);
    w->freelist = reinterpret_cast<int*>(base + o_fl);
    w->lmiss = reinterpret_cast<int*>(base + o_lm);
    w->nch = nch;
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
  int sl[kPer];   // all sixteen lookups in flight (clamped addresses; only tokens in the row used)
#pragma unroll
  for (int i = 0; i < kPer; ++i) sl[i] = tok2slot[min(max(g0 + t_first + i, (int64_t)0), P - 1)];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int t = t_first + i;
    res[i] = t < len && g0 + t < P && sl[i] >= 0 && sl[i] < C;
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

// ------------------------------------------------------------------ begin: alloc
constexpr int kA = 1024;        // threads of the one-workgroup steps
constexpr int kWin = kA * 16;   // ring positions per window

__global__ __launch_bounds__(kA) void early_alloc_kernel(const int32_t* __restrict__ slot_pin, int32_t C, int B,
                                                         int32_t M_early, int32_t* ctr,
                                                         int32_t* __restrict__ stats, EWs ws) {
  __shared__ int scr[kA / 64];
  __shared__ __align__(16) uint8_t s_fr[kWin];
  const int tid = threadIdx.x;
  const int ep = ctr[ECH_CTR_EPOCH] + 1;
  int head = ctr[ECH_CTR_HEAD];
  if (head < 0 || head >= C) head = 0;   // only a corrupted state; keeps every slot index in range
  // hits per sequence (the pinned slots: one per resident token above theta)
  int hit_all = 0;
  for (int b0 = 0; b0 < B; b0 += kA) {
    const int b = b0 + tid;
    int h = 0;
    if (b < B) {
      const int* hb = ws.hitblk + (size_t)b * ws.nch;
      int c = 0;
      for (; c + 8 <= ws.nch; c += 8) {
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = hb[c + u];   // all in flight
#pragma unroll
        for (int u = 0; u < 8; ++u) h += v[u];
      }
      for (; c < ws.nch; ++c) h += hb[c];
      int32_t* st = stats + 4 * b;
      st[0] = h;
      st[1] = 0;
      st[2] = 0;
      st[3] = 0;
    }
    hit_all += ech::block_sum<kA>(h, scr);
  }
  // free slots in ring order from the head, up to the early demand bound
  int found = 0;
  for (int i0 = 0; i0 < C && found < M_early; i0 += kWin) {   // block-uniform
#pragma unroll
    for (int j = 0; j < kWin / kA; ++j) {   // coalesced loads, all in flight
      const int pos = i0 + j * kA + tid;
      int p = head + min(pos, C - 1);
      if (p >= C) p -= C;
      const int pv = slot_pin[p];
      s_fr[j * kA + tid] = (pos < C && pv != ep) ? 1 : 0;
    }
    __syncthreads();
    const uint4 f0 = reinterpret_cast<const uint4*>(s_fr)[tid];   // positions i0 + 16 tid .. +15
    const uint32_t fw[4] = {f0.x, f0.y, f0.z, f0.w};
    int cnt = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) cnt += __popc(fw[q]);   // flags are 0/1 bytes
    int tot;
    int rank = found + ech::block_excl_scan<kA>(cnt, scr, &tot);
    if (rank < M_early) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if ((fw[q] >> (8 * e)) & 1u) {
            if (rank < M_early) {
              int p = head + i0 + 16 * tid + 4 * q + e;
              if (p >= C) p -= C;
              ws.freelist[rank] = p;
            }
            ++rank;
          }
        }
      }
    }
    found += tot;
    __syncthreads();   // s_fr is rewritten by the next window
  }
  if (tid == 0) {
    ws.sc[E_EP] = ep;
    ws.sc[E_NFREE] = min(found, M_early);   // the free slots any rank can take
    ws.sc[E_RUN] = 0;
    ws.sc[E_HEAD0] = head;
    ctr[ECH_CTR_EPOCH] = ep;
    ctr[ECH_CTR_NPINNED] = hit_all;
    ctr[ECH_CTR_NEVICT] = 0;
    ctr[ECH_CTR_NWANT] = 0;
    ctr[ECH_CTR_NMISS_EARLY] = 0;
  }
}

// ------------------------------------------------------------------ group
// grid (nch, b1 - b0): 16 consecutive tokens per thread; a miss is a
// non-resident token above theta (strict) inside the row. The block's
// misses are listed in order and counted.
__global__ __launch_bounds__(kT) void early_want_kernel(int b0, const float* __restrict__ logits, int64_t ld,
                                                        const float* __restrict__ theta,
                                                        const int64_t* __restrict__ tok0,
                                                        const int32_t* __restrict__ lens,
                                                        const int32_t* __restrict__ tok2slot, int64_t P, EWs ws) {
  __shared__ int scr[kT / 64];
  const int b = b0 + blockIdx.y, c = blockIdx.x;
  const size_t blk = (size_t)b * ws.nch + c;
  const int len = lens[b];
  const float th = theta[b];
  const int t = c * kBlk + threadIdx.x * kPer;
  const int64_t g0 = tok0[b] + t;
  uint32_t mm = 0;
  int n = 0;
  if (th == th && t < len) {
    const float* row = logits + (size_t)b * ld;
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
    uint32_t above = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) above |= (t + i < len && v[i] > th && g0 + i < P) ? 1u << i : 0u;
    if (above) {
      int sl[kPer];   // all sixteen lookups in flight (clamped addresses; only flagged ones used)
#pragma unroll
      for (int i = 0; i < kPer; ++i) sl[i] = tok2slot[min(max(g0 + i, (int64_t)0), P - 1)];
#pragma unroll
      for (int i = 0; i < kPer; ++i) mm |= (((above >> i) & 1u) && sl[i] < 0) ? 1u << i : 0u;
      n = __popc(mm);
    }
  }
  int tot;
  int r = ech::block_excl_scan<kT>(n, scr, &tot);
  for (; mm != 0u; mm &= mm - 1u, ++r) ws.lmiss[blk * kBlk + r] = (int)(g0 + __builtin_ctz(mm));
  if (threadIdx.x == 0) ws.want[blk] = tot;
}

// One workgroup: rank ranges of the group's sequences, continuing earlier
// groups; every block's first rank; statistics; the group's range.
__global__ __launch_bounds__(kA) void early_rank_kernel(int group, int b0, int nb, int cap, int32_t* ctr,
                                                        int32_t* __restrict__ stats, EWs ws) {
  __shared__ int scr[kA / 64];
  __shared__ int s_seg[kMaxB + 1], s_off[kMaxB];
  const int tid = threadIdx.x;
  const int nch = ws.nch;
  const int n = nb * nch;
  const int* want = ws.want + (size_t)b0 * nch;
  int* off = ws.off + (size_t)b0 * nch;
  // flat exclusive scan of the group's block counts (sequence-major), four
  // blocks per thread; each sequence's first block leaves its prefix in s_seg
  int wv[4], ew[4];
  int run = 0;
  for (int i0 = 0; i0 < n; i0 += 4 * kA) {
    const int i = i0 + 4 * tid;
    int sum = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      wv[u] = want[min(i + u, n - 1)];
      if (i + u >= n) wv[u] = 0;
      sum += wv[u];
    }
    int tot;
    int pw = run + ech::block_excl_scan<kA>(sum, scr, &tot);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      ew[u] = pw;
      if (i + u < n && (i + u) % nch == 0) s_seg[(i + u) / nch] = pw;
      pw += wv[u];
    }
    run += tot;
  }
  if (tid == 0) s_seg[nb] = run;
  __syncthreads();
  // per sequence: capped take, rank of its first miss, statistics
  const int start = ws.sc[E_RUN], nfree = ws.sc[E_NFREE];
  int rank_run = start;
  for (int j0 = 0; j0 < nb; j0 += kA) {
    const int j = j0 + tid;
    int take = 0, want_b = 0;
    if (j < nb) {
      want_b = s_seg[j + 1] - s_seg[j];
      take = min(cap, want_b);
    }
    int tot;
    const int seq_off = rank_run + ech::block_excl_scan<kA>(take, scr, &tot);
    if (j < nb) {
      const int bb = b0 + j;
      s_off[j] = seq_off;
      ws.lim[bb] = seq_off + take;
      const int fetched = max(0, min(nfree - seq_off, take));
      stats[4 * bb + 1] = fetched;
      stats[4 * bb + 2] = want_b - fetched;
    }
    rank_run += tot;
  }
  __syncthreads();
  // every block's first rank
  if (n <= 4 * kA) {
    const int i = 4 * tid;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i + u < n) off[i + u] = s_off[(i + u) / nch] + (ew[u] - s_seg[(i + u) / nch]);
  } else {
    run = 0;   // the same scan again
    for (int i0 = 0; i0 < n; i0 += 4 * kA) {
      const int i = i0 + 4 * tid;
      int sum = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        wv[u] = want[min(i + u, n - 1)];
        if (i + u >= n) wv[u] = 0;
        sum += wv[u];
      }
      int tot;
      int pw = run + ech::block_excl_scan<kA>(sum, scr, &tot);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (i + u < n) off[i + u] = s_off[(i + u) / nch] + (pw - s_seg[(i + u) / nch]);
        pw += wv[u];
      }
      run += tot;
    }
  }
  if (tid == 0) {
    ws.sc[E_RUN] = rank_run;
    ws.grp[2 * group] = min(start, nfree);
    ws.grp[2 * group + 1] = min(rank_run, nfree);
    ctr[ECH_CTR_NWANT] += rank_run - start;
    ctr[ECH_CTR_NMISS_EARLY] = min(rank_run, nfree);
  }
}

// grid (nch, b1 - b0): block (c, j) places its listed misses by rank.
__global__ __launch_bounds__(kT) void early_apply_kernel(int group, int b0, int32_t* __restrict__ tok2slot,
                                                         int64_t P, int32_t* __restrict__ slot2tok, int32_t C,
                                                         int32_t* __restrict__ miss, int32_t M_early, int32_t* ctr,
                                                         int32_t* __restrict__ stats, EWs ws) {
  const int b = b0 + blockIdx.y, c = blockIdx.x;
  const size_t blk = (size_t)b * ws.nch + c;
  const int cnt = min(ws.want[blk], kBlk);
  const int base = ws.off[blk];
  const int lim = min(ws.lim[b], min(ws.grp[2 * group + 1], M_early));
  if (cnt == 0 || base >= lim) return;   // block-uniform
  const int last = ws.grp[2 * group + 1] - 1;
  for (int i = threadIdx.x; i < cnt; i += kT) {   // trips differ only in the last pass
    const int m = base + i;
    bool evicted = false;
    if (m < lim) {
      const int g = ws.lmiss[blk * kBlk + i];
      const int p = ws.freelist[m];
      if (g < 0 || g >= P || p < 0 || p >= C) {
        atomicOr(&ctr[ECH_CTR_STATUS], ECH_ST_OVERFLOW);   // unreachable unless counts and lists disagree
      } else {
        const int u = slot2tok[p];
        if (u >= 0 && u < P) {
          tok2slot[u] = -1;   // evict; the host row stays where it is
          evicted = true;
        }
        slot2tok[p] = g;
        tok2slot[g] = p;
        miss[2 * m] = g;
        miss[2 * m + 1] = p;
        if (m == last) ctr[ECH_CTR_HEAD] = (p + 1 == C) ? 0 : p + 1;
      }
    }
    ech::wave_count(&ctr[ECH_CTR_NEVICT], evicted);
    ech::wave_count(&stats[4 * b + 3], evicted);
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
  hipLaunchKernelGGL(early_alloc_kernel, dim3(1), dim3(kA), 0, s, slot_pin, C, B, M_early, ctr, stats, e);
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
  hipLaunchKernelGGL(early_want_kernel, gg, dim3(kT), 0, s, b0, logits, ld, theta, seq_tok0, seq_len, tok2slot, P,
                     e);
  ECH_LAUNCH_CHECK();
  hipLaunchKernelGGL(early_rank_kernel, dim3(1), dim3(kA), 0, s, group, b0, b1 - b0, cap, ctr, stats, e);
  ECH_LAUNCH_CHECK();
  hipLaunchKernelGGL(early_apply_kernel, gg, dim3(kT), 0, s, group, b0, tok2slot, P, slot2tok, C, miss_early,
                     M_early, ctr, stats, e);
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
