// GPU-resident per-layer slot map and recall (ECHO explainer: "One layer, one
// step: free -> allocate -> recall", "Five fixed-size integer tensors on the
// GPU", "Decode: fetch above a predicted threshold").
//
// A phase is a fixed sequence of kernels with grids sized from host-known
// maxima; every data-dependent count lives in device memory, so the phase can
// be captured in a hipGraph and replayed.
//
//   pin      mark the slots of the phase's resident selection with the new
//            epoch (slot_pin[s] = epoch) and count hits / wanted misses per
//            block. EARLY: tokens with score > theta; FINAL: idx entries;
//            PREFILL: idx entries of all rows, misses claimed once per token
//            by marking tok2slot -1 -> -2 (union), then counted by a
//            token scan.
//   free     count unpinned slots per block in ring order from the head.
//   scan     one workgroup: exclusive scans of the block counts give every
//            miss its rank (ascending sequence, token; EARLY keeps the first
//            `cap` per sequence) and every free slot its rank in ring order;
//            n_alloc = min(wanted, free). Writes stats and counters.
//   emit     recompute the same flags in order: miss of rank m -> mcand[m],
//            free slot of rank m -> freelist[m].
//   apply    miss m takes freelist[m]: the slot's old token is unmapped (no
//            write-back), the maps point at each other, miss[m] = (g, slot).
// Ranks come from scans, not from atomics, so the maps are a deterministic
// function of the inputs: bit-identical run to run.

#include <algorithm>

#include "common.hpp"

namespace {

constexpr int kT = 256;
constexpr int kPer = 16;
constexpr int kBlk = kT * kPer;   // tokens or slots per block in ordered kernels
constexpr int kMaxK = 4096;
constexpr int kMaxB = 1024;

enum { S_EP = 0, S_NWANT = 1, S_NALLOC = 2, S_HEAD = 3, S_NFREE = 4, S_N = 16 };

struct CWs {
  int* want;     // [ne] wanted misses per entry block
  int* hit;      // [ne] hits per entry block
  int* off;      // [ne] rank of the block's first miss
  int* lim;      // [ne] rank limit of the block's sequence (EARLY cap)
  int* nfree;    // [ns] unpinned slots per slot block
  int* soff;     // [ns] rank of the block's first free slot
  int* freelist; // [M_max]
  int2* mcand;   // [M_max] (g, aux): aux = entry index (FINAL), sequence (EARLY), 0 (PREFILL)
  int* sc;       // [S_N] scalars
  int ne, ns, nbr;  // entry blocks, slot blocks, entry blocks per sequence
  int P, C, M_max;  // bounds every index is checked against
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

void block_counts(int phase, int B, int R, int k, int max_len, int32_t C, int* ne, int* ns, int* nbr) {
  const int nbj = (k + kT - 1) / kT;
  const int nch = std::max(1, (max_len + kBlk - 1) / kBlk);
  if (phase == ECH_FINAL) {
    *nbr = nbj;
    *ne = B * nbj;
  } else if (phase == ECH_EARLY) {
    *nbr = nch;
    *ne = B * nch;
  } else {
    *nbr = nch;
    *ne = nch;
  }
  (void)R;
  *ns = (int)((C + kBlk - 1) / kBlk);
}

size_t layout(int phase, int B, int R, int k, int max_len, int32_t C, int32_t M_max, CWs* w, char* base) {
  int ne, ns, nbr;
  block_counts(phase, B, R, k, max_len, C, &ne, &ns, &nbr);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  size_t o_want = take(4 * (size_t)ne), o_hit = take(4 * (size_t)ne), o_off = take(4 * (size_t)ne),
         o_lim = take(4 * (size_t)ne), o_nf = take(4 * (size_t)ns), o_so = take(4 * (size_t)ns),
         o_fl = take(4 * (size_t)M_max), o_mc = take(8 * (size_t)M_max), o_sc = take(4 * S_N);
  if (w && base) {
    w->want = reinterpret_cast<int*>(base + o_want);
    w->hit = reinterpret_cast<int*>(base + o_hit);
    w->off = reinterpret_cast<int*>(base + o_off);
    w->lim = reinterpret_cast<int*>(base + o_lim);
    w->nfree = reinterpret_cast<int*>(base + o_nf);
    w->soff = reinterpret_cast<int*>(base + o_so);
    w->freelist = reinterpret_cast<int*>(base + o_fl);
    w->mcand = reinterpret_cast<int2*>(base + o_mc);
    w->sc = reinterpret_cast<int*>(base + o_sc);
    w->ne = ne;
    w->ns = ns;
    w->nbr = nbr;
  }
  return o;
}

__device__ __forceinline__ void set_status(int32_t* ctr, int bit) { atomicOr(&ctr[ECH_CTR_STATUS], bit); }

// ------------------------------------------------------------------ pin / count
// FINAL: grid (nbj, B), one idx entry per thread.
__global__ __launch_bounds__(kT) void pin_final_kernel(const int32_t* __restrict__ idx, int k,
                                                       const int64_t* __restrict__ tok0,
                                                       const int32_t* __restrict__ lens,
                                                       const int32_t* __restrict__ tok2slot,
                                                       int32_t* __restrict__ slot_pin, int32_t* __restrict__ sel_slot,
                                                       int32_t* ctr, CWs w) {
  __shared__ int scr[kT / 64];
  const int b = blockIdx.y, j = blockIdx.x * kT + threadIdx.x;
  const int ep = ctr[ECH_CTR_EPOCH] + 1;
  int hit = 0, miss = 0;
  if (j < k) {
    const size_t e = (size_t)b * k + j;
    const int t = idx[e];
    int sl = -1;
    if (t >= 0) {
      if (t >= lens[b]) {
        set_status(ctr, ECH_ST_BADTOK);
      } else {
        const int64_t g = tok0[b] + t;
        if (g < 0 || g >= w.P) {
          set_status(ctr, ECH_ST_BADTOK);
        } else {
          sl = tok2slot[g];
          if (sl >= 0 && sl < w.C) {
            slot_pin[sl] = ep;
            hit = 1;
          } else {
            sl = -1;
            miss = 1;
          }
        }
      }
    }
    sel_slot[e] = sl;
  }
  const int nh = ech::block_sum<kT>(hit, scr);
  const int nm = ech::block_sum<kT>(miss, scr);
  if (threadIdx.x == 0) {
    const int blk = b * gridDim.x + blockIdx.x;
    w.hit[blk] = nh;
    w.want[blk] = nm;
  }
}

// EARLY: grid (nch, B), 16 consecutive tokens per thread.
__device__ __forceinline__ void load16(const float* p, int t, int len, float (&v)[kPer]) {
  if (t + kPer <= len) {
#pragma unroll
    for (int i = 0; i < kPer / 4; ++i) {
      const float4 x = reinterpret_cast<const float4*>(p + t)[i];
      v[4 * i] = x.x;
      v[4 * i + 1] = x.y;
      v[4 * i + 2] = x.z;
      v[4 * i + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kPer; ++i) v[i] = (t + i < len) ? p[t + i] : 0.f;
  }
}

__global__ __launch_bounds__(kT) void pin_early_kernel(const float* __restrict__ logits, int64_t ld,
                                                       const float* __restrict__ theta,
                                                       const int64_t* __restrict__ tok0,
                                                       const int32_t* __restrict__ lens,
                                                       const int32_t* __restrict__ tok2slot,
                                                       int32_t* __restrict__ slot_pin, int32_t* ctr, CWs w) {
  __shared__ int scr[kT / 64];
  const int b = blockIdx.y;
  const int len = lens[b];
  const float th = theta[b];
  const int ep = ctr[ECH_CTR_EPOCH] + 1;
  const int t = blockIdx.x * kBlk + threadIdx.x * kPer;
  int hit = 0, want = 0;
  if (th == th && t < len) {
    float v[kPer];
    load16(logits + (size_t)b * ld, t, len, v);
    const int64_t g0 = tok0[b] + t;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (t + i < len && v[i] > th && g0 + i < w.P) {
        const int sl = tok2slot[g0 + i];
        if (sl >= 0 && sl < w.C) {
          slot_pin[sl] = ep;
          ++hit;
        } else {
          ++want;
        }
      }
    }
  }
  const int nh = ech::block_sum<kT>(hit, scr);
  const int nw = ech::block_sum<kT>(want, scr);
  if (threadIdx.x == 0) {
    const int blk = b * gridDim.x + blockIdx.x;
    w.hit[blk] = nh;
    w.want[blk] = nw;
  }
}

// PREFILL: grid (nbj, R). Pins resident tokens of every row; marks each
// missing token as claimed (tok2slot -1 -> -2) so the union has no
// duplicates. Many rows select the same tokens; a plain store suffices since
// every claimer stores the same value and nothing else writes these entries
// during the kernel (an atomic compare-and-swap serialised the duplicates).
__global__ __launch_bounds__(kT) void pin_prefill_kernel(const int32_t* __restrict__ idx, int k,
                                                         const int64_t* __restrict__ tok0p,
                                                         const int32_t* __restrict__ lenp,
                                                         int32_t* __restrict__ tok2slot,
                                                         int32_t* __restrict__ slot_pin, int32_t* ctr, CWs w) {
  const int r = blockIdx.y, j = blockIdx.x * kT + threadIdx.x;
  if (j >= k) return;
  const int64_t tok0 = tok0p[0];
  const int len = lenp[0];
  const int t = idx[(size_t)r * k + j];
  if (t < 0) return;
  const int64_t g = tok0 + t;
  if (t >= len || g >= w.P) {
    set_status(ctr, ECH_ST_BADTOK);
    return;
  }
  const int ep = ctr[ECH_CTR_EPOCH] + 1;
  const int sl = tok2slot[g];
  if (sl >= 0 && sl < w.C) slot_pin[sl] = ep;
  else if (sl == -1) tok2slot[g] = -2;   // every claimer writes the same value: no atomic needed
}

// PREFILL: grid (nch), count claimed tokens per block of the token range.
__global__ __launch_bounds__(kT) void count_claimed_kernel(const int64_t* __restrict__ tok0p,
                                                           const int32_t* __restrict__ lenp,
                                                           const int32_t* __restrict__ tok2slot, CWs w) {
  __shared__ int scr[kT / 64];
  const int64_t tok0 = tok0p[0];
  const int len = lenp[0];
  const int t = blockIdx.x * kBlk + threadIdx.x * kPer;
  int n = 0;
  for (int i = 0; i < kPer; ++i)
    if (t + i < len && tok0 + t + i < w.P && tok2slot[tok0 + t + i] == -2) ++n;
  const int tot = ech::block_sum<kT>(n, scr);
  if (threadIdx.x == 0) {
    w.want[blockIdx.x] = tot;
    w.hit[blockIdx.x] = 0;
  }
}

// grid (ns): unpinned slots per block, ring positions i -> slot (head + i) % C.
__global__ __launch_bounds__(kT) void count_free_kernel(const int32_t* __restrict__ slot_pin, int32_t C,
                                                        const int32_t* ctr, CWs w) {
  __shared__ int scr[kT / 64];
  const int head = ctr[ECH_CTR_HEAD];
  const int ep = ctr[ECH_CTR_EPOCH] + 1;
  const int i0 = blockIdx.x * kBlk + threadIdx.x * kPer;
  int n = 0;
  for (int i = 0; i < kPer; ++i) {
    const int pos = i0 + i;
    if (pos < C) {
      int p = head + pos;
      if (p >= C) p -= C;
      n += slot_pin[p] != ep;
    }
  }
  const int tot = ech::block_sum<kT>(n, scr);
  if (threadIdx.x == 0) w.nfree[blockIdx.x] = tot;
}

// ------------------------------------------------------------------ scan

template <int NT>
__global__ __launch_bounds__(NT) void scan_kernel(int phase, int B, int cap, int32_t C, int32_t* ctr,
                                                   int32_t* __restrict__ stats, CWs w) {
  __shared__ int scr[NT / 64];
  __shared__ int s_rowoff[NT], s_take[NT], s_seg[NT];
  // free slots: exclusive scan over slot blocks (chunks of NT)
  int nfree_tot = 0;
  for (int b0 = 0; b0 < w.ns; b0 += NT) {
    const int i = b0 + threadIdx.x;
    const int v = i < w.ns ? w.nfree[i] : 0;
    int tot;
    const int ex = ech::block_excl_scan<NT>(v, scr, &tot);
    if (i < w.ns) w.soff[i] = nfree_tot + ex;
    nfree_tot += tot;
  }
  // misses: the entry blocks are sequence-major (b * nbr + c). One flat
  // exclusive scan of the want counts gives every block's prefix (kept in off
  // for now) and, at the segment boundaries, every sequence's total; the hit
  // counts get the same scan (prefixes kept in lim for now). All threads
  // take part, however many blocks a sequence has.
  const int nseq = (phase == ECH_PREFILL) ? 1 : B;
  const int n = nseq * w.nbr;
  int want_all = 0, hit_all = 0;
  for (int i0 = 0; i0 < n; i0 += NT) {
    const int i = i0 + threadIdx.x;
    int tw, th;
    const int ew = ech::block_excl_scan<NT>(i < n ? w.want[i] : 0, scr, &tw);
    const int eh = ech::block_excl_scan<NT>(i < n ? w.hit[i] : 0, scr, &th);
    if (i < n) {
      w.off[i] = want_all + ew;
      w.lim[i] = hit_all + eh;
    }
    want_all += tw;
    hit_all += th;
  }
  __syncthreads();   // the prefixes in off and lim are read across threads below
  const int b = threadIdx.x;
  int want_b = 0, hit_b = 0, seg = 0;
  if (b < nseq) {
    seg = w.off[b * w.nbr];
    want_b = (b + 1 < nseq ? w.off[(b + 1) * w.nbr] : want_all) - seg;
    hit_b = (b + 1 < nseq ? w.lim[(b + 1) * w.nbr] : hit_all) - w.lim[b * w.nbr];
  }
  const int take_b = (phase == ECH_EARLY) ? min(cap, want_b) : want_b;
  int n_want;
  const int row_off = ech::block_excl_scan<NT>(b < nseq ? take_b : 0, scr, &n_want);
  const bool clamped = n_want > w.M_max;   // only when a caller contract is broken
  if (clamped) n_want = w.M_max;
  const int n_alloc = min(n_want, nfree_tot);
  if (b < nseq) {
    s_rowoff[b] = row_off;
    s_take[b] = take_b;
    s_seg[b] = seg;
  }
  __syncthreads();
  // every block: its first miss's rank and its sequence's rank limit
  for (int i = threadIdx.x; i < n; i += NT) {
    const int bi = i / w.nbr;
    w.off[i] = s_rowoff[bi] + (w.off[i] - s_seg[bi]);
    w.lim[i] = s_rowoff[bi] + s_take[bi];
  }
  if (b < nseq) {
    const int fetched = max(0, min(n_alloc - row_off, take_b));
    int32_t* s = stats + 4 * b;
    if (phase == ECH_PREFILL) {
      s[0] = C - nfree_tot;          // resident union tokens = pinned slots
    } else {
      s[0] = hit_b;
    }
    s[1] = fetched;
    s[2] = want_b - fetched;
    s[3] = 0;
  }
  if (threadIdx.x == 0) {
    const int ep = ctr[ECH_CTR_EPOCH] + 1;
    w.sc[S_EP] = ep;
    w.sc[S_NWANT] = n_want;
    w.sc[S_NALLOC] = n_alloc;
    w.sc[S_HEAD] = ctr[ECH_CTR_HEAD];
    w.sc[S_NFREE] = nfree_tot;
    ctr[phase == ECH_EARLY ? ECH_CTR_NMISS_EARLY : ECH_CTR_NMISS] = n_alloc;
    ctr[ECH_CTR_NWANT] = n_want;
    ctr[ECH_CTR_NPINNED] = C - nfree_tot;
    ctr[ECH_CTR_NEVICT] = 0;
    if ((phase != ECH_EARLY && n_want > nfree_tot) || clamped) ctr[ECH_CTR_STATUS] |= ECH_ST_OVERFLOW;
  }
}

// ------------------------------------------------------------------ emit
// Blocks [0, ne) are entry blocks, [ne, ne + ns) slot blocks.
struct EmitArgs {
  int phase;
  const int32_t* idx;
  int k;
  const int64_t* tok0;
  const int32_t* lens;
  const float* logits;
  int64_t ld;
  const float* theta;
  const int32_t* tok2slot;
  const int32_t* slot_pin;
  int32_t C;
  int nbj;
};

__global__ __launch_bounds__(kT) void emit_kernel(EmitArgs a, CWs w) {
  __shared__ int scr[kT / 64];
  const int n_want = w.sc[S_NWANT];
  const int n_alloc = w.sc[S_NALLOC];
  if ((int)blockIdx.x >= w.ne) {
    // ---- slot role
    const int sb = blockIdx.x - w.ne;
    const int head = w.sc[S_HEAD], ep = w.sc[S_EP];
    const int i0 = sb * kBlk + threadIdx.x * kPer;
    bool fr[kPer];
    int n = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int pos = i0 + i;
      fr[i] = false;
      if (pos < a.C) {
        int p = head + pos;
        if (p >= a.C) p -= a.C;
        fr[i] = a.slot_pin[p] != ep;
      }
      n += fr[i];
    }
    int tot;
    int rank = w.soff[sb] + ech::block_excl_scan<kT>(n, scr, &tot);
    if (w.soff[sb] >= n_alloc) return;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (!fr[i]) continue;
      if (rank < n_alloc) {
        int p = head + i0 + i;
        if (p >= a.C) p -= a.C;
        w.freelist[rank] = p;
        if (rank == n_alloc - 1) w.sc[S_HEAD] = (p + 1 == a.C) ? 0 : p + 1;
      }
      ++rank;
    }
    return;
  }
  // ---- entry role
  const int blk = blockIdx.x;
  const int base = w.off[blk], lim = w.lim[blk];
  if (a.phase == ECH_FINAL) {
    const int b = blk / a.nbj, jb = blk % a.nbj;
    const int j = jb * kT + threadIdx.x;
    int g = -1;
    bool m = false;
    size_t e = 0;
    if (j < a.k) {
      e = (size_t)b * a.k + j;
      const int t = a.idx[e];
      if (t >= 0 && t < a.lens[b] && a.tok0[b] + t < w.P) {
        g = (int)(a.tok0[b] + t);
        m = a.tok2slot[g] < 0;
      }
    }
    int tot;
    const int rank = base + ech::block_excl_scan<kT>(m ? 1 : 0, scr, &tot);
    if (m && rank < lim && rank < w.M_max) w.mcand[rank] = make_int2(g, (int)e);
    (void)n_want;
    return;
  }
  // EARLY / PREFILL: 16 consecutive tokens per thread
  const int b = (a.phase == ECH_EARLY) ? blk / w.nbr : 0;
  const int c = (a.phase == ECH_EARLY) ? blk % w.nbr : blk;
  const int t = c * kBlk + threadIdx.x * kPer;
  bool m[kPer];
  int n = 0;
  int64_t g0;
  if (a.phase == ECH_EARLY) {
    const int len = a.lens[b];
    const float th = a.theta[b];
    g0 = a.tok0[b] + t;
    float v[kPer];
    const bool live = th == th && t < len;
    if (live) load16(a.logits + (size_t)b * a.ld, t, len, v);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      m[i] = live && t + i < len && v[i] > th && g0 + i < w.P && a.tok2slot[g0 + i] < 0;
      n += m[i];
    }
  } else {
    const int plen = a.lens[0];
    g0 = a.tok0[0] + t;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      m[i] = t + i < plen && g0 + i < w.P && a.tok2slot[g0 + i] == -2;
      n += m[i];
    }
  }
  int tot;
  int rank = base + ech::block_excl_scan<kT>(n, scr, &tot);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (!m[i]) continue;
    if (rank < lim && rank < w.M_max) w.mcand[rank] = make_int2((int)(g0 + i), b);
    ++rank;
  }
}

// ------------------------------------------------------------------ apply
__global__ __launch_bounds__(kT) void apply_kernel(int phase, int k, int nseq, int32_t* __restrict__ tok2slot,
                                                   int32_t* __restrict__ slot2tok, int32_t* __restrict__ slot_pin,
                                                   int32_t* __restrict__ miss, int32_t* ctr,
                                                   int32_t* __restrict__ sel_slot, int32_t* __restrict__ stats,
                                                   CWs w) {
  const int n_want = w.sc[S_NWANT];
  const int n_alloc = w.sc[S_NALLOC];
  const int ep = w.sc[S_EP];
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    ctr[ECH_CTR_EPOCH] = ep;
    if (n_alloc > 0) ctr[ECH_CTR_HEAD] = w.sc[S_HEAD];
  }
  for (int m = blockIdx.x * kT + threadIdx.x; m < n_want; m += gridDim.x * kT) {
    const int2 mc = w.mcand[m];
    const int g = mc.x;
    const int owner = (phase == ECH_FINAL) ? mc.y / k : (phase == ECH_EARLY ? mc.y : 0);
    if (g < 0 || g >= w.P || owner < 0 || owner >= nseq || (phase == ECH_FINAL && mc.y >= nseq * k)) {
      set_status(ctr, ECH_ST_OVERFLOW);   // unreachable unless counts and ranks disagree
      continue;
    }
    if (m < n_alloc) {
      const int p = w.freelist[m];
      if (p < 0 || p >= w.C) {
        set_status(ctr, ECH_ST_OVERFLOW);
        continue;
      }
      const int u = slot2tok[p];
      if (u >= 0 && u < w.P) {
        tok2slot[u] = -1;   // evict; the host row stays where it is
        atomicAdd(&ctr[ECH_CTR_NEVICT], 1);
        atomicAdd(&stats[4 * owner + 3], 1);
      }
      slot2tok[p] = g;
      tok2slot[g] = p;
      slot_pin[p] = ep;
      miss[2 * m] = g;
      miss[2 * m + 1] = p;
      if (phase == ECH_FINAL) sel_slot[mc.y] = p;
    } else if (phase == ECH_PREFILL) {
      tok2slot[g] = -1;     // release the claim of a miss that got no slot
    }
  }
}

// PREFILL: sel_slot for every row entry once the maps are final.
__global__ __launch_bounds__(kT) void selfill_kernel(const int32_t* __restrict__ idx, int k,
                                                     const int64_t* __restrict__ tok0p,
                                                     const int32_t* __restrict__ lenp,
                                                     const int32_t* __restrict__ tok2slot, int64_t P,
                                                     int32_t* __restrict__ sel_slot) {
  const int r = blockIdx.y, j = blockIdx.x * kT + threadIdx.x;
  if (j >= k) return;
  const int64_t tok0 = tok0p[0];
  const int len = lenp[0];
  const size_t e = (size_t)r * k + j;
  const int t = idx[e];
  sel_slot[e] = (t >= 0 && t < len && tok0 + t < P) ? tok2slot[tok0 + t] : -1;
}

// ------------------------------------------------------------------ reset / recall
__global__ void reset_kernel(int32_t* tok2slot, int64_t P, int32_t* slot2tok, int32_t* slot_pin, int32_t C,
                             int32_t* ctr) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < P; i += stride) tok2slot[i] = -1;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < C; i += stride) {
    slot2tok[i] = -1;
    slot_pin[i] = 0;
  }
  if (blockIdx.x == 0 && threadIdx.x < ECH_CTR_LEN) ctr[threadIdx.x] = 0;
}

constexpr int kRecallUnroll = 8;
constexpr int kRecallBlocks = 48;
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kT) void recall_kernel(const v4u* __restrict__ host, int64_t P, int row16,
                                                    v4u* __restrict__ dev, int32_t C,
                                                    const int32_t* __restrict__ miss, int32_t* ctr, int cidx,
                                                    int32_t M_max) {
  const int n = min(ctr[cidx], M_max);
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
        const int m = (int)(i / row16);
        const int c = (int)(i - (int64_t)m * row16);
        const int g = miss[2 * m], p = miss[2 * m + 1];
        if (g >= 0 && g < P && p >= 0 && p < C) {
          v[u] = __builtin_nontemporal_load(host + (int64_t)g * row16 + c);
          dst[u] = (int64_t)p * row16 + c;
        } else if (c == 0) {
          set_status(ctr, ECH_ST_BADMISS);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kRecallUnroll; ++u)
      if (dst[u] >= 0) __builtin_nontemporal_store(v[u], dev + dst[u]);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) atomicAdd(&ctr[ECH_CTR_RECALLED], n);
}

}  // namespace

extern "C" int ech_cache_reset(int32_t* tok2slot, int64_t P, int32_t* slot2tok, int32_t* slot_pin, int32_t C,
                               int32_t* ctr, void* stream) {
  if (!tok2slot || !slot2tok || !slot_pin || !ctr || P < 1 || C < 1 || P >= INT32_MAX) return ECH_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t n = std::max<int64_t>(P, C);
  const int blocks = (int)std::min<int64_t>(4096, (n + kT - 1) / kT);
  hipLaunchKernelGGL(reset_kernel, dim3(blocks), dim3(kT), 0, s, tok2slot, P, slot2tok, slot_pin, C, ctr);
  ECH_LAUNCH_CHECK();
  return ECH_OK;
}

extern "C" size_t ech_cache_step_ws_bytes(int phase, int B, int R, int k, int max_len, int32_t C, int32_t M_max) {
  if (phase < ECH_EARLY || phase > ECH_PREFILL || B < 1 || k < 1 || max_len < 0 || C < 1 || M_max < 0) return 0;
  return layout(phase, B, R, k, max_len, C, M_max, nullptr, nullptr);
}

extern "C" int ech_cache_step(int phase, int32_t* tok2slot, int64_t P, int32_t* slot2tok, int32_t* slot_pin,
                              int32_t C, int32_t* miss, int32_t M_max, int32_t* ctr, const int64_t* seq_tok0,
                              const int32_t* seq_len, int B, int max_len, const int32_t* idx, int R, int k,
                              const float* logits, int64_t ld, const float* theta, int cap, int32_t* sel_slot,
                              int32_t* stats, void* ws, size_t ws_bytes, void* stream) {
  if (phase != ECH_EARLY && phase != ECH_FINAL && phase != ECH_PREFILL) return ECH_EINVAL;
  if (!tok2slot || !slot2tok || !slot_pin || !miss || !ctr || !stats || !ws) return ECH_EINVAL;
  if (P < 1 || P >= INT32_MAX || C < 1 || C > (1 << 30) || M_max < 0) return ECH_EINVAL;
  if (B < 1 || B > kMaxB || k < 1 || k > kMaxK || max_len < 0) return ECH_EINVAL;
  if (reinterpret_cast<uintptr_t>(ws) & 255u) return ECH_EINVAL;
  int64_t demand = 0;
  if (phase == ECH_EARLY) {
    if (!logits || !theta || !seq_tok0 || !seq_len || cap < 0 || ld < max_len || ld % 4 != 0) return ECH_EINVAL;
    if (reinterpret_cast<uintptr_t>(logits) & 15u) return ECH_EINVAL;
    demand = (int64_t)B * std::min(cap, max_len);
  } else if (phase == ECH_FINAL) {
    if (!idx || !sel_slot || !seq_tok0 || !seq_len || R != B) return ECH_EINVAL;
    demand = (int64_t)B * std::min(k, max_len);
    if (demand > C) return ECH_ENOSPC;
  } else {
    if (!idx || !sel_slot || !seq_tok0 || B != 1 || R < 1 || R > 65535) return ECH_EINVAL;
    demand = std::min<int64_t>(max_len, (int64_t)R * k);
    if (demand > C) return ECH_ENOSPC;
  }
  if ((int64_t)M_max < demand) return ECH_EINVAL;
  if (ws_bytes < ech_cache_step_ws_bytes(phase, B, R, k, max_len, C, M_max)) return ECH_EINVAL;
  CWs w;
  layout(phase, B, R, k, max_len, C, M_max, &w, static_cast<char*>(ws));
  w.P = (int)P;
  w.C = C;
  w.M_max = M_max;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int nbj = (k + kT - 1) / kT;
  if (phase == ECH_FINAL) {
    hipLaunchKernelGGL(pin_final_kernel, dim3(nbj, B), dim3(kT), 0, s, idx, k, seq_tok0, seq_len, tok2slot, slot_pin,
                       sel_slot, ctr, w);
  } else if (phase == ECH_EARLY) {
    hipLaunchKernelGGL(pin_early_kernel, dim3(w.nbr, B), dim3(kT), 0, s, logits, ld, theta, seq_tok0, seq_len,
                       tok2slot, slot_pin, ctr, w);
  } else {
    hipLaunchKernelGGL(pin_prefill_kernel, dim3(nbj, R), dim3(kT), 0, s, idx, k, seq_tok0, seq_len, tok2slot,
                       slot_pin, ctr, w);
    ECH_LAUNCH_CHECK();
    hipLaunchKernelGGL(count_claimed_kernel, dim3(w.ne), dim3(kT), 0, s, seq_tok0, seq_len, tok2slot, w);
  }
  ECH_LAUNCH_CHECK();
  hipLaunchKernelGGL(count_free_kernel, dim3(w.ns), dim3(kT), 0, s, slot_pin, C, ctr, w);
  ECH_LAUNCH_CHECK();
  // one thread per sequence: 1024 for decode batches, 256 for the single
  // prefill sequence (fits beside other work on a CU)
  if (phase == ECH_PREFILL)
    hipLaunchKernelGGL(scan_kernel<256>, dim3(1), dim3(256), 0, s, phase, B, cap, C, ctr, stats, w);
  else
    hipLaunchKernelGGL(scan_kernel<1024>, dim3(1), dim3(1024), 0, s, phase, B, cap, C, ctr, stats, w);
  ECH_LAUNCH_CHECK();
  EmitArgs ea;
  ea.phase = phase;
  ea.idx = idx;
  ea.k = k;
  ea.tok0 = seq_tok0;
  ea.lens = seq_len;
  ea.logits = logits;
  ea.ld = ld;
  ea.theta = theta;
  ea.tok2slot = tok2slot;
  ea.slot_pin = slot_pin;
  ea.C = C;
  ea.nbj = nbj;
  hipLaunchKernelGGL(emit_kernel, dim3(w.ne + w.ns), dim3(kT), 0, s, ea, w);
  ECH_LAUNCH_CHECK();
  const int apply_blocks = (int)std::max<int64_t>(1, std::min<int64_t>(1024, (demand + kT - 1) / kT));
  hipLaunchKernelGGL(apply_kernel, dim3(apply_blocks), dim3(kT), 0, s, phase, k, phase == ECH_PREFILL ? 1 : B,
                     tok2slot, slot2tok, slot_pin, miss,
                     ctr, sel_slot, stats, w);
  ECH_LAUNCH_CHECK();
  if (phase == ECH_PREFILL) {
    hipLaunchKernelGGL(selfill_kernel, dim3(nbj, R), dim3(kT), 0, s, idx, k, seq_tok0, seq_len, tok2slot, P,
                       sel_slot);
    ECH_LAUNCH_CHECK();
  }
  return ECH_OK;
}

extern "C" int ech_recall(int phase, const void* host_pool, int64_t P, int64_t row_bytes, void* dev_cache,
                          int32_t C, const int32_t* miss, int32_t* ctr, int32_t M_max, void* stream) {
  if (phase != ECH_EARLY && phase != ECH_FINAL && phase != ECH_PREFILL) return ECH_EINVAL;
  if (!host_pool || !dev_cache || !miss || !ctr || P < 1 || C < 1 || M_max < 0) return ECH_EINVAL;
  if (row_bytes <= 0 || row_bytes % 16 != 0 || row_bytes / 16 > INT32_MAX) return ECH_EINVAL;
  if ((reinterpret_cast<uintptr_t>(host_pool) & 15u) || (reinterpret_cast<uintptr_t>(dev_cache) & 15u))
    return ECH_EINVAL;
  void* dptr = nullptr;
  if (hipHostGetDevicePointer(&dptr, const_cast<void*>(host_pool), 0) != hipSuccess || !dptr) {
    (void)hipGetLastError();
    return ECH_EINVAL;
  }
  if (M_max == 0) return ECH_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int row16 = (int)(row_bytes / 16);
  const int64_t work = (int64_t)M_max * row16;
  // A PCIe-bound gather needs only ~1-2 MB of loads in flight (48 blocks x
  // 256 threads x 8 x 16 B = 1.5 MB, the best of the shapes measured in the
  // decode step); more blocks would just park waves on host loads and keep
  // the kernels of the other stream off the CUs.
  const int blocks = (int)std::max<int64_t>(1, std::min<int64_t>(kRecallBlocks, (work + kT * kRecallUnroll - 1) /
                                                                                    (kT * kRecallUnroll)));
  hipLaunchKernelGGL(recall_kernel, dim3(blocks), dim3(kT), 0, s, static_cast<const v4u*>(dptr), P, row16,
                     static_cast<v4u*>(dev_cache), C, miss, ctr,
                     phase == ECH_EARLY ? ECH_CTR_NMISS_EARLY : ECH_CTR_NMISS, M_max);
  ECH_LAUNCH_CHECK();
  return ECH_OK;
}
