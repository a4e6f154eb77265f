// GPU-resident per-layer slot map and recall (ECHO explainer: "One layer, one
// step: free -> allocate -> recall", "Five fixed-size integer tensors on the
// GPU", "Decode: fetch above a predicted threshold").
//
// A phase is a fixed sequence of kernels with grids sized from host-known
// maxima; every data-dependent count lives in device memory, so the phase can
// be captured in a hipGraph and replayed.
//
//   count    each block marks the slots of its part of the phase's resident
//            selection with the new epoch (slot_pin[s] = epoch), counts hits
//            and misses, and lists its misses in order. EARLY: tokens with
//            score > theta; FINAL: idx entries; PREFILL: idx entries of all
//            rows, misses claimed once per token by marking tok2slot -1 -> -2
//            (union), then listed by a token scan.
//   place    every block with misses takes its ranks from the counts
//            (ascending sequence, token; EARLY keeps the first `cap` per
//            sequence) and ranks the unpinned slots in ring order from the
//            head, window by window, only as far as its own ranks; miss m
//            takes the free slot of rank m: the slot's old token is unmapped
//            (no write-back), the maps point at each other, miss[m] =
//            (g, slot). One more block writes the statistics, counters, head
//            and epoch; n_alloc = min(wanted, free).
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

enum { S_EP = 0, S_HEAD = 1, S_N = 16 };

struct CWs {
  int* want;     // [ne] misses per entry block (all of them)
  int* hit;      // [ne] hits (pinned slots) per entry block
  int2* lmiss;   // [ne][lcap] the block's misses in order: (g, aux), aux = entry index (FINAL)
  int* sc;       // [S_N] the phase's epoch and head, published by its counting kernel
  int ne, nbr, lcap;  // entry blocks, entry blocks per sequence, list capacity per block
  int P, C, M_max;    // bounds every index is checked against
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

void block_counts(int phase, int B, int k, int max_len, int* ne, int* nbr, int* lcap) {
  const int nbj = (k + kT - 1) / kT;
  const int nch = std::max(1, (max_len + kBlk - 1) / kBlk);
  if (phase == ECH_FINAL) {
    *nbr = nbj;
    *ne = B * nbj;
    *lcap = kT;
  } else if (phase == ECH_EARLY) {
    *nbr = nch;
    *ne = B * nch;
    *lcap = kBlk;
  } else {
    *nbr = nch;
    *ne = nch;
    *lcap = kBlk;
  }
}

size_t layout(int phase, int B, int k, int max_len, CWs* w, char* base) {
  int ne, nbr, lcap;
  block_counts(phase, B, k, max_len, &ne, &nbr, &lcap);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  size_t o_want = take(4 * (size_t)ne), o_hit = take(4 * (size_t)ne), o_lm = take(8 * (size_t)ne * lcap),
         o_sc = take(4 * S_N);
  if (w && base) {
    w->want = reinterpret_cast<int*>(base + o_want);
    w->hit = reinterpret_cast<int*>(base + o_hit);
    w->lmiss = reinterpret_cast<int2*>(base + o_lm);
    w->sc = reinterpret_cast<int*>(base + o_sc);
    w->ne = ne;
    w->nbr = nbr;
    w->lcap = lcap;
  }
  return o;
}

__device__ __forceinline__ void set_status(int32_t* ctr, int bit) { atomicOr(&ctr[ECH_CTR_STATUS], bit); }

// Relaxed device-scope stores and loads: coherent across the XCDs' L2s, so a
// word written in a launch is seen by a workgroup of a launch running beside
// it (the live copier) without a release fence.
__device__ __forceinline__ void st_dev(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_vm_zero() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Start of a phase, by one thread of its counting kernel: publish the epoch
// and the head (the placing kernel's blocks read them while its bookkeeping
// block rewrites ctr) and clear the eviction count.
__device__ __forceinline__ void publish_phase(int32_t* ctr, int ep, CWs w) {
  int head = ctr[ECH_CTR_HEAD];
  if (head < 0 || head >= w.C) head = 0;   // only a corrupted state; keeps every slot index in range
  w.sc[S_EP] = ep;
  w.sc[S_HEAD] = head;
  ctr[ECH_CTR_NEVICT] = 0;
}

// ------------------------------------------------------------------ ring scan
// Free (unpinned) slots in ring order from the head, a window of kWin
// positions at a time, until `need` are counted or the ring ends. For every
// free slot whose rank r lies in [lo, hi), fn(r, slot) runs in the thread
// that ranks it. Returns the number counted; *s_last (LDS) gets the slot of
// the last one counted. Block-wide (kT threads, contains barriers); s_fr is
// kWin bytes of LDS, scr kT/64 ints.
constexpr int kWin = kT * 32;

template <class Fn>
__device__ int ring_scan(const int32_t* __restrict__ slot_pin, int C, int head, int ep, int need, int lo, int hi,
                         uint8_t* s_fr, int* scr, int* s_last, Fn fn) {
  const int tid = threadIdx.x;
  int found = 0;
  for (int i0 = 0; i0 < C && found < need; i0 += kWin) {   // block-uniform
#pragma unroll
    for (int j = 0; j < kWin / kT; ++j) {   // coalesced loads, all in flight
      const int pos = i0 + j * kT + tid;
      int p = head + min(pos, C - 1);
      if (p >= C) p -= C;
      const int pv = slot_pin[p];
      s_fr[j * kT + tid] = (pos < C && pv != ep) ? 1 : 0;
    }
    __syncthreads();
    // thread t ranks positions i0 + 32t .. +31 (two 16-byte LDS reads)
    const uint4 f0 = reinterpret_cast<const uint4*>(s_fr)[2 * tid];
    const uint4 f1 = reinterpret_cast<const uint4*>(s_fr)[2 * tid + 1];
    const uint32_t fw[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
    int cnt = 0;
#pragma unroll
    for (int q = 0; q < 8; ++q) cnt += __popc(fw[q]);   // flags are 0/1 bytes
    int tot;
    int rank = found + ech::block_excl_scan<kT>(cnt, scr, &tot);
    const int wlast = found + tot - 1;
    if (cnt > 0 && (rank < hi || rank + cnt > wlast)) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if ((fw[q] >> (8 * e)) & 1u) {
            int p = head + i0 + 32 * tid + 4 * q + e;
            if (p >= C) p -= C;
            if (rank >= lo && rank < hi) fn(rank, p);
            if (rank == wlast) *s_last = p;
            ++rank;
          }
        }
      }
    }
    found += tot;
    __syncthreads();   // s_fr is rewritten by the next window
  }
  return found;
}

// ------------------------------------------------------------------ pin / count
// Each block pins the slots of its resident selection with the new epoch
// (slot_pin[s] = epoch), counts hits and misses and lists its misses in
// order.

// FINAL: grid (nbj, B), one idx entry per thread.
__global__ __launch_bounds__(kT) void pin_final_kernel(const int32_t* __restrict__ idx, int k,
                                                       const int64_t* __restrict__ tok0,
                                                       const int32_t* __restrict__ lens,
                                                       const int32_t* __restrict__ tok2slot,
                                                       int32_t* __restrict__ slot_pin, int32_t* __restrict__ sel_slot,
                                                       int32_t* ctr, int32_t* __restrict__ stats, CWs w) {
  __shared__ int scr[kT / 64];
  const int b = blockIdx.y, j = blockIdx.x * kT + threadIdx.x;
  const int blk = b * gridDim.x + blockIdx.x;
  const int ep = ctr[ECH_CTR_EPOCH] + 1;
  int hit = 0, miss = 0, g = -1;
  size_t e = 0;
  if (j < k) {
    e = (size_t)b * k + j;
    const int t = idx[e];
    int sl = -1;
    if (t >= 0) {
      if (t >= lens[b]) {
        set_status(ctr, ECH_ST_BADTOK);
      } else {
        const int64_t gg = tok0[b] + t;
        if (gg < 0 || gg >= w.P) {
          set_status(ctr, ECH_ST_BADTOK);
        } else {
          g = (int)gg;
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
  int nm;
  const int r = ech::block_excl_scan<kT>(miss, scr, &nm);
  if (miss) w.lmiss[(size_t)blk * w.lcap + r] = make_int2(g, (int)e);
  const int nh = ech::block_sum<kT>(hit, scr);
  if (threadIdx.x == 0) {
    w.hit[blk] = nh;
    w.want[blk] = nm;
    if (blockIdx.x == 0) {
      stats[4 * b + 3] = 0;   // evictions, counted by the placing kernel
      if (b == 0) {
        publish_phase(ctr, ep, w);
        ctr[ECH_CTR_NCOPIED_FINAL] = 0;   // nothing of this list is copied yet
        ctr[ECH_CTR_FINAL_READY] = 0;     // the placing kernel's last workgroup sets it
        ctr[ECH_CTR_FINAL_DONE] = 0;
      }
    }
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
                                                       int32_t* __restrict__ slot_pin, int32_t* ctr,
                                                       int32_t* __restrict__ stats, CWs w) {
  __shared__ int scr[kT / 64];
  const int b = blockIdx.y;
  const int blk = b * gridDim.x + blockIdx.x;
  const int len = lens[b];
  const float th = theta[b];
  const int ep = ctr[ECH_CTR_EPOCH] + 1;
  const int t = blockIdx.x * kBlk + threadIdx.x * kPer;
  const int64_t g0 = tok0[b] + t;
  int hit = 0, want = 0;
  uint32_t miss_mask = 0;   // bit i: token t + i is a miss
  if (th == th && t < len) {
    float v[kPer];
    load16(logits + (size_t)b * ld, t, len, v);
    uint32_t above = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      above |= (t + i < len && v[i] > th && g0 + i < w.P) ? 1u << i : 0u;
    if (above) {
      // all sixteen lookups in flight at once (addresses clamped into the
      // map; only the flagged ones are used)
      int sl[kPer];
#pragma unroll
      for (int i = 0; i < kPer; ++i) sl[i] = tok2slot[min(max(g0 + i, (int64_t)0), (int64_t)w.P - 1)];
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        if ((above >> i) & 1u) {
          if (sl[i] >= 0 && sl[i] < w.C) {
            slot_pin[sl[i]] = ep;
            ++hit;
          } else {
            miss_mask |= 1u << i;
            ++want;
          }
        }
      }
    }
  }
  int nw;
  int r = ech::block_excl_scan<kT>(want, scr, &nw);
  for (uint32_t mm = miss_mask; mm != 0u && r < w.lcap; mm &= mm - 1u, ++r)
    w.lmiss[(size_t)blk * w.lcap + r] = make_int2((int)(g0 + __builtin_ctz(mm)), b);
  const int nh = ech::block_sum<kT>(hit, scr);
  if (threadIdx.x == 0) {
    w.hit[blk] = nh;
    w.want[blk] = nw;
    if (blockIdx.x == 0) {
      stats[4 * b + 3] = 0;   // evictions, counted by the placing kernel
      if (b == 0) publish_phase(ctr, ep, w);
    }
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

// PREFILL: grid (nch), 16 consecutive tokens per thread: the claimed tokens
// of each block of the token range (its misses, in order) and its pinned
// resident tokens (one per pinned slot: a slot holds one token).
__global__ __launch_bounds__(kT) void count_claimed_kernel(const int64_t* __restrict__ tok0p,
                                                           const int32_t* __restrict__ lenp,
                                                           const int32_t* __restrict__ tok2slot,
                                                           const int32_t* __restrict__ slot_pin, int32_t* ctr,
                                                           int32_t* __restrict__ stats, CWs w) {
  __shared__ int scr[kT / 64];
  const int64_t tok0 = tok0p[0];
  const int len = lenp[0];
  const int ep = ctr[ECH_CTR_EPOCH] + 1;
  const int t = blockIdx.x * kBlk + threadIdx.x * kPer;
  const int64_t g0 = tok0 + t;
  int want = 0, pinned = 0;
  uint32_t miss_mask = 0;   // bit i: token t + i is claimed
  if (t < len && g0 < w.P) {
    int sl[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) sl[i] = tok2slot[min(max(g0 + i, (int64_t)0), (int64_t)w.P - 1)];   // all in flight
    int pe[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) pe[i] = slot_pin[min(max(sl[i], 0), w.C - 1)];   // clamped, used only for slots in range
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (t + i < len && g0 + i < w.P) {
        if (sl[i] == -2) {
          miss_mask |= 1u << i;
          ++want;
        } else if (sl[i] >= 0 && sl[i] < w.C && pe[i] == ep) {
          ++pinned;
        }
      }
    }
  }
  int nw;
  int r = ech::block_excl_scan<kT>(want, scr, &nw);
  for (uint32_t mm = miss_mask; mm != 0u; mm &= mm - 1u, ++r)
    w.lmiss[(size_t)blockIdx.x * w.lcap + r] = make_int2((int)(g0 + __builtin_ctz(mm)), 0);
  const int np = ech::block_sum<kT>(pinned, scr);
  if (threadIdx.x == 0) {
    w.want[blockIdx.x] = nw;
    w.hit[blockIdx.x] = np;
    if (blockIdx.x == 0) {
      stats[3] = 0;   // evictions, counted by the placing kernel
      publish_phase(ctr, ep, w);
    }
  }
}

// ------------------------------------------------------------------ place
// grid (ne + 1, S). Block (i, y), i < ne, places the misses of entry block i
// in the slice y of its list (S > 1 splits the long lists of PREFILL token
// blocks). Ranks come from the counts: the capped totals of the sequences
// before i's (EARLY keeps the first `cap` misses of each sequence) plus the
// misses of i's sequence before block i. The block then ranks the free slots
// itself, in ring order from the head, only as far as its own ranks: miss of
// rank m takes the m-th free slot; its old token is unmapped (no
// write-back), the maps point at each other, miss[m] = (g, slot). Block
// (ne, 0) does the bookkeeping: per-sequence statistics, counts, the new head
// and epoch. Nothing in this kernel writes slot_pin, so every block ranks the
// same free slots.

// s_tot[b] = the sum of cnt[b * nbr + c] over c, for b < nb (LDS), by the
// whole block: thread t sums a contiguous run of the counts (all its loads
// in flight) and adds each sequence's part with one LDS atomic.
__device__ void seq_totals(const int* __restrict__ cnt, int nb, int nbr, int* s_tot) {
  const int tid = threadIdx.x;
  for (int b = tid; b < nb; b += kT) s_tot[b] = 0;
  __syncthreads();
  const int n = nb * nbr;
  const int m = (n + kT - 1) / kT;
  const int i_lo = min(n, tid * m), i_hi = min(n, i_lo + m);
  int cur = -1, acc = 0;
  for (int i0 = i_lo; i0 < i_hi; i0 += 8) {
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = cnt[min(i0 + u, n - 1)];   // clamped: all issued at once
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (i0 + u < i_hi) {
        const int sq = (i0 + u) / nbr;
        if (sq != cur) {
          if (acc) atomicAdd(&s_tot[cur], acc);
          cur = sq;
          acc = 0;
        }
        acc += v[u];
      }
    }
  }
  if (acc) atomicAdd(&s_tot[cur], acc);
  __syncthreads();
}

__device__ void bookkeep(int phase, int nseq, int cap, const int32_t* __restrict__ slot_pin, int32_t* ctr,
                         int32_t* __restrict__ stats, CWs w, uint8_t* smem, int* scr) {
  int* s_take = reinterpret_cast<int*>(smem);
  int* s_want = s_take + kMaxB;
  int* s_hit = s_want + kMaxB;
  int* s_row = s_hit + kMaxB;
  uint8_t* s_fr = reinterpret_cast<uint8_t*>(s_row + kMaxB);
  __shared__ int s_last, s_lastw;
  const int tid = threadIdx.x;
  const int ep = w.sc[S_EP], head = w.sc[S_HEAD];
  seq_totals(w.want, nseq, w.nbr, s_want);
  seq_totals(w.hit, nseq, w.nbr, s_hit);
  int n_want = 0, hit_all = 0;
  for (int b0 = 0; b0 < nseq; b0 += kT) {
    const int b = b0 + tid;
    int take = 0, h = 0;
    if (b < nseq) {
      const int wb = s_want[b];
      h = s_hit[b];
      take = (phase == ECH_EARLY) ? min(cap, wb) : wb;
      s_take[b] = take;
    }
    int tot;
    const int ex = ech::block_excl_scan<kT>(take, scr, &tot);
    if (b < nseq) s_row[b] = n_want + ex;
    n_want += tot;
    hit_all += ech::block_sum<kT>(h, scr);
  }
  const bool clamped = n_want > w.M_max;   // only when a caller contract is broken
  if (clamped) n_want = w.M_max;
  const int found = ring_scan(slot_pin, w.C, head, ep, n_want, n_want - 1, n_want, s_fr, scr, &s_lastw,
                              [&](int, int p) { s_last = p; });
  const int n_alloc = min(n_want, found);
  for (int b = tid; b < nseq; b += kT) {
    const int fetched = max(0, min(n_alloc - s_row[b], s_take[b]));
    int32_t* st = stats + 4 * b;
    st[0] = s_hit[b];
    st[1] = fetched;
    st[2] = s_want[b] - fetched;   // wanted (before the cap) and not fetched
  }
  if (tid == 0) {
    if (phase == ECH_EARLY) {
      ctr[ECH_CTR_NMISS_EARLY] = n_alloc;
      ctr[ECH_CTR_NCOPIED_EARLY] = 0;   // nothing of this list is copied yet
    } else if (phase == ECH_FINAL) {
      st_dev(&ctr[ECH_CTR_NMISS], n_alloc);   // read beside this launch once the list is complete
    } else {
      ctr[ECH_CTR_NMISS] = n_alloc;
    }
    ctr[ECH_CTR_NWANT] = n_want;
    ctr[ECH_CTR_NPINNED] = hit_all;
    ctr[ECH_CTR_EPOCH] = ep;
    int walk = 0;   // ring positions from the head to the last slot allocated
    if (n_alloc > 0) {
      const int last = (n_alloc == n_want) ? s_last : s_lastw;
      ctr[ECH_CTR_HEAD] = (last + 1 == w.C) ? 0 : last + 1;
      walk = (last - head + w.C) % w.C + 1;
    }
    if (phase == ECH_EARLY) ctr[ECH_CTR_EARLY_WALK] = walk;
    // The FINAL walk starts where the EARLY one ended; together longer than
    // the ring, it reached slots the EARLY phase allocated.
    if (phase == ECH_FINAL && walk > 0) {
      const int we = ctr[ECH_CTR_EARLY_WALK];
      if (we > 0 && (int64_t)we + walk > w.C) atomicOr(&ctr[ECH_CTR_FINAL_READY], 2);
    }
    if ((phase != ECH_EARLY && n_want > found) || clamped) ctr[ECH_CTR_STATUS] |= ECH_ST_OVERFLOW;
  }
}

__device__ __forceinline__ void place_block(int phase, int nseq, int cap, int32_t* __restrict__ tok2slot,
                                            int32_t* __restrict__ slot2tok, const int32_t* __restrict__ slot_pin,
                                            int32_t* __restrict__ miss, int32_t* ctr, int32_t* __restrict__ sel_slot,
                                            int32_t* __restrict__ stats, CWs w) {
  // placing blocks: s_slot [kBlk ints] | s_fr [kWin bytes] | s_tot [kMaxB ints];
  // the bookkeeping block: 4 x [kMaxB ints] | s_fr [kWin bytes]
  __shared__ __align__(16) uint8_t smem[4 * kBlk + kWin + 4 * kMaxB];
  __shared__ int scr[kT / 64];
  __shared__ int s_lastw;
  static_assert(4 * kBlk >= 4 * 4 * kMaxB, "bookkeeping arrays fit");
  const int i = blockIdx.x;
  if (i == w.ne) {
    if (blockIdx.y == 0) bookkeep(phase, nseq, cap, slot_pin, ctr, stats, w, smem, scr);
    return;
  }
  const int cnt = min(w.want[i], w.lcap);
  const int span = (gridDim.y == 1) ? w.lcap : kT;
  const int j_lo = blockIdx.y * span;
  if (j_lo >= cnt) return;   // block-uniform: most blocks have no misses
  const int j_hi = min(cnt, j_lo + span);
  const int tid = threadIdx.x;
  const int b = i / w.nbr, c = i % w.nbr;
  // ranks: capped totals of the sequences before b, then b's misses before block i
  int* s_tot = reinterpret_cast<int*>(smem + 4 * kBlk + kWin);
  seq_totals(w.want, b + 1, w.nbr, s_tot);
  int prev = 0;
  for (int bb = tid; bb < b; bb += kT) prev += (phase == ECH_EARLY) ? min(cap, s_tot[bb]) : s_tot[bb];
  int pre = 0;
  for (int cc = tid; cc < c; cc += kT) pre += w.want[(size_t)b * w.nbr + cc];
  prev = ech::block_sum<kT>(prev, scr);
  pre = ech::block_sum<kT>(pre, scr);
  const int tot_b = s_tot[b];
  const int take = (phase == ECH_EARLY) ? min(cap, tot_b) : tot_b;
  const int base = prev + pre;                      // rank of list entry 0
  const int lim = min(prev + take, w.M_max);        // ranks at or past lim are not placed
  const int r_lo = base + j_lo, r_hi = min(base + j_hi, lim);
  if (r_lo >= r_hi) return;                         // block-uniform: all past the cap
  // the free slots of ranks [r_lo, r_hi)
  int* s_slot = reinterpret_cast<int*>(smem);
  uint8_t* s_fr = smem + 4 * kBlk;
  for (int j = tid; j < r_hi - r_lo; j += kT) s_slot[j] = -1;
  __syncthreads();
  const int ep = w.sc[S_EP], head = w.sc[S_HEAD];
  ring_scan(slot_pin, w.C, head, ep, r_hi, r_lo, r_hi, s_fr, scr, &s_lastw,
            [&](int r, int p) { s_slot[r - r_lo] = p; });
  const int owner = (phase == ECH_PREFILL) ? 0 : b;
  for (int j = tid; j < r_hi - r_lo; j += kT) {   // trips differ only in the last pass
    const int m = r_lo + j;
    const int2 mc = w.lmiss[(size_t)i * w.lcap + j_lo + j];
    const int g = mc.x;
    const int p = s_slot[j];
    bool evicted = false;
    if (g < 0 || g >= w.P) {
      set_status(ctr, ECH_ST_OVERFLOW);   // unreachable unless counts and lists disagree
    } else if (p >= 0) {
      const int u = slot2tok[p];
      if (u >= 0 && u < w.P) {
        tok2slot[u] = -1;   // evict; the host row stays where it is
        evicted = true;
      }
      slot2tok[p] = g;
      tok2slot[g] = p;
      if (phase == ECH_FINAL) {   // read beside this launch once the list is complete
        st_dev(&miss[2 * m], g);
        st_dev(&miss[2 * m + 1], p);
        sel_slot[mc.y] = p;
      } else {
        miss[2 * m] = g;
        miss[2 * m + 1] = p;
      }
    } else if (phase == ECH_PREFILL) {
      tok2slot[g] = -1;     // release the claim of a miss that got no slot
    }
    ech::wave_count(&ctr[ECH_CTR_NEVICT], evicted);
    ech::wave_count(&stats[4 * owner + 3], evicted);
  }
}

__global__ __launch_bounds__(kT) void place_kernel(int phase, int nseq, int cap, int32_t* __restrict__ tok2slot,
                                                   int32_t* __restrict__ slot2tok,
                                                   const int32_t* __restrict__ slot_pin, int32_t* __restrict__ miss,
                                                   int32_t* ctr, int32_t* __restrict__ sel_slot,
                                                   int32_t* __restrict__ stats, CWs w) {
  place_block(phase, nseq, cap, tok2slot, slot2tok, slot_pin, miss, ctr, sel_slot, stats, w);
  if (phase == ECH_FINAL) {
    // The last workgroup to finish marks the list complete (bit 0) for a
    // copier running beside this launch: every workgroup's coherent stores
    // (entries, count, bit 1) have completed before it arrives.
    wait_vm_zero();
    __syncthreads();
    if (threadIdx.x == 0 &&
        atomicAdd(&ctr[ECH_CTR_FINAL_DONE], 1) == (int)(gridDim.x * gridDim.y) - 1)
      atomicOr(&ctr[ECH_CTR_FINAL_READY], 1);
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
                                                    int ccopied, int32_t M_max) {
  const int n = min(ctr[cidx], M_max);
  // EARLY, FINAL: entries the live copier already copied are skipped
  const int n0 = (ccopied >= 0) ? min(max(ctr[ccopied], 0), n) : 0;
  const int64_t total = (int64_t)(n - n0) * row16;
  const int64_t stride = (int64_t)gridDim.x * kT * kRecallUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kT * kRecallUnroll + threadIdx.x; base < total; base += stride) {
    v4u v[kRecallUnroll];
    int64_t dst[kRecallUnroll];
#pragma unroll
    for (int u = 0; u < kRecallUnroll; ++u) {
      const int64_t i = base + (int64_t)u * kT;
      dst[u] = -1;
      if (i < total) {
        const int m = n0 + (int)(i / row16);
        const int c = (int)(i % row16);
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
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    atomicAdd(&ctr[ECH_CTR_RECALLED], n - n0);
    if (cidx == ECH_CTR_NMISS_EARLY) ctr[ECH_CTR_LIVE] = 0;   // this step's early list is complete
  }
}

// The rows the live copier left of both lists of a step, in one launch,
// after the FINAL phase: early entries from ctr[NCOPIED_EARLY] on whose slot
// still holds their token (a slot the FINAL phase gave to another token
// gets that token's row from the FINAL list instead, so no two rows of the
// launch go to one slot), then FINAL entries from ctr[NCOPIED_FINAL] on.
__global__ __launch_bounds__(kT) void recall_rest_kernel(const v4u* __restrict__ host, int64_t P, int row16,
                                                         v4u* __restrict__ dev, int32_t C,
                                                         const int32_t* __restrict__ miss_e, int32_t M_early,
                                                         const int32_t* __restrict__ miss_f, int32_t M_max,
                                                         const int32_t* __restrict__ slot2tok, int32_t* ctr) {
  const int ne = min(ctr[ECH_CTR_NMISS_EARLY], M_early), nf = min(ctr[ECH_CTR_NMISS], M_max);
  const int n0e = min(max(ctr[ECH_CTR_NCOPIED_EARLY], 0), ne), n0f = min(max(ctr[ECH_CTR_NCOPIED_FINAL], 0), nf);
  const int re = ne - n0e;   // early rows, then FINAL rows
  const int64_t total = (int64_t)(re + nf - n0f) * row16;
  const int64_t stride = (int64_t)gridDim.x * kT * kRecallUnroll;
  int copied = 0;
  for (int64_t base = (int64_t)blockIdx.x * kT * kRecallUnroll + threadIdx.x; base < total; base += stride) {
    v4u v[kRecallUnroll];
    int64_t dst[kRecallUnroll];
#pragma unroll
    for (int u = 0; u < kRecallUnroll; ++u) {
      const int64_t i = base + (int64_t)u * kT;
      dst[u] = -1;
      if (i < total) {
        const int r = (int)(i / row16);
        const int c = (int)(i % row16);
        const bool early = r < re;
        const int32_t* e = early ? miss_e + 2 * (n0e + r) : miss_f + 2 * (n0f + r - re);
        const int g = e[0], p = e[1];
        if (g >= 0 && g < P && p >= 0 && p < C) {
          if (!early || slot2tok[p] == g) {
            v[u] = __builtin_nontemporal_load(host + (int64_t)g * row16 + c);
            dst[u] = (int64_t)p * row16 + c;
            copied += (c == 0);
          }
        } else if (c == 0) {
          set_status(ctr, ECH_ST_BADMISS);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kRecallUnroll; ++u)
      if (dst[u] >= 0) __builtin_nontemporal_store(v[u], dev + dst[u]);
  }
  copied = ech::wave_sum(copied);
  if ((threadIdx.x & 63) == 0 && copied) atomicAdd(&ctr[ECH_CTR_RECALLED], copied);
  if (blockIdx.x == 0 && threadIdx.x == 0) ctr[ECH_CTR_LIVE] = 0;   // this step's early list is complete
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
  (void)R;
  return layout(phase, B, k, max_len, nullptr, nullptr);
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
  layout(phase, B, k, max_len, &w, static_cast<char*>(ws));
  w.P = (int)P;
  w.C = C;
  w.M_max = M_max;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int nbj = (k + kT - 1) / kT;
  // count, then place (the ranks, the free slots and the maps)
  if (phase == ECH_FINAL) {
    hipLaunchKernelGGL(pin_final_kernel, dim3(nbj, B), dim3(kT), 0, s, idx, k, seq_tok0, seq_len, tok2slot,
                       slot_pin, sel_slot, ctr, stats, w);
  } else if (phase == ECH_EARLY) {
    hipLaunchKernelGGL(pin_early_kernel, dim3(w.nbr, B), dim3(kT), 0, s, logits, ld, theta, seq_tok0, seq_len,
                       tok2slot, slot_pin, ctr, stats, w);
  } else {
    hipLaunchKernelGGL(pin_prefill_kernel, dim3(nbj, R), dim3(kT), 0, s, idx, k, seq_tok0, seq_len, tok2slot,
                       slot_pin, ctr, w);
    ECH_LAUNCH_CHECK();
    hipLaunchKernelGGL(count_claimed_kernel, dim3(w.ne), dim3(kT), 0, s, seq_tok0, seq_len, tok2slot, slot_pin, ctr,
                       stats, w);
  }
  ECH_LAUNCH_CHECK();
  const int slices = (phase == ECH_PREFILL) ? w.lcap / kT : 1;
  hipLaunchKernelGGL(place_kernel, dim3(w.ne + 1, slices), dim3(kT), 0, s, phase, phase == ECH_PREFILL ? 1 : B, cap,
                     tok2slot, slot2tok, slot_pin, miss, ctr, sel_slot, stats, w);
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
                     phase == ECH_EARLY ? ECH_CTR_NMISS_EARLY : ECH_CTR_NMISS,
                     phase == ECH_EARLY ? ECH_CTR_NCOPIED_EARLY : phase == ECH_FINAL ? ECH_CTR_NCOPIED_FINAL : -1,
                     M_max);
  ECH_LAUNCH_CHECK();
  return ECH_OK;
}

extern "C" int ech_recall_rest(const void* host_pool, int64_t P, int64_t row_bytes, void* dev_cache, int32_t C,
                               const int32_t* miss_early, int32_t M_early, const int32_t* miss, int32_t M_max,
                               const int32_t* slot2tok, int32_t* ctr, void* stream) {
  if (!host_pool || !dev_cache || !miss_early || !miss || !slot2tok || !ctr || P < 1 || C < 1 || M_early < 0 ||
      M_max < 0)
    return ECH_EINVAL;
  if (row_bytes <= 0 || row_bytes % 16 != 0 || row_bytes / 16 > INT32_MAX) return ECH_EINVAL;
  if ((reinterpret_cast<uintptr_t>(host_pool) & 15u) || (reinterpret_cast<uintptr_t>(dev_cache) & 15u))
    return ECH_EINVAL;
  void* dptr = nullptr;
  if (hipHostGetDevicePointer(&dptr, const_cast<void*>(host_pool), 0) != hipSuccess || !dptr) {
    (void)hipGetLastError();
    return ECH_EINVAL;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int row16 = (int)(row_bytes / 16);
  const int64_t work = ((int64_t)M_early + M_max) * row16;
  const int blocks = (int)std::max<int64_t>(1, std::min<int64_t>(kRecallBlocks, (work + kT * kRecallUnroll - 1) /
                                                                                    (kT * kRecallUnroll)));
  hipLaunchKernelGGL(recall_rest_kernel, dim3(blocks), dim3(kT), 0, s, static_cast<const v4u*>(dptr), P, row16,
                     static_cast<v4u*>(dev_cache), C, miss_early, M_early, miss, M_max, slot2tok, ctr);
  ECH_LAUNCH_CHECK();
  return ECH_OK;
}
