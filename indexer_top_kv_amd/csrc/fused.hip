// Decode scores fused with the early fetch (ECHO explainer, "Decode: fetch
// above a predicted threshold": tokens scoring above the predicted threshold
// are fetched before the exact top-k is known, to hide the dependency of the
// recall on the top-k; "Fused indexer kernel (extends DeepGEMM)" and the
// artifact README's fused prefetch kernels: the scores and the prefetch in one
// kernel).
//
// The result is exactly that of ech_index_logits followed by one ECH_EARLY
// phase of ech_cache_step over sequences [e0, e1): pins = slots of resident
// tokens scoring above theta; misses = per sequence the first `cap`
// non-resident tokens above theta, ascending; misses in ascending (sequence,
// token) order take the unpinned slots in ring order from the head. What
// changes is when things happen: the allocation of a sequence's misses and the
// PCIe copy of their rows start while later sequences are still being scored.
//
//   pin    grid (chunks, e1-e0): each 4096-token chunk lists its resident
//          tokens, scores them with the scores kernel's own tile arithmetic
//          (decode.hpp / score.hpp: the same bit patterns), pins those above
//          theta (slot_pin = epoch), counts hits.
//   rank   one workgroup: hits per sequence, the unpinned slots in ring order
//          from the head (as many as the early demand bound needs), the
//          epoch; clears the fused kernel's control words and the early miss
//          list (every entry (-1, -1)).
//   fused  one launch, three kinds of workgroups (1-D grid, in this order):
//     alloc  (one per early sequence, at most 64, each taking every 64th)
//            waits for the masks its sequence's scoring waves publish,
//            lists the sequence's first `cap` misses in token order, takes its
//            first rank from the sequences before it (decoupled look-back on
//            one word per sequence), gives miss m the m-th ranked free slot
//            (evicting its old token, no write-back) and writes miss m.
//     copy   (32) claim groups of consecutive miss ranks in order, wait for
//            their entries and copy the rows from pinned host memory over
//            PCIe; once every alloc workgroup is done they stop claiming, so
//            the launch ends soon after the scoring. ctr[NCOPIED_EARLY] says
//            how many leading entries were copied; ech_recall(ECH_EARLY)
//            copies the rest.
//     score  the fp8 decode scores kernel's waves (256 tokens each); a wave
//            of an early sequence then looks up the residency of its tokens
//            above theta and publishes its misses as a 256-bit mask in 8
//            tagged words.
//
// Workgroups of one launch communicate through words that carry their own
// validity (a tag bit, a flag, or a (-1, -1) sentinel), read and written with
// relaxed device-scope atomics (coherent across the chiplets' L2 caches), so
// no release fence - which writes back a whole L2 on MI355X - is needed. The
// scoring waves never wait; alloc workgroups wait only on scoring waves and
// on alloc workgroups of earlier sequences; copy workgroups wait only on
// alloc workgroups. Every wait is bounded (0.5 s of the constant-rate clock):
// past it the workgroup sets ECH_ST_TIMEOUT and carries on, so the launch
// always ends.

#include <algorithm>

#include "decode.hpp"

namespace {

constexpr int kT = 256;
constexpr int kPer = 16;
constexpr int kBlk = kT * kPer;          // tokens per pin block
constexpr int kTPW = 16;                 // tiles per scoring wave
constexpr int kNS = 4;                   // ring slots per scoring wave
constexpr int kWavesF = 4;               // waves per scoring workgroup
constexpr int kWaveTok = kTPW * 16;      // 256 tokens per scoring wave
constexpr int kWords = kWaveTok / 32;    // mask words per wave
constexpr int kMaxCap = 4096;
constexpr int kMaxB = 1024;
constexpr int kMaxAlloc = 64;            // alloc workgroups at most
constexpr int kCopy = 32;                // copy workgroups
constexpr int kCopyUnroll = 8;           // 16-byte pieces per thread per group
constexpr int kA = 1024;                 // threads of the rank workgroup
constexpr int kWinA = kA * 16;           // ring positions per window

typedef unsigned long long u64;
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
constexpr u64 kTag = 1ull << 32;         // a published mask word: tag in the high half
constexpr u64 kAgg = 1ull << 62;         // look-back word: aggregate (this sequence's take)
constexpr u64 kInc = 1ull << 63;         // look-back word: inclusive prefix
constexpr u64 kFin = 1ull << 63;         // finished word: every alloc workgroup is done
constexpr u64 kNone = ~0ull;             // an early miss entry not written yet: (-1, -1)
constexpr u64 kSpinTicks = 50000000ull;  // 0.5 s at the 100 MHz constant-rate clock

struct Ctl {                             // control words at the start of the workspace
  int next_group;                        // copy groups claimed
  int a_done;                            // alloc workgroups finished
  int c_done;                            // copy workgroups finished
  int nfree;                             // free slots ranked (<= M_early)
  int pad[4];
  u64 finished;                          // kFin | n_alloc
};

struct FWs {
  Ctl* ctl;
  u64* lb;                               // [R] look-back word per sequence
  int* hitblk;                           // [R * nch] hits per pin block
  int* freelist;                         // [M_early] free slots in ring order from the head
  u64* masks;                            // [R * wpr * kWords] published miss masks
  int nch, wpr;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t fused_layout(int R, int max_len, int32_t M_early, FWs* w, char* base) {
  const int nch = std::max(1, (max_len + kBlk - 1) / kBlk);
  const int wpr = std::max(1, (max_len + kWaveTok - 1) / kWaveTok);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  const size_t o_ctl = take(sizeof(Ctl)), o_lb = take(8 * (size_t)R), o_hit = take(4 * (size_t)R * nch),
               o_fl = take(4 * (size_t)std::max(M_early, 1)), o_m = take(8 * (size_t)R * wpr * kWords);
  if (w && base) {
    w->ctl = reinterpret_cast<Ctl*>(base + o_ctl);
    w->lb = reinterpret_cast<u64*>(base + o_lb);
    w->hitblk = reinterpret_cast<int*>(base + o_hit);
    w->freelist = reinterpret_cast<int*>(base + o_fl);
    w->masks = reinterpret_cast<u64*>(base + o_m);
    w->nch = nch;
    w->wpr = wpr;
  }
  return o;
}

__device__ __forceinline__ u64 ld_dev(const u64* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(u64* p, u64 v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_dev(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void set_status(int32_t* ctr, int bit) { atomicOr(&ctr[ECH_CTR_STATUS], bit); }

// Wait until pred(load()) holds, sleeping between polls; false (and the
// timeout status) once the bound has passed.
template <class Load, class Pred>
__device__ __forceinline__ bool spin_until(Load load, Pred pred, int32_t* ctr, u64 t0, decltype(load())* out) {
  for (;;) {
    const auto v = load();
    if (pred(v)) {
      *out = v;
      return true;
    }
    if (wall_clock64() - t0 > kSpinTicks) {
      set_status(ctr, ECH_ST_TIMEOUT);
      *out = v;
      return false;
    }
    __builtin_amdgcn_s_sleep(16);
  }
}

// ------------------------------------------------------------------ pin
// grid (nch, e1 - e0). Chunk c of sequence b covers tokens [c*kBlk, +kBlk).
// The resident tokens of the chunk are listed in order, then each wave
// scores tiles of 16 of them, four tiles at a time with all their (gathered)
// key rows in flight together.
constexpr int kPinBatch = 4;

__global__ __launch_bounds__(kT) void fused_pin_kernel(const uint16_t* __restrict__ q, const float* __restrict__ w,
                                                       const uint8_t* __restrict__ kc, const float* __restrict__ ksc,
                                                       const int64_t* __restrict__ tok0,
                                                       const int32_t* __restrict__ lens,
                                                       const float* __restrict__ theta, int e0,
                                                       const int32_t* __restrict__ tok2slot, int64_t P, int32_t C,
                                                       int32_t* __restrict__ slot_pin, const int32_t* ctr, FWs ws) {
  __shared__ int rt[kBlk];          // resident token offsets of the chunk, ascending
  __shared__ int scr[kT / 64];
  const int b = e0 + blockIdx.y, c = blockIdx.x;
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
  // ordered compaction of the chunk's resident tokens
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
  __syncthreads();
  int hits = 0;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ntile = (nres + 15) / 16;
  if (wave < ntile) {   // wave-uniform
    const int col = lane & 15, grp = lane >> 4;
    // query fragments and head weights straight into registers, in the
    // scores kernel's operand layout (the same products, the same sums)
    bf16x8_t a[4][4];
    float wv[4][4];
    const uint8_t* qb = reinterpret_cast<const uint8_t*>(q + (size_t)b * kH * kD);
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2)
        a[ht][s2] = as_bf16x8(*reinterpret_cast<const uint4*>(qb + (16 * ht + col) * (kD * 2) +
                                                               2 * dim0_of<ECH_KEY_FP8>(grp, s2)));
#pragma unroll
      for (int u = 0; u < 4; ++u) wv[ht][u] = w[(size_t)b * kH + 16 * ht + 4 * grp + u];
    }
    const uint8_t* kbase = kc + (size_t)g0 * kD;
    for (int j0 = wave; j0 < ntile; j0 += kPinBatch * (kT / 64)) {
      KeyFrag<ECH_KEY_FP8> f[kPinBatch];
      float sc[kPinBatch];
      int tt[kPinBatch];
#pragma unroll
      for (int u = 0; u < kPinBatch; ++u) {   // the batch's gathers, all in flight
        const int e = 16 * (j0 + u * (kT / 64)) + col;
        tt[u] = rt[min(e, nres - 1)];
        load_key<ECH_KEY_FP8>(f[u], kbase + (size_t)tt[u] * kD, grp);
        sc[u] = ksc[g0 + tt[u]];
      }
#pragma unroll
      for (int u = 0; u < kPinBatch; ++u) {
        const int j = j0 + u * (kT / 64);
        if (j < ntile) {   // wave-uniform
          const int e = 16 * j + col;
          bf16x8_t kb[4];
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) kb[s2] = key_step<ECH_KEY_FP8>(f[u], s2);
          const float v = tile_score(a, wv, kb, sc[u]);
          if (grp == 0 && e < nres && v > th) {
            slot_pin[tok2slot[g0 + tt[u]]] = ep;
            ++hits;
          }
        }
      }
    }
  }
  const int tot = ech::block_sum<kT>(hits, scr);
  if (threadIdx.x == 0) *out = tot;
}

// ------------------------------------------------------------------ rank
__global__ __launch_bounds__(kA) void fused_rank_kernel(const int32_t* __restrict__ slot_pin, int32_t C, int e0,
                                                        int e1, int32_t* __restrict__ miss_early, int32_t M_early,
                                                        int32_t* ctr, int32_t* __restrict__ stats, FWs ws) {
  __shared__ int scr[kA / 64];
  __shared__ __align__(16) uint8_t s_fr[kWinA];
  const int tid = threadIdx.x;
  const int ep = ctr[ECH_CTR_EPOCH] + 1;
  int head = ctr[ECH_CTR_HEAD];
  if (head < 0 || head >= C) head = 0;   // only a corrupted state; keeps every slot index in range
  // hits per sequence (the pinned slots: one per resident token above
  // theta): every pin block's count in flight at once, summed in LDS
  __shared__ int s_hit[kMaxB];
  const int nb = e1 - e0;
  for (int i = tid; i < nb; i += kA) s_hit[i] = 0;
  __syncthreads();
  int hit_all = 0;
  for (int i = tid; i < nb * ws.nch; i += kA) {
    const int h = ws.hitblk[(size_t)e0 * ws.nch + i];
    if (h) atomicAdd(&s_hit[i / ws.nch], h);
    hit_all += h;
  }
  hit_all = ech::block_sum<kA>(hit_all, scr);   // contains the barrier s_hit needs
  for (int i = tid; i < nb; i += kA) {
    int32_t* st = stats + 4 * (e0 + i);
    st[0] = s_hit[i];
    st[1] = 0;
    st[2] = 0;
    st[3] = 0;
    ws.lb[e0 + i] = 0;
  }
  // the early miss list starts empty: every entry (-1, -1)
  for (int i = tid; i < 2 * M_early; i += kA) miss_early[i] = -1;
  // free slots in ring order from the head, up to the early demand bound
  int found = 0;
  for (int i0 = 0; i0 < C && found < M_early; i0 += kWinA) {   // block-uniform
#pragma unroll
    for (int j = 0; j < kWinA / kA; ++j) {   // coalesced loads, all in flight
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
    for (int qq = 0; qq < 4; ++qq) cnt += __popc(fw[qq]);   // flags are 0/1 bytes
    int tot;
    int rank = found + ech::block_excl_scan<kA>(cnt, scr, &tot);
    if (rank < M_early) {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if ((fw[qq] >> (8 * e)) & 1u) {
            if (rank < M_early) {
              int p = head + i0 + 16 * tid + 4 * qq + e;
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
    Ctl* cl = ws.ctl;
    cl->next_group = 0;
    cl->a_done = 0;
    cl->c_done = 0;
    cl->nfree = min(found, M_early);
    cl->finished = 0;
    ctr[ECH_CTR_EPOCH] = ep;
    ctr[ECH_CTR_NPINNED] = hit_all;
    ctr[ECH_CTR_NEVICT] = 0;
    ctr[ECH_CTR_NWANT] = 0;
    ctr[ECH_CTR_NMISS_EARLY] = 0;
    ctr[ECH_CTR_NCOPIED_EARLY] = 0;
  }
}

// ------------------------------------------------------------------ fused
struct FusedArgs {
  // scores
  const uint16_t* q;
  const float* w;
  const uint8_t* kc;
  const float* ksc;
  const int64_t* tok0;
  const int32_t* lens;
  float* out;
  int64_t ld;
  int gx;                  // scoring workgroups per row
  // early fetch
  int e0, e1, cap;
  const float* theta;
  int32_t* tok2slot;
  int64_t P;
  int32_t* slot2tok;
  int32_t C;
  int32_t* miss;           // [M_early, 2]
  int32_t M_early;
  int32_t* ctr;
  int32_t* stats;
  // recall
  const v4u* host;         // device view of the pinned pool
  v4u* dev;
  int row16;
  int n_alloc_wg, n_copy_wg;
  FWs ws;
};

constexpr int kFusedLds = kWavesF * kNS * kDecTile + kWavesF * 2 * 64 * 4;
static_assert(kFusedLds >= 4 * kMaxCap + 64, "alloc list fits");
static_assert(kFusedLds >= 8 * (kT * kCopyUnroll), "copy entries fit");

// One early sequence: its misses in token order, its ranks, its slots.
__device__ void alloc_sequence(const FusedArgs& a, int b, int* s_list, int* scr, u64* s_bcast) {
  const int tid = threadIdx.x;
  const int len = a.lens[b];
  const float th = a.theta[b];
  const int nw = (th == th && len > 0) ? min((len + kWaveTok - 1) / kWaveTok, a.ws.wpr) : 0;
  const int64_t g0 = a.tok0[b];
  const u64* mk = a.ws.masks + (size_t)b * a.ws.wpr * kWords;
  const u64 t0 = wall_clock64();
  int want = 0;
  for (int base = 0; base < nw; base += kT) {   // block-uniform
    const int i = base + tid;
    // One thread waits for the window's last wave (the waves of a row are
    // scored in order, so it is about the last to publish), then every
    // thread reads its own wave: few polls while the scoring runs.
    if (tid == 0) {
      const u64* wl = mk + (size_t)(min(base + kT, nw) - 1) * kWords;
      u64 v;
      spin_until([&] { return ld_dev(wl); }, [](u64 x) { return (x >> 32) == 1ull; }, a.ctr, t0, &v);
    }
    __syncthreads();
    u64 wd[kWords];
    int c = 0;
    if (i < nw) {
      u64* wp = const_cast<u64*>(mk) + (size_t)i * kWords;
      u64 v;
      spin_until([&] { return ld_dev(wp); }, [](u64 x) { return (x >> 32) == 1ull; }, a.ctr, t0, &v);
      wd[0] = v;
#pragma unroll
      for (int k = 1; k < kWords; ++k) {
        spin_until([&] { return ld_dev(wp + k); }, [](u64 x) { return (x >> 32) == 1ull; }, a.ctr, t0, &v);
        wd[k] = v;
      }
#pragma unroll
      for (int k = 0; k < kWords; ++k) {
        c += __popc((uint32_t)wd[k]);
        st_dev(wp + k, 0ull);   // consumed: the next step finds it empty
      }
    }
    int tot;
    int r = want + ech::block_excl_scan<kT>(c, scr, &tot);
    if (i < nw && c > 0 && r < a.cap) {
#pragma unroll
      for (int k = 0; k < kWords; ++k) {
        for (uint32_t m = (uint32_t)wd[k]; m != 0u && r < a.cap; m &= m - 1u, ++r)
          s_list[r] = (int)(g0 + (int64_t)i * kWaveTok + 32 * k + __builtin_ctz(m));
      }
    }
    want += tot;
  }
  const int take = min(a.cap, want);
  // this sequence's first rank: the takes of the early sequences before it
  if (tid == 0) {
    st_dev(&a.ws.lb[b], kAgg | (u64)take);
    u64 base = 0;
    for (int bb = b - 1; bb >= a.e0; --bb) {
      u64 v;
      spin_until([&] { return ld_dev(&a.ws.lb[bb]); }, [](u64 x) { return (x & (kAgg | kInc)) != 0ull; }, a.ctr,
                 t0, &v);
      base += v & 0xffffffffull;
      if (v & kInc) break;
    }
    st_dev(&a.ws.lb[b], kInc | (base + (u64)take));
    *s_bcast = base;
  }
  __syncthreads();   // s_list complete, base published in LDS
  const int base = (int)*s_bcast;
  const int nfree = a.ws.ctl->nfree;
  const int fetched = max(0, min(nfree - base, take));
  int ev = 0;
  for (int r = tid; r < fetched; r += kT) {
    const int m = base + r;
    const int p = a.ws.freelist[m];
    const int g = s_list[r];
    if (p < 0 || p >= a.C || g < 0 || g >= a.P) {
      set_status(a.ctr, ECH_ST_OVERFLOW);   // unreachable unless the rank phase and the masks disagree
      continue;
    }
    const int u = a.slot2tok[p];
    if (u >= 0 && u < a.P) {
      a.tok2slot[u] = -1;   // evict; the host row stays where it is
      ++ev;
    }
    a.slot2tok[p] = g;
    a.tok2slot[g] = p;
    st_dev(reinterpret_cast<u64*>(a.miss) + m, (u64)(uint32_t)g | ((u64)(uint32_t)p << 32));
  }
  const int evs = ech::block_sum<kT>(ev, scr);
  if (tid == 0) {
    int32_t* st = a.stats + 4 * b;
    st[1] = fetched;
    st[2] = want - fetched;   // wanted (before the cap) and not fetched
    st[3] = evs;
    if (evs) atomicAdd(&a.ctr[ECH_CTR_NEVICT], evs);
  }
  __syncthreads();   // s_list and s_bcast are reused by the next sequence
}

__device__ void alloc_role(const FusedArgs& a, int j, uint8_t* smem) {
  __shared__ int scr[kT / 64];
  __shared__ u64 s_bcast;
  int* s_list = reinterpret_cast<int*>(smem);
  for (int b = a.e0 + j; b < a.e1; b += a.n_alloc_wg) alloc_sequence(a, b, s_list, scr, &s_bcast);
  if (threadIdx.x == 0) {
    const int prev = atomicAdd(&a.ws.ctl->a_done, 1);
    if (prev == a.n_alloc_wg - 1) {   // the last alloc workgroup: totals, head, and the end mark
      u64 v;
      spin_until([&] { return ld_dev(&a.ws.lb[a.e1 - 1]); }, [](u64 x) { return (x & kInc) != 0ull; }, a.ctr,
                 wall_clock64(), &v);
      const int total = (int)(v & 0xffffffffull);
      const int n_alloc = min(total, a.ws.ctl->nfree);
      a.ctr[ECH_CTR_NWANT] = total;
      a.ctr[ECH_CTR_NMISS_EARLY] = n_alloc;
      if (n_alloc > 0) {
        const int last = a.ws.freelist[n_alloc - 1];
        a.ctr[ECH_CTR_HEAD] = (last + 1 == a.C) ? 0 : last + 1;
      }
      st_dev(&a.ws.ctl->finished, kFin | (u64)n_alloc);
    }
  }
}

__device__ void copy_role(const FusedArgs& a, uint8_t* smem) {
  __shared__ int s_g, s_stop;
  u64* s_e = reinterpret_cast<u64*>(smem);
  const int tid = threadIdx.x;
  const int rg = max(1, (kT * kCopyUnroll) / a.row16);   // rows per group
  const u64 t0 = wall_clock64();
  u64* fin = &a.ws.ctl->finished;
  const u64* ent = reinterpret_cast<const u64*>(a.miss);
  for (;;) {
    if (tid == 0) {
      if (ld_dev(fin) & kFin) {
        s_stop = 1;
      } else {
        s_stop = 0;
        s_g = atomicAdd(&a.ws.ctl->next_group, 1);
      }
    }
    __syncthreads();
    if (s_stop) break;
    const int m0 = s_g * rg;
    // One thread waits for the group's last entry (entries are written in
    // about rank order) or the end mark, then one thread per row reads its
    // entry: few polls while the allocation runs.
    if (tid == 0) {
      const int m = min(m0 + rg, a.M_early) - 1;
      for (;;) {
        if (m < m0 || ld_dev(ent + m) != kNone) break;
        const u64 f = ld_dev(fin);
        if ((f & kFin) && m >= (int)(f & 0xffffffffull)) break;
        if (wall_clock64() - t0 > kSpinTicks) {
          set_status(a.ctr, ECH_ST_TIMEOUT);
          break;
        }
        __builtin_amdgcn_s_sleep(16);
      }
    }
    __syncthreads();
    if (tid < rg) {   // one thread per row of the group reads its entry
      const int m = m0 + tid;
      u64 e = kNone;
      if (m < a.M_early) {
        for (;;) {
          e = ld_dev(ent + m);
          if (e != kNone) break;
          const u64 f = ld_dev(fin);
          if ((f & kFin) && m >= (int)(f & 0xffffffffull)) break;   // past the end: nothing to copy
          if (wall_clock64() - t0 > kSpinTicks) {
            set_status(a.ctr, ECH_ST_TIMEOUT);
            break;
          }
          __builtin_amdgcn_s_sleep(16);
        }
      }
      s_e[tid] = e;
    }
    __syncthreads();
    v4u v[kCopyUnroll];
    int64_t dst[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {   // all host loads in flight, then the stores
      const int i = tid + u * kT;
      dst[u] = -1;
      if (i < rg * a.row16) {
        const int row = i / a.row16, c = i - row * a.row16;
        const u64 e = s_e[row];
        if (e != kNone) {
          const int g = (int)(uint32_t)e, p = (int)(uint32_t)(e >> 32);
          if (g >= 0 && g < a.P && p >= 0 && p < a.C) {
            v[u] = __builtin_nontemporal_load(a.host + (int64_t)g * a.row16 + c);
            dst[u] = (int64_t)p * a.row16 + c;
          } else if (c == 0) {
            set_status(a.ctr, ECH_ST_BADMISS);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u)
      if (dst[u] >= 0) __builtin_nontemporal_store(v[u], a.dev + dst[u]);
    __syncthreads();   // s_g, s_e are rewritten by the next group
  }
  if (tid == 0) {
    const int prev = atomicAdd(&a.ws.ctl->c_done, 1);
    if (prev == a.n_copy_wg - 1) {   // the last copy workgroup: every claimed group is copied
      const int n_alloc = (int)(ld_dev(fin) & 0xffffffffull);
      const int claimed = ld_dev(&a.ws.ctl->next_group);
      const int ncopied = (int)min((int64_t)claimed * rg, (int64_t)n_alloc);
      a.ctr[ECH_CTR_NCOPIED_EARLY] = ncopied;
      atomicAdd(&a.ctr[ECH_CTR_RECALLED], ncopied);
    }
  }
}

__device__ void score_role(const FusedArgs& a, int fb, uint8_t* smem) {
  const int r = fb / a.gx, bx = fb - r * a.gx;
  const int len = a.lens[r];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wi = bx * kWavesF + wave;        // wave index within the row
  const int wt0 = wi * kWaveTok;
  if (wt0 >= len) return;
  uint8_t (*ring)[kDecTile] = reinterpret_cast<uint8_t (*)[kDecTile]>(smem + wave * kNS * kDecTile);
  float (*sring)[64] = reinterpret_cast<float (*)[64]>(smem + kWavesF * kNS * kDecTile + wave * 2 * 64 * 4);
  float keep[kTPW / 4];
  const int64_t g0 = a.tok0[r];
  fp8_wave_scores<kTPW, kNS>(a.q, a.w, a.kc, a.ksc, r, g0, len, wt0, ring, sring, keep);
  fp8_wave_store<kTPW>(keep, &ring[0][0], a.out + (size_t)r * a.ld + wt0, min(kWaveTok, len - wt0));
  if (r < a.e0 || r >= a.e1) return;
  const float th = a.theta[r];
  if (th != th) return;
  // misses of this wave: tokens above theta (strict) that are not resident
  const int lane = threadIdx.x & 63;
  bool above[kTPW / 4];
  int sl[kTPW / 4];
#pragma unroll
  for (int j = 0; j < kTPW / 4; ++j) {
    const int t = wt0 + 64 * j + lane;
    above[j] = t < len && keep[j] > th && g0 + t < a.P;
    sl[j] = above[j] ? a.tok2slot[g0 + t] : 0;   // the lookups of the four tokens in flight together
  }
  u64 bal[kTPW / 4];
#pragma unroll
  for (int j = 0; j < kTPW / 4; ++j) bal[j] = __ballot(above[j] && !(sl[j] >= 0 && sl[j] < a.C));
  if (lane < kWords) {
    u64 m = bal[0];
#pragma unroll
    for (int j = 1; j < kTPW / 4; ++j)
      if ((lane >> 1) == j) m = bal[j];
    const uint32_t half = (lane & 1) ? (uint32_t)(m >> 32) : (uint32_t)m;
    st_dev(a.ws.masks + ((size_t)r * a.ws.wpr + wi) * kWords + lane, kTag | half);
  }
}

__global__ __launch_bounds__(kT) void fused_kernel(FusedArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kFusedLds];
  const int bid = blockIdx.x;
  if (bid < a.n_alloc_wg) {
    alloc_role(a, bid, smem);
  } else if (bid < a.n_alloc_wg + a.n_copy_wg) {
    copy_role(a, smem);
  } else {
    score_role(a, bid - a.n_alloc_wg - a.n_copy_wg, smem);
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" size_t ech_index_logits_early_ws_bytes(int R, int max_len, int32_t M_early) {
  if (R < 1 || max_len < 0 || M_early < 0) return 0;
  return fused_layout(R, max_len, M_early, nullptr, nullptr);
}

extern "C" int ech_index_logits_early(const void* q, const float* w, const void* kcache, int kdtype,
                                      const float* kscale, const int64_t* row_tok0, const int32_t* row_len, int R,
                                      int H, int D, int max_len, float* logits, int64_t ld, int e0, int e1,
                                      const float* theta, int cap, int32_t* tok2slot, int64_t P, int32_t* slot2tok,
                                      int32_t* slot_pin, int32_t C, int32_t* miss_early, int32_t M_early,
                                      int32_t* ctr, int32_t* stats, const void* host_pool, int64_t row_bytes,
                                      void* dev_cache, void* ws, size_t ws_bytes, void* stream) {
  if (!q || !w || !kcache || !row_tok0 || !row_len || !logits || !theta || !tok2slot || !slot2tok || !slot_pin ||
      !miss_early || !ctr || !stats || !host_pool || !dev_cache || !ws)
    return ECH_EINVAL;
  if (kdtype != ECH_KEY_FP8) return ECH_EUNSUPPORTED;
  if (!kscale || H != kH || D != kD || R < 1 || R > kMaxB || max_len < 0 || ld < max_len) return ECH_EINVAL;
  if (e0 < 0 || e1 <= e0 || e1 > R || cap < 0 || cap > kMaxCap) return ECH_EINVAL;
  if (P < 1 || P >= INT32_MAX || C < 1 || C > (1 << 30) || M_early < 0) return ECH_EINVAL;
  if ((int64_t)M_early < (int64_t)(e1 - e0) * std::min(cap, max_len)) return ECH_EINVAL;
  if (row_bytes < 16 || row_bytes % 16 != 0 || row_bytes > 16 * kT * kCopyUnroll) return ECH_EINVAL;
  if (!aligned16(q) || !aligned16(kcache) || !aligned16(dev_cache) || !aligned16(host_pool)) return ECH_EINVAL;
  if ((reinterpret_cast<uintptr_t>(miss_early) & 7u) || (reinterpret_cast<uintptr_t>(ws) & 255u)) return ECH_EINVAL;
  if (ws_bytes < ech_index_logits_early_ws_bytes(R, max_len, M_early)) return ECH_EINVAL;
  void* hdev = nullptr;
  if (hipHostGetDevicePointer(&hdev, const_cast<void*>(host_pool), 0) != hipSuccess || !hdev) {
    (void)hipGetLastError();
    return ECH_EINVAL;
  }
  FWs fw;
  fused_layout(R, max_len, M_early, &fw, static_cast<char*>(ws));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint8_t* kk = static_cast<const uint8_t*>(kcache);
  hipLaunchKernelGGL(fused_pin_kernel, dim3(fw.nch, e1 - e0), dim3(kT), 0, s, qq, w, kk, kscale, row_tok0, row_len,
                     theta, e0, tok2slot, P, C, slot_pin, ctr, fw);
  ECH_LAUNCH_CHECK();
  hipLaunchKernelGGL(fused_rank_kernel, dim3(1), dim3(kA), 0, s, slot_pin, C, e0, e1, miss_early, M_early, ctr,
                     stats, fw);
  ECH_LAUNCH_CHECK();
  FusedArgs a;
  a.q = qq;
  a.w = w;
  a.kc = kk;
  a.ksc = kscale;
  a.tok0 = row_tok0;
  a.lens = row_len;
  a.out = logits;
  a.ld = ld;
  a.gx = (max_len + kWavesF * kWaveTok - 1) / (kWavesF * kWaveTok);
  a.e0 = e0;
  a.e1 = e1;
  a.cap = cap;
  a.theta = theta;
  a.tok2slot = tok2slot;
  a.P = P;
  a.slot2tok = slot2tok;
  a.C = C;
  a.miss = miss_early;
  a.M_early = M_early;
  a.ctr = ctr;
  a.stats = stats;
  a.host = static_cast<const v4u*>(hdev);
  a.dev = static_cast<v4u*>(dev_cache);
  a.row16 = (int)(row_bytes / 16);
  a.n_alloc_wg = std::min(e1 - e0, kMaxAlloc);
  a.n_copy_wg = kCopy;
  a.ws = fw;
  const int64_t blocks = (int64_t)a.n_alloc_wg + a.n_copy_wg + (int64_t)a.gx * R;
  if (blocks > INT32_MAX) return ECH_EINVAL;
  hipLaunchKernelGGL(fused_kernel, dim3((unsigned)blocks), dim3(kT), 0, s, a);
  ECH_LAUNCH_CHECK();
  return ECH_OK;
}
