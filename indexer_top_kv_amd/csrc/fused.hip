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
// changes is when things happen: a sequence's early misses get their slots,
// and appear in the early miss list, while later sequences are still being
// scored, and a copier launch on another stream moves their rows meanwhile.
//
//   pins    (min(e1-e0, 64) x 4 workgroups) only slots the allocation can
//           reach need their pin status, so the ring is taken in windows of
//           32768 positions from the head, a quarter per workgroup: each
//           workgroup finds its sequence's tokens in its quarter (slot2tok),
//           scores them with the scores
//           kernel's own tile arithmetic (decode.hpp / score.hpp: the same bit
//           patterns) and pins those above theta (slot_pin = epoch); the
//           workgroups then agree, through two counters, whether the windows
//           so far hold enough unpinned slots for the early demand bound, else
//           take the next window. Also clears the control words, the early
//           miss list (every entry (-1, -1)) and the free list.
//   fused   one launch, three kinds of workgroups (1-D grid, in this order):
//     rank    (16) the unpinned slots in ring order from the head, as many as
//             the early demand bound (ring slices with a decoupled look-back),
//             published one by one: the free list, then its length.
//     alloc   (one per early sequence, at most 64, each taking every 64th)
//             waits for the masks its sequence's scoring waves publish, lists
//             the sequence's first `cap` misses in token order, takes its
//             first rank from the sequences before it (decoupled look-back,
//             the predecessors' words read in parallel), gives miss m the m-th
//             free slot (evicting its old token, no write-back) and writes miss
//             m. The last early sequence publishes the list's length.
//     score   the fp8 decode scores kernel's waves (256 tokens each); a wave
//             of an early sequence then looks up the residency of its tokens
//             above theta and publishes its misses as a 256-bit mask in 8
//             tagged words, with the count of its resident tokens above theta
//             (hits).
//   copier  a separate launch on a second stream (ech_recall_early_live):
//           claims groups of consecutive ranks in order and copies their rows
//           from pinned host memory over PCIe as their entries appear, so the
//           transfer runs beside the scoring and on beside the top-k.
//
// Workgroups communicate through words that carry their own validity (a tag
// bit, a flag, or a (-1, -1) / 0 sentinel), read and written with relaxed
// device-scope atomics (coherent across the chiplets' L2 caches), so no
// release fence - which writes back a whole L2 on MI355X - is needed inside a
// launch. Scoring waves and rank workgroups wait on nothing but rank
// look-backs; alloc workgroups wait on scoring waves, rank workgroups and
// earlier sequences; the pins workgroups wait on one another (64 at most, all
// resident). Every wait is bounded (0.5 s of the constant-rate clock): past it
// the workgroup sets ECH_ST_TIMEOUT and carries on, so every launch ends. The
// copier only ever waits with a short patience and then leaves the rest to
// ech_recall(ECH_EARLY), so it is correct whichever way the two streams are
// scheduled.
//
// Measured on MI355X (32 x 131072 fp8, 260000 slots): PCIe reads in flight
// slow the HBM stream and stretch every dependent memory round trip several
// times over, so the copier is kept to 32 workgroups (1 MB in flight).

#include <algorithm>

#include "bins.hpp"
#include "decode.hpp"
#include "lists.hpp"

namespace {

constexpr int kT = 256;
constexpr int kTPW = 16;                 // tiles per scoring wave
constexpr int kNS = 4;                   // ring slots per scoring wave
constexpr int kWavesF = 4;               // waves per scoring workgroup
constexpr int kWaveTok = kTPW * 16;      // 256 tokens per scoring wave
constexpr int kWords = kWaveTok / 32;    // mask words per wave
constexpr int kListSlice = 64;           // band entries a scoring wave lists for the top-k, at most
constexpr int kMaxCap = 4096;
constexpr int kMaxB = 1024;
constexpr int kMaxAlloc = 64;            // alloc workgroups at most
constexpr int kCopyUnroll = 8;           // 16-byte pieces per thread per copied group
constexpr int kPinPart = 8192;           // ring positions per pins workgroup and window
constexpr int kPinParts = 4;             // pins workgroups per early sequence (parts of a window)
constexpr int kPinWin = kPinPart * kPinParts;   // ring positions per window of the pins kernel
constexpr int kMaxPinWg = 64;            // early sequences the pins grid covers at once
constexpr int kRankSlice = kT * 16;      // ring positions per slice of a rank workgroup
constexpr int kRankWg = 16;              // rank workgroups

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
  int c_done;                            // copy workgroups finished
  int ep;                                // the phase's epoch
  int head;                              // the ring head at the phase's start
  int pin_done;                          // pins kernel: window arrivals (all workgroups, all windows)
  int pin_total;                         // pins kernel: slots pinned so far
  int first_incomplete;                  // live copier: the first group it gave up on
  int next_fgroup;                       // live copier: FINAL copy groups claimed
  u64 finished;                          // kFin | n_alloc
  u64 nfree;                             // kFin | free slots ranked (<= M_early)
};

struct FWs {
  Ctl* ctl;
  u64* lb;                               // [R] look-back word per sequence
  u64* rlb;                              // [ceil(C / kRankSlice)] look-back word per ring slice
  int* freelist;                         // [M_early] slot + 1 of the free slot of each rank (0: not yet)
  u64* masks;                            // [R * wpr * kWords] published miss masks
  int2* lmeta;                           // [R * wpr] per scoring wave: (band tokens listed, floor bin)
  int2* lpool;                           // [R * wpr * kListSlice] listed (score bits, token), per wave
  float* lth;                            // [R] the theta each row's band was listed against
  int wpr;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t fused_layout(int R, int max_len, int32_t C, int32_t M_early, FWs* w, char* base) {
  const int wpr = std::max(1, (max_len + kWaveTok - 1) / kWaveTok);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  const size_t o_ctl = take(sizeof(Ctl)), o_lb = take(8 * (size_t)R),
               o_rlb = take(8 * (size_t)((std::max(C, 1) + kRankSlice - 1) / kRankSlice)),
               o_fl = take(4 * (size_t)std::max(M_early, 1)),
               o_m = take(8 * (size_t)R * wpr * kWords), o_lm = take(8 * (size_t)R * wpr),
               o_lp = take(8 * (size_t)R * wpr * kListSlice), o_lt = take(4 * (size_t)R);
  if (w && base) {
    w->ctl = reinterpret_cast<Ctl*>(base + o_ctl);
    w->lb = reinterpret_cast<u64*>(base + o_lb);
    w->rlb = reinterpret_cast<u64*>(base + o_rlb);
    w->freelist = reinterpret_cast<int*>(base + o_fl);
    w->masks = reinterpret_cast<u64*>(base + o_m);
    w->lmeta = reinterpret_cast<int2*>(base + o_lm);
    w->lpool = reinterpret_cast<int2*>(base + o_lp);
    w->lth = reinterpret_cast<float*>(base + o_lt);
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
__device__ __forceinline__ void st_dev(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

// ------------------------------------------------------------------ pins
// grid (min(e1 - e0, kMaxPinWg), kPinParts); workgroup (j, part) handles
// part `part` (kPinPart positions) of every window for the early sequences
// e0 + j, e0 + j + gridDim.x, ... A window covers twice the early demand
// bound of a full batch, so one window normally suffices. Every workgroup
// takes part in every window's count (two counters that only grow, so
// nothing is cleared between windows); every workgroup reads the same totals
// after a window and so takes the same decision.
constexpr int kPinBatch = 4;

__device__ int pin_sequence_window(const uint16_t* __restrict__ q, const float* __restrict__ w,
                                   const uint8_t* __restrict__ kc, const float* __restrict__ ksc, int b, int64_t g0,
                                   int len, float th, const int32_t* __restrict__ slot2tok, int32_t C, int head, int p0,
                                   int wsz, int ep, int32_t* __restrict__ slot_pin, int* s_pos, int* scr) {
  const int tid = threadIdx.x;
  // the part's slots holding a token of sequence b
  constexpr int kU = kPinPart / kT;
  static_assert(kU % 32 == 0, "whole mask words");
  int n = 0;
  uint32_t mine[kU / 32];
#pragma unroll
  for (int k = 0; k < kU / 32; ++k) mine[k] = 0;
#pragma unroll
  for (int u0 = 0; u0 < kU; u0 += 16) {
    int gv[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {   // coalesced, sixteen in flight
      const int pos = p0 + (u0 + u) * kT + tid;
      int p = head + min(pos, C - 1);
      if (p >= C) p -= C;
      gv[u] = slot2tok[p];
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const bool in = (u0 + u) * kT + tid < wsz && gv[u] >= g0 && (int64_t)gv[u] < g0 + len;
      if (in) mine[(u0 + u) >> 5] |= 1u << ((u0 + u) & 31);
      n += in;
    }
  }
  int nres;
  int pos = ech::block_excl_scan<kT>(n, scr, &nres);
#pragma unroll
  for (int k = 0; k < kU / 32; ++k)
    for (uint32_t m = mine[k]; m != 0u; m &= m - 1u) s_pos[pos++] = (32 * k + __builtin_ctz(m)) * kT + tid;
  __syncthreads();
  int pinned = 0;
  const int lane = tid & 63, wave = tid >> 6;
  const int ntile = (nres + 15) / 16;
  if (wave < ntile) {   // wave-uniform
    const int col = lane & 15, grp = lane >> 4;
    // query fragments and head weights in the scores kernel's operand layout
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
    for (int j0 = wave; j0 < ntile; j0 += kPinBatch * (kT / 64)) {
      KeyFrag<ECH_KEY_FP8> f[kPinBatch];
      float sc[kPinBatch];
      int pp[kPinBatch];
      int64_t gg[kPinBatch];
#pragma unroll
      for (int u = 0; u < kPinBatch; ++u) {   // the batch's gathers, all in flight
        const int e = 16 * (j0 + u * (kT / 64)) + col;
        int p = head + p0 + s_pos[min(e, nres - 1)];
        p = (int)((int64_t)p % C);
        pp[u] = p;
        gg[u] = slot2tok[p];
        load_key<ECH_KEY_FP8>(f[u], kc + (size_t)gg[u] * kD, grp);
        sc[u] = ksc[gg[u]];
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
            slot_pin[pp[u]] = ep;
            ++pinned;
          }
        }
      }
    }
  }
  __syncthreads();   // s_pos is rewritten by the next sequence or window
  return pinned;
}

__global__ __launch_bounds__(kT) void fused_pins_kernel(const uint16_t* __restrict__ q, const float* __restrict__ w,
                                                        const uint8_t* __restrict__ kc, const float* __restrict__ ksc,
                                                        const int64_t* __restrict__ tok0,
                                                        const int32_t* __restrict__ lens,
                                                        const float* __restrict__ theta, int e0, int e1,
                                                        const int32_t* __restrict__ slot2tok, int32_t C,
                                                        int32_t* __restrict__ slot_pin, int32_t* __restrict__ miss_early,
                                                        int32_t M_early, int32_t* ctr, FWs ws) {
  __shared__ int s_pos[kPinPart];
  __shared__ int scr[kT / 64];
  __shared__ int s_tot;
  const int tid = threadIdx.x, j = blockIdx.x, part = blockIdx.y;
  const int lid = blockIdx.y * gridDim.x + blockIdx.x, nwg = gridDim.x * gridDim.y;
  const int ep = ctr[ECH_CTR_EPOCH] + 1;
  int head = ctr[ECH_CTR_HEAD];
  if (head < 0 || head >= C) head = 0;   // only a corrupted state; keeps every slot index in range
  // the launch starts from empty lists and cleared control words
  for (int i = lid * kT + tid; i < 2 * M_early; i += nwg * kT) miss_early[i] = -1;
  for (int i = lid * kT + tid; i < M_early; i += nwg * kT) ws.freelist[i] = 0;
  for (int b = e0 + lid * kT + tid; b < e1; b += nwg * kT) ws.lb[b] = 0;
  for (int i = lid * kT + tid; i < (C + kRankSlice - 1) / kRankSlice; i += nwg * kT) ws.rlb[i] = 0;
  if (lid == 0 && tid == 0) {
    Ctl* cl = ws.ctl;
    cl->next_group = 0;
    cl->c_done = 0;
    cl->ep = ep;
    cl->head = head;
    cl->finished = 0;
    cl->nfree = 0;
    cl->first_incomplete = INT32_MAX;
    cl->next_fgroup = 0;
    ctr[ECH_CTR_FINAL_READY] = 0;   // the FINAL phase after this launch sets it again
    ctr[ECH_CTR_EARLY_WALK] = 0;
    ctr[ECH_CTR_NEVICT] = 0;
    ctr[ECH_CTR_NWANT] = 0;
    ctr[ECH_CTR_NMISS_EARLY] = 0;
    ctr[ECH_CTR_NCOPIED_EARLY] = 0;
    ctr[ECH_CTR_NPINNED] = 0;
  }
  const u64 t0 = wall_clock64();
  int covered = 0;
  for (int win = 0;; ++win) {   // block-uniform
    const int w0 = win * kPinWin;
    if (w0 >= C) break;
    const int p0 = w0 + part * kPinPart;
    const int wsz = max(0, min(kPinPart, C - p0));
    int pinned = 0;
    for (int b = e0 + j; b < e1 && wsz > 0; b += gridDim.x) {
      const float th = theta[b];
      if (th != th) continue;
      pinned += pin_sequence_window(q, w, kc, ksc, b, tok0[b], lens[b], th, slot2tok, C, head, p0, wsz, ep, slot_pin,
                                    s_pos, scr);
    }
    pinned = ech::block_sum<kT>(pinned, scr);
    if (tid == 0) {
      if (pinned) atomicAdd(&ws.ctl->pin_total, pinned);
      atomicAdd(&ws.ctl->pin_done, 1);
      for (;;) {   // every workgroup's count of this window is in
        if (ld_dev(&ws.ctl->pin_done) >= nwg * (win + 1)) break;
        if (wall_clock64() - t0 > kSpinTicks) {
          set_status(ctr, ECH_ST_TIMEOUT);
          break;
        }
        __builtin_amdgcn_s_sleep(4);
      }
      s_tot = ld_dev(&ws.ctl->pin_total);
    }
    __syncthreads();
    covered += min(kPinWin, C - w0);
    const int enough = covered - s_tot >= M_early;
    __syncthreads();   // s_tot is rewritten after the next window
    if (enough) break;
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
  const int32_t* slot_pin;
  int n_alloc_wg;
  FWs ws;
};

constexpr int kFusedLds = kWavesF * kNS * kDecTile + kWavesF * 2 * 64 * 4;
static_assert(kFusedLds >= 4 * kMaxCap + 64, "alloc list fits");
static_assert(kFusedLds >= kRankSlice, "rank flags fit");

// The free list: unpinned slots in ring order from the head (the pins kernel
// stamped every pinned slot of the windows it took, and those hold enough
// unpinned ones). Rank workgroup i takes ring slices i, i + kRankWg, ... of
// kRankSlice positions; a slice's first rank comes from the slices before it
// (decoupled look-back); entries are published one by one as slot + 1, and
// the slice holding the last needed rank (or the ring's end) publishes the
// count.
__device__ void rank_role(const FusedArgs& a, int i, uint8_t* smem) {
  __shared__ int scr[kT / 64];
  __shared__ u64 s_ex;
  uint8_t* s_fr = smem;
  const int tid = threadIdx.x;
  const int ep = a.ws.ctl->ep, head = a.ws.ctl->head, C = a.C, M = a.M_early;
  const int nslice = (C + kRankSlice - 1) / kRankSlice;
  const u64 t0 = wall_clock64();
  for (int k = i; k < nslice; k += kRankWg) {   // block-uniform
    const int i0 = k * kRankSlice;
#pragma unroll
    for (int j = 0; j < kRankSlice / kT; ++j) {   // coalesced loads, all in flight
      const int pos = i0 + j * kT + tid;
      int p = head + min(pos, C - 1);
      if (p >= C) p -= C;
      const int pv = a.slot_pin[p];
      s_fr[j * kT + tid] = (pos < C && pv != ep) ? 1 : 0;
    }
    __syncthreads();
    // thread t ranks positions i0 + 16t .. +15
    const uint4 f0 = reinterpret_cast<const uint4*>(s_fr)[tid];
    const uint32_t fw[4] = {f0.x, f0.y, f0.z, f0.w};
    int cnt = 0;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) cnt += __popc(fw[qq]);   // flags are 0/1 bytes
    int tot;
    int local = ech::block_excl_scan<kT>(cnt, scr, &tot);
    if (tid == 0) {   // this slice's first rank
      st_dev(&a.ws.rlb[k], kAgg | (u64)tot);
      u64 ex = 0;
      for (int kk = k - 1; kk >= 0; --kk) {
        u64 v;
        spin_until([&] { return ld_dev(&a.ws.rlb[kk]); }, [](u64 x) { return (x & (kAgg | kInc)) != 0ull; }, a.ctr,
                   t0, &v);
        ex += v & 0xffffffffull;
        if (v & kInc) break;
      }
      st_dev(&a.ws.rlb[k], kInc | (ex + (u64)tot));
      if ((ex < (u64)M && ex + (u64)tot >= (u64)M) || (k == nslice - 1 && ex < (u64)M))
        st_dev(&a.ws.ctl->nfree, kFin | min(ex + (u64)tot, (u64)M));
      s_ex = ex;
    }
    __syncthreads();
    const int ex = (int)min(s_ex, (u64)M);
    int rank = ex + local;
    if (rank < M) {
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if ((fw[qq] >> (8 * e)) & 1u) {
            if (rank < M) {
              int p = head + i0 + 16 * tid + 4 * qq + e;
              if (p >= C) p -= C;
              st_dev(&a.ws.freelist[rank], p + 1);
            }
            ++rank;
          }
        }
      }
    }
    const bool done = s_ex + (u64)tot >= (u64)M;
    __syncthreads();   // s_fr and s_ex are rewritten by the next slice
    if (done) break;
  }
  if (i == 0 && tid == 0) {
    a.ctr[ECH_CTR_EPOCH] = ep;
    a.ws.ctl->pin_done = 0;   // the pins kernel of the next call starts from zero
    a.ws.ctl->pin_total = 0;
  }
}

// The first rank of early sequence b: the takes of the early sequences before
// it, read back to the nearest one that has published its inclusive prefix.
// The words of up to kT predecessors are read at once, one per thread (a
// walk of one dependent load per predecessor costs tens of microseconds while
// the PCIe copy loads the memory system).
__device__ int first_rank(const FusedArgs& a, int b, u64 t0, int* scr, int* s_min) {
  const int tid = threadIdx.x;
  int base = 0;
  for (int off = 0; off < b - a.e0; off += kT) {   // block-uniform
    const int bb = b - 1 - off - tid;
    u64 v = 0;
    if (bb >= a.e0)
      spin_until([&] { return ld_dev(&a.ws.lb[bb]); }, [](u64 x) { return (x & (kAgg | kInc)) != 0ull; }, a.ctr,
                 t0, &v);
    if (tid == 0) *s_min = kT;
    __syncthreads();
    if (bb >= a.e0 && (v & kInc)) atomicMin(s_min, tid);
    __syncthreads();
    const int nearest = *s_min;   // the nearest inclusive prefix in this chunk, or kT
    base += ech::block_sum<kT>((bb >= a.e0 && tid <= nearest) ? (int)(v & 0xffffffffull) : 0, scr);
    if (nearest < kT) break;
  }
  return base;
}

// One early sequence: its misses in token order, its ranks, its slots.
__device__ void alloc_sequence(const FusedArgs& a, int b, int nfree, int* s_list, int* scr, int* s_min) {
  const int tid = threadIdx.x;
  const int len = a.lens[b];
  const float th = a.theta[b];
  const int nw = (th == th && len > 0) ? min((len + kWaveTok - 1) / kWaveTok, a.ws.wpr) : 0;
  const int64_t g0 = a.tok0[b];
  const u64* mk = a.ws.masks + (size_t)b * a.ws.wpr * kWords;
  const u64 t0 = wall_clock64();
  int want = 0, hits = 0;
  for (int base = 0; base < nw; base += kT) {   // block-uniform
    const int i = base + tid;
    // One thread waits for the window's last wave (the waves of a row are
    // scored in order, so it is about the last to publish), then every
    // thread reads its own wave: few polls while the scoring runs.
    if (tid == 0) {
      const u64* wl = mk + (size_t)(min(base + kT, nw) - 1) * kWords;
      u64 v;
      spin_until([&] { return ld_dev(wl); }, [](u64 x) { return (x & kTag) != 0ull; }, a.ctr, t0, &v);
    }
    __syncthreads();
    u64 wd[kWords];
    int c = 0;
    if (i < nw) {
      u64* wp = const_cast<u64*>(mk) + (size_t)i * kWords;
      u64 v;
      spin_until([&] { return ld_dev(wp); }, [](u64 x) { return (x & kTag) != 0ull; }, a.ctr, t0, &v);
      wd[0] = v;
#pragma unroll
      for (int k = 1; k < kWords; ++k) {
        spin_until([&] { return ld_dev(wp + k); }, [](u64 x) { return (x & kTag) != 0ull; }, a.ctr, t0, &v);
        wd[k] = v;
      }
      hits += (int)(wd[0] >> 33);   // the wave's resident tokens above theta
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
  hits = ech::block_sum<kT>(hits, scr);
  if (tid == 0) st_dev(&a.ws.lb[b], kAgg | (u64)take);   // later sequences need only this
  const int base = first_rank(a, b, t0, scr, s_min);
  if (tid == 0) {
    st_dev(&a.ws.lb[b], kInc | (u64)(base + take));
    if (b == a.e1 - 1) {   // the last early sequence knows the list's length
      const int total = base + take;
      const int n_alloc = min(total, nfree);
      st_dev(&a.ws.ctl->finished, kFin | (u64)n_alloc);
      a.ctr[ECH_CTR_NWANT] = total;
      a.ctr[ECH_CTR_NMISS_EARLY] = n_alloc;
      if (n_alloc > 0) {
        int pv;
        spin_until([&] { return ld_dev(&a.ws.freelist[n_alloc - 1]); }, [](int x) { return x != 0; }, a.ctr, t0,
                   &pv);
        const int last = pv - 1;
        a.ctr[ECH_CTR_HEAD] = (last + 1 == a.C) ? 0 : last + 1;
        a.ctr[ECH_CTR_EARLY_WALK] = (last - a.ws.ctl->head + a.C) % a.C + 1;
      }
    }
  }
  const int fetched = max(0, min(nfree - base, take));
  int ev = 0;
  for (int r = tid; r < fetched; r += kT) {
    const int m = base + r;
    int pv;
    spin_until([&] { return ld_dev(&a.ws.freelist[m]); }, [](int x) { return x != 0; }, a.ctr, t0, &pv);
    const int p = pv - 1;
    const int g = s_list[r];
    if (p < 0 || p >= a.C || g < 0 || g >= a.P) {
      set_status(a.ctr, ECH_ST_OVERFLOW);   // unreachable unless the rank workgroups and the masks disagree
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
    st[0] = hits;
    st[1] = fetched;
    st[2] = want - fetched;   // wanted (before the cap) and not fetched
    st[3] = evs;
    if (evs) atomicAdd(&a.ctr[ECH_CTR_NEVICT], evs);
    if (hits) atomicAdd(&a.ctr[ECH_CTR_NPINNED], hits);
  }
  __syncthreads();   // s_list is reused by the next sequence
}

__device__ void alloc_role(const FusedArgs& a, int j, uint8_t* smem) {
  __shared__ int scr[kT / 64];
  __shared__ int s_min, s_nfree;
  int* s_list = reinterpret_cast<int*>(smem);
  if (threadIdx.x == 0) {   // the free count, published by the rank workgroups early in the launch
    u64 nf;
    spin_until([&] { return ld_dev(&a.ws.ctl->nfree); }, [](u64 x) { return (x & kFin) != 0ull; }, a.ctr,
               wall_clock64(), &nf);
    s_nfree = (int)(nf & 0xffffffffull);
  }
  __syncthreads();
  const int nfree = s_nfree;
  for (int b = a.e0 + j; b < a.e1; b += a.n_alloc_wg) alloc_sequence(a, b, nfree, s_list, scr, &s_min);
}

// For the top-k (ech_topk_early): the wave's tokens in the row's band, the
// bins at and above the floor theta implies (the one-pass top-k's band), in
// token order into the wave's slice, and the wave's (count, floor). A NaN
// theta, or more band tokens than the slice holds, leaves (0, 256): no bin
// is known to be complete there, and the selection takes the whole row.
__device__ __forceinline__ void list_band(const FusedArgs& a, int r, int wi, int wt0, int len,
                                          const float (&keep)[kTPW / 4]) {
  const Shift shf = make_shift(a.theta[r]);
  const uint32_t blo = band_lo(shf);
  const int lane = threadIdx.x & 63;
  u64 bal[kTPW / 4];
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < kTPW / 4; ++j) {
    const int t = wt0 + 64 * j + lane;
    bal[j] = __ballot(t < len && shifted_bin_one(keep[j], shf) >= blo);
    cnt += __popcll(bal[j]);
  }
  const bool ok = shf.on && cnt <= kListSlice;
  const size_t wslot = (size_t)r * a.ws.wpr + wi;
  if (ok) {
    int2* lp = a.ws.lpool + wslot * kListSlice;
    int base = 0;
#pragma unroll
    for (int j = 0; j < kTPW / 4; ++j) {
      if ((bal[j] >> lane) & 1ull) {
        const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal[j] >> 32),
                                                              __builtin_amdgcn_mbcnt_lo((uint32_t)bal[j], 0u));
        lp[pos] = make_int2(__float_as_int(keep[j]), wt0 + 64 * j + lane);
      }
      base += __popcll(bal[j]);
    }
  }
  if (lane == 0) {
    a.ws.lmeta[wslot] = ok ? make_int2(cnt, (int)blo) : make_int2(0, 256);
    if (wi == 0) a.ws.lth[r] = shf.th;
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
  list_band(a, r, wi, wt0, len, keep);
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
  int hits = 0;
#pragma unroll
  for (int j = 0; j < kTPW / 4; ++j) {
    const bool res = sl[j] >= 0 && sl[j] < a.C;
    bal[j] = __ballot(above[j] && !res);
    hits += __popcll(__ballot(above[j] && res));
  }
  if (lane < kWords) {
    u64 m = bal[0];
#pragma unroll
    for (int j = 1; j < kTPW / 4; ++j)
      if ((lane >> 1) == j) m = bal[j];
    const uint32_t half = (lane & 1) ? (uint32_t)(m >> 32) : (uint32_t)m;
    // word 0 also carries the wave's hits (resident tokens above theta)
    st_dev(a.ws.masks + ((size_t)r * a.ws.wpr + wi) * kWords + lane,
           kTag | half | (lane == 0 ? (u64)hits << 33 : 0ull));
  }
}

__global__ __launch_bounds__(kT) void fused_kernel(FusedArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[kFusedLds];
  const int bid = blockIdx.x;
  if (bid == 0 && threadIdx.x == 0) st_dev(&a.ctr[ECH_CTR_LIVE], 1);   // the live copier may start
  if (bid < kRankWg) {
    rank_role(a, bid, smem);
  } else if (bid < kRankWg + a.n_alloc_wg) {
    alloc_role(a, bid - kRankWg, smem);
  } else {
    score_role(a, bid - kRankWg - a.n_alloc_wg, smem);
  }
}


// ------------------------------------------------------------------ live copier
// A separate launch on another stream, beside the fused launch: copies the
// early rows over PCIe as the alloc workgroups write their miss-list entries.
// It starts copying only once the fused launch has started this step's list
// (ctr[ECH_CTR_LIVE] = 1; ech_recall(ECH_EARLY) clears it at the end of the
// step), claims groups of consecutive ranks in order, waits for each group's
// entries, and stops at the end of the list. Any wait without progress for
// kPatienceTicks (the fused launch not running, e.g. queued behind this one)
// makes it give up: the copied groups form a prefix of the list
// (ctr[ECH_CTR_NCOPIED_EARLY]) and ech_recall(ECH_EARLY) copies the rest, so
// the result never depends on how the two launches are scheduled.
//
// Given the FINAL list, a workgroup that reached the end of the early list
// then waits (same patience) for the FINAL phase of the step to complete its
// list (ctr[ECH_CTR_FINAL_READY] bit 0, set by that phase's last placing
// workgroup after every entry and ctr[ECH_CTR_NMISS] went out with coherent
// stores) and copies it group by group; every claimed group is copied whole,
// so the copied groups are again a prefix (ctr[ECH_CTR_NCOPIED_FINAL]). The
// FINAL rows go to slots no early row is written to: the FINAL allocation
// walks the ring on from where the early one stopped, and if it walked onto
// the early one's slots (bit 1) no FINAL row is copied here. The PCIe link
// thus stays busy from the first early row to the last FINAL one, with no
// launch boundary and no cross-stream wait between the two lists.
constexpr int kLive = 32;                     // copier workgroups (more slow the scoring beside them more than they gain)
constexpr u64 kPatienceTicks = 100000ull;     // 1 ms at the 100 MHz constant-rate clock

struct LiveArgs {
  const v4u* host;                            // device view of the pinned pool
  v4u* dev;
  int row16;
  int64_t P;
  int32_t C;
  const int32_t* miss;
  int32_t M_early;
  const int32_t* missf;                       // the FINAL list, or null
  int32_t M_final;
  int32_t* ctr;
  Ctl* ctl;
};

// Copies the rows of the group's entries s_e[0..rg) (kNone: nothing), all
// host loads in flight before the stores.
__device__ __forceinline__ void copy_group(const LiveArgs& a, const u64* s_e, int rg) {
  const int tid = threadIdx.x;
  v4u v[kCopyUnroll];
  int64_t dst[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
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
}

__global__ __launch_bounds__(kT) void early_live_copy_kernel(LiveArgs a) {
  __shared__ u64 s_e[kT * kCopyUnroll];
  __shared__ int s_g, s_state;                // state: 0 copy group s_g, 1 end of list, 2 gave up
  __shared__ int s_nf;
  const int tid = threadIdx.x;
  const int rg = max(1, (kT * kCopyUnroll) / a.row16);   // rows per group
  u64* fin = &a.ctl->finished;
  const u64* ent = reinterpret_cast<const u64*>(a.miss);
  if (tid == 0) {   // wait for the fused launch to start this step's list
    const u64 t0 = wall_clock64();
    s_state = 0;
    while (ld_dev(&a.ctr[ECH_CTR_LIVE]) == 0) {
      if (wall_clock64() - t0 > kPatienceTicks) {
        s_state = 2;
        break;
      }
      __builtin_amdgcn_s_sleep(16);
    }
  }
  __syncthreads();
  int gave_up_at = -1;
  if (s_state == 0) {
    for (;;) {
      if (tid == 0) {
        const int g = atomicAdd(&a.ctl->next_group, 1);
        const int m0 = g * rg;
        const u64 f0 = ld_dev(fin);
        s_g = g;
        s_state = ((f0 & kFin) && m0 >= (int)(f0 & 0xffffffffull)) || m0 >= a.M_early ? 1 : 0;
        if (s_state == 0) {
          // the group's last entry (entries are written in about rank order)
          // or the end mark; patience restarts with every change seen
          const int m = min(m0 + rg, a.M_early) - 1;
          u64 t0 = wall_clock64();
          for (;;) {
            if (ld_dev(ent + m) != kNone) break;
            const u64 f = ld_dev(fin);
            if ((f & kFin) && m >= (int)(f & 0xffffffffull)) break;
            if (wall_clock64() - t0 > kPatienceTicks) {
              s_state = 2;
              break;
            }
            __builtin_amdgcn_s_sleep(16);
          }
        }
      }
      __syncthreads();
      if (s_state != 0) {
        if (s_state == 2) gave_up_at = s_g;
        break;
      }
      const int m0 = s_g * rg;
      if (tid < rg) {   // one thread per row of the group reads its entry
        const int m = m0 + tid;
        u64 e = kNone;
        if (m < a.M_early) {
          const u64 t0 = wall_clock64();
          for (;;) {
            e = ld_dev(ent + m);
            if (e != kNone) break;
            const u64 f = ld_dev(fin);
            if ((f & kFin) && m >= (int)(f & 0xffffffffull)) break;   // past the end: nothing to copy
            if (wall_clock64() - t0 > kPatienceTicks) {
              atomicOr(&s_state, 2);
              break;
            }
            __builtin_amdgcn_s_sleep(16);
          }
        }
        s_e[tid] = e;
      }
      __syncthreads();
      if (s_state != 0) {   // a row of this group never came: the group is not copied
        gave_up_at = s_g;
        break;
      }
      copy_group(a, s_e, rg);
      __syncthreads();   // s_g, s_e, s_state are rewritten by the next group
    }
  }
  // the FINAL rows, by the workgroups that reached the end of the early list
  const bool final_rows = a.missf != nullptr && s_state == 1;
  __syncthreads();   // every thread has read s_state
  if (final_rows) {
    if (tid == 0) {
      const u64 t0 = wall_clock64();
      int r;
      for (;;) {
        r = ld_dev(&a.ctr[ECH_CTR_FINAL_READY]);
        if ((r & 1) || wall_clock64() - t0 > kPatienceTicks) break;
        __builtin_amdgcn_s_sleep(16);
      }
      s_state = (r & 3) == 1 ? 0 : 2;
      s_nf = min(max(ld_dev(&a.ctr[ECH_CTR_NMISS]), 0), a.M_final);
    }
    __syncthreads();
    const u64* entf = reinterpret_cast<const u64*>(a.missf);
    for (;;) {
      if (tid == 0 && s_state == 0) {
        const int g = atomicAdd(&a.ctl->next_fgroup, 1);
        s_g = g;
        if ((int64_t)g * rg >= s_nf) s_state = 1;
      }
      __syncthreads();
      if (s_state != 0) break;
      if (tid < rg) {
        const int m = s_g * rg + tid;
        s_e[tid] = m < s_nf ? ld_dev(entf + m) : kNone;
      }
      __syncthreads();
      copy_group(a, s_e, rg);
      __syncthreads();
    }
  }
  if (tid == 0) {
    if (gave_up_at >= 0) atomicMin(&a.ctl->first_incomplete, gave_up_at);
    const int prev = atomicAdd(&a.ctl->c_done, 1);
    if (prev == kLive - 1) {   // the last copier workgroup: the copied prefixes
      const u64 f = ld_dev(fin);
      int64_t groups = min(ld_dev(&a.ctl->next_group), ld_dev(&a.ctl->first_incomplete));
      int64_t ncopied = groups * rg;
      if (f & kFin) ncopied = min(ncopied, (int64_t)(f & 0xffffffffull));
      ncopied = min(ncopied, (int64_t)a.M_early);
      a.ctr[ECH_CTR_NCOPIED_EARLY] = (int)ncopied;
      int64_t nfin = 0;
      const int fg = ld_dev(&a.ctl->next_fgroup);
      if (fg > 0) {   // some workgroup saw the FINAL list complete: its length is final
        nfin = min((int64_t)fg * rg, (int64_t)min(max(ld_dev(&a.ctr[ECH_CTR_NMISS]), 0), a.M_final));
        a.ctr[ECH_CTR_NCOPIED_FINAL] = (int)nfin;
      }
      atomicAdd(&a.ctr[ECH_CTR_RECALLED], (int)(ncopied + nfin));
    }
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" size_t ech_index_logits_early_ws_bytes(int R, int max_len, int32_t C, int32_t M_early) {
  if (R < 1 || max_len < 0 || C < 1 || M_early < 0) return 0;
  return fused_layout(R, max_len, C, M_early, nullptr, nullptr);
}

extern "C" int ech_index_logits_early(const void* q, const float* w, const void* kcache, int kdtype,
                                      const float* kscale, const int64_t* row_tok0, const int32_t* row_len, int R,
                                      int H, int D, int max_len, float* logits, int64_t ld, int e0, int e1,
                                      const float* theta, int cap, int32_t* tok2slot, int64_t P, int32_t* slot2tok,
                                      int32_t* slot_pin, int32_t C, int32_t* miss_early, int32_t M_early,
                                      int32_t* ctr, int32_t* stats, void* ws, size_t ws_bytes, void* stream) {
  if (!q || !w || !kcache || !row_tok0 || !row_len || !logits || !theta || !tok2slot || !slot2tok || !slot_pin ||
      !miss_early || !ctr || !stats || !ws)
    return ECH_EINVAL;
  if (kdtype != ECH_KEY_FP8) return ECH_EUNSUPPORTED;
  if (!kscale || H != kH || D != kD || R < 1 || R > kMaxB || max_len < 0 || ld < max_len) return ECH_EINVAL;
  if (e0 < 0 || e1 <= e0 || e1 > R || cap < 0 || cap > kMaxCap) return ECH_EINVAL;
  if (P < 1 || P >= INT32_MAX || C < 1 || C > (1 << 30) || M_early < 0) return ECH_EINVAL;
  if ((int64_t)M_early < (int64_t)(e1 - e0) * std::min(cap, max_len)) return ECH_EINVAL;
  if (!aligned16(q) || !aligned16(kcache)) return ECH_EINVAL;
  if ((reinterpret_cast<uintptr_t>(miss_early) & 7u) || (reinterpret_cast<uintptr_t>(ws) & 255u)) return ECH_EINVAL;
  if (ws_bytes < ech_index_logits_early_ws_bytes(R, max_len, C, M_early)) return ECH_EINVAL;
  FWs fw;
  fused_layout(R, max_len, C, M_early, &fw, static_cast<char*>(ws));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
  const uint8_t* kk = static_cast<const uint8_t*>(kcache);
  hipLaunchKernelGGL(fused_pins_kernel, dim3(std::min(e1 - e0, kMaxPinWg), kPinParts), dim3(kT), 0, s, qq, w, kk, kscale,
                     row_tok0, row_len, theta, e0, e1, slot2tok, C, slot_pin, miss_early, M_early, ctr, fw);
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
  a.slot_pin = slot_pin;
  a.n_alloc_wg = std::min(e1 - e0, kMaxAlloc);
  a.ws = fw;
  const int64_t blocks = kRankWg + (int64_t)a.n_alloc_wg + (int64_t)a.gx * R;
  if (blocks > INT32_MAX) return ECH_EINVAL;
  hipLaunchKernelGGL(fused_kernel, dim3((unsigned)blocks), dim3(kT), 0, s, a);
  ECH_LAUNCH_CHECK();
  return ECH_OK;
}

extern "C" int ech_topk_early(const float* logits, int64_t ld, const int32_t* row_len, int R, int max_len, int k,
                              const float* theta_in, float* theta_out, int32_t* idx, float* kth, const void* ws,
                              size_t ws_bytes, int32_t C, int32_t M_early, void* stream) {
  if (!logits || !row_len || !idx || !kth || !ws || !theta_in) return ECH_EINVAL;
  if (R < 1 || R > kMaxB || k < 1 || k > ech::kListMaxK || max_len < 0 || ld < max_len || C < 1 || M_early < 0)
    return ECH_EINVAL;
  if (ld % 4 != 0 || !aligned16(logits) || (reinterpret_cast<uintptr_t>(ws) & 255u)) return ECH_EINVAL;
  if ((max_len + kWaveTok - 1) / kWaveTok > ech::kListMaxChunks) return ECH_EINVAL;
  if (ws_bytes < ech_index_logits_early_ws_bytes(R, max_len, C, M_early)) return ECH_EINVAL;
  FWs fw;
  fused_layout(R, max_len, C, M_early, &fw, static_cast<char*>(const_cast<void*>(ws)));
  return ech::topk_lists_launch(logits, ld, row_len, R, max_len, k, theta_in, theta_out, idx, kth, fw.lmeta, fw.lpool,
                                fw.lth, fw.wpr, kListSlice, kWaveTok, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int ech_recall_early_live(const void* host_pool, int64_t P, int64_t row_bytes, void* dev_cache, int32_t C,
                                     const int32_t* miss_early, int32_t M_early, const int32_t* miss_final,
                                     int32_t M_final, int32_t* ctr, void* ws, void* stream) {
  if (!host_pool || !dev_cache || !miss_early || !ctr || !ws || P < 1 || P >= INT32_MAX || C < 1 || M_early < 0)
    return ECH_EINVAL;
  if (miss_final && (M_final < 0 || (reinterpret_cast<uintptr_t>(miss_final) & 7u))) return ECH_EINVAL;
  if (row_bytes < 16 || row_bytes % 16 != 0 || row_bytes > 16 * kT * kCopyUnroll) return ECH_EINVAL;
  if (!aligned16(dev_cache) || !aligned16(host_pool) || (reinterpret_cast<uintptr_t>(miss_early) & 7u) ||
      (reinterpret_cast<uintptr_t>(ws) & 255u))
    return ECH_EINVAL;
  void* hdev = nullptr;
  if (hipHostGetDevicePointer(&hdev, const_cast<void*>(host_pool), 0) != hipSuccess || !hdev) {
    (void)hipGetLastError();
    return ECH_EINVAL;
  }
  if (M_early == 0) return ECH_OK;
  LiveArgs a;
  a.host = static_cast<const v4u*>(hdev);
  a.dev = static_cast<v4u*>(dev_cache);
  a.row16 = (int)(row_bytes / 16);
  a.P = P;
  a.C = C;
  a.miss = miss_early;
  a.M_early = M_early;
  a.missf = miss_final;
  a.M_final = miss_final ? M_final : 0;
  a.ctr = ctr;
  a.ctl = reinterpret_cast<Ctl*>(ws);   // the control words lead the fused launch's workspace
  hipLaunchKernelGGL(early_live_copy_kernel, dim3(kLive), dim3(kT), 0, reinterpret_cast<hipStream_t>(stream), a);
  ECH_LAUNCH_CHECK();
  return ECH_OK;
}
