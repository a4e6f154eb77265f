// Exact top-k per score row on gfx950.
//
// ECHO explainer, "Prefill: one-round histogram": a single 256-bin histogram
// pass keyed by the high byte of the score minus the predicted threshold
// theta; the selection must be exact (the explainer's opening summary). The
// k-th element (s*, t*) of the order (score descending, token ascending)
// defines the set exactly:
//     t selected  <=>  s_t > s*  or  (s_t == s* and t among the first
//                      need_eq tokens with score s*)
// so the kernels find s* and need_eq, then compact in ascending t.
//
// Three launch shapes, by the call's rows:
//   - a few rows of at most 16384 tokens: one workgroup per row holds the row
//     in registers (topk_small_kernel, one launch);
//   - a few long rows (decode): one pass over the scores (topk_one_kernel,
//     after a one-block reset), each workgroup a 16384-token chunk; the last
//     workgroup of a row selects from the chunks' band lists;
//   - many rows (a prefill block), in five launches:
//   T1 hist     grid (chunks, R): LDS histogram of bin(t) = high byte of
//               the order key of fp16(fl32(s_t - theta)) per 4096-token chunk.
//               Every step is monotone in s, so higher bins hold strictly
//               larger scores.
//   T2 rowsel   grid (R): sum the chunk histograms, boundary bin b* where the
//               count from the top reaches k, need = k - count above b*.
//               The chunk histograms also give, per chunk, the number of
//               tokens in bins >= b*, hence each chunk's offset in T3's list.
//   T3 list     grid (chunks, R): every token in a bin >= b* is written, in
//               token order, to the row's list at its chunk's offset (block
//               scans, no atomics): the tokens certainly selected and the
//               boundary-bin tokens, at most k + cap entries.
//   T4 resolve  grid (R): radix-select the need-th largest score among the
//               list's b* entries in LDS (4 rounds of 8 bits of ord(s)), then
//               write the selection in token order by one ordered pass over
//               the list. Writes kth and the EMA update of theta.
//   T5 compact  grid (chunks, R): only for rows the list does not serve:
//               rows no longer than k (all tokens; padded with -1) and rows
//               whose boundary bin holds more than cap tokens (no or poor
//               theta), for which T4 ran the radix rounds over the whole row
//               and left per-chunk offsets.
//   A good theta puts only a few hundred tokens in b* (bins are logarithmic
//   around the threshold), so the row is read twice (T1, T3).

#include <algorithm>
#include <mutex>

#include "bins.hpp"
#include "lists.hpp"

namespace {

constexpr int kChunk = 4096;        // tokens per chunk (T1, T3, T5)
static_assert(kChunk == 4 * 4 * 256, "four float4 loads per thread per chunk");
constexpr int kVec = kChunk / (4 * 256);   // float4 loads per thread
constexpr int kT = 256;             // threads for chunk kernels
constexpr int kMaxK = 4096;
constexpr int kMaxChunks = 1024;    // max_len <= 4M

// kNormal: resolved from T3's list. kWide: the boundary bin holds more than
// cap tokens; resolved over the whole row, compacted by T5. With many rows a
// wide row whose boundary is the lumped bin 0 is first refined (T2b): its
// lumped tokens are binned again without lumping, and if the boundary
// sub-bin d0 fits, the row is served by the list after all (refine = 1).
enum RowMode : int { kNormal = 0, kAll = 1, kEmpty = 2, kWide = 3 };

struct RowState {
  int mode;
  int bstar;
  int need;      // rank of the k-th token within b*
  int nlist;     // list entries (tokens in bins >= b*)
  float spred;   // T5: scores > spred are selected (-inf in kAll mode)
  int refine;    // boundary = lumped tokens whose unlumped bin is d0
  int d0;
  int pad;
};

struct Ws {
  RowState* rs;
  int* hist;     // [R][nch][256]
  int* off;      // [R][nch] list offsets (kNormal) or output offsets (T5 rows)
  int* take;     // [R][nch]
  int2* list;    // [R][lcap] (score bits, token)
  int cap;       // largest boundary bin served by the list
  int lcap;      // k + cap, rounded up to 8 entries
  int nch;
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Largest boundary bin the list serves (T4 selects it in LDS).
constexpr int kListCap = 4096;

size_t layout(int R, int max_len, int k, Ws* w, char* base) {
  const int nch = std::max(1, (max_len + kChunk - 1) / kChunk);
  const int cap = kListCap;
  const int lcap = (k + cap + 7) & ~7;   // rows of the list stay 64-byte aligned
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  size_t o_rs = take(sizeof(RowState) * R);
  size_t o_hist = take(sizeof(int) * (size_t)R * nch * 256);
  size_t o_off = take(sizeof(int) * (size_t)R * nch);
  size_t o_take = take(sizeof(int) * (size_t)R * nch);
  size_t o_list = take(sizeof(int2) * (size_t)R * lcap);
  if (w && base) {
    w->rs = reinterpret_cast<RowState*>(base + o_rs);
    w->hist = reinterpret_cast<int*>(base + o_hist);
    w->off = reinterpret_cast<int*>(base + o_off);
    w->take = reinterpret_cast<int*>(base + o_take);
    w->list = reinterpret_cast<int2*>(base + o_list);
    w->cap = cap;
    w->lcap = lcap;
    w->nch = nch;
  }
  return o;
}

// The 256 bins are the high byte of the order key of fp16(d): sign, 5
// exponent bits and 2 mantissa bits, i.e. four bins per binade of |d| (the
// high byte of the fp32 key would give one bin per two binades). fp32 -> fp16
// rounding is monotone, so the binning stays monotone in s; overflow goes to
// the infinities, the outermost bins. Finite negative d never reaches bin 0
// (its order key is at least 0x0400), so bin 0 is free for the lumped scores.
__device__ __forceinline__ uint32_t bin16(float d) {
  const _Float16 h = (_Float16)d;
  uint32_t u = __builtin_bit_cast(uint16_t, h);
  if ((u & 0x7fffu) == 0u) u = 0u;               // -0 -> +0
  const uint32_t key = (u & 0x8000u) ? (~u & 0xffffu) : (u | 0x8000u);
  return key >> 8;
}

__device__ __forceinline__ uint32_t shifted_bin(float x, const Shift& sh) {
  if (!sh.on) return bin16(x);
  const float d = x - sh.th;
  return d < sh.cut ? 0u : bin16(d);
}

__device__ __forceinline__ float row_theta(const float* th, int r) {
  return th ? th[r] : __builtin_nanf("");
}

// ------------------------------------------------------------------ T1
// Load a chunk's 16 scores per thread (4 float4, issued before any use);
// element j*4 + e of thread tid is token lo + 4*(j*256 + tid) + e.
__device__ __forceinline__ void load_chunk(const float* row, int lo, int hi, float4 (&v)[kVec]) {
#pragma unroll
  for (int j = 0; j < kVec; ++j) {
    const int t = lo + 4 * (j * kT + (int)threadIdx.x);
    if (t + 3 < hi) {
      // nontemporal: each load instruction covers a contiguous 1 KiB, the
      // pattern where the hint raises the stream rate on MI355X
      typedef float f4v __attribute__((ext_vector_type(4)));
      const f4v x = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(row + t));
      v[j] = make_float4(x.x, x.y, x.z, x.w);
    } else {
      v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (t < hi) v[j].x = row[t];
      if (t + 1 < hi) v[j].y = row[t + 1];
      if (t + 2 < hi) v[j].z = row[t + 2];
    }
  }
}

__device__ __forceinline__ float f4(const float4& v, int e) { return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w; }

__global__ __launch_bounds__(kT) void topk_hist_kernel(const float* __restrict__ logits, int64_t ld,
                                                       const int32_t* __restrict__ lens, int k,
                                                       const float* __restrict__ theta, Ws ws) {
  const int r = blockIdx.y, c = blockIdx.x;
  const int len = lens[r];
  const int lo = c * kChunk;
  if (len <= k || lo >= len) return;
  const int hi = min(lo + kChunk, len);
  __shared__ int h[256];
  h[threadIdx.x] = 0;
  const Shift sh = make_shift(row_theta(theta, r));
  float4 v[kVec];
  load_chunk(logits + (size_t)r * ld, lo, hi, v);
  __syncthreads();
  int lumped = 0;
#pragma unroll
  for (int j = 0; j < kVec; ++j) {
    const int t = lo + 4 * (j * kT + (int)threadIdx.x);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = f4(v[j], e);
      const bool ok = t + e < hi;
      const float d = sh.on ? x - sh.th : x;
      const bool lump = ok && d < sh.cut;
      lumped += lump;
      ech::lds_hist_add(h, bin16(d), ok && !lump);
    }
  }
  lumped = ech::wave_sum(lumped);
  if (ech::lane_id() == 0 && lumped) atomicAdd(&h[0], lumped);
  __syncthreads();
  ws.hist[((size_t)r * ws.nch + c) * 256 + threadIdx.x] = h[threadIdx.x];
}

// ------------------------------------------------------------------ T2
// T2 for calls with many rows (a prefill block: rows of at most a few dozen
// chunks), 256 threads: thread b sums bin (255 - b) over the row's chunks,
// eight independent loads in flight; four adjacent threads then share a
// chunk for its count over bins >= b* (16 int4 loads each). Few registers, so
// its workgroups fit beside the matrix-core kernel of the next block.
__global__ __launch_bounds__(256) void topk_rowsel_many_kernel(const int32_t* __restrict__ lens, int k, Ws ws) {
  constexpr int NT = 256;
  constexpr int kParts = NT / 256;
  const int r = blockIdx.x;
  const int len = lens[r];
  RowState& st = ws.rs[r];
  if (len <= k) {
    if (threadIdx.x == 0) {
      st.mode = len == 0 ? kEmpty : kAll;
      st.bstar = 0;
      st.need = 0;
      st.nlist = 0;
      st.refine = 0;
    }
    return;
  }
  const int nch = (len + kChunk - 1) / kChunk;
  __shared__ int part_sum[kParts][256];
  __shared__ int scratch[NT / 64];
  __shared__ int s_bstar, s_nbin;
  const int b = threadIdx.x & 255, part = threadIdx.x >> 8;
  const int bin = 255 - b;
  const int* h = ws.hist + (size_t)r * ws.nch * 256 + bin;
  int acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int c = part;
  for (; c + 7 * kParts < nch; c += 8 * kParts) {
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] += h[(size_t)(c + kParts * u) * 256];
  }
  for (; c < nch; c += kParts) acc[0] += h[(size_t)c * 256];
  part_sum[part][b] = acc[0] + acc[1] + acc[2] + acc[3] + acc[4] + acc[5] + acc[6] + acc[7];
  __syncthreads();
  // threads 0..255 hold bins 255..0 in order; the rest add zeros after them
  int cnt = 0;
  if (threadIdx.x < 256) {
#pragma unroll
    for (int pp = 0; pp < kParts; ++pp) cnt += part_sum[pp][b];
  }
  int tot;
  const int above = ech::block_excl_scan<NT>(cnt, scratch, &tot);
  if (threadIdx.x < 256 && above < k && above + cnt >= k) {
    s_bstar = bin;
    s_nbin = cnt;
    st.bstar = bin;
    st.need = k - above;
  }
  __syncthreads();
  const int bstar = s_bstar;
  const bool wide = s_nbin > ws.cap;
  if (threadIdx.x == 0) {
    st.mode = wide ? kWide : kNormal;
    st.refine = 0;
  }
  // List offsets: chunk c holds the sum over bins >= b* of its histogram.
  // Wide rows keep instead, per chunk, the count of bins > b* (in take), for
  // the refinement. Four adjacent threads share a chunk (16 int4 loads each,
  // all in flight).
  const int tb = wide ? bstar + 1 : bstar;
  int run = 0;
  const int sub = threadIdx.x & 3;
  for (int c0 = 0; c0 < nch; c0 += NT / 4) {
    const int c = c0 + (int)threadIdx.x / 4;
    int n = 0;
    if (c < nch) {
      const int4* hc = reinterpret_cast<const int4*>(ws.hist + ((size_t)r * ws.nch + c) * 256) + 16 * sub;
      int4 q[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) q[i] = hc[i];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int b0 = 64 * sub + 4 * i;
        n += (b0 >= tb ? q[i].x : 0) + (b0 + 1 >= tb ? q[i].y : 0) + (b0 + 2 >= tb ? q[i].z : 0) +
             (b0 + 3 >= tb ? q[i].w : 0);
      }
    }
    n += __shfl_xor(n, 1, 64);
    n += __shfl_xor(n, 2, 64);
    int t;
    const int pre = ech::block_excl_scan<NT>(sub == 0 ? n : 0, scratch, &t);
    if (c < nch && sub == 0) {
      if (wide) ws.take[(size_t)r * ws.nch + c] = n;
      else ws.off[(size_t)r * ws.nch + c] = run + pre;
    }
    run += t;
  }
  if (threadIdx.x == 0 && !wide) st.nlist = run;
}

// ------------------------------------------------------------------ T2b
// Refinement of wide rows whose boundary is the lumped bin 0 (a prediction
// far above the k-th score), for calls with many rows. Histogram, per chunk,
// of the lumped tokens by bin16(d) without lumping, into the row's T1
// histogram space (no longer read).
__global__ __launch_bounds__(kT) void topk_refine_hist_kernel(const float* __restrict__ logits, int64_t ld,
                                                              const int32_t* __restrict__ lens,
                                                              const float* __restrict__ theta, Ws ws) {
  const int r = blockIdx.y, c = blockIdx.x;
  const int len = lens[r];
  const int lo = c * kChunk;
  if (lo >= len) return;
  const RowState st = ws.rs[r];
  if (st.mode != kWide || st.bstar != 0) return;
  const Shift sh = make_shift(row_theta(theta, r));
  if (!sh.on) return;
  const int hi = min(lo + kChunk, len);
  __shared__ int h[256];
  h[threadIdx.x] = 0;
  float4 v[kVec];
  load_chunk(logits + (size_t)r * ld, lo, hi, v);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kVec; ++j) {
    const int t = lo + 4 * (j * kT + (int)threadIdx.x);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float d = f4(v[j], e) - sh.th;
      ech::lds_hist_add(h, bin16(d), t + e < hi && d < sh.cut);
    }
  }
  __syncthreads();
  ws.hist[((size_t)r * ws.nch + c) * 256 + threadIdx.x] = h[threadIdx.x];
}

// The boundary sub-bin d0 of a refined row and, if it holds at most cap
// tokens, the row's list offsets: per chunk, the tokens above the lumped bin
// (take) plus the lumped ones with unlumped bin >= d0.
template <int NT>
__global__ __launch_bounds__(NT) void topk_refine_sel_kernel(const int32_t* __restrict__ lens,
                                                             const float* __restrict__ theta, Ws ws) {
  constexpr int kParts = NT / 256;
  const int r = blockIdx.x;
  const int len = lens[r];
  RowState& st = ws.rs[r];
  if (st.mode != kWide || st.bstar != 0 || !make_shift(row_theta(theta, r)).on) return;
  const int nch = (len + kChunk - 1) / kChunk;
  __shared__ int part_sum[kParts][256];
  __shared__ int scratch[NT / 64];
  __shared__ int s_d0, s_n2, s_need;
  const int b = threadIdx.x & 255, part = threadIdx.x >> 8;
  const int* h = ws.hist + (size_t)r * ws.nch * 256 + (255 - b);
  int acc = 0;
  for (int c = part; c < nch; c += kParts) acc += h[(size_t)c * 256];
  part_sum[part][b] = acc;
  __syncthreads();
  int cnt = 0;
  if (threadIdx.x < 256) {
#pragma unroll
    for (int pp = 0; pp < kParts; ++pp) cnt += part_sum[pp][b];
  }
  int tot;
  const int above = ech::block_excl_scan<NT>(cnt, scratch, &tot);
  const int need = st.need;
  if (threadIdx.x < 256 && above < need && above + cnt >= need) {
    s_d0 = 255 - b;
    s_n2 = cnt;
    s_need = need - above;
  }
  __syncthreads();
  if (s_n2 > ws.cap) return;   // still wider than the list: resolved over the whole row
  const int d0 = s_d0;
  int run = 0;
  const int sub = threadIdx.x & 3;
  for (int c0 = 0; c0 < nch; c0 += NT / 4) {
    const int c = c0 + (int)threadIdx.x / 4;
    int n = 0;
    if (c < nch) {
      const int4* hc = reinterpret_cast<const int4*>(ws.hist + ((size_t)r * ws.nch + c) * 256) + 16 * sub;
      int4 q[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) q[i] = hc[i];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int b0 = 64 * sub + 4 * i;
        n += (b0 >= d0 ? q[i].x : 0) + (b0 + 1 >= d0 ? q[i].y : 0) + (b0 + 2 >= d0 ? q[i].z : 0) +
             (b0 + 3 >= d0 ? q[i].w : 0);
      }
      if (sub == 0) n += ws.take[(size_t)r * ws.nch + c];
    }
    n += __shfl_xor(n, 1, 64);
    n += __shfl_xor(n, 2, 64);
    int t;
    const int pre = ech::block_excl_scan<NT>(sub == 0 ? n : 0, scratch, &t);
    if (c < nch && sub == 0) ws.off[(size_t)r * ws.nch + c] = run + pre;
    run += t;
  }
  if (threadIdx.x == 0) {
    st.need = s_need;
    st.refine = 1;
    st.d0 = d0;
    st.nlist = run;
    st.mode = kNormal;
  }
}

// ------------------------------------------------------------------ T3
// Wave w of the block takes tokens [lo + 1024w, +1024) of the chunk: load j
// of lane l covers tokens +256j + 4l .. +3 (each instruction still reads a
// contiguous 1 KiB). The listing order (wave, j, lane, element) is the token
// order, so ranks come from wave scans and one exchange of wave totals.
__global__ __launch_bounds__(kT) void topk_list_kernel(const float* __restrict__ logits, int64_t ld,
                                                       const int32_t* __restrict__ lens,
                                                       const float* __restrict__ theta, Ws ws) {
  const int r = blockIdx.y, c = blockIdx.x;
  const int len = lens[r];
  const int lo = c * kChunk;
  if (lo >= len) return;
  const int hi = min(lo + kChunk, len);
  const int lane = ech::lane_id(), wave = threadIdx.x >> 6;
  const float* row = logits + (size_t)r * ld;
  const int wlo = lo + 1024 * wave;
  // scores first, so their latency overlaps that of the row state
  float4 v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = wlo + 256 * j + 4 * lane;
    if (t + 3 < hi) {
      typedef float f4v __attribute__((ext_vector_type(4)));
      const f4v x = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(row + t));
      v[j] = make_float4(x.x, x.y, x.z, x.w);
    } else {
      v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (t < hi) v[j].x = row[t];
      if (t + 1 < hi) v[j].y = row[t + 1];
      if (t + 2 < hi) v[j].z = row[t + 2];
    }
  }
  const RowState st = ws.rs[r];
  const int o = ws.off[(size_t)r * ws.nch + c];   // loaded beside the row state
  if (st.mode != kNormal) return;
  const Shift sh = make_shift(row_theta(theta, r));
  const uint32_t bstar = (uint32_t)st.bstar;
  const bool refine = st.refine;
  const uint32_t d0 = (uint32_t)st.d0;
  __shared__ int wtot[kT / 64];
  // The chunk's entries are gathered in LDS and leave as consecutive 8-byte
  // stores: written one by one from the lanes that hold them they cost more
  // than the whole read of the chunk. Chunks with more entries than the
  // buffer (rows barely longer than k) write directly.
  constexpr int kStage = 1024;
  __shared__ int2 stage[kStage];
  uint32_t in = 0;   // bit 4j + e: element e of load j is in a bin >= b*
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = wlo + 256 * j + 4 * lane;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = f4(v[j], e);
      const uint32_t b = shifted_bin(x, sh);
      const bool listed = b > bstar || (b == bstar && (!refine || bin16(x - sh.th) >= d0));
      in |= (t + e < hi && listed) ? 1u << (4 * j + e) : 0u;
    }
  }
  int n[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) n[j] = __popc((in >> (4 * j)) & 15u);
  const int i01 = ech::wave_incl_scan(n[0] | (n[1] << 16));
  const int i23 = ech::wave_incl_scan(n[2] | (n[3] << 16));
  const int t01 = __shfl(i01, 63, 64), t23 = __shfl(i23, 63, 64);
  const int p01 = i01 - (n[0] | (n[1] << 16)), p23 = i23 - (n[2] | (n[3] << 16));
  const int tj[4] = {t01 & 0xffff, t01 >> 16, t23 & 0xffff, t23 >> 16};
  const int pj[4] = {p01 & 0xffff, p01 >> 16, p23 & 0xffff, p23 >> 16};
  if (lane == 0) wtot[wave] = tj[0] + tj[1] + tj[2] + tj[3];
  __syncthreads();
  int base = 0;   // this wave's first entry within the chunk
  for (int w = 0; w < wave; ++w) base += wtot[w];
  const int total = wtot[0] + wtot[1] + wtot[2] + wtot[3];
  const bool staged = total <= kStage;
  const int room = ws.lcap - o;   // the offsets bound the list by k + cap; guard only
  int2* dst = ws.list + (size_t)r * ws.lcap + o;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int pos = base + pj[j];
    const int t = wlo + 256 * j + 4 * lane;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if ((in >> (4 * j + e)) & 1u) {
        const int2 entry = make_int2(__float_as_int(f4(v[j], e)), t + e);
        if (staged) stage[pos] = entry;
        else if (pos < room) dst[pos] = entry;
        ++pos;
      }
    }
    base += tj[j];
  }
  if (staged) {
    __syncthreads();
    const int n_out = min(total, room);
    for (int i = threadIdx.x; i < n_out; i += kT) dst[i] = stage[i];
  }
}

// ------------------------------------------------------------------ T4
// fn(t, x) for every score of a row, NT threads, four float4 loads in flight
// per thread (a loop with one scalar load per iteration waits a full memory
// round trip each time). Rows are 16-byte aligned (ld % 4 == 0).
template <int NT, typename Fn>
__device__ __forceinline__ void for_each_score(const float* __restrict__ row, int len, Fn fn) {
  constexpr int kU = 4;
  for (int b0 = 0; b0 < len; b0 += 4 * NT * kU) {
    float4 v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int t = b0 + 4 * (u * NT + (int)threadIdx.x);
      if (t + 3 < len) {
        v[u] = *reinterpret_cast<const float4*>(row + t);
      } else {
        v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (t < len) v[u].x = row[t];
        if (t + 1 < len) v[u].y = row[t + 1];
        if (t + 2 < len) v[u].z = row[t + 2];
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int t = b0 + 4 * (u * NT + (int)threadIdx.x);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (t + e < len) fn(t + e, f4(v[u], e));
    }
  }
}

// Radix-select helpers over a key set; `hist` is 256 ints of LDS.
// Finds the digit d (bits [shift, shift+8) of ord) at which the count from
// the top reaches `need`; updates need to the rank within that digit.
__device__ __forceinline__ void pick_digit(int* hist, int* sh, int need, int* out_digit, int* out_need) {
  // thread i < 256 owns digit 255 - i
  int cnt = 0, above = 0, tot = 0;
  if (threadIdx.x < 256) cnt = hist[255 - threadIdx.x];
  // block-wide exclusive scan over the first 256 threads (4 waves)
  const int lane = ech::lane_id(), wave = threadIdx.x / 64;
  int incl = ech::wave_incl_scan(cnt);
  if (threadIdx.x < 256 && lane == 63) sh[wave] = incl;
  __syncthreads();
  if (threadIdx.x < 256) {
    int wb = 0;
    for (int i = 0; i < wave; ++i) wb += sh[i];
    above = wb + incl - cnt;
    if (above < need && above + cnt >= need) {
      *out_digit = 255 - threadIdx.x;
      *out_need = need - above;
    }
  }
  (void)tot;
  __syncthreads();
}

// The need-th largest of the first n scores of cl, by wave 0 alone (4
// rounds of 8 bits of the order key, histogram in LDS). One wave's LDS
// operations execute in order, so the rounds need no block barrier; the
// wavefront fences keep the compiler from moving LDS accesses across phases.
// Returns the order key of the score; *need_out = its rank among equals.
__device__ __forceinline__ uint32_t wave_select(const int2* cl, int n, int need, int* hist, int* need_out) {
  const int lane = ech::lane_id();
  uint32_t prefix = 0, mask = 0;
#pragma unroll 1
  for (int round = 0; round < 4; ++round) {
    const int shift = 24 - 8 * round;
#pragma unroll
    for (int q = 0; q < 4; ++q) hist[4 * lane + q] = 0;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    for (int i = lane; i < n; i += 64) {
      const uint32_t key = ech::ord_key(__int_as_float(cl[i].x));
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    // lane l owns digits 255 - 4l - q, q = 0..3 (descending)
    int cnt[4], sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      cnt[q] = hist[255 - 4 * lane - q];
      sum += cnt[q];
    }
    int above = ech::wave_incl_scan(sum) - sum;
    int digit = -1, nneed = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (above < need && above + cnt[q] >= need) {
        digit = 255 - 4 * lane - q;
        nneed = need - above;
      }
      above += cnt[q];
    }
    const uint64_t m = __ballot(digit >= 0);
    const int src = __ffsll((unsigned long long)m) - 1;
    digit = __shfl(digit, src, 64);
    need = __shfl(nneed, src, 64);
    prefix |= (uint32_t)digit << shift;
    mask |= 255u << shift;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  }
  *need_out = need;
  return prefix;
}

template <int NT>
__global__ __launch_bounds__(NT) void topk_resolve_kernel(const float* __restrict__ logits, int64_t ld,
                                                           const int32_t* __restrict__ lens, int k,
                                                           const float* theta_in,
                                                           float* theta_out, float* __restrict__ kth,
                                                           int32_t* __restrict__ idx, Ws ws) {
  extern __shared__ int2 cl[];                     // candidate list [cap]
  __shared__ int hist[256];
  __shared__ int sh[16];
  __shared__ int gt_c[kMaxChunks];
  __shared__ int eq_c[kMaxChunks];
  __shared__ int s_digit, s_need, s_nb;
  __shared__ uint32_t s_prefix;
  __shared__ float s_min;

  const int r = blockIdx.x;
  const int len = lens[r];
  RowState& st = ws.rs[r];
  const int mode = st.mode;
  const float th_in = row_theta(theta_in, r);
  const float* row = logits + (size_t)r * ld;
  const int nch = (len + kChunk - 1) / kChunk;

  if (mode == kEmpty) {
    if (threadIdx.x == 0) {
      kth[r] = __builtin_nanf("");
      if (theta_out) theta_out[r] = th_in;
    }
    return;
  }
  for (int c = threadIdx.x; c < nch; c += NT) {
    gt_c[c] = 0;
    eq_c[c] = 0;
  }
  float sstar, spred;
  int need_eq;
  if (mode == kAll) {
    // every visible token is selected; kth is the row minimum
    float m = __builtin_inff();
    for_each_score<NT>(row, len, [&](int, float x) { m = fminf(m, x); });
    for (int d = 32; d > 0; d >>= 1) m = fminf(m, __shfl_xor(m, d, 64));
    float* wmin = reinterpret_cast<float*>(hist);
    if (ech::lane_id() == 0) wmin[threadIdx.x / 64] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
      float mm = __builtin_inff();
      for (int i = 0; i < NT / 64; ++i) mm = fminf(mm, wmin[i]);
      s_min = mm;
    }
    __syncthreads();
    sstar = s_min;
    spred = -__builtin_inff();
    need_eq = 0;
    for (int c = threadIdx.x; c < nch; c += NT) gt_c[c] = min(kChunk, len - c * kChunk);
    __syncthreads();
  } else {
    int need = st.need;
    uint32_t prefix = 0, mask = 0;
    const bool in_lds = mode == kNormal;
    const Shift shf = make_shift(th_in);
    const uint32_t bstar = (uint32_t)st.bstar;
    const int nlist = in_lds ? st.nlist : 0;
    const bool refine = st.refine;
    const uint32_t d0 = (uint32_t)st.d0;
    const int2* lst = ws.list + (size_t)r * ws.lcap;
    int cnt = 0;
    if (in_lds) {
      // the list's b* entries (at most cap) into LDS, in any order
      if (threadIdx.x == 0) s_nb = 0;
      __syncthreads();
      for (int i0 = 0; i0 < nlist; i0 += 8 * NT) {
        int2 e[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int i = i0 + u * NT + (int)threadIdx.x;
          e[u] = i < nlist ? lst[i] : make_int2(0, -1);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const float x = __int_as_float(e[u].x);
          if (e[u].y >= 0 && shifted_bin(x, shf) == bstar && (!refine || bin16(x - shf.th) == d0)) {
            const int p = atomicAdd(&s_nb, 1);
            if (p < ws.cap) cl[p] = e[u];   // the histogram bounds b* by cap; guard only
          }
        }
      }
      __syncthreads();
      cnt = min(s_nb, ws.cap);
      if (threadIdx.x < 64) {
        int nq;
        const uint32_t pf = wave_select(cl, cnt, need, hist, &nq);
        if (threadIdx.x == 0) {
          s_prefix = pf;
          s_need = nq;
        }
      }
      __syncthreads();
      prefix = s_prefix;
      need = s_need;
    }
    __syncthreads();
#pragma unroll 1
    for (int round = 0; round < 4 && !in_lds; ++round) {   // wide rows: the same rounds over the whole row
      const int shift = 24 - 8 * round;
      for (int i = threadIdx.x; i < 256; i += NT) hist[i] = 0;
      __syncthreads();
      for_each_score<NT>(row, len, [&](int, float x) {
        const uint32_t key = ech::ord_key(x);
        const bool act = shifted_bin(x, shf) == bstar && (key & mask) == prefix;
        ech::lds_hist_add(hist, (key >> shift) & 255u, act);
      });
      __syncthreads();
      pick_digit(hist, sh, need, &s_digit, &s_need);
      prefix |= (uint32_t)s_digit << shift;
      mask |= 255u << shift;
      need = s_need;
      __syncthreads();
    }
    sstar = ech::ord_to_float(prefix);
    spred = sstar;
    need_eq = need;
    if (in_lds) {
      // The selection in token order, by one ordered pass over the list:
      // every entry above b*, and the b* entries above s* or among the first
      // need_eq equal to it.
      // Thread i holds 8 consecutive entries per round, so one block scan
      // serves 8 * NT entries.
      int32_t* orow = idx + (size_t)r * k;
      int gt_run = 0, eq_run = 0;
      for (int i0 = 0; i0 < nlist; i0 += 8 * NT) {
        const int ib = i0 + 8 * (int)threadIdx.x;
        int2 e[8];
        if (ib + 7 < nlist) {
          const int4* q = reinterpret_cast<const int4*>(lst + ib);   // 64-byte aligned (lcap and ib multiples of 8)
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int4 x = q[u];
            e[2 * u] = make_int2(x.x, x.y);
            e[2 * u + 1] = make_int2(x.z, x.w);
          }
        } else {
#pragma unroll
          for (int u = 0; u < 8; ++u) e[u] = ib + u < nlist ? lst[ib + u] : make_int2(0, -1);
        }
        uint32_t gtm = 0, eqm = 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (e[u].y < 0) continue;
          // every list entry outside the boundary set scores above it
          const float x = __int_as_float(e[u].x);
          gtm |= x > sstar ? 1u << u : 0u;
          eqm |= x == sstar ? 1u << u : 0u;
        }
        int tot;
        const int pre = ech::block_excl_scan<NT>(__popc(gtm) | (__popc(eqm) << 16), sh, &tot);
        int gt_b = gt_run + (pre & 0xffff), eq_b = eq_run + (pre >> 16);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const bool gt = (gtm >> u) & 1u, eq = (eqm >> u) & 1u;
          const int pos = gt_b + min(eq_b, need_eq);
          if ((gt || (eq && eq_b < need_eq)) && pos < k) orow[pos] = e[u].y;
          gt_b += gt;
          eq_b += eq;
        }
        gt_run += tot & 0xffff;
        eq_run += tot >> 16;
      }
      if (threadIdx.x == 0) {
        st.spred = spred;
        kth[r] = sstar;
        if (theta_out) theta_out[r] = (th_in == th_in) ? (sstar + th_in) * 0.5f : sstar;
      }
      return;
    } else {
      for_each_score<NT>(row, len, [&](int t, float x) {
        if (x > sstar) atomicAdd(&gt_c[t / kChunk], 1);
        else if (x == sstar) atomicAdd(&eq_c[t / kChunk], 1);
      });
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    int run = 0, eq_before = 0;
    int* off = ws.off + (size_t)r * ws.nch;
    int* tk = ws.take + (size_t)r * ws.nch;
    for (int c = 0; c < nch; ++c) {
      const int tkc = max(0, min(eq_c[c], need_eq - eq_before));
      off[c] = run;
      tk[c] = tkc;
      run += gt_c[c] + tkc;
      eq_before += eq_c[c];
    }
    st.spred = spred;
    kth[r] = sstar;
    if (theta_out) theta_out[r] = (th_in == th_in) ? (sstar + th_in) * 0.5f : sstar;
  }
}

// ------------------------------------------------------------------ T5
// grid (gx, R): block x takes the chunks x, x + gx, ... of row r. Rows
// written from the list leave at once, so gx stays small: with long rows a
// block per chunk would be hundreds of workgroups that only read the mode.
__global__ __launch_bounds__(kT) void topk_compact_kernel(const float* __restrict__ logits, int64_t ld,
                                                          const int32_t* __restrict__ lens, int k,
                                                          int32_t* __restrict__ idx, Ws ws) {
  const int r = blockIdx.y;
  const int len = lens[r];
  int32_t* orow = idx + (size_t)r * k;
  if (blockIdx.x == 0) {
    for (int j = min(k, len) + threadIdx.x; j < k; j += kT) orow[j] = -1;
  }
  // Most rows were written by T4 from the list: check before reading scores.
  const RowState st = ws.rs[r];
  if (st.mode == kEmpty || st.mode == kNormal) return;
  const float sp = st.spred;
  __shared__ int scratch[kT / 64];
  for (int c = blockIdx.x; c * kChunk < len; c += gridDim.x) {   // block-uniform trip count
    const int lo = c * kChunk;
    const int hi = min(lo + kChunk, len);
    float4 v[kVec];
    load_chunk(logits + (size_t)r * ld, lo, hi, v);
    const int base = ws.off[(size_t)r * ws.nch + c];
    const int te = ws.take[(size_t)r * ws.nch + c];
    int gt_run = 0, eq_run = 0;   // block-uniform running counts
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
      const int t = lo + 4 * (j * kT + (int)threadIdx.x);
      int ngt = 0, neq = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = f4(v[j], e);
        const bool ok = t + e < hi;
        ngt += (ok && x > sp) ? 1 : 0;
        neq += (ok && x == sp) ? 1 : 0;
      }
      int tot;
      const int pre = ech::block_excl_scan<kT>(ngt | (neq << 16), scratch, &tot);
      int gt_b = gt_run + (pre & 0xffff);
      int eq_b = eq_run + (pre >> 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = f4(v[j], e);
        if (t + e >= hi) continue;
        const bool gt = x > sp, eq = x == sp;
        const bool sel = gt || (eq && eq_b < te);
        const int pos = base + gt_b + min(eq_b, te);
        if (sel && pos < k) orow[pos] = t + e;
        gt_b += gt;
        eq_b += eq;
      }
      gt_run += tot & 0xffff;
      eq_run += tot >> 16;
    }
  }
}

// ------------------------------------------------------------------ short rows
// A few rows of at most kSmallMax tokens: one workgroup per row, each thread
// holding 16 consecutive scores of the row in registers for the whole
// selection. The same steps as the multi-kernel path: histogram of the
// shifted bins, boundary bin b*, radix rounds on the exact order keys of the
// b* tokens (listed in LDS and selected by one wave when there are at most
// kSmallCand of them, else block-wide over the registers, so b* may be any
// width), then the selection written in token order by one ordered pass.
constexpr int kSmallNT = 1024;
constexpr int kSmallPer = 16;
constexpr int kSmallMax = kSmallNT * kSmallPer;   // 16384 tokens
constexpr int kSmallCand = 4096;                  // boundary tokens listed for the radix rounds

// LDS of a 1024-thread selection workgroup (short rows and the one-pass path).
struct SelLds {
  int2 cand[kSmallCand + 64];   // (score bits, token): boundary tokens, or a chunk's list being
                                // staged (+ a junk entry per lane)
  int hist[256 + 64];           // + a junk word per lane
  int sh[kSmallNT / 64];
  int s_digit, s_need, s_nc, s_last;
  uint32_t s_prefix;
  float s_min;
};

// The whole selection of one row of at most kSmallMax tokens by one
// workgroup of kSmallNT threads: idx (k entries, -1 padded), kth and the EMA
// update of theta (theta_out may be null).
__device__ void small_row(const float* __restrict__ row, int len, int k, float th_in, float* kth_out,
                          float* theta_out, int32_t* __restrict__ orow, SelLds& L) {
  constexpr int NT = kSmallNT;
  const int tid = threadIdx.x;
  for (int j = min(k, len) + tid; j < k; j += NT) orow[j] = -1;
  if (len == 0) {
    if (tid == 0) {
      *kth_out = __builtin_nanf("");
      if (theta_out) *theta_out = th_in;
    }
    return;
  }
  // tokens t0 .. t0+15 of this thread (16-byte aligned rows: ld % 4 == 0)
  const int t0 = kSmallPer * tid;
  float v[kSmallPer];
  if (t0 + kSmallPer <= len) {
#pragma unroll
    for (int q = 0; q < kSmallPer / 4; ++q) {
      const float4 x = reinterpret_cast<const float4*>(row + t0)[q];
      v[4 * q] = x.x;
      v[4 * q + 1] = x.y;
      v[4 * q + 2] = x.z;
      v[4 * q + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < kSmallPer; ++e) v[e] = t0 + e < len ? row[t0 + e] : 0.f;
  }
  uint32_t valid = 0;   // bit e: token t0 + e is in the row
#pragma unroll
  for (int e = 0; e < kSmallPer; ++e) valid |= (t0 + e < len) ? 1u << e : 0u;
  float sstar;
  int need_eq = 0;
  if (len <= k) {
    // every token is selected; kth is the row minimum
    float m = __builtin_inff();
#pragma unroll
    for (int e = 0; e < kSmallPer; ++e)
      if ((valid >> e) & 1u) m = fminf(m, v[e]);
    for (int d = 32; d > 0; d >>= 1) m = fminf(m, __shfl_xor(m, d, 64));
    float* wmin = reinterpret_cast<float*>(L.hist);
    if (ech::lane_id() == 0) wmin[tid / 64] = m;
#pragma unroll
    for (int e = 0; e < kSmallPer; ++e)
      if ((valid >> e) & 1u) orow[t0 + e] = t0 + e;
    __syncthreads();
    if (tid == 0) {
      float mm = __builtin_inff();
      for (int i = 0; i < NT / 64; ++i) mm = fminf(mm, wmin[i]);
      L.s_min = mm;
    }
    __syncthreads();
    sstar = L.s_min;
  } else {
    // 1. histogram of the shifted bins (lumped tokens counted per wave); the
    // thread keeps its bins
    const Shift shf = make_shift(th_in);
    if (tid < 256) L.hist[tid] = 0;
    if (tid == 0) L.s_nc = 0;
    __syncthreads();
    uint32_t bins[kSmallPer];
    int lumped = 0;
#pragma unroll
    for (int e = 0; e < kSmallPer; ++e) {
      bins[e] = shifted_bin(v[e], shf);
      const bool ok = (valid >> e) & 1u;
      const bool lump = ok && shf.on && bins[e] == 0u;
      lumped += lump;
      ech::lds_hist_add(L.hist, bins[e], ok && !lump);
    }
    lumped = ech::wave_sum(lumped);
    if (ech::lane_id() == 0 && lumped) atomicAdd(&L.hist[0], lumped);
    __syncthreads();
    // 2. boundary bin and the rank of the k-th token within it
    pick_digit(L.hist, L.sh, k, &L.s_digit, &L.s_need);
    const uint32_t bstar = (uint32_t)L.s_digit;
    int need = L.s_need;
    // list the boundary tokens (one LDS atomic per wave)
    uint32_t bm = 0;
#pragma unroll
    for (int e = 0; e < kSmallPer; ++e) bm |= (((valid >> e) & 1u) && bins[e] == bstar) ? 1u << e : 0u;
    const int cnt = __popc(bm);
    const int incl = ech::wave_incl_scan(cnt);
    int wbase = 0;
    if (ech::lane_id() == 63 && incl > 0) wbase = atomicAdd(&L.s_nc, incl);
    wbase = __shfl(wbase, 63, 64);
    int p = wbase + incl - cnt;
#pragma unroll
    for (int e = 0; e < kSmallPer; ++e) {
      if ((bm >> e) & 1u) {
        if (p < kSmallCand) L.cand[p] = make_int2(__float_as_int(v[e]), t0 + e);
        ++p;
      }
    }
    __syncthreads();
    const int nc = L.s_nc;
    // 3. the need-th largest boundary score: one wave over the list, or
    // block-wide rounds over the registers when the bin is wider than it
    uint32_t prefix = 0;
    if (nc <= kSmallCand) {   // block-uniform
      if (tid < 64) {
        int nq;
        const uint32_t pf = wave_select(L.cand, nc, need, L.hist, &nq);
        if (tid == 0) {
          L.s_prefix = pf;
          L.s_need = nq;
        }
      }
      __syncthreads();
      prefix = L.s_prefix;
      need = L.s_need;
    } else {
      uint32_t mask = 0;
#pragma unroll 1
      for (int round = 0; round < 4; ++round) {
        const int shift = 24 - 8 * round;
        if (tid < 256) L.hist[tid] = 0;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < kSmallPer; ++e) {
          const uint32_t key = ech::ord_key(v[e]);
          ech::lds_hist_add(L.hist, (key >> shift) & 255u, ((bm >> e) & 1u) && (key & mask) == prefix);
        }
        __syncthreads();
        pick_digit(L.hist, L.sh, need, &L.s_digit, &L.s_need);
        prefix |= (uint32_t)L.s_digit << shift;
        mask |= 255u << shift;
        need = L.s_need;
        __syncthreads();
      }
    }
    sstar = ech::ord_to_float(prefix);
    need_eq = need;
    // 4. the selection in token order: every score above s*, and the first
    // need_eq equal to it
    uint32_t gtm = 0, eqm = 0;
#pragma unroll
    for (int e = 0; e < kSmallPer; ++e) {
      const bool ok = (valid >> e) & 1u;
      gtm |= (ok && v[e] > sstar) ? 1u << e : 0u;
      eqm |= (ok && v[e] == sstar) ? 1u << e : 0u;
    }
    int tot;
    const int pre = ech::block_excl_scan<NT>(__popc(gtm) | (__popc(eqm) << 16), L.sh, &tot);
    int gt_b = pre & 0xffff, eq_b = pre >> 16;
#pragma unroll
    for (int e = 0; e < kSmallPer; ++e) {
      const bool gt = (gtm >> e) & 1u, eq = (eqm >> e) & 1u;
      const int pos = gt_b + min(eq_b, need_eq);
      if ((gt || (eq && eq_b < need_eq)) && pos < k) orow[pos] = t0 + e;
      gt_b += gt;
      eq_b += eq;
    }
  }
  if (tid == 0) {
    *kth_out = sstar;
    if (theta_out) *theta_out = (th_in == th_in) ? (sstar + th_in) * 0.5f : sstar;
  }
}

__global__ __launch_bounds__(kSmallNT) void topk_small_kernel(const float* __restrict__ logits, int64_t ld,
                                                              const int32_t* __restrict__ lens, int k,
                                                              const float* theta_in, float* theta_out,
                                                              float* __restrict__ kth, int32_t* __restrict__ idx) {
  __shared__ SelLds L;
  const int r = blockIdx.x;
  small_row(logits + (size_t)r * ld, min(lens[r], kSmallMax), k, row_theta(theta_in, r), kth + r,
            theta_out ? theta_out + r : nullptr, idx + (size_t)r * k, L);
}

// ------------------------------------------------------------------ few long rows: one pass
// grid (chunks of kOneChunk tokens, R), kSmallNT threads, after a one-block
// reset of the row counters and histograms. Each workgroup reads its chunk
// once (16 scores per thread in registers) and
//   - adds its histogram of shifted bins to the row's histogram (global
//     atomics, only the bins it holds),
//   - lists, in token order, its tokens in the bins at and above a floor
//     into its slice of the row's pool (the pool split evenly over the row's
//     chunks, at most kSmallCand entries each): the floor is the bin of
//     theta - |theta|/8 (the band the prediction implies), raised where
//     needed so that the chunk's tokens fit its slice,
//   - counts itself done. The last workgroup of the row to finish takes b*
//     from the row histogram. If b* is at or above every chunk's floor (every
//     bin from b* up is listed), the selection comes from the lists alone:
//     radix rounds on the b* entries give s* and need_eq, and one ordered
//     pass over the lists writes the selection. Otherwise (a floor above b*)
//     the same workgroup selects over the whole row: radix rounds restricted
//     to b*, then an ordered pass.
// The decode prediction moves by a few percent of the k-th score per step
// (the EMA of the explainer's "Decode: fetch above a predicted threshold"),
// so the band holds b* and each score is read once. Rows of a ragged call
// no longer than kSmallMax are selected whole by their first workgroup.
constexpr int kOneChunk = kSmallNT * kSmallPer;                  // 16384 tokens per workgroup
constexpr int kOneMaxChunks = kMaxChunks * kChunk / kOneChunk;   // 256 (4M tokens)
constexpr int kOneMaxRows = 256;
constexpr int kPool = 32768;         // listed entries per row, at most

struct OneWs {
  int* ctl;      // [R] * 32: per row, one 128-byte line: [0] chunks done
  int* hist;     // [R][256] row histograms
  int2* meta;    // [R][nch] per chunk: entries listed, floor
  int2* pool;    // [R][npool] (score bits, token): chunk c's slice at c * slice
  int nch;       // chunks of the longest row
  int npool;     // entries per row
};

// Pool entries per row for rows of at most nch chunks.
int one_pool(int nch) { return std::min(kPool, nch * kSmallCand); }

size_t one_layout(int R, int max_len, OneWs* w, char* base) {
  const int nch = std::max(1, (max_len + kOneChunk - 1) / kOneChunk);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  size_t o_ctl = take(sizeof(int) * 32 * (size_t)R);
  size_t o_hist = take(sizeof(int) * 256 * (size_t)R);
  size_t o_meta = take(sizeof(int2) * (size_t)R * nch);
  size_t o_pool = take(sizeof(int2) * (size_t)R * one_pool(nch));
  if (w && base) {
    w->ctl = reinterpret_cast<int*>(base + o_ctl);
    w->hist = reinterpret_cast<int*>(base + o_hist);
    w->meta = reinterpret_cast<int2*>(base + o_meta);
    w->pool = reinterpret_cast<int2*>(base + o_pool);
    w->nch = nch;
    w->npool = one_pool(nch);
  }
  return o;
}

// Wait until this wave's global stores and atomics have completed.
__device__ __forceinline__ void wait_vm_zero() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// What a chunk workgroup hands to the last one goes through device-coherent
// (agent-scope) stores, loads and atomics: once a wave's stores have
// completed they are visible to such loads on every XCD, so the hand-over
// needs no cache write-back or invalidation, only the wait before the count.
__device__ __forceinline__ void st_agent(int2* p, int2 v) {
  const uint64_t u = (uint64_t)(uint32_t)v.x | ((uint64_t)(uint32_t)v.y << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int2 ld_agent(const int2* p) {
  const uint64_t u = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return make_int2((int)(uint32_t)u, (int)(uint32_t)(u >> 32));
}
__device__ __forceinline__ int ld_agent(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Inclusive scan over a wave through DPP row shifts (within rows of 16
// lanes) and row broadcasts (rows 1, 3 take row 0, 2's total; rows 2, 3 take
// lane 31's): a few cycles per step where a lane shuffle is an LDS round
// trip. Every lane of the wave must be active.
__device__ __forceinline__ int wave_scan_dpp(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return v;
}

__device__ __forceinline__ int wave_sum_dpp(int v) { return __builtin_amdgcn_readlane(wave_scan_dpp(v), 63); }

// Exclusive scan over a workgroup of NT threads (all active) with the DPP
// wave scan; the total goes to *total.
template <int NT>
__device__ __forceinline__ int block_scan_dpp(int v, int* scratch, int* total) {
  constexpr int NW = NT / 64;
  const int lane = ech::lane_id(), wave = threadIdx.x / 64;
  const int incl = wave_scan_dpp(v);
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  int wbase = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int x = scratch[i];
    wbase += i < wave ? x : 0;
    tot += x;
  }
  __syncthreads();
  *total = tot;
  return wbase + incl - v;
}

__global__ __launch_bounds__(256) void topk_one_reset_kernel(OneWs ws) {
  const int r = blockIdx.x;
  ws.hist[(size_t)r * 256 + threadIdx.x] = 0;
  if (threadIdx.x < 32) ws.ctl[32 * r + threadIdx.x] = 0;
}

// Ordered pass over a whole row by one workgroup: every score above s* and
// the first need_eq equal to it, in token order. Thread tid takes 16
// consecutive tokens of each 16384-token block, so one block scan orders them.
__device__ void row_compact(const float* __restrict__ row, int len, float sstar, int need_eq, int k,
                            int32_t* __restrict__ orow, int* sh) {
  constexpr int NT = kSmallNT;
  int gt_run = 0, eq_run = 0;
  for (int b0 = 0; b0 < len; b0 += kOneChunk) {
    const int t0 = b0 + kSmallPer * (int)threadIdx.x;
    float v[kSmallPer];
    if (t0 + kSmallPer <= len) {
#pragma unroll
      for (int q = 0; q < kSmallPer / 4; ++q) {
        const float4 x = reinterpret_cast<const float4*>(row + t0)[q];
        v[4 * q] = x.x;
        v[4 * q + 1] = x.y;
        v[4 * q + 2] = x.z;
        v[4 * q + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int e = 0; e < kSmallPer; ++e) v[e] = t0 + e < len ? row[t0 + e] : 0.f;
    }
    uint32_t gtm = 0, eqm = 0;
#pragma unroll
    for (int e = 0; e < kSmallPer; ++e) {
      const bool ok = t0 + e < len;
      gtm |= (ok && v[e] > sstar) ? 1u << e : 0u;
      eqm |= (ok && v[e] == sstar) ? 1u << e : 0u;
    }
    int tot;
    const int pre = ech::block_excl_scan<NT>(__popc(gtm) | (__popc(eqm) << 16), sh, &tot);
    int gt_b = gt_run + (pre & 0xffff), eq_b = eq_run + (pre >> 16);
#pragma unroll
    for (int e = 0; e < kSmallPer; ++e) {
      const bool gt = (gtm >> e) & 1u, eq = (eqm >> e) & 1u;
      const int pos = gt_b + min(eq_b, need_eq);
      if ((gt || (eq && eq_b < need_eq)) && pos < k) orow[pos] = t0 + e;
      gt_b += gt;
      eq_b += eq;
    }
    gt_run += tot & 0xffff;
    eq_run += tot >> 16;
  }
}

// A row's chunk lists: chunk c's n_out entries (score bits, token) start at
// pool[c * slice], entry i of the concatenation is in chunk a with
// off[a] <= i < off[a + 1] (off in LDS, nch + 1 entries).
struct ListView {
  const int2* pool;
  const int* off;
  int nch, slice, nlist;
  bool coherent;   // written by workgroups of this launch: device-coherent loads
  // Entries ib .. ib + 7 (token -1 past the end).
  __device__ __forceinline__ void load8(int ib, int2 (&e)[8]) const {
    int a = 0, b = nch;   // off[a] <= ib < off[b]
    if (ib < nlist) {
      while (b - a > 1) {
        const int mid = (a + b) >> 1;
        if (off[mid] <= ib) a = mid;
        else b = mid;
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = ib + u;
      if (i < nlist) {
        while (off[a + 1] <= i) ++a;
        const int2* p = &pool[a * slice + (i - off[a])];
        e[u] = coherent ? ld_agent(p) : *p;
      } else {
        e[u] = make_int2(0, -1);
      }
    }
  }
};

// The selection of one row once its boundary bin b* and need (the rank of s*
// among the b* tokens) are known, by a whole workgroup of kSmallNT threads:
// from the lists when `lists` (every token of the row in b* and above is
// listed; `first` holds list entries 8 tid .. 8 tid + 7), else from the whole
// row (radix rounds restricted to b*, then an ordered pass). Writes the
// row's indices, kth and the EMA update of theta.
__device__ void select_bstar(bool lists, uint32_t bstar, int need, int nb, const float* __restrict__ row, int len,
                             int k, const Shift& shf, float th_in, const ListView& lv, const int2 (&first)[8],
                             int32_t* __restrict__ orow, float* kth_r, float* theta_out_r, SelLds& L) {
  constexpr int NT = kSmallNT;
  const int tid = threadIdx.x;
  const int nlist = lv.nlist;
  auto load8 = [&](int ib, int2 (&e)[8]) { lv.load8(ib, e); };
  float sstar;
  int need_eq;
  if (lists) {
    uint32_t prefix = 0;
    if (nb <= kSmallCand) {   // the b* entries into LDS
      if (tid == 0) L.s_nc = 0;
      __syncthreads();
      for (int i0 = 0; i0 < nlist; i0 += 8 * NT) {
        int2 e[8];
        if (i0 == 0) {
#pragma unroll
          for (int u = 0; u < 8; ++u) e[u] = first[u];
        } else {
          load8(i0 + 8 * tid, e);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          if (e[u].y >= 0 && shifted_bin_one(__int_as_float(e[u].x), shf) == bstar) {
            const int p = atomicAdd(&L.s_nc, 1);
            if (p < kSmallCand) L.cand[p] = e[u];   // the histogram bounds them by nb; guard only
          }
        }
      }
      __syncthreads();
      const int nc = min(L.s_nc, kSmallCand);
      if (tid < 64) {
        uint32_t pf;
        int nq;
        if (nc <= 64) {
          // A few: lane l takes entry l and counts the keys above and at or
          // above its own; the lane where the count from the top reaches
          // need holds s*.
          const uint32_t key = tid < nc ? ech::ord_key(__int_as_float(L.cand[tid].x)) : 0u;
          int gt = 0, ge = 0;
          for (int j = 0; j < nc; ++j) {
            const uint32_t kj = __builtin_amdgcn_readlane(key, j);
            gt += kj > key;
            ge += kj >= key;
          }
          const uint64_t hit = __ballot(tid < nc && gt < need && need <= ge);
          const int src = __ffsll((unsigned long long)hit) - 1;
          pf = __shfl(key, src, 64);
          nq = need - __shfl(gt, src, 64);
        } else {
          pf = wave_select(L.cand, nc, need, L.hist, &nq);
        }
        if (tid == 0) {
          L.s_prefix = pf;
          L.s_need = nq;
        }
      }
      __syncthreads();
      prefix = L.s_prefix;
      need = L.s_need;
    } else {   // a wide b*: block-wide rounds over the lists
      uint32_t mask = 0;
#pragma unroll 1
      for (int round = 0; round < 4; ++round) {
        const int shift = 24 - 8 * round;
        if (tid < 256) L.hist[tid] = 0;
        __syncthreads();
        for (int i0 = 0; i0 < nlist; i0 += 8 * NT) {
          int2 e[8];
          load8(i0 + 8 * tid, e);
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const float x = __int_as_float(e[u].x);
            const uint32_t key = ech::ord_key(x);
            ech::lds_hist_add(L.hist, (key >> shift) & 255u,
                              e[u].y >= 0 && shifted_bin_one(x, shf) == bstar && (key & mask) == prefix);
          }
        }
        __syncthreads();
        pick_digit(L.hist, L.sh, need, &L.s_digit, &L.s_need);
        prefix |= (uint32_t)L.s_digit << shift;
        mask |= 255u << shift;
        need = L.s_need;
        __syncthreads();
      }
    }
    sstar = ech::ord_to_float(prefix);
    need_eq = need;
    // The selection in token order by one ordered pass over the lists: listed
    // entries above b* score above s*, those below b* under it.
    int gt_run = 0, eq_run = 0;
    for (int i0 = 0; i0 < nlist; i0 += 8 * NT) {
      int2 e[8];
      if (i0 == 0) {
#pragma unroll
        for (int u = 0; u < 8; ++u) e[u] = first[u];
      } else {
        load8(i0 + 8 * tid, e);
      }
      uint32_t gtm = 0, eqm = 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (e[u].y < 0) continue;
        const float x = __int_as_float(e[u].x);
        gtm |= x > sstar ? 1u << u : 0u;
        eqm |= x == sstar ? 1u << u : 0u;
      }
      int tot;
      const int pre = block_scan_dpp<NT>(__popc(gtm) | (__popc(eqm) << 16), L.sh, &tot);
      int gt_b = gt_run + (pre & 0xffff), eq_b = eq_run + (pre >> 16);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const bool gt = (gtm >> u) & 1u, eq = (eqm >> u) & 1u;
        const int pos = gt_b + min(eq_b, need_eq);
        if ((gt || (eq && eq_b < need_eq)) && pos < k) orow[pos] = e[u].y;
        gt_b += gt;
        eq_b += eq;
      }
      gt_run += tot & 0xffff;
      eq_run += tot >> 16;
    }
  } else {
    // The lists miss b*: radix rounds over the row's b* tokens, then an
    // ordered pass over the row.
    uint32_t prefix = 0, mask = 0;
#pragma unroll 1
    for (int round = 0; round < 4; ++round) {
      const int shift = 24 - 8 * round;
      if (tid < 256) L.hist[tid] = 0;
      __syncthreads();
      for_each_score<NT>(row, len, [&](int, float x) {
        const uint32_t key = ech::ord_key(x);
        ech::lds_hist_add(L.hist, (key >> shift) & 255u,
                          shifted_bin_one(x, shf) == bstar && (key & mask) == prefix);
      });
      __syncthreads();
      pick_digit(L.hist, L.sh, need, &L.s_digit, &L.s_need);
      prefix |= (uint32_t)L.s_digit << shift;
      mask |= 255u << shift;
      need = L.s_need;
      __syncthreads();
    }
    sstar = ech::ord_to_float(prefix);
    need_eq = need;
    row_compact(row, len, sstar, need_eq, k, orow, L.sh);
  }
  if (tid == 0) {
    *kth_r = sstar;
    if (theta_out_r) *theta_out_r = (th_in == th_in) ? (sstar + th_in) * 0.5f : sstar;
  }
}


__global__ __launch_bounds__(kSmallNT) void topk_one_kernel(const float* __restrict__ logits, int64_t ld,
                                                            const int32_t* __restrict__ lens, int max_len, int k,
                                                            const float* theta_in, float* theta_out,
                                                            float* __restrict__ kth, int32_t* __restrict__ idx,
                                                            OneWs ws) {
  constexpr int NT = kSmallNT;
  __shared__ SelLds L;
  __shared__ int s_off[kOneMaxChunks + 1];   // the last workgroup: chunk c's entries start at s_off[c]
  __shared__ int s_fmax;
  const int r = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
  const int len = min(lens[r], max_len);   // the grid and workspace are sized by max_len
  const float th_in = row_theta(theta_in, r);
  const float* row = logits + (size_t)r * ld;
  int32_t* orow = idx + (size_t)r * k;
  if (len <= kSmallMax) {
    if (c == 0) small_row(row, len, k, th_in, kth + r, theta_out ? theta_out + r : nullptr, orow, L);
    return;
  }
  const int nch = (len + kOneChunk - 1) / kOneChunk;
  if (c >= nch) return;
  const Shift shf = make_shift(th_in);
  int* ctl = ws.ctl + 32 * r;
  int2* pool = ws.pool + (size_t)r * ws.npool;
  const int slice = min(kSmallCand, ws.npool / nch);   // this row's entries per chunk

  // ---- the chunk: histogram, floor, listed tokens
  // Thread tid holds the 16 consecutive tokens from t0, so one scan of the
  // per-thread counts orders the list. The per-token work is branch-free
  // (the pass is bound by instruction issue, not by the read): lumped and
  // absent tokens add to a junk word of their lane, unlisted ones stage into
  // a junk entry of their lane.
  const int lane = ech::lane_id();
  const int lo = c * kOneChunk, hi = min(lo + kOneChunk, len);
  const int t0 = lo + kSmallPer * tid;
  const int nv = min(kSmallPer, max(0, hi - t0));   // this thread's tokens in the row
  float v[kSmallPer];
  if (nv == kSmallPer) {
#pragma unroll
    for (int q = 0; q < kSmallPer / 4; ++q) {
      typedef float f4v __attribute__((ext_vector_type(4)));
      const f4v x = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(row + t0) + q);
      v[4 * q] = x.x;
      v[4 * q + 1] = x.y;
      v[4 * q + 2] = x.z;
      v[4 * q + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < kSmallPer; ++e) v[e] = e < nv ? row[t0 + e] : 0.f;
  }
  const uint32_t blo = band_lo(shf);
  if (tid < 256) L.hist[tid] = 0;
  __syncthreads();
  uint32_t in = 0;   // bit e: token t0 + e is listed
  int lumped = 0;
#pragma unroll
  for (int e = 0; e < kSmallPer; ++e) {
    const bool ok = e < nv;
    const float d = shf.on ? v[e] - shf.th : v[e];
    const bool lump = d < shf.cut;
    const uint32_t b = bin_one(d);
    atomicAdd(&L.hist[(ok && !lump) ? b : 256 + lane], 1);
    lumped += (ok && lump) ? 1 : 0;
    in |= (ok && !lump && b >= blo) ? 1u << e : 0u;
  }
  lumped = wave_sum_dpp(lumped);
  if (lane == 0 && lumped) atomicAdd(&L.hist[0], lumped);
  int total;
  int pre = block_scan_dpp<NT>(__popc(in), L.sh, &total);   // its barriers also close the histogram
  uint32_t floor_c = blo;
  if (total > slice) {   // the band does not fit the slice (block-uniform): raise the floor
    // to the lowest bin whose count from the top fits (threads 0..255 take bins 255..0)
    const int hb = tid < 256 ? L.hist[255 - tid] : 0;
    int hall;
    const int hex = block_scan_dpp<NT>(hb, L.sh, &hall);
    const int fit = __syncthreads_count(tid < 256 && hex + hb <= slice);
    floor_c = max(blo, 256u - (uint32_t)fit);
    in = 0;
#pragma unroll
    for (int e = 0; e < kSmallPer; ++e)
      in |= (e < nv && shifted_bin_one(v[e], shf) >= floor_c) ? 1u << e : 0u;
    pre = block_scan_dpp<NT>(__popc(in), L.sh, &total);
  }
  {
    int pos = pre;
#pragma unroll
    for (int e = 0; e < kSmallPer; ++e) {
      const bool listed = (in >> e) & 1u;
      L.cand[(listed && pos < slice) ? pos : kSmallCand + lane] = make_int2(__float_as_int(v[e]), t0 + e);
      pos += listed ? 1 : 0;
    }
  }
  __syncthreads();
  const int n_out = min(total, slice);   // the floor bounds total by slice; guard only
  for (int i = tid; i < n_out; i += NT) st_agent(&pool[c * slice + i], L.cand[i]);
  if (tid == 0) st_agent(&ws.meta[(size_t)r * ws.nch + c], make_int2(n_out, (int)floor_c));
  if (tid < 256) {
    const int hv = L.hist[tid];
    if (hv) atomicAdd(&ws.hist[(size_t)r * 256 + tid], hv);
  }
  // Publish: every wave's coherent stores and atomics complete, then the
  // count; the last workgroup reads with coherent loads.
  wait_vm_zero();
  __syncthreads();
  if (tid == 0)
    L.s_last = __hip_atomic_fetch_add(&ctl[0], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nch - 1;
  __syncthreads();
  if (!L.s_last) return;

  // ---- the last workgroup of the row: b* and the selection
  if (tid < 256) L.hist[tid] = ld_agent(&ws.hist[(size_t)r * 256 + tid]);
  const int2 m = tid < nch ? ld_agent(&ws.meta[(size_t)r * ws.nch + tid]) : make_int2(0, 0);
  if (tid == 0) s_fmax = 0;
  __syncthreads();
  pick_digit(L.hist, L.sh, k, &L.s_digit, &L.s_need);
  const uint32_t bstar = (uint32_t)L.s_digit;
  const int need = L.s_need;
  const int nb = L.hist[bstar];
  if (tid < nch) atomicMax(&s_fmax, m.y);
  int nlist;
  const int off = block_scan_dpp<NT>(m.x, L.sh, &nlist);
  if (tid < nch) s_off[tid] = off;
  if (tid == 0) s_off[nch] = nlist;
  __syncthreads();
  ListView lv{pool, s_off, nch, slice, nlist, true};
  int2 first[8];
  const bool lists = (uint32_t)s_fmax <= bstar;
  if (lists) lv.load8(8 * tid, first);
  select_bstar(lists, bstar, need, nb, row, len, k, shf, th_in, lv, first, orow, kth + r,
               theta_out ? theta_out + r : nullptr, L);
}

// ------------------------------------------------------------------ rows listed while scored
// grid (R), kSmallNT threads: the selection of rows whose band the scoring
// kernel listed as it scored them, in the one-pass layout with its scoring
// waves as the chunks. Every token of the row at or above the highest floor
// is listed, so the histogram of those entries is the row's histogram there:
// if they are at least k, b* is among them and the selection comes from the
// lists; otherwise (a NaN theta, an overflowing wave, or a band that holds
// fewer than k tokens) one pass over the row gives its whole histogram and
// the row path selects. Rows no longer than kSmallMax are selected whole.
__global__ __launch_bounds__(kSmallNT) void topk_lists_kernel(const float* __restrict__ logits, int64_t ld,
                                                              const int32_t* __restrict__ lens, int max_len, int k,
                                                              const float* theta_in, float* theta_out,
                                                              float* __restrict__ kth, int32_t* __restrict__ idx,
                                                              const int2* __restrict__ meta,
                                                              const int2* __restrict__ pool,
                                                              const float* __restrict__ list_theta, int cpr,
                                                              int slice, int chunk_tok) {
  constexpr int NT = kSmallNT;
  constexpr int kPerT = ech::kListMaxChunks / NT;   // chunks per thread
  __shared__ SelLds L;
  __shared__ int s_off[ech::kListMaxChunks + 1];
  __shared__ int s_fmax;
  const int r = blockIdx.x, tid = threadIdx.x;
  const int len = min(lens[r], max_len);
  const float th_in = row_theta(theta_in, r);
  const float* row = logits + (size_t)r * ld;
  int32_t* orow = idx + (size_t)r * k;
  if (len <= kSmallMax) {
    small_row(row, len, k, th_in, kth + r, theta_out ? theta_out + r : nullptr, orow, L);
    return;
  }
  const int nch = min((len + chunk_tok - 1) / chunk_tok, cpr);
  const Shift shf = make_shift(th_in);
  // lists made against another theta prove nothing here: the whole row then
  const bool same_theta = __float_as_uint(list_theta[r]) == __float_as_uint(th_in);
  // chunk offsets (thread tid sums chunks kPerT tid .. +kPerT) and the highest floor
  int cnt[kPerT];
  int mine = 0, fl = 0;
#pragma unroll
  for (int u = 0; u < kPerT; ++u) {
    const int c = kPerT * tid + u;
    const int2 m = c < nch ? (same_theta ? meta[(size_t)r * cpr + c] : make_int2(0, 256)) : make_int2(0, 0);
    cnt[u] = m.x;
    mine += m.x;
    fl = max(fl, m.y);
  }
  if (tid == 0) s_fmax = 0;
  if (tid < 256) L.hist[tid] = 0;
  __syncthreads();
  if (fl) atomicMax(&s_fmax, fl);
  int nlist;
  int off = block_scan_dpp<NT>(mine, L.sh, &nlist);
#pragma unroll
  for (int u = 0; u < kPerT; ++u) {
    const int c = kPerT * tid + u;
    if (c < nch) s_off[c] = off;
    off += cnt[u];
  }
  if (tid == 0) s_off[nch] = nlist;
  __syncthreads();
  const uint32_t fmax = (uint32_t)s_fmax;
  const ListView lv{pool + (size_t)r * cpr * slice, s_off, nch, slice, nlist, false};
  int2 first[8];
  lv.load8(8 * tid, first);
  int above = 0;
  for (int i0 = 0; i0 < nlist; i0 += 8 * NT) {
    int2 e[8];
    if (i0 == 0) {
#pragma unroll
      for (int u = 0; u < 8; ++u) e[u] = first[u];
    } else {
      lv.load8(i0 + 8 * tid, e);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t b = e[u].y >= 0 ? shifted_bin_one(__int_as_float(e[u].x), shf) : 0u;
      const bool at = e[u].y >= 0 && b >= fmax;
      ech::lds_hist_add(L.hist, b, at);
      above += at ? 1 : 0;
    }
  }
  int n_above;
  (void)block_scan_dpp<NT>(above, L.sh, &n_above);   // its barriers also close the histogram
  const bool lists = n_above >= k;
  if (!lists) {   // the row's whole histogram, by one pass over the row
    if (tid < 256) L.hist[tid] = 0;
    __syncthreads();
    for_each_score<NT>(row, len, [&](int, float x) { ech::lds_hist_add(L.hist, shifted_bin_one(x, shf), true); });
    __syncthreads();
  }
  pick_digit(L.hist, L.sh, k, &L.s_digit, &L.s_need);
  const uint32_t bstar = (uint32_t)L.s_digit;
  const int need = L.s_need;
  const int nb = L.hist[bstar];
  select_bstar(lists, bstar, need, nb, row, len, k, shf, th_in, lv, first, orow, kth + r,
               theta_out ? theta_out + r : nullptr, L);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Which launches serve a call: a few short rows (one launch, no workspace
// use), a few long rows (the one-pass launch), or many rows (T1..T5).
enum class TopkPath { kSmall, kOne, kMany };

TopkPath topk_path(int R, int max_len) {
  if (R <= kOneMaxRows) return max_len <= kSmallMax ? TopkPath::kSmall : TopkPath::kOne;
  return TopkPath::kMany;
}

}  // namespace

extern "C" size_t ech_topk_ws_bytes(int R, int max_len, int k) {
  if (R < 1 || max_len < 0) return 0;
  if (k < 1 || k > kMaxK) return 0;
  if (topk_path(R, max_len) == TopkPath::kMany) return layout(R, max_len, k, nullptr, nullptr);
  return std::max<size_t>(256, one_layout(R, max_len, nullptr, nullptr));
}

namespace {

// Arguments of ech_topk other than the workspace.
bool topk_args_ok(const float* logits, int64_t ld, const int32_t* row_len, int R, int max_len, int k,
                  const int32_t* idx, const float* kth) {
  if (!logits || !row_len || !idx || !kth) return false;
  if (R < 1 || R > 65535 || k < 1 || k > kMaxK || max_len < 0 || ld < max_len) return false;
  if ((int64_t)max_len > (int64_t)kChunk * kMaxChunks) return false;
  return ld % 4 == 0 && aligned16(logits);
}

// The launches of one ech_topk call on a checked workspace.
int topk_launch(const float* logits, int64_t ld, const int32_t* row_len, int R, int max_len, int k,
                const float* theta_in, float* theta_out, int32_t* idx, float* kth, void* ws, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const TopkPath path = topk_path(R, max_len);
  if (path == TopkPath::kSmall) {
    hipLaunchKernelGGL(topk_small_kernel, dim3(R), dim3(kSmallNT), 0, s, logits, ld, row_len, k, theta_in,
                       theta_out, kth, idx);
    ECH_LAUNCH_CHECK();
    return ECH_OK;
  }
  if (path == TopkPath::kOne) {
    OneWs w;
    one_layout(R, max_len, &w, static_cast<char*>(ws));
    hipLaunchKernelGGL(topk_one_reset_kernel, dim3(R), dim3(256), 0, s, w);
    ECH_LAUNCH_CHECK();
    hipLaunchKernelGGL(topk_one_kernel, dim3(w.nch, R), dim3(kSmallNT), 0, s, logits, ld, row_len, max_len, k, theta_in,
                       theta_out, kth, idx, w);
    ECH_LAUNCH_CHECK();
    return ECH_OK;
  }
  // Many rows (a prefill block): 256-thread per-row kernels, so they fit
  // beside other work on a CU.
  Ws w;
  layout(R, max_len, k, &w, static_cast<char*>(ws));
  const dim3 gch(w.nch, R);
  hipLaunchKernelGGL(topk_hist_kernel, gch, dim3(kT), 0, s, logits, ld, row_len, k, theta_in, w);
  ECH_LAUNCH_CHECK();
  hipLaunchKernelGGL(topk_rowsel_many_kernel, dim3(R), dim3(256), 0, s, row_len, k, w);
  ECH_LAUNCH_CHECK();
  // refine rows with a lumped boundary in parallel over chunks
  hipLaunchKernelGGL(topk_refine_hist_kernel, gch, dim3(kT), 0, s, logits, ld, row_len, theta_in, w);
  ECH_LAUNCH_CHECK();
  hipLaunchKernelGGL(topk_refine_sel_kernel<256>, dim3(R), dim3(256), 0, s, row_len, theta_in, w);
  ECH_LAUNCH_CHECK();
  hipLaunchKernelGGL(topk_list_kernel, gch, dim3(kT), 0, s, logits, ld, row_len, theta_in, w);
  ECH_LAUNCH_CHECK();
  hipLaunchKernelGGL(topk_resolve_kernel<256>, dim3(R), dim3(256), sizeof(int2) * w.cap, s, logits, ld, row_len,
                     k, theta_in, theta_out, kth, idx, w);
  ECH_LAUNCH_CHECK();
  const int gx = std::max(1, std::min(w.nch, std::max(8, 256 / R)));
  hipLaunchKernelGGL(topk_compact_kernel, dim3(gx, R), dim3(kT), 0, s, logits, ld, row_len, k, idx, w);
  ECH_LAUNCH_CHECK();
  return ECH_OK;
}

}  // namespace

extern "C" int ech_topk(const float* logits, int64_t ld, const int32_t* row_len, int R, int max_len, int k,
                        const float* theta_in, float* theta_out, int32_t* idx, float* kth, void* ws,
                        size_t ws_bytes, void* stream) {
  if (!topk_args_ok(logits, ld, row_len, R, max_len, k, idx, kth)) return ECH_EINVAL;
  if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255u)) return ECH_EINVAL;
  if (ws_bytes < ech_topk_ws_bytes(R, max_len, k)) return ECH_EINVAL;
  return topk_launch(logits, ld, row_len, R, max_len, k, theta_in, theta_out, idx, kth, ws, stream);
}

// ------------------------------------------------------------------ no allocation
// The workspace of ech_topk_noalloc: a static device array, one per GPU the
// library runs on (held until the process ends). In host code `scratch`
// names a host-side stand-in, not the device address: the device address of
// each GPU's copy is looked up once per device (hipGetSymbolAddress, with
// that device current) and only that address is passed to kernels.
namespace {

constexpr size_t kScratchBytes = ECH_TOPK_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of the current device's scratch array; ECH_EHIP if the
// device or the symbol lookup fails.
int scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return ECH_EHIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return ECH_EHIP;
    }
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return ECH_OK;
}

}  // namespace

extern "C" int ech_topk_noalloc(const float* logits, int64_t ld, const int32_t* row_len, int R, int max_len, int k,
                                const float* theta_in, float* theta_out, int32_t* idx, float* kth, void* stream) {
  if (!topk_args_ok(logits, ld, row_len, R, max_len, k, idx, kth)) return ECH_EINVAL;
  if (ech_topk_ws_bytes(R, max_len, k) > kScratchBytes) return ECH_ESCRATCH;
  void* ws = nullptr;
  const int rc = scratch_of_current_device(&ws);
  if (rc != ECH_OK) return rc;
  return topk_launch(logits, ld, row_len, R, max_len, k, theta_in, theta_out, idx, kth, ws, stream);
}

int ech::topk_lists_launch(const float* logits, int64_t ld, const int32_t* row_len, int R, int max_len, int k,
                           const float* theta_in, float* theta_out, int32_t* idx, float* kth, const int2* meta,
                           const int2* pool, const float* list_theta, int cpr, int slice, int chunk_tok,
                           hipStream_t stream) {
  hipLaunchKernelGGL(topk_lists_kernel, dim3(R), dim3(kSmallNT), 0, stream, logits, ld, row_len, max_len, k,
                     theta_in, theta_out, kth, idx, meta, pool, list_theta, cpr, slice, chunk_tok);
  ECH_LAUNCH_CHECK();
  return ECH_OK;
}
